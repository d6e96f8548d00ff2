"""The C ABI without a GPU: libmhcb.so loads, exports every entry point that
include/*.h declares, and rejects bad arguments before touching the device
(no compute call is made here)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    for header in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(header).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(mhcb_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_symbols()
    for want in ("mhcb_boundary", "mhcb_boundary_glm", "mhcb_finalize", "mhcb_finalize_ex", "mhcb_mixes",
                 "mhcb_quant_mxfp8", "mhcb_mailbox_init", "mhcb_publish", "mhcb_last_error"):
        assert want in names


def test_library_exports_every_declared_symbol():
    import tp_reduce_mhc_amd as mhc
    lib = ctypes.CDLL(mhc.LIBRARY_PATH)
    for name in declared_symbols():
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"
    assert set(mhc.EXPORTED) == set(declared_symbols())


def test_host_only_helpers():
    import tp_reduce_mhc_amd as mhc
    assert mhc.mhcb_mxfp8_scale_bytes(8192, 5120) == 8192 * 160
    assert mhc.mhcb_mxfp8_scale_bytes(100, 5120) == 128 * 160
    assert mhc.mhcb_mxfp8_scale_bytes(1, 128) == 128 * 4
    base = mhc.mhcb_workspace_bytes(10, 512, 4, 0)   # sync state + 8 MiB scratch
    assert base > 8 << 20 and base % 256 == 0
    sync = base - (8 << 20)
    # The two-shot areas share the scratch: 8 MiB unless they need more.
    assert mhc.mhcb_workspace_bytes(10, 512, 4, 1) == base
    big = (8 * 8 * 512 + 4096) * 8192 * 2
    assert mhc.mhcb_workspace_bytes(4096, 8192, 8, 1) == sync + big
    assert mhc.mhcb_workspace_bytes(10, 512, 0, 1) == -1
    prev = mhc.mhcb_set_token_slices(4)
    assert mhc.mhcb_set_token_slices(prev) == 4
    assert mhc.mhcb_version().count(".") == 2
    for args in ((10, 512, 4, 0), (10, 512, 4, 1), (4096, 8192, 8, 1), (10, 512, 0, 1)):
        assert mhc.mhcb_finalize_workspace_bytes(*args) == mhc.mhcb_workspace_bytes(*args)


def test_token_slices_setting_is_per_thread():
    """mhcb_set_token_slices changes the calling thread's setting only."""
    import threading
    import tp_reduce_mhc_amd as mhc
    prev = mhc.mhcb_set_token_slices(7)
    seen = {}

    def other():
        seen["initial"] = mhc.mhcb_set_token_slices(3)
        seen["own"] = mhc.mhcb_set_token_slices(0)

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen == {"initial": 0, "own": 3}
    assert mhc.mhcb_set_token_slices(prev) == 7


def test_status_and_spin_limit_validation():
    """The status reads and the spin-limit setter validate before launching."""
    import tp_reduce_mhc_amd as mhc
    with pytest.raises(mhc.MhcbError, match="required"):
        mhc.mhcb_workspace_status(FAKE, None, 0)
    with pytest.raises(mhc.MhcbError, match="required"):
        mhc.mhcb_workspace_status(None, FAKE, 0)
    with pytest.raises(mhc.MhcbError, match="256-byte"):
        mhc.mhcb_workspace_status(FAKE + 16, FAKE, 0)
    with pytest.raises(mhc.MhcbError, match="required"):
        mhc.mhcb_workspace_set_spin_limit(None, 5, 0)
    mb = mhc.mhcb_mailbox(FAKE, FAKE, FAKE, 3, 2, 8, 512, 0)
    with pytest.raises(mhc.MhcbError, match="required"):
        mhc.mhcb_mailbox_status(mb, None, 0)
    with pytest.raises(mhc.MhcbError, match="aligned"):
        mhc.mhcb_mailbox_status(mb, FAKE + 2, 0)


FAKE = 0x10000  # an aligned non-null address; validation fails before any use of it


def _boundary(**kw):
    import tp_reduce_mhc_amd as mhc
    args = dict(partials=FAKE, rank_stride=4 * 512, mailbox=None, residual=FAKE, post=FAKE,
                comb=FAKE, pre=FAKE, norm_weight=FAKE, residual_out=FAKE, layer_input=FAKE,
                mxfp8_values=None, mxfp8_scales=None, workspace=None, workspace_bytes=0, M=4,
                hidden_size=512, hc_mult=4, tp=2, norm_eps=1e-6, stream=0)
    args.update(kw)
    return mhc.mhcb_boundary(**args)


@pytest.mark.parametrize("kw,code,text", [
    (dict(M=0), 1, "M=0"),
    (dict(hc_mult=3), 3, "hc_mult"),
    (dict(hc_mult=16), 3, "1, 2, 4 or 8"),
    (dict(hidden_size=100), 3, "multiple of 8"),
    (dict(hidden_size=32768, rank_stride=4 * 32768), 3, "exceeds"),
    (dict(tp=0), 1, "tp=0"),
    (dict(tp=65), 1, "tp=65"),
    (dict(pre=None), 1, "pre and norm_weight"),
    (dict(mxfp8_values=FAKE), 1, "both given"),
    (dict(pre=None, norm_weight=None, layer_input=None, mxfp8_values=FAKE, mxfp8_scales=FAKE), 1,
     "residual-only"),
    (dict(mxfp8_values=FAKE, mxfp8_scales=FAKE, hidden_size=520, rank_stride=4 * 520), 3, "% 128"),
    (dict(residual=FAKE + 2), 2, "aligned"),
    (dict(partials=None), 1, "exactly one"),
    (dict(rank_stride=100), 1, "overlaps"),
    (dict(rank_stride=4 * 512 + 4), 2, "rank_stride"),
    (dict(residual_out=None), 1, "required"),
    (dict(workspace=FAKE, workspace_bytes=100), 1, "workspace_bytes"),
    (dict(workspace=FAKE + 16, workspace_bytes=1 << 23), 2, "256-byte"),
])
def test_boundary_validation(kw, code, text):
    import tp_reduce_mhc_amd as mhc
    with pytest.raises(mhc.MhcbError) as e:
        _boundary(**kw)
    assert e.value.code == code
    assert text in str(e.value)


def test_mailbox_validation():
    import tp_reduce_mhc_amd as mhc
    mb = mhc.mhcb_mailbox(FAKE, FAKE, FAKE, 3, 2, 8, 512, 0)
    with pytest.raises(mhc.MhcbError, match="outside"):
        _boundary(partials=None, mailbox=mb, M=9)
    with pytest.raises(mhc.MhcbError, match="tp=2 but tp=4"):
        _boundary(partials=None, mailbox=mb, tp=4)
    bad = mhc.mhcb_mailbox(FAKE, FAKE, FAKE, 2, 2, 8, 512, 0)
    with pytest.raises(mhc.MhcbError, match="generations"):
        _boundary(partials=None, mailbox=bad)
    with pytest.raises(mhc.MhcbError, match="exactly one"):
        _boundary(mailbox=mb)
    with pytest.raises(mhc.MhcbError, match="ranks"):
        mhc.mhcb_publish(mb, FAKE, 4 * 512, 1, 2, 4, 0)
    with pytest.raises(mhc.MhcbError, match="M=0"):
        mhc.mhcb_publish(mb, FAKE, 4 * 512, 0, 2, 0, 0)


def test_glm_mixes_finalize_quant_validation():
    import tp_reduce_mhc_amd as mhc
    glm = dict(partials=FAKE, rank_stride=4 * 512, residual=FAKE, post=FAKE, comb=FAKE, hc_fn=FAKE,
               scale=FAKE, base=FAKE, norm_weight=FAKE, residual_out=FAKE, mixes_out=FAKE,
               layer_input=FAKE, workspace=None, workspace_bytes=0, M=4, hidden_size=512, hc_mult=4,
               tp=2, rms_eps=1e-6, hc_eps=1e-6, norm_eps=1e-6, stream=0)
    for kw, text in ((dict(tokens_per_wg=3), "tokens_per_wg"), (dict(hc_fn=None), "required"),
                     (dict(tokens_per_wg=16), "needs a workspace"),
                     (dict(tokens_per_wg=-16), "needs a workspace"),
                     (dict(tokens_per_wg=-16, workspace=FAKE, workspace_bytes=1 << 23),
                      "needs a workspace"),
                     (dict(hidden_size=8200, rank_stride=4 * 8200), "exceeds"),
                     (dict(tokens_per_wg=4, hidden_size=8192, rank_stride=4 * 8192), "tokens_per_wg=4")):
        with pytest.raises(mhc.MhcbError, match=text):
            mhc.mhcb_boundary_glm(**{**glm, **kw})
    with pytest.raises(mhc.MhcbError, match="sinkhorn_repeat"):
        mhc.mhcb_mixes(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 1e-6, 2.0, -1, 0)
    with pytest.raises(mhc.MhcbError, match="hc_mult"):
        mhc.mhcb_mixes(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 3, 1e-6, 2.0, 20, 0)
    with pytest.raises(mhc.MhcbError, match="only 4"):
        mhc.mhcb_boundary_glm(**{**glm, "hc_mult": 2})
    fin = dict(gemm2_permuted=FAKE, gemm2_rank_stride=32 * 512, rows=32, expert_weights=FAKE,
               weights_rank_stride=0, permuted_idx=FAKE, idx_rank_stride=0, shared_output=FAKE,
               shared_rank_stride=4 * 512, residual=FAKE, post=FAKE, comb=FAKE, pre=FAKE,
               norm_weight=FAKE, residual_out=FAKE, layer_input=FAKE, mxfp8_values=None,
               mxfp8_scales=None, two_shot=0, workspace=None, workspace_bytes=0, M=4,
               hidden_size=512, hc_mult=4, tp=2, top_k=8, norm_eps=1e-6, stream=0)
    for kw, text in ((dict(top_k=0), "top_k"), (dict(tp=64, top_k=32), "exceeds"),
                     (dict(two_shot=1), "workspace"), (dict(rows=-1), "rows"),
                     (dict(two_shot=1, workspace=FAKE + 8, workspace_bytes=1 << 24), "aligned"),
                     (dict(two_shot=1, workspace=FAKE, workspace_bytes=1 << 10), "workspace_bytes")):
        with pytest.raises(mhc.MhcbError, match=text):
            mhc.mhcb_finalize(**{**fin, **kw})
    fglm = dict(gemm2_permuted=FAKE, gemm2_rank_stride=32 * 512, rows=32, expert_weights=FAKE,
                weights_rank_stride=0, weights_bf16=0, routed_scaling_factor=1.0,
                permuted_idx=FAKE, idx_rank_stride=0, shared_output=FAKE,
                shared_rank_stride=4 * 512, residual=FAKE, post=FAKE, comb=FAKE, hc_fn=FAKE,
                scale=FAKE, base=FAKE, norm_weight=FAKE, residual_out=FAKE, mixes_out=FAKE,
                layer_input=FAKE, workspace=FAKE, workspace_bytes=1 << 30, M=4, hidden_size=512,
                hc_mult=4, tp=2, top_k=8, rms_eps=1e-6, hc_eps=1e-6, norm_eps=1e-6, stream=0)
    need = mhc.mhcb_finalize_glm_workspace_bytes(4, 512, 2)
    assert need == mhc.mhcb_workspace_bytes(4, 512, 2, 0) + 2 * 4 * 512 * 2
    for kw, text in ((dict(workspace=None), "workspace"), (dict(workspace_bytes=need - 1), "workspace_bytes"),
                     (dict(workspace=FAKE + 64), "256-byte"), (dict(top_k=0), "top_k"),
                     (dict(hc_mult=8), "only 4"), (dict(hc_fn=None), "required"),
                     (dict(hidden_size=8200, shared_rank_stride=4 * 8200), "exceeds"),
                     (dict(weights_bf16=2), "weights_bf16"),
                     (dict(routed_scaling_factor=float("nan")), "finite")):
        with pytest.raises(mhc.MhcbError, match=text):
            mhc.mhcb_finalize_glm(**{**fglm, **kw})
    fin_ex = {**fin, "weights_bf16": 1, "routed_scaling_factor": 2.5}
    for kw, text in ((dict(weights_bf16=2), "weights_bf16"),
                     (dict(routed_scaling_factor=float("inf")), "finite"),
                     (dict(routed_scaling_factor=float("nan")), "finite"),
                     (dict(expert_weights=FAKE + 1), "aligned"),
                     (dict(weights_bf16=0, expert_weights=FAKE + 2), "aligned"),
                     (dict(top_k=0), "top_k")):
        with pytest.raises(mhc.MhcbError, match=text):
            mhc.mhcb_finalize_ex(**{**fin_ex, **kw})
    with pytest.raises(mhc.MhcbError, match="multiple of 128"):
        mhc.mhcb_quant_mxfp8(FAKE, FAKE, FAKE, 4, 520, 0)
    with pytest.raises(mhc.MhcbError, match="at least"):
        mhc.mhcb_workspace_init(FAKE, 64, 0)
    with pytest.raises(mhc.MhcbError, match="256-byte"):
        mhc.mhcb_workspace_init(FAKE + 64, 1 << 23, 0)


def _indexer(**kw):
    import tp_reduce_mhc_amd as mhc
    args = dict(x=FAKE, weight=FAKE, key_out=FAKE, heads_out=FAKE, gate_out=FAKE, workspace=None,
                workspace_bytes=0, M=16, K=6144, key_rows=128, heads=32, gate_rows=128, stream=0)
    args.update(kw)
    return mhc.mhcb_indexer_projection(**args)


@pytest.mark.parametrize("kw,code,text", [
    (dict(M=0), "EINVAL", "M=0"),
    (dict(K=100), "EUNSUPPORTED", "multiple of 128"),
    (dict(K=65536 + 128), "EUNSUPPORTED", "multiple of 128"),
    (dict(key_rows=4096, heads=1, gate_rows=0), "EUNSUPPORTED", "rows exceed"),
    (dict(key_rows=0, heads=0, gate_rows=0), "EINVAL", "at least one"),
    (dict(key_rows=-1), "EINVAL", "at least one"),
    (dict(x=None), "EINVAL", "required"),
    (dict(heads_out=None), "EINVAL", "required"),
    (dict(x=FAKE + 8), "EALIGN", "16-byte"),
    (dict(heads_out=FAKE + 2), "EALIGN", "element-aligned"),
    (dict(workspace=FAKE, workspace_bytes=16), "EINVAL", "mhcb_indexer_workspace_bytes"),
    (dict(workspace=FAKE + 64, workspace_bytes=1 << 30), "EALIGN", "256-byte"),
])
def test_indexer_validation(kw, code, text):
    """The indexer projection validates its sizes, pointers, alignment and
    workspace before anything is launched."""
    import tp_reduce_mhc_amd as mhc
    with pytest.raises(mhc.MhcbError, match=text) as e:
        _indexer(**kw)
    assert e.value.code == getattr(mhc, "MHCB_" + code)


def test_indexer_workspace_bytes():
    """No workspace where K is not split: the one-workgroup-per-row form
    (M <= 4) and more output blocks than the counter area holds; a fixed
    counter area plus the partials otherwise, growing with M; -1 for sizes
    the call rejects."""
    import tp_reduce_mhc_amd as mhc
    assert mhc.mhcb_indexer_workspace_bytes(4, 6144, 128, 32, 128) == 0
    assert mhc.mhcb_indexer_workspace_bytes(24576, 6144, 128, 32, 128) == 0  # 1152 4x6 blocks
    small = mhc.mhcb_indexer_workspace_bytes(16, 6144, 128, 32, 128)
    large = mhc.mhcb_indexer_workspace_bytes(256, 6144, 128, 32, 128)
    assert 4096 < small < large and small % 4 == 0
    with pytest.raises(mhc.MhcbError):
        mhc.mhcb_indexer_workspace_bytes(16, 100, 128, 32, 128)
    with pytest.raises(mhc.MhcbError, match="required"):
        mhc.mhcb_indexer_workspace_init(None, 256, 0)


def test_indexer_projection_object_validates_shapes():
    """IndexerProjection rejects weights that are not 2-D BF16 with one K,
    before any device work."""
    import torch
    import tp_reduce_mhc_amd as mhc
    k, h, g = (torch.zeros((r, 256), dtype=torch.bfloat16) for r in (16, 8, 8))
    with pytest.raises(ValueError, match="share K"):
        mhc.IndexerProjection(k, h, torch.zeros((8, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="BF16"):
        mhc.IndexerProjection(k, h.float(), g)
    proj = mhc.IndexerProjection(k, h, g)
    assert (proj.key, proj.heads, proj.gate) == (16, 8, 8) and proj.weight.shape == (32, 256)
    with pytest.raises(ValueError, match="K"):
        proj(torch.zeros((2, 128), dtype=torch.bfloat16))


def test_workspace_cache_grows_by_doubling_and_keeps_replaced_buffers():
    """The binding's per-(device, stream) workspace caches: a request no
    larger than the cached buffer reuses it; a larger one replaces it with a
    buffer at least twice its size and keeps the old one alive (a captured
    graph or queued call may still use it), so the retired buffers never add
    up to more than the live one."""
    from tp_reduce_mhc_amd import mhcb

    class Buf:
        def __init__(self, n):
            self.n = n

        def numel(self):
            return self.n

    made, cache, retired_before = [], {}, len(mhcb._RETIRED)

    def make(n):
        made.append(n)
        return Buf(n)

    try:
        for need in (100, 150, 90, 400, 1000, 1001):
            live = mhcb._cached(cache, ("dev", 0), need, make)
            assert live.numel() >= need
        assert made == [100, 200, 400, 1000, 2000]
        retired = mhcb._RETIRED[retired_before:]
        assert [b.numel() for b in retired] == [100, 200, 400, 1000]
        assert sum(b.numel() for b in retired) <= live.numel()
        assert mhcb._cached(cache, ("dev", 1), 10, make).numel() == 10  # another stream
    finally:
        del mhcb._RETIRED[retired_before:]


def test_product_path_does_not_touch_the_oracle():
    """The binding and the HIP sources never import, load or name the
    oracle's library or module."""
    pkg = os.path.join(ROOT, "tp_reduce_mhc_amd")
    for path in glob.glob(os.path.join(pkg, "**", "*"), recursive=True):
        if os.path.isfile(path) and path.endswith((".py", ".hip", ".h", ".cpp")):
            text = open(path).read()
            assert "import oracle" not in text and "from oracle" not in text, path
            assert "liboracle" not in text and "oracle_" not in text, path


def test_binding_fails_loudly_without_the_library(tmp_path):
    """The Python binding has no fallback: without libmhcb.so it refuses to
    import."""
    import shutil
    import subprocess
    import sys
    src = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tp_reduce_mhc_amd")
    pkg = tmp_path / "tp_reduce_mhc_amd"
    pkg.mkdir()
    for name in ("__init__.py", "mhcb.py"):
        shutil.copy(os.path.join(src, name), pkg / name)
    r = subprocess.run([sys.executable, "-c", "import tp_reduce_mhc_amd"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "libmhcb.so is missing" in r.stderr
