"""Parity of the HIP path (through the C ABI) with the oracle, on seeded
workloads of the pages' shapes.  Needs an MI355X: marked gpu.

Bars: the BF16 rank sum and the MXFP8 codes/scales bit-exact; post-mixed
streams and the delayed layer input within 1 BF16 ulp (they come out
bit-exact here); GLM layer input within 1 ulp of the oracle's collapse and
RMSNorm run on the pre-mix the kernel derived from its own raw mixes (and,
secondary, within the tie-aware band of the oracle's own layer input with a
capped count of 2-ulp elements); raw GLM mixes |d| <= 1e-5 (|ref| + 1);
side mixes |d| <= 1e-5 |ref| + 1e-7.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import (assert_bits_equal, assert_within_ulp, check_glm_outputs, dev, host,
                            u16)
from tests.numerics import bf16_ulp_distance, bf16_value

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import tp_reduce_mhc_amd as mhc


def run_boundary(b, mxfp8=False, pre=True):
    out = mhc.boundary(dev(b.partials), dev(b.residual), dev(b.post), dev(b.comb),
                       dev(b.pre) if pre else None, dev(b.gamma) if pre else None, b.norm_eps,
                       mxfp8=mxfp8)
    torch.cuda.synchronize()
    ro, li, mx = out
    return u16(ro), (u16(li) if li is not None else None), (
        (host(mx[0]), host(mx[1])) if mx else None)


def check_boundary(b, mxfp8=False, threads=8):
    print(f"[gpu] {b.name} mxfp8={mxfp8}", flush=True)
    ro, li, mx = run_boundary(b, mxfp8)
    ro_ref, li_ref, mx_ref = oracle.boundary(b.partials, b.residual, b.post, b.comb, b.pre, b.gamma,
                                             b.norm_eps, mxfp8=mxfp8, threads=threads)
    assert_bits_equal(ro, ro_ref, "residual_out")
    assert_within_ulp(li, li_ref, 1, "layer_input")
    if mxfp8:
        v_q, s_q = oracle.quant_mxfp8(li)          # the oracle quantizes the GPU's BF16 output
        assert_bits_equal(mx[0], v_q, "mxfp8 values")
        assert_bits_equal(mx[1], s_q, "mxfp8 scales")
    return ro, li, mx


# ---------------------------------------------------------------------------
# Delayed-mHC boundary
# ---------------------------------------------------------------------------

def test_tiny_delayed_boundary():
    check_boundary(synth.tiny_delayed(), mxfp8=True)


@pytest.mark.parametrize("M", [1, 8, 32, 64, 128])
def test_dsv41_delayed_boundary_sweep(M):
    check_boundary(synth.dsv41_delayed(M))


@pytest.mark.parametrize("M,H,mxfp8", [(130, 1024, False), (129, 3072, False), (200, 5120, False),
                                       (256, 5120, False), (131, 7168, False), (1030, 1024, True),
                                       (1100, 3072, True), (1024, 5120, True), (1025, 7168, True)])
def test_balanced_forms(M, H, mxfp8):
    """The balanced forms for unsplit tokens of 256 FF + 128 fragments and
    eight ranks: eight waves at H = 5120 (every M), four waves at the other
    widths (FF = 0, 1, 3; more than 128 tokens, 1024 with MXFP8).  Every
    element against the oracle (streams bit-exact, layer input within 1 ulp;
    MXFP8 codes and scales, padding rows included, bit-exact)."""
    check_boundary(synth.boundary(80 + H // 1024, M, H, 8, 0.5, f"balanced-H{H}-tp8-M{M}"),
                   mxfp8=mxfp8)


@pytest.mark.parametrize("M,mxfp8", [(1, True), (3, False), (26, True), (51, False), (52, True),
                                     (64, False)])
def test_split_half_form(M, mxfp8):
    """H = 5120 tokens split with a workspace, as chosen on 256 compute
    units: five slices of 128 fragments (four columns a thread) up to
    M = 51, four one-fragment slices beyond.  Every element against the
    oracle, MXFP8 codes and scales with the padding rows included; the
    unsplit call gives the same bits."""
    b = synth.boundary(90, M, 5120, 8, 0.5, f"split-half-H5120-tp8-M{M}")
    ro, li, mx = check_boundary(b, mxfp8=mxfp8)
    out = mhc.boundary(dev(b.partials), dev(b.residual), dev(b.post), dev(b.comb), dev(b.pre),
                       dev(b.gamma), b.norm_eps, mxfp8=mxfp8, split=False)
    torch.cuda.synchronize()
    assert_bits_equal(u16(out[0]), ro, "unsplit residual_out")
    assert_bits_equal(u16(out[1]), li, "unsplit layer_input")
    if mxfp8:
        assert_bits_equal(host(out[2][0]), mx[0], "unsplit mxfp8 values")
        assert_bits_equal(host(out[2][1]), mx[1], "unsplit mxfp8 scales")


def test_bf16_sum_is_bit_exact_through_the_probe():
    """post = 1, comb = 0 expose the BF16 rank sum in every output stream."""
    b = synth.dsv41_delayed(32)
    b.post = np.ones_like(b.post)
    b.comb = np.zeros_like(b.comb)
    ro, _, _ = run_boundary(b)
    xr = np.array([[oracle.rank_sum_element(b.partials[:, t:t + 1], c) for c in range(0, b.H, 37)]
                   for t in range(b.M)], np.uint16)
    for j in range(4):
        assert_bits_equal(ro[:, j, ::37], xr, f"stream {j}")


def test_rank_order_designed_case():
    """Ranks (1, 2^-8, 2^-24, 2^-24): only the in-order FP32 sum gives 1.0."""
    b = synth.boundary(11, 2, 512, 4, 0.5)
    b.partials[:, :, 5] = np.array([0x3F80, 0x3B80, 0x3380, 0x3380], np.uint16)[:, None]
    b.post = np.ones_like(b.post)
    b.comb = np.zeros_like(b.comb)
    ro, _, _ = run_boundary(b)
    assert (ro[:, :, 5] == 0x3F80).all()


@pytest.mark.parametrize("tp", [1, 2, 3, 5, 8, 9, 16])
def test_tp_variants(tp):
    check_boundary(synth.boundary(12, 5, 1024, tp, 0.5, f"tp{tp}"))


@pytest.mark.parametrize("H", [8, 520, 1032, 4104, 6144, 8200, 16384])
def test_ragged_and_wide_hidden(H):
    """Fragments not a multiple of the workgroup (ragged last trip), one
    fragment, and the 1/2/4 fragments-per-thread geometries."""
    check_boundary(synth.boundary(13, 3, H, 2, 0.5, f"H{H}"))


def test_residual_only_variant():
    b = synth.dsv41_delayed(8)
    ro, li, _ = run_boundary(b, pre=False)
    ro_ref, _, _ = oracle.boundary(b.partials, b.residual, b.post, b.comb, None, None, 1e-6)
    assert li is None
    assert_bits_equal(ro, ro_ref, "residual_out")


def test_negative_zero_and_rounding_edges():
    """Partials that are -0, subnormal, exact BF16 ties of the FP32 sum and
    sums that cancel to zero."""
    b = synth.boundary(14, 4, 256, 2, 0.5)
    p = b.partials
    p[0, :, 0:8] = 0x8000                                   # -0 + x
    p[1, :, 8:16] = 0x8000
    p[:, :, 16:24] = 0x8000                                 # -0 + -0
    p[0, :, 24:32], p[1, :, 24:32] = 0x0001, 0x0002        # subnormal sums
    p[0, :, 32:40], p[1, :, 32:40] = 0x3F80, 0x3B80        # 1 + 2^-8: BF16 tie
    p[0, :, 40:48], p[1, :, 40:48] = 0x3F81, 0x3B80        # 1+2^-7 + 2^-8: tie to even up
    p[0, :, 48:56] = 0x4000
    p[1, :, 48:56] = 0xC000                                 # cancellation
    b.residual[:, :, 60:64] = 0x0003                        # subnormal residuals
    check_boundary(b)


def test_mxfp8_epilogue_with_padding_rows():
    for M in (100, 128, 129, 256):
        b = synth.boundary(4, M, 5120, 8, 0.5, f"mxfp8-M{M}")
        check_boundary(b, mxfp8=True)


def test_standalone_quant_matches_oracle():
    for M, H in ((1, 128), (3, 512), (130, 5120)):
        x = synth.bf16_matrix(M, H, 2.0)
        x[0, :32] = 0                                        # zero block
        values, scales = mhc.quant_mxfp8(dev(x))
        torch.cuda.synchronize()
        v_ref, s_ref = oracle.quant_mxfp8(x)
        assert_bits_equal(host(values), v_ref, "values")
        assert_bits_equal(host(scales), s_ref, "scales")


def test_large_m_full_size():
    """M = 8192 (H=5120, tp=8) with the MXFP8 epilogue in the benchmark's
    launch configuration, every token against the oracle.  The codes and
    scales are compared with the oracle's quantization of its own layer
    input wherever the GPU's layer input is bit-equal to it (every token
    here), and with the oracle's quantization of the GPU's rows elsewhere."""
    b = synth.large_m_delayed(8192)
    ro, li, (vals, scales) = run_boundary(b, mxfp8=True)
    ro_ref, li_ref, (v_ref, s_ref) = oracle.boundary(
        b.partials, b.residual, b.post, b.comb, b.pre, b.gamma, b.norm_eps, mxfp8=True,
        threads=oracle.default_threads())
    assert_bits_equal(ro, ro_ref, "residual_out")
    off = assert_within_ulp(li, li_ref, 1, "layer_input")
    same = (li == li_ref).all(axis=1)
    assert_bits_equal(vals[same], v_ref[same], "mxfp8 values (rows equal to the oracle's)")
    K = 5120 // 32
    idx = np.array([[oracle.sf_index(int(t), k, K) for k in range(K)] for t in range(8192)])
    assert_bits_equal(scales[idx[same]], s_ref[idx[same]], "mxfp8 scales (rows equal)")
    for t in np.flatnonzero(~same):
        v_q, s_q = oracle.quant_mxfp8(li[t:t + 1])
        assert_bits_equal(vals[t:t + 1], v_q, f"mxfp8 values of token {t}")
        assert_bits_equal(scales[idx[t]], s_q[idx[0]], f"mxfp8 scales of token {t}")
    print(f"[gpu] M=8192: layer_input {off} elements 1 ulp off, {int((~same).sum())} rows "
          "quantized separately", flush=True)


@pytest.mark.parametrize("M", [1, 8, 64, 100])
def test_token_split_gives_identical_bits(M):
    """Every number of workgroups per token (1 = no split, no workspace)
    gives the same bits: each square is exact in binary64, and the sums'
    rounding (near 2^-53 relative) lies far below the binary32 rounding of
    the RMSNorm factor.
    The bounded cross-workgroup waits never gave up."""
    b = synth.boundary(15, M, 5120, 8, 0.5, f"split-M{M}")
    ref = run_boundary_split(b, None)
    ws = mhc.new_workspace(mhc.mhcb_workspace_bytes(M, 5120, 8, 0), "cuda")
    try:
        for S in (0, 2, 3, 5, 8, 16):
            mhc.mhcb_set_token_slices(S)
            got = run_boundary_split(b, ws)
            for g, r, what in zip(got, ref, ("residual_out", "layer_input", "values", "scales")):
                assert_bits_equal(g, r, f"S={S} {what}")
    finally:
        mhc.mhcb_set_token_slices(0)
    assert mhc.workspace_status(ws) == mhc.MHCB_OK
    ro_ref, li_ref, _ = oracle.boundary(b.partials, b.residual, b.post, b.comb, b.pre, b.gamma,
                                        b.norm_eps, threads=8)
    assert_bits_equal(ref[0], ro_ref, "residual_out")
    assert_within_ulp(ref[1], li_ref, 1, "layer_input")


def run_boundary_split(b, ws):
    M, H = b.M, b.H
    ro = torch.empty((M, 4, H), dtype=torch.bfloat16, device="cuda")
    li = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    vals = torch.empty((M, H), dtype=torch.uint8, device="cuda")
    scales = torch.empty(mhc.mhcb_mxfp8_scale_bytes(M, H), dtype=torch.uint8, device="cuda")
    mhc.mhcb_boundary(dev(b.partials), M * H, None, dev(b.residual), dev(b.post), dev(b.comb),
                      dev(b.pre), dev(b.gamma), ro, li, vals, scales, ws,
                      ws.numel() if ws is not None else 0, M, H, 4, b.tp, b.norm_eps)
    torch.cuda.synchronize()
    return u16(ro), u16(li), host(vals), host(scales)


# The sync state: a 256-byte header, then a 4 KiB slot per token holding the
# epoch word (split calls on the slot, low 32 bits; the last one's slice
# count, high 32 bits) at +0 and two 1792-byte copies of the exchange area at
# +128 and +1920; a call uses copy epoch % 2.
EMPTY = 0x7FC0DEAD


def sync_state(ws):
    """(epochs [1024], last slice counts [1024], copies [1024, 2, 448] as
    32-bit words, status)."""
    torch.cuda.synchronize()
    raw = ws[:256 + 4096 * 1024].cpu().numpy()
    slots = raw[256:].reshape(1024, 4096)
    epoch_word = slots[:, :8].copy().view(np.uint64)[:, 0]     # (epoch << 8) | slices
    copies = np.stack([slots[:, 128:1920].copy().view(np.uint32),
                       slots[:, 1920:3712].copy().view(np.uint32)], axis=1)
    return ((epoch_word >> np.uint64(8)).astype(np.int64),
            (epoch_word & np.uint64(0xFF)).astype(np.int64), copies,
            int(raw[:4].view(np.uint32)[0]))


def run_glm_on(g, G, ws):
    M, H = g.M, g.H
    out = (torch.empty((M, 4, H), dtype=torch.bfloat16, device="cuda"),
           torch.empty((M, 24), dtype=torch.float32, device="cuda"),
           torch.empty((M, H), dtype=torch.bfloat16, device="cuda"))
    mhc.mhcb_boundary_glm(dev(g.partials), M * H, dev(g.residual), dev(g.post), dev(g.comb),
                          dev(g.fn), dev(g.scale), dev(g.base), dev(g.gamma), *out, ws,
                          ws.numel(), M, H, 4, g.tp, g.rms_eps, g.hc_eps, g.norm_eps, G)
    torch.cuda.synchronize()
    return u16(out[0]), host(out[1]), u16(out[2])


def effective_slices(F, S):
    """The library's slice count for a requested S over F fragments: slices
    of ceil(F/S) fragments rounded up to a multiple of 4."""
    frags = -(-F // S)
    frags = -(-frags // 4) * 4
    return -(-F // frags)


def check_call_state(ws, want_epochs, want_slices, what):
    """After a call: every slot's epoch counts its split calls and records the
    last one's slice count, and the copy the next call on the slot will use
    is entirely empty (so it starts clean whatever its slice count)."""
    epochs, slices, copies, status = sync_state(ws)
    assert status == 0, f"a wait gave up ({what})"
    assert np.array_equal(epochs, want_epochs), f"epochs after {what}"
    assert np.array_equal(slices, want_slices), f"last slice counts after {what}"
    nxt = copies[np.arange(1024), epochs % 2]
    assert (nxt == EMPTY).all(), f"the next call's copy is not empty after {what}"


def test_workspace_epochs_and_clean_copies():
    """mhcb_workspace_init writes the epochs 0 and every exchange word empty.
    Every split call advances the epoch of its tokens' slots and leaves the
    copy the next call will use empty, with no reset at its end: the slices
    clear the previous call's entries while they work.  The slice count
    changes from call to call (16, 3, 1, 16, 2, ...), every result still
    matches (the delayed boundary bit for bit with the unsplit call) and no
    wait gives up."""
    ws = mhc.new_workspace(mhc.mhcb_workspace_bytes(0, 0, 1, 0), "cuda")
    want = np.zeros(1024, np.int64)
    want_s = np.zeros(1024, np.int64)
    epochs, slices, copies, status = sync_state(ws)
    assert status == 0 and not epochs.any() and not slices.any() and (copies == EMPTY).all()

    b = synth.boundary(16, 8, 5120, 8, 0.5, "state-delayed")
    ref = run_boundary_split(b, None)
    for S in (16, 3, 1, 16, 2, 5, 16):
        mhc.mhcb_set_token_slices(S)
        try:
            got = run_boundary_split(b, ws)
        finally:
            mhc.mhcb_set_token_slices(0)
        for x, y, what in zip(got, ref, ("residual_out", "layer_input", "values", "scales")):
            assert_bits_equal(x, y, f"delayed S={S} {what}")
        if S > 1:
            want[:b.M] += 1
            want_s[:b.M] = effective_slices(640, S)
        check_call_state(ws, want, want_s, f"delayed S={S}")

    # (GLM input, tokens per workgroup, slices); 16 = tiles.
    for g, G, S in ((synth.glm(7), 1, 2), (synth.glm(7), 2, 16), (synth.glm(7), 4, 5),
                    (synth.glm(20, H=2048), 16, 3), (synth.glm(20, H=2048), 16, 16),
                    (synth.glm(20, H=2048), 16, 4), (synth.glm(300), 16, 8)):
        print(f"[gpu] {g.name} G={G} S={S}", flush=True)
        mhc.mhcb_set_token_slices(S)
        try:
            ro, mixes, li = run_glm_on(g, G, ws)
        finally:
            mhc.mhcb_set_token_slices(0)
        check_glm_against_oracle(g, ro, mixes, li, f"G={G} S={S}")
        F = g.H // 8
        want[:g.M] += 1
        want_s[:g.M] = effective_slices(F, S if G == 16 else min(S, F // 64))
        check_call_state(ws, want, want_s, f"{g.name} G={G} S={S}")


def test_graph_replays_match_eager_calls():
    """Split calls captured in one HIP graph (delayed boundary with MXFP8,
    MoE finalize, GLM exchanging tiles and two passes with the side mixes,
    all through one workspace; the GLM boundary of an MoE sublayer on its
    own) and
    replayed three times, with eager calls on the same workspace in between,
    give the eager results every time (the tags the exchanges wait for are
    read from the workspace at each replay, not frozen into the graph), and
    those results match the oracle to each call's parity bar.  The DSA
    indexer projection with K ranges is in the graph too; its counters are
    zero again after the last replay."""
    b = synth.boundary(17, 8, 1024, 8, 0.5, "graph-delayed")
    f = synth.moe_finalize(8, H=1024)
    g = synth.glm(40, H=2048)
    ws = mhc.new_workspace(mhc.mhcb_workspace_bytes(0, 0, 1, 0), "cuda")
    db = {k: dev(getattr(b, k)) for k in ("partials", "residual", "post", "comb", "pre", "gamma")}
    df = {k: dev(getattr(f, k)) for k in ("gemm2", "weights", "idx", "shared", "residual", "post",
                                          "comb", "pre", "gamma")}
    dg = {k: dev(getattr(g, k)) for k in ("partials", "residual", "post", "comb", "fn", "scale",
                                          "base", "gamma")}
    outs = {
        "b_ro": torch.empty((b.M, 4, b.H), dtype=torch.bfloat16, device="cuda"),
        "b_li": torch.empty((b.M, b.H), dtype=torch.bfloat16, device="cuda"),
        "b_v": torch.empty((b.M, b.H), dtype=torch.uint8, device="cuda"),
        "b_s": torch.empty(mhc.mhcb_mxfp8_scale_bytes(b.M, b.H), dtype=torch.uint8, device="cuda"),
        "f_ro": torch.empty((f.M, 4, f.H), dtype=torch.bfloat16, device="cuda"),
        "f_li": torch.empty((f.M, f.H), dtype=torch.bfloat16, device="cuda"),
        "g_ro": torch.empty((g.M, 4, g.H), dtype=torch.bfloat16, device="cuda"),
        "g_mx": torch.empty((g.M, 24), dtype=torch.float32, device="cuda"),
        "g_li": torch.empty((g.M, g.H), dtype=torch.bfloat16, device="cuda"),
        "g2_ro": torch.empty((g.M, 4, g.H), dtype=torch.bfloat16, device="cuda"),
        "g2_mx": torch.empty((g.M, 24), dtype=torch.float32, device="cuda"),
        "g2_li": torch.empty((g.M, g.H), dtype=torch.bfloat16, device="cuda"),
        "x_post": torch.empty((g.M, 4, 1), dtype=torch.float32, device="cuda"),
        "x_comb": torch.empty((g.M, 4, 4), dtype=torch.float32, device="cuda"),
        "m_ro": torch.empty((f.M, 4, f.H), dtype=torch.bfloat16, device="cuda"),
        "m_mx": torch.empty((f.M, 24), dtype=torch.float32, device="cuda"),
        "m_li": torch.empty((f.M, f.H), dtype=torch.bfloat16, device="cuda"),
    }
    rows = f.M * f.top_k
    # The GLM boundary of an MoE sublayer on f's routes (H=1024, tp=4).
    gm = synth.glm(f.M, H=f.H, tp=f.tp)
    dgm = {k: dev(getattr(gm, k)) for k in ("fn", "scale", "base", "gamma")}
    ws_moe = mhc.new_workspace(mhc.mhcb_finalize_glm_workspace_bytes(f.M, f.H, f.tp), "cuda")
    # The DSA indexer projection with K ranges (its counters must be back
    # at zero after every call and replay).
    ix = synth.indexer(16, K=2048)
    dix = {"x": dev(ix.x), "w": dev(ix.w)}
    ix_bytes = mhc.mhcb_indexer_workspace_bytes(ix.M, ix.K, ix.key, ix.heads, ix.gate)
    assert ix_bytes > 0
    ws_ix = torch.empty(ix_bytes, dtype=torch.uint8, device="cuda")
    mhc.mhcb_indexer_workspace_init(ws_ix, ix_bytes)
    outs["i_key"] = torch.empty((ix.M, ix.key), dtype=torch.bfloat16, device="cuda")
    outs["i_heads"] = torch.empty((ix.M, ix.heads), dtype=torch.float32, device="cuda")
    outs["i_gate"] = torch.empty((ix.M, ix.gate), dtype=torch.bfloat16, device="cuda")
    eager_ix = [torch.empty_like(outs[k]) for k in ("i_key", "i_heads", "i_gate")]

    def calls():
        mhc.mhcb_boundary(db["partials"], b.M * b.H, None, db["residual"], db["post"], db["comb"],
                          db["pre"], db["gamma"], outs["b_ro"], outs["b_li"], outs["b_v"],
                          outs["b_s"], ws, ws.numel(), b.M, b.H, 4, b.tp, b.norm_eps)
        mhc.mhcb_finalize(df["gemm2"], rows * f.H, rows, df["weights"], 0, df["idx"], 0,
                          df["shared"], f.M * f.H, df["residual"], df["post"], df["comb"],
                          df["pre"], df["gamma"], outs["f_ro"], outs["f_li"], None, None, 0, ws,
                          ws.numel(), f.M, f.H, 4, f.tp, f.top_k, f.norm_eps)
        mhc.mhcb_boundary_glm(dg["partials"], g.M * g.H, dg["residual"], dg["post"], dg["comb"],
                              dg["fn"], dg["scale"], dg["base"], dg["gamma"], outs["g_ro"],
                              outs["g_mx"], outs["g_li"], ws, ws.numel(), g.M, g.H, 4, g.tp,
                              g.rms_eps, g.hc_eps, g.norm_eps, 16)
        mhc.mhcb_boundary_glm(dg["partials"], g.M * g.H, dg["residual"], dg["post"], dg["comb"],
                              dg["fn"], dg["scale"], dg["base"], dg["gamma"], outs["g2_ro"],
                              outs["g2_mx"], outs["g2_li"], ws, ws.numel(), g.M, g.H, 4, g.tp,
                              g.rms_eps, g.hc_eps, g.norm_eps, -16)
        mhc.mhcb_mixes(outs["g2_mx"], dg["scale"], dg["base"], outs["x_post"], outs["x_comb"], g.M,
                       4, g.hc_eps, g.post_mult, g.sinkhorn_repeat)
        mhc.mhcb_finalize_glm(df["gemm2"], rows * f.H, rows, df["weights"], 0, 0, 1.0, df["idx"], 0,
                              df["shared"], f.M * f.H, df["residual"], df["post"], df["comb"],
                              dgm["fn"], dgm["scale"], dgm["base"], dgm["gamma"], outs["m_ro"],
                              outs["m_mx"], outs["m_li"], ws_moe, ws_moe.numel(), f.M, f.H, 4,
                              f.tp, f.top_k, gm.rms_eps, gm.hc_eps, gm.norm_eps)
        mhc.mhcb_indexer_projection(dix["x"], dix["w"], outs["i_key"], outs["i_heads"],
                                    outs["i_gate"], ws_ix, ix_bytes, ix.M, ix.K, ix.key, ix.heads,
                                    ix.gate)

    calls()
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in outs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in outs.values():
            v.fill_(0x5A if v.dtype == torch.uint8 else float("nan"))
        run_boundary_split(b, ws)                       # eager work on the same workspace
        mhc.mhcb_indexer_projection(dix["x"], dix["w"], *eager_ix, ws_ix, ix_bytes, ix.M, ix.K,
                                    ix.key, ix.heads, ix.gate)  # and on the indexer's
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v.view(torch.uint8), want[k].view(torch.uint8)), f"replay {rep}: {k}"
    assert mhc.workspace_status(ws) == mhc.MHCB_OK
    epochs, _, copies, status = sync_state(ws)
    assert status == 0 and epochs.max() > 0
    assert (copies[np.arange(1024), epochs % 2] == EMPTY).all(), "the next call's copy is empty"

    # The replayed results (bit-equal to the eager ones) against the oracle.
    ro_ref, li_ref, _ = oracle.boundary(b.partials, b.residual, b.post, b.comb, b.pre, b.gamma,
                                        b.norm_eps, threads=8)
    assert_bits_equal(u16(outs["b_ro"]), ro_ref, "graph delayed residual_out")
    assert_within_ulp(u16(outs["b_li"]), li_ref, 1, "graph delayed layer_input")
    v_q, s_q = oracle.quant_mxfp8(u16(outs["b_li"]))
    assert_bits_equal(outs["b_v"].cpu().numpy(), v_q, "graph mxfp8 values")
    assert_bits_equal(outs["b_s"].cpu().numpy(), s_q, "graph mxfp8 scales")
    ro_ref, li_ref, _ = oracle.finalize(f.gemm2, f.weights, f.idx, f.shared, f.residual, f.post,
                                        f.comb, f.pre, f.gamma, f.norm_eps, threads=8)
    assert_bits_equal(u16(outs["f_ro"]), ro_ref, "graph finalize residual_out")
    assert_within_ulp(u16(outs["f_li"]), li_ref, 1, "graph finalize layer_input")
    check_glm_against_oracle(g, u16(outs["g_ro"]), host(outs["g_mx"]), u16(outs["g_li"]),
                             "graph glm tiles")
    check_glm_against_oracle(g, u16(outs["g2_ro"]), host(outs["g2_mx"]), u16(outs["g2_li"]),
                             "graph glm two passes")
    p_ref, c_ref = oracle.side_mixes(host(outs["g2_mx"]), g.scale, g.base, g.hc_eps, g.post_mult,
                                     g.sinkhorn_repeat)
    post_n, comb_n = host(outs["x_post"]).reshape(-1, 4), host(outs["x_comb"])
    assert (np.abs(post_n - p_ref) <= 1e-5 * np.abs(p_ref) + 1e-7).all(), "graph side post"
    assert (np.abs(comb_n - c_ref) <= 1e-5 * np.abs(c_ref) + 1e-7).all(), "graph side comb"
    ro_ref, mix_ref, li_ref, pre_ref = oracle.boundary_glm_moe(
        f.gemm2, f.weights, f.idx, f.shared, f.residual, f.post, f.comb, gm.fn, gm.scale, gm.base,
        gm.gamma, gm.rms_eps, gm.hc_eps, gm.norm_eps, threads=8)
    check_glm_outputs("graph glm moe", u16(outs["m_ro"]), host(outs["m_mx"]), u16(outs["m_li"]),
                      ro_ref, mix_ref, li_ref, pre_ref, gm.scale, gm.base, gm.gamma, gm.hc_eps,
                      gm.norm_eps)
    check_indexer(ix, (u16(outs["i_key"]), host(outs["i_heads"]), u16(outs["i_gate"])))
    assert not ws_ix[:4096].any(), "indexer counters back at zero"


def test_cross_token_independence_and_determinism():
    b = synth.dsv41_delayed(128)
    ro1, li1, _ = run_boundary(b)
    ro2, li2, _ = run_boundary(b)
    assert_bits_equal(ro1, ro2, "run-to-run residual_out")
    assert_bits_equal(li1, li2, "run-to-run layer_input")
    s = synth.dsv41_delayed(128)
    s.M = 8
    s.partials, s.residual, s.post, s.comb, s.pre = (b.partials[:, :8], b.residual[:8], b.post[:8],
                                                    b.comb[:8], b.pre[:8])
    ro3, li3, _ = run_boundary(s)
    assert_bits_equal(ro3, ro1[:8], "prefix residual_out")
    assert_bits_equal(li3, li1[:8], "prefix layer_input")


# ---------------------------------------------------------------------------
# MoE finalize and the two-shot emulation
# ---------------------------------------------------------------------------

def run_finalize(f, two_shot=False, mxfp8=False, split=True):
    out = mhc.finalize(dev(f.gemm2), dev(f.weights), dev(f.idx), dev(f.shared), dev(f.residual),
                       dev(f.post), dev(f.comb), dev(f.pre), dev(f.gamma), f.norm_eps,
                       two_shot=two_shot, mxfp8=mxfp8, split=split)
    torch.cuda.synchronize()
    ro, li, mx = out
    return u16(ro), u16(li), ((host(mx[0]), host(mx[1])) if mx else None)


@pytest.mark.parametrize("M", [64, 512])
def test_moe_finalize_matches_oracle_and_two_shot(M):
    f = synth.moe_finalize(M)
    print(f"[gpu] {f.name}", flush=True)
    ro, li, mx = run_finalize(f, mxfp8=True)
    ro_ref, li_ref, _ = oracle.finalize(f.gemm2, f.weights, f.idx, f.shared, f.residual, f.post,
                                        f.comb, f.pre, f.gamma, f.norm_eps, threads=8)
    assert_bits_equal(ro, ro_ref, "residual_out")
    assert_within_ulp(li, li_ref, 1, "layer_input")
    ro2, li2, mx2 = run_finalize(f, two_shot=True, mxfp8=True)
    assert_bits_equal(ro2, ro, "two-shot residual_out")
    assert_bits_equal(li2, li, "two-shot layer_input")
    assert_bits_equal(mx2[0], mx[0], "two-shot mxfp8 values")
    assert_bits_equal(mx2[1], mx[1], "two-shot mxfp8 scales")
    ro3, li3, mx3 = run_finalize(f, mxfp8=True, split=False)
    assert_bits_equal(ro3, ro, "one workgroup per token: residual_out")
    assert_bits_equal(li3, li, "one workgroup per token: layer_input")
    assert_bits_equal(mx3[1], mx[1], "one workgroup per token: mxfp8 scales")


def test_moe_finalize_per_rank_routing_with_dropped_experts():
    f = synth.moe_finalize(37, H=1024, tp=4, top_k=8, replicated_routing=False, drop_fraction=0.15)
    ro, li, _ = run_finalize(f)
    ro_ref, li_ref, _ = oracle.finalize(f.gemm2, f.weights, f.idx, f.shared, f.residual, f.post,
                                        f.comb, f.pre, f.gamma, f.norm_eps,
                                        replicated_routing=False, threads=8)
    assert_bits_equal(ro, ro_ref, "residual_out")
    assert_within_ulp(li, li_ref, 1, "layer_input")
    ro2, li2, _ = run_finalize(f, two_shot=True)
    assert_bits_equal(ro2, ro, "two-shot residual_out")
    assert_bits_equal(li2, li, "two-shot layer_input")


def test_moe_finalize_large_m_full_size():
    """M = 4096 (H=5120, tp=4, top_k=8): every token against the oracle;
    two-shot equal."""
    f = synth.moe_finalize(4096)
    ro, li, _ = run_finalize(f)
    ro2, li2, _ = run_finalize(f, two_shot=True)
    assert_bits_equal(ro2, ro, "two-shot residual_out")
    assert_bits_equal(li2, li, "two-shot layer_input")
    n = oracle.default_threads()
    contrib = oracle.finalize_contributions(f.gemm2, f.weights, f.idx, f.shared, threads=n)
    ro_ref, li_ref, _ = oracle.boundary(contrib, f.residual, f.post, f.comb, f.pre, f.gamma,
                                        f.norm_eps, threads=n)
    assert_bits_equal(ro, ro_ref, "residual_out")
    assert_within_ulp(li, li_ref, 1, "layer_input")


# ---------------------------------------------------------------------------
# GLM boundary and side mixes
# ---------------------------------------------------------------------------

def run_glm(g, G, workspace=True):
    """Outputs are pre-filled with NaN so that an element the kernel misses
    cannot pass on a previous call's bits."""
    M, H = g.M, g.H
    ro = torch.full((M, 4, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    mixes = torch.full((M, 24), float("nan"), dtype=torch.float32, device="cuda")
    li = torch.full((M, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = mhc.workspace("cuda") if workspace else None
    mhc.mhcb_boundary_glm(dev(g.partials), M * H, dev(g.residual), dev(g.post), dev(g.comb),
                          dev(g.fn), dev(g.scale), dev(g.base), dev(g.gamma), ro, mixes, li, ws,
                          ws.numel() if workspace else 0, M, H, 4, g.tp, g.rms_eps, g.hc_eps,
                          g.norm_eps, G)
    torch.cuda.synchronize()
    if workspace:
        assert mhc.workspace_status(ws) == mhc.MHCB_OK
    return u16(ro), host(mixes), u16(li)


@pytest.mark.parametrize("M", [1, 16, 64, 7])
def test_glm_boundary_matches_oracle(M):
    g = synth.glm(M)
    print(f"[gpu] {g.name}", flush=True)
    ro_ref, mix_ref, li_ref, pre_ref = oracle.boundary_glm(
        g.partials, g.residual, g.post, g.comb, g.fn, g.scale, g.base, g.gamma, g.rms_eps,
        g.hc_eps, g.norm_eps, threads=8)
    first = None
    for G in (1, 2, 4):
        ro, mixes, li = run_glm(g, G)
        check_glm_outputs(f"G={G}", ro, mixes, li, ro_ref, mix_ref, li_ref, pre_ref, g.scale,
                          g.base, g.gamma, g.hc_eps, g.norm_eps)
        if first is None:
            first = (ro, mixes, li)
        else:   # outputs do not depend on the tokens per workgroup
            assert_bits_equal(ro, first[0], f"G={G} residual_out vs G=1")
            assert np.array_equal(mixes, first[1]), f"G={G} mixes vs G=1"
            assert_bits_equal(li, first[2], f"G={G} layer_input vs G=1")


def check_glm_against_oracle(g, ro, mixes, li, what, toks=None):
    """The GLM outputs of every token (or of tokens `toks`) against the oracle."""
    sel = slice(None) if toks is None else toks
    ro_ref, mix_ref, li_ref, pre_ref = oracle.boundary_glm(
        g.partials[:, sel], g.residual[sel], g.post[sel], g.comb[sel], g.fn, g.scale, g.base,
        g.gamma, g.rms_eps, g.hc_eps, g.norm_eps, threads=8)
    return check_glm_outputs(what, ro[sel], mixes[sel], li[sel], ro_ref, mix_ref, li_ref, pre_ref,
                             g.scale, g.base, g.gamma, g.hc_eps, g.norm_eps)


@pytest.mark.parametrize("M,H,G,workspace", [(100, 6144, 1, True), (100, 6144, 2, True),
                                              (9, 6144, 2, False), (9, 1024, 4, False)])
def test_glm_one_thread_per_fragment_and_no_workspace(M, H, G, workspace):
    """Whole tokens in one workgroup: one thread per fragment (H=6144) or a
    quad per fragment (H=1024); without a workspace nothing is split."""
    g = synth.glm(M, H=H)
    print(f"[gpu] {g.name} G={G} workspace={workspace}", flush=True)
    ro, mixes, li = run_glm(g, G, workspace)
    check_glm_against_oracle(g, ro, mixes, li, f"G={G}")


@pytest.mark.parametrize("M,H,tp", [(1, 6144, 8), (17, 6144, 8), (40, 2048, 3), (33, 512, 8),
                                    (16, 8192, 8), (5, 1024, 1), (3, 64, 2)])
def test_glm_tiles_match_oracle(M, H, tp):
    """16-token matrix-core tiles (tokens_per_wg=16): ragged last tiles,
    runtime and fixed rank counts, one to four steps per wave."""
    g = synth.glm(M, H=H, tp=tp)
    print(f"[gpu] {g.name} tiles", flush=True)
    ro, mixes, li = run_glm(g, 16)
    check_glm_against_oracle(g, ro, mixes, li, "tiles")


@pytest.mark.parametrize("S", [1, 3, 16])
def test_glm_tiles_any_slice_count(S):
    g = synth.glm(20, H=2048, tp=8)
    prev = mhc.mhcb_set_token_slices(S)
    try:
        print(f"[gpu] {g.name} tiles, slices {S}", flush=True)
        ro, mixes, li = run_glm(g, 16)
    finally:
        mhc.mhcb_set_token_slices(prev)
    check_glm_against_oracle(g, ro, mixes, li, f"tiles S={S}")


def test_glm_tiles_more_tokens_than_one_launch():
    """M above the per-launch token limit of the split kernels (1024): the
    call is issued as several launches."""
    g = synth.glm(1100, H=256, tp=2)
    print(f"[gpu] {g.name} tiles", flush=True)
    ro, mixes, li = run_glm(g, 16)
    check_glm_against_oracle(g, ro, mixes, li, "tiles M=1100")


@pytest.mark.parametrize("M,H,tp,S", [(1, 6144, 8, 0), (17, 6144, 8, 0), (40, 2048, 3, 0),
                                      (33, 512, 8, 0), (16, 8192, 8, 0), (5, 1024, 1, 0),
                                      (3, 64, 2, 0), (20, 2048, 8, 4), (20, 2048, 4, 8),
                                      (37, 6144, 8, 48), (19, 6144, 4, 16),
                                      (600, 2048, 8, 0), (333, 6144, 8, 0), (200, 8192, 4, 0),
                                      (400, 6144, 8, 48), (1100, 6144, 4, 0), (250, 1000, 8, 0)])
def test_glm_two_pass_tiles_match_oracle(M, H, tp, S):
    """16-token tiles in two passes (tokens_per_wg=-16): a stream pass that
    leaves per-slice partials in the workspace, then one workgroup per token.
    Slices of 16 to 64 fragments, ragged last slices and tiles, fixed (4, 8)
    and runtime rank counts, tile counts that are not multiples of eight and
    more tokens than one launch takes."""
    g = synth.glm(M, H=H, tp=tp)
    prev = mhc.mhcb_set_token_slices(S)
    try:
        print(f"[gpu] {g.name} two-pass tiles, slices {S}", flush=True)
        ro, mixes, li = run_glm(g, -16)
    finally:
        mhc.mhcb_set_token_slices(prev)
    check_glm_against_oracle(g, ro, mixes, li, f"two-pass S={S}")


def test_glm_two_pass_more_tokens_than_one_launch():
    g = synth.glm(1100, H=256, tp=2)
    print(f"[gpu] {g.name} two-pass tiles", flush=True)
    ro, mixes, li = run_glm(g, -16)
    check_glm_against_oracle(g, ro, mixes, li, "two-pass M=1100")


def test_glm_two_pass_full_size():
    """M = 512, H=6144, tp=8 in two passes, every token against the oracle,
    and its streams equal to the exchanging tiles' bit for bit."""
    g = synth.glm(512)
    print(f"[gpu] {g.name} two-pass tiles", flush=True)
    ro, mixes, li = run_glm(g, -16)
    ro16, mixes16, _ = run_glm(g, 16)
    assert_bits_equal(ro, ro16, "two-pass vs exchanging tiles residual_out")
    assert (np.abs(mixes - mixes16) <= 2e-5 * (np.abs(mixes16) + 1)).all()
    check_glm_against_oracle(g, ro, mixes, li, "two-pass M=512")


@pytest.mark.parametrize("M", [256, 512])
def test_glm_full_size_automatic(M):
    """The GLM workload's larger sizes (H=6144, tp=8) with the automatic
    choice, every token against the oracle."""
    g = synth.glm(M)
    print(f"[gpu] {g.name} automatic", flush=True)
    ro, mixes, li = run_glm(g, 0)
    check_glm_against_oracle(g, ro, mixes, li, f"auto M={M}")


@pytest.mark.parametrize("M,spread", [(1, 1.0), (64, 1.0), (513, 1.0), (256, 4.0)])
def test_side_mixes_match_oracle(M, spread):
    """The side kernel uses FP32 hardware reciprocals and FP32 exp; spread
    widens the raw mixes (and so the Sinkhorn logits) to stress them."""
    raw, scale, base = synth.raw_mixes(M)
    raw = (raw * np.float32(spread)).astype(np.float32)
    post, comb = mhc.mixes(dev(raw), dev(scale), dev(base), 1e-6, 2.0, 20)
    torch.cuda.synchronize()
    p_ref, c_ref = oracle.side_mixes(raw, scale, base, 1e-6, 2.0, 20)
    post, comb = host(post).reshape(M, 4), host(comb)
    assert (np.abs(post - p_ref) <= 1e-5 * np.abs(p_ref) + 1e-7).all()
    assert (np.abs(comb - c_ref) <= 1e-5 * np.abs(c_ref) + 1e-7).all()
    rel = np.abs(comb - c_ref) / np.maximum(np.abs(c_ref), 1e-30)
    print(f"[gpu] side mixes M={M} spread {spread}: bit-exact post {np.array_equal(post, p_ref)}, "
          f"comb {np.array_equal(comb, c_ref)}, max comb rel err {rel.max():.2e}", flush=True)


def test_glm_boundary_object_side_stream_and_join():
    g = synth.glm(16)
    gb = mhc.GlmBoundary(rms_eps=g.rms_eps, hc_eps=g.hc_eps, post_mult=g.post_mult,
                         sinkhorn_repeat=g.sinkhorn_repeat, norm_eps=g.norm_eps, device="cuda")
    for _ in range(3):
        ro, post_n, comb_n, li, raw = gb(dev(g.partials), dev(g.residual), dev(g.post),
                                         dev(g.comb), dev(g.fn), dev(g.scale), dev(g.base),
                                         dev(g.gamma))
        gb.join()
        torch.cuda.synchronize()
        p_ref, c_ref = oracle.side_mixes(host(raw), g.scale, g.base, g.hc_eps, g.post_mult,
                                         g.sinkhorn_repeat)
        assert (np.abs(host(post_n).reshape(-1, 4) - p_ref) <= 1e-5 * np.abs(p_ref) + 1e-7).all()
        assert (np.abs(host(comb_n) - c_ref) <= 1e-5 * np.abs(c_ref) + 1e-7).all()


# ---------------------------------------------------------------------------
# Mailbox stand-in
# ---------------------------------------------------------------------------

def _hc_inputs(hc, M, H, tp, seed):
    """Seeded delayed-boundary inputs with hc residual streams."""
    rng = np.random.default_rng(seed)
    partials = synth.to_bf16_bits(rng.standard_normal((tp, M, H)).astype(np.float32) * 0.5)
    residual = synth.to_bf16_bits(rng.standard_normal((M, hc, H)).astype(np.float32))
    post = rng.uniform(0, 1, (M, hc)).astype(np.float32)
    comb = (rng.uniform(0, 1, (M, hc, hc)) / hc).astype(np.float32)
    pre = rng.uniform(0, 1, (M, hc)).astype(np.float32)
    gamma = synth.to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    return partials, residual, post, comb, pre, gamma


@pytest.mark.parametrize("hc", [1, 2, 8])
def test_general_hc_delayed_finalize_and_mailbox(hc):
    """hc_mult = 1, 2 and 8 streams: the delayed boundary (split and unsplit,
    MXFP8 epilogue), the MoE finalize (one-shot split and unsplit, two-shot)
    and the mailbox-fed consumer, against the oracle."""
    M, H, tp = 37, 1024, 4
    partials, residual, post, comb, pre, gamma = _hc_inputs(hc, M, H, tp, 70 + hc)
    print(f"[gpu] general hc={hc} M={M} H={H}", flush=True)
    ro_ref, li_ref, (v_ref, s_ref) = oracle.boundary(partials, residual, post, comb, pre, gamma,
                                                     1e-6, mxfp8=True, threads=8)
    d = [dev(x) for x in (partials, residual, post, comb, pre, gamma)]
    for split in (True, False):
        ro, li, (vals, scales) = mhc.boundary(*d, 1e-6, mxfp8=True, split=split)
        torch.cuda.synchronize()
        assert_bits_equal(u16(ro), ro_ref, f"residual_out split={split}")
        assert_within_ulp(u16(li), li_ref, 1, f"layer_input split={split}")
        v_q, s_q = oracle.quant_mxfp8(u16(li))
        assert_bits_equal(host(vals), v_q, "mxfp8 values")
        assert_bits_equal(host(scales), s_q, "mxfp8 scales")

    f = synth.moe_finalize(M, H=H, tp=tp, top_k=4, replicated_routing=False, drop_fraction=0.1)
    fro_ref, fli_ref, _ = oracle.finalize(f.gemm2, f.weights, f.idx, f.shared, residual, post, comb,
                                          pre, gamma, 1e-6, replicated_routing=False, threads=8)
    for two_shot, split in ((False, True), (False, False), (True, True)):
        out = mhc.finalize(dev(f.gemm2), dev(f.weights), dev(f.idx), dev(f.shared), d[1], d[2],
                           d[3], d[4], d[5], 1e-6, two_shot=two_shot, split=split)
        torch.cuda.synchronize()
        assert_bits_equal(u16(out[0]), fro_ref, f"finalize residual_out two_shot={two_shot} split={split}")
        assert_within_ulp(u16(out[1]), fli_ref, 1, f"finalize layer_input two_shot={two_shot}")

    mb = mhc.Mailbox(tp, 64, H, "cuda")
    mb.init()
    mb.publish(d[0])
    ro, li, _ = mb.boundary(M, d[1], d[2], d[3], d[4], d[5], 1e-6)
    torch.cuda.synchronize()
    assert mb.status_ok()
    assert_bits_equal(u16(ro), ro_ref, "mailbox residual_out")
    assert_within_ulp(u16(li), li_ref, 1, "mailbox layer_input")


@pytest.mark.parametrize("hc", [1, 2, 8])
def test_general_hc_dsv41_shape(hc):
    """hc_mult = 1, 2 and 8 at H=5120, tp=8 (ranks held in registers; eight
    streams in two trips when unsplit): split and unsplit against the oracle."""
    b = synth.dsv41_delayed(16, hc)
    print(f"[gpu] {b.name}", flush=True)
    ro_ref, li_ref, _ = oracle.boundary(b.partials, b.residual, b.post, b.comb, b.pre, b.gamma,
                                        b.norm_eps, threads=8)
    d = [dev(x) for x in (b.partials, b.residual, b.post, b.comb, b.pre, b.gamma)]
    for split in (True, False):
        ro, li, _ = mhc.boundary(*d, b.norm_eps, split=split)
        torch.cuda.synchronize()
        assert_bits_equal(u16(ro), ro_ref, f"residual_out split={split}")
        assert_within_ulp(u16(li), li_ref, 1, f"layer_input split={split}")


def test_mailbox_generations_cycle_and_match_direct():
    from oracle.mailbox_model import MailboxModel
    cap, H, tp = 64, 1024, 4
    mb = mhc.Mailbox(tp, cap, H, "cuda")
    mb.init()
    model = MailboxModel(tp, cap, H)
    for call, M in enumerate((5, 64, 17, 1, 33)):
        b = synth.boundary(20 + call, M, H, tp, 0.5, f"mailbox-call{call}")
        b.partials[0, 0, :8] = 0x8000                       # a -0 payload must not stall
        print(f"[gpu] mailbox call {call} M={M}", flush=True)
        mb.publish(dev(b.partials))
        ro, li, _ = mb.boundary(M, dev(b.residual), dev(b.post), dev(b.comb), dev(b.pre),
                                dev(b.gamma), b.norm_eps)
        torch.cuda.synchronize()
        model.publish(b.partials)
        model.consume(M)
        assert mb.status_ok()
        assert_bits_equal(u16(mb.slots), model.slots, "mailbox slots after consume")
        assert np.array_equal(host(mb.stage_state), model.stage), "stage_state"
        ro_ref, li_ref, _ = oracle.boundary(b.partials, b.residual, b.post, b.comb, b.pre, b.gamma,
                                            b.norm_eps)
        assert_bits_equal(u16(ro), ro_ref, "residual_out")
        assert_within_ulp(u16(li), li_ref, 1, "layer_input")


def test_mailbox_large_m_with_mxfp8():
    """Mailbox-fed boundary at M = 8192 with the MXFP8 epilogue, three calls
    cycling the generations; equal to the direct path."""
    b = synth.large_m_delayed(8192)
    mb = mhc.Mailbox(8, 8192, 5120, "cuda")
    mb.init()
    ro_d, li_d, mx_d = run_boundary(b, mxfp8=True)
    parts, res, post, comb, pre, gam = (dev(b.partials), dev(b.residual), dev(b.post),
                                        dev(b.comb), dev(b.pre), dev(b.gamma))
    for call in range(3):
        mb.publish(parts)
        ro, li, mx = mb.boundary(8192, res, post, comb, pre, gam, b.norm_eps, mxfp8=True)
        torch.cuda.synchronize()
        assert mb.status_ok()
        assert host(mb.stage_state).tolist() == [call, (call + 1) % 3]
        assert_bits_equal(u16(ro), ro_d, "mailbox residual_out")
        assert_bits_equal(u16(li), li_d, "mailbox layer_input")
        assert_bits_equal(host(mx[0]), mx_d[0], "mailbox mxfp8 values")
        assert_bits_equal(host(mx[1]), mx_d[1], "mailbox mxfp8 scales")
    assert (u16(mb.slots) == 0x8000).all()


def test_workspace_cache_growth_keeps_a_captured_graph_valid():
    """A graph captured with the binding's cached workspace of a stream keeps
    working after a larger request on that stream replaces the workspace:
    the replaced buffer stays allocated (new allocations on the stream,
    filled with garbage, do not land on it), and replays give the eager
    results bit for bit."""
    b = synth.boundary(51, 9, 1024, 8, 0.5, "cache-growth")
    st = torch.cuda.Stream()
    ws = mhc.workspace("cuda", stream=st)
    d = {k: dev(getattr(b, k)) for k in ("partials", "residual", "post", "comb", "pre", "gamma")}
    ro = torch.empty((b.M, 4, b.H), dtype=torch.bfloat16, device="cuda")
    li = torch.empty((b.M, b.H), dtype=torch.bfloat16, device="cuda")

    def call():
        mhc.mhcb_boundary(d["partials"], b.M * b.H, None, d["residual"], d["post"], d["comb"],
                          d["pre"], d["gamma"], ro, li, None, None, ws, ws.numel(), b.M, b.H, 4,
                          b.tp, b.norm_eps, st)

    st.wait_stream(torch.cuda.current_stream())
    call()
    torch.cuda.synchronize()
    want_ro, want_li = ro.clone(), li.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        call()
    torch.cuda.synchronize()
    old_ptr, n = ws.data_ptr(), ws.numel()
    bigger = mhc.workspace("cuda", stream=st, nbytes=n + 1)
    assert bigger.data_ptr() != old_ptr and bigger.numel() >= 2 * n
    del ws  # only the cache's record of the replaced buffer is left
    with torch.cuda.stream(st):
        junk = [torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda") for _ in range(4)]
    torch.cuda.synchronize()
    assert all(j.data_ptr() != old_ptr for j in junk), "the replaced workspace was handed out again"
    for rep in range(2):
        ro.fill_(float("nan"))
        li.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ro.view(torch.int16), want_ro.view(torch.int16)), f"replay {rep}"
        assert torch.equal(li.view(torch.int16), want_li.view(torch.int16)), f"replay {rep}"
    ro_ref, li_ref, _ = oracle.boundary(b.partials, b.residual, b.post, b.comb, b.pre, b.gamma,
                                        b.norm_eps)
    assert_bits_equal(u16(ro), ro_ref, "residual_out")
    assert_within_ulp(u16(li), li_ref, 1, "layer_input")


def test_graph_replays_mailbox_publish_and_consume():
    """The mailbox chain captured in one HIP graph: the producer's publish of
    all tp ranks, then the mailbox-fed boundary split over slices of a
    workspace.  Four replays, with an eager publish + consume pair on other
    inputs after the first and third (so replays start from different
    generations): the kernels read the generation from stage_state at run
    time, so after every replay stage_state and every slot equal the host
    model's, and the outputs equal the oracle's to the parity bar."""
    from oracle.mailbox_model import MailboxModel
    cap, H, tp, M = 32, 1024, 4, 9
    b = synth.boundary(41, M, H, tp, 0.5, "graph-mailbox")
    e = synth.boundary(42, M, H, tp, 0.5, "graph-mailbox-eager")
    mb = mhc.Mailbox(tp, cap, H, "cuda")
    mb.init()
    model = MailboxModel(tp, cap, H)
    ws = mhc.new_workspace(mhc.mhcb_workspace_bytes(0, 0, 1, 0), "cuda")
    names = ("partials", "residual", "post", "comb", "pre", "gamma")
    db, de = ({k: dev(getattr(x, k)) for k in names} for x in (b, e))
    ro = torch.empty((M, 4, H), dtype=torch.bfloat16, device="cuda")
    li = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ro_e, li_e = torch.empty_like(ro), torch.empty_like(li)

    def chain(d, ro_out, li_out):
        mhc.mhcb_publish(mb, d["partials"], M * H, 0, tp, M)
        mhc.mhcb_boundary(None, 0, mb, d["residual"], d["post"], d["comb"], d["pre"], d["gamma"],
                          ro_out, li_out, None, None, ws, ws.numel(), M, H, 4, tp, b.norm_eps)

    def check(label, x, ro_got, li_got):
        assert mb.status_ok(), label
        assert np.array_equal(host(mb.stage_state), model.stage), f"{label}: stage_state"
        assert_bits_equal(u16(mb.slots), model.slots, f"{label}: slots")
        ro_ref, li_ref, _ = oracle.boundary(x.partials, x.residual, x.post, x.comb, x.pre,
                                            x.gamma, x.norm_eps)
        assert_bits_equal(u16(ro_got), ro_ref, f"{label}: residual_out")
        assert_within_ulp(u16(li_got), li_ref, 1, f"{label}: layer_input")

    chain(db, ro, li)  # eager first call (and warm-up)
    torch.cuda.synchronize()
    model.publish(b.partials)
    model.consume(M)
    check("eager", b, ro, li)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        chain(db, ro, li)
    torch.cuda.synchronize()
    assert np.array_equal(host(mb.stage_state), model.stage), "capture ran nothing"
    for rep in range(4):
        print(f"[gpu] mailbox graph replay {rep}", flush=True)
        ro.fill_(float("nan"))
        li.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        model.publish(b.partials)
        model.consume(M)
        check(f"replay {rep}", b, ro, li)
        if rep % 2 == 0:
            chain(de, ro_e, li_e)
            torch.cuda.synchronize()
            model.publish(e.partials)
            model.consume(M)
            check(f"eager after replay {rep}", e, ro_e, li_e)
    assert mhc.workspace_status(ws) == mhc.MHCB_OK


def test_mailbox_poll_gives_up_with_a_bounded_spin():
    """A consumer whose producer never publishes: a tiny spin limit makes
    every poll give up (all kernels exit normally), the status words count
    the time-outs, and the outputs are NaN, not sums of sentinels."""
    mb = mhc.Mailbox(2, 4, 256, "cuda", spin_limit=4)
    mb.init()
    b = synth.boundary(30, 2, 256, 2, 0.5)
    ro, li, _ = mb.boundary(2, dev(b.residual), dev(b.post), dev(b.comb), dev(b.pre), dev(b.gamma),
                            1e-6)
    timeouts, late = mhc.mailbox_status(mb)
    assert timeouts > 0 and late > 0 and not mb.status_ok()
    assert torch.isnan(ro.float()).all() and torch.isnan(li.float()).all()


def test_mailbox_eight_wave_consumer_gives_up_with_a_bounded_spin():
    """The same give-up on the eight-wave consumer (H=5120, tp=8, unsplit:
    no workspace): every chunk's poll gives up, the kernel ends, the
    outputs are NaN, the status counts the time-outs and late chunks, and
    the consumed slots are back to the sentinel."""
    M, H, tp = 3, 5120, 8
    mb = mhc.Mailbox(tp, M, H, "cuda", spin_limit=4)
    mb.init()
    b = synth.dsv41_delayed(M)
    ro = torch.zeros((M, 4, H), dtype=torch.bfloat16, device="cuda")
    li = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    mhc.mhcb_boundary(None, 0, mb, dev(b.residual), dev(b.post), dev(b.comb), dev(b.pre),
                      dev(b.gamma), ro, li, None, None, None, 0, M, H, 4, tp, b.norm_eps)
    torch.cuda.synchronize()
    timeouts, late = mhc.mailbox_status(mb)
    assert timeouts > 0 and late > 0 and not mb.status_ok()
    assert torch.isnan(ro.float()).all() and torch.isnan(li.float()).all()
    assert (u16(mb.slots) == 0x8000).all()
    assert host(mb.stage_state).tolist() == [0, 1]


@pytest.mark.parametrize("M", [8, 160])
def test_mailbox_consumer_polls_fragments_that_land_late(M):
    """The consumer's spin on fragments still landing (the DSV4.1 page's
    _LamportMHCDeviceKernel poll loop, the GLM page's _PublishDeviceKernel):
    ranks 0..tp/2-1 are published on the consumer's stream before it, ranks
    tp/2..tp-1 by a peer on a second stream with no ordering against the
    consumer, behind a 256 MiB copy, so they land while the consumer polls.
    The peer publishes through its own view of the slots (its own stage
    state, as each rank keeps on the pages).  Three calls cycle the
    generations; each is bit-equal to the direct path, no poll gives up,
    and late fragments are counted."""
    tp, H = 8, 5120
    b = synth.dsv41_delayed(M)
    ro_d, li_d, _ = run_boundary(b)
    mb = mhc.Mailbox(tp, M, H, "cuda")
    mb.init()
    peer = mb.peer_view()
    parts = dev(b.partials)
    residual, post, comb, pre, gamma = (dev(b.residual), dev(b.post), dev(b.comb), dev(b.pre),
                                        dev(b.gamma))
    big_src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
    big_dst = torch.empty_like(big_src)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    late_total = 0
    for call in range(3):
        print(f"[gpu] mailbox live poll, call {call}", flush=True)
        with torch.cuda.stream(side):
            peer.stage_state.fill_(call % 3)   # the peer's own consumer advanced it
            big_dst.copy_(big_src)              # the peer is busy a while
            mhc.mhcb_publish(peer, parts[tp // 2:], M * H, tp // 2, tp - tp // 2, M, side)
        mb.publish(parts[:tp // 2], 0)
        ro, li, _ = mb.boundary(M, residual, post, comb, pre, gamma, b.norm_eps)
        torch.cuda.synchronize()
        timeouts, late = mhc.mailbox_status(mb)
        assert timeouts == 0, f"call {call}: {timeouts} polls gave up"
        assert_bits_equal(u16(ro), ro_d, f"call {call} residual_out")
        assert_bits_equal(u16(li), li_d, f"call {call} layer_input")
        assert (u16(mb.slots)[call % 3] == 0x8000).all()
        late_total = late
    print(f"[gpu] mailbox live poll: {late_total} late fragments re-read over 3 calls", flush=True)
    assert late_total > 0


@pytest.mark.parametrize("S", [16, 5])
def test_split_wait_gives_up_with_a_tiny_spin_limit(S):
    """A workspace spin limit of one re-read on token-split delayed calls
    (M = 1024; 16 slices of 40 fragments, or 5 of 128 in the form with
    four columns a thread): slices that find a partner's value missing
    give up.  Every
    kernel exits; the streams stay exact; each slice's block of the layer
    input is either the oracle's bits or all NaN; the status counts the
    time-outs."""
    M, H = 1024, 5120
    b = synth.boundary(32, M, H, 8, 0.5, "split-timeout-H5120-tp8-M1024")
    print(f"[gpu] {b.name} slices={S}", flush=True)
    ro_ref, li_ref, _ = oracle.boundary(b.partials, b.residual, b.post, b.comb, b.pre, b.gamma,
                                        b.norm_eps, threads=oracle.default_threads())
    ws = mhc.new_workspace(mhc.mhcb_workspace_bytes(0, 0, 1, 0), "cuda")
    block = -(-(H // 8) // S)
    block = (block + 3) // 4 * 4 * 8          # columns per slice
    args = [dev(b.partials), M * H, None, dev(b.residual), dev(b.post), dev(b.comb), dev(b.pre),
            dev(b.gamma)]
    prev = mhc.mhcb_set_token_slices(S)
    gave_up = 0
    try:
        mhc.mhcb_workspace_set_spin_limit(ws, 1)
        for attempt in range(6):
            ro = torch.empty((M, 4, H), dtype=torch.bfloat16, device="cuda")
            li = torch.full((M, H), 12345.0, dtype=torch.bfloat16, device="cuda")  # "not written"
            mhc.mhcb_boundary(*args, ro, li, None, None, ws, ws.numel(), M, H, 4, 8, b.norm_eps)
            out = torch.zeros(1, dtype=torch.int32, device="cuda")
            mhc.mhcb_workspace_status(ws, out)
            torch.cuda.synchronize()
            n = int(out.item())
            got = u16(li).reshape(M, -1, block)
            nan = np.isnan(bf16_value(got))
            good = ~nan.all(axis=2)
            want = li_ref.reshape(M, -1, block)
            bad = good & ~(got == want).all(axis=2)
            unwritten = (got == u16(torch.full((1,), 12345.0, dtype=torch.bfloat16))[0]).all(axis=2)
            print(f"[gpu] spin limit 1, attempt {attempt}: {n} time-outs, "
                  f"{int((~good).sum())} NaN slice blocks, {int(bad.sum())} wrong blocks "
                  f"({int((bad & unwritten).sum())} unwritten, "
                  f"{int((bad & (np.abs(bf16_value(got)) == 0).all(axis=2)).sum())} all zero); "
                  f"wrong (token, slice): {np.argwhere(bad)[:12].tolist()}; "
                  f"NaN (token, slice): {np.argwhere(~good)[:12].tolist()}", flush=True)
            assert_bits_equal(u16(ro), ro_ref, f"attempt {attempt} residual_out")
            whole = nan.all(axis=2) | ~nan.any(axis=2)
            assert whole.all(), f"attempt {attempt}: a slice block is partly NaN"
            assert not bad.any(), f"attempt {attempt}: wrong bits"
            # every wait that gave up left its slice's block NaN (a slice that
            # started after its token's slot broke is NaN without waiting)
            assert int((~good).sum()) >= n, f"attempt {attempt}: {n} time-outs"
            if n > 0:
                gave_up = n
                broken = ~good.all(axis=1)          # tokens with a NaN block
                break
        assert gave_up > 0, "no wait gave up with a spin limit of one re-read"
        # A give-up breaks its token's slot: with the default spin limit, the
        # next call gives those tokens NaN (never sums of stale entries) and
        # every other token the oracle's bits, until the workspace is
        # initialized again.
        mhc.mhcb_workspace_set_spin_limit(ws, 0)
        li = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
        mhc.mhcb_boundary(*args, ro, li, None, None, ws, ws.numel(), M, H, 4, 8, b.norm_eps)
        torch.cuda.synchronize()
        got = u16(li)
        assert np.isnan(bf16_value(got[broken])).all(), "a broken token slot gave numbers"
        assert_bits_equal(got[~broken], li_ref[~broken], "tokens with intact slots")
        mhc.mhcb_workspace_init(ws, ws.numel())
        mhc.mhcb_boundary(*args, ro, li, None, None, ws, ws.numel(), M, H, 4, 8, b.norm_eps)
        assert mhc.workspace_status(ws) == mhc.MHCB_OK
        assert_bits_equal(u16(li), li_ref, "after mhcb_workspace_init")
        print(f"[gpu] {int(broken.sum())} broken token slots gave NaN on the next call; "
              "clean after init", flush=True)
    finally:
        mhc.mhcb_set_token_slices(prev)
        mhc.mhcb_workspace_set_spin_limit(ws, 0)
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# Errors leave state untouched
# ---------------------------------------------------------------------------

def test_bad_arguments_leave_mailbox_untouched():
    mb = mhc.Mailbox(2, 8, 256, "cuda")
    mb.init()
    b = synth.boundary(31, 4, 256, 2, 0.5)
    mb.publish(dev(b.partials))
    torch.cuda.synchronize()
    before_slots, before_stage = u16(mb.slots).copy(), host(mb.stage_state).copy()
    with pytest.raises(mhc.MhcbError):
        mb.boundary(9, dev(np.zeros((9, 4, 256), np.uint16)), dev(np.zeros((9, 4), np.float32)),
                    dev(np.zeros((9, 4, 4), np.float32)), dev(np.zeros((9, 4), np.float32)),
                    dev(b.gamma), 1e-6)                     # M > capacity
    with pytest.raises(mhc.MhcbError):
        mb.boundary(4, dev(b.residual), dev(b.post), dev(b.comb), dev(b.pre), None, 1e-6)
    torch.cuda.synchronize()
    assert_bits_equal(u16(mb.slots), before_slots, "slots")
    assert np.array_equal(host(mb.stage_state), before_stage)


# ---------------------------------------------------------------------------
# Seeded random shapes
# ---------------------------------------------------------------------------

def _random_shapes(seed, count):
    rng = np.random.default_rng([seed, 20260])
    for i in range(count):
        H = int(rng.choice([8, 24, 136, 512, 1000, 2048, 3072, 5120, 7168, 8192, 12288, 16384]))
        M = int(rng.integers(1, 300))
        tp = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16]))
        slices = int(rng.choice([0, 1, 2, 3, 16]))
        yield i, M, H, tp, slices


@pytest.mark.parametrize("case", list(_random_shapes(1, 12)), ids=lambda c: f"M{c[1]}-H{c[2]}-tp{c[3]}-S{c[4]}")
def test_delayed_random_shapes(case):
    """Delayed boundary on seeded random (M, hidden, tp, slices): residual
    streams bit-exact, layer input within 1 ulp (bit-exact in practice), and
    the MXFP8 epilogue bit-exact wherever hidden % 128 == 0."""
    i, M, H, tp, S = case
    b = synth.boundary(40 + i, M, H, tp, 0.5, f"random-{i}")
    mxfp8 = H % 128 == 0
    ws = mhc.workspace("cuda")
    prev = mhc.mhcb_set_token_slices(S)
    try:
        got = run_boundary_split(b, ws) if mxfp8 else None
        if not mxfp8:
            ro = torch.empty((M, 4, H), dtype=torch.bfloat16, device="cuda")
            li = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
            mhc.mhcb_boundary(dev(b.partials), M * H, None, dev(b.residual), dev(b.post),
                              dev(b.comb), dev(b.pre), dev(b.gamma), ro, li, None, None, ws,
                              ws.numel(), M, H, 4, tp, b.norm_eps)
            torch.cuda.synchronize()
            got = (u16(ro), u16(li), None, None)
    finally:
        mhc.mhcb_set_token_slices(prev)
    print(f"[gpu] {b.name} M={M} H={H} tp={tp} S={S} mxfp8={mxfp8}", flush=True)
    ro_ref, li_ref, _ = oracle.boundary(b.partials, b.residual, b.post, b.comb, b.pre, b.gamma,
                                        b.norm_eps, threads=8)
    assert_bits_equal(got[0], ro_ref, "residual_out")
    assert_within_ulp(got[1], li_ref, 1, "layer_input")
    if mxfp8:
        v_q, s_q = oracle.quant_mxfp8(got[1])
        assert_bits_equal(got[2], v_q, "mxfp8 values")
        assert_bits_equal(got[3], s_q, "mxfp8 scales")
    assert mhc.workspace_status(ws) == mhc.MHCB_OK


@pytest.mark.parametrize("case", [(0, 5, 1024, 3, 1), (1, 33, 3072, 8, 2), (2, 2, 8192, 2, 4),
                                  (3, 70, 512, 8, 16), (4, 300, 2048, 5, 0), (5, 17, 6144, 12, 16),
                                  (6, 45, 1536, 6, -16), (7, 129, 4096, 16, -16), (8, 7, 256, 7, -16)],
                         ids=lambda c: f"M{c[1]}-H{c[2]}-tp{c[3]}-G{c[4]}")
def test_glm_random_shapes(case):
    """GLM on mixed shapes, tokens per workgroup, exchanging tiles and two
    passes (-16; tp = 16 takes the runtime rank loop in two rounds of eight),
    against the oracle."""
    i, M, H, tp, G = case
    g = synth.glm(M, H=H, tp=tp, name=f"glm-random-{i}")
    if G == 4 and H > 6144:
        G = 2
    print(f"[gpu] {g.name} M={M} H={H} tp={tp} G={G}", flush=True)
    ro, mixes, li = run_glm(g, G)
    check_glm_against_oracle(g, ro, mixes, li, f"G={G}")


@pytest.mark.parametrize("bf16_weights,scale", [(True, 1.0), (True, 0.3), (False, 2.5),
                                                 (True, 2.5)])
def test_finalize_routing_weight_options(bf16_weights, scale):
    """mhcb_finalize_ex: BF16 or FP32 routing weights and a routed scaling
    factor, per-rank routing with dropped routes; one-shot split and unsplit
    and two-shot all match the oracle."""
    f = synth.moe_finalize(40, H=1024, tp=4, top_k=8, replicated_routing=False,
                           drop_fraction=0.1)
    w = synth.to_bf16_bits(f.weights) if bf16_weights else f.weights
    print(f"[gpu] {f.name} bf16_weights={bf16_weights} scale={scale}", flush=True)
    ro_ref, li_ref, _ = oracle.finalize(f.gemm2, w, f.idx, f.shared, f.residual, f.post, f.comb,
                                        f.pre, f.gamma, f.norm_eps, replicated_routing=False,
                                        routed_scaling_factor=scale, threads=8)
    for two_shot, split in ((False, True), (False, False), (True, True)):
        out = mhc.finalize(dev(f.gemm2), dev(w), dev(f.idx), dev(f.shared), dev(f.residual),
                           dev(f.post), dev(f.comb), dev(f.pre), dev(f.gamma), f.norm_eps,
                           two_shot=two_shot, split=split, routed_scaling_factor=scale)
        torch.cuda.synchronize()
        assert_bits_equal(u16(out[0]), ro_ref, f"residual_out two_shot={two_shot} split={split}")
        assert_within_ulp(u16(out[1]), li_ref, 1, f"layer_input two_shot={two_shot} split={split}")


@pytest.mark.parametrize("case", [(3, 1024, 1, 1, True, 0.0), (17, 2048, 2, 16, False, 0.3),
                                  (64, 5120, 4, 6, True, 0.0), (40, 3072, 8, 2, False, 0.5),
                                  (130, 512, 3, 8, True, 0.0)],
                         ids=lambda c: f"M{c[0]}-H{c[1]}-tp{c[2]}-k{c[3]}")
def test_finalize_random_shapes(case):
    """MoE finalize on mixed (M, hidden, tp, top_k, routing): split and
    unsplit, hoisted and runtime-rank gathers, dropped routes; one-shot and
    two-shot give the same bits and match the oracle."""
    M, H, tp, k, replicated, drop = case
    f = synth.moe_finalize(M, H=H, tp=tp, top_k=k, replicated_routing=replicated,
                           drop_fraction=drop)
    print(f"[gpu] {f.name} M={M} H={H} tp={tp} top_k={k}", flush=True)
    ro_ref, li_ref, _ = oracle.finalize(f.gemm2, f.weights, f.idx, f.shared, f.residual, f.post,
                                        f.comb, f.pre, f.gamma, f.norm_eps,
                                        replicated_routing=replicated, threads=8)
    for two_shot, split in ((False, True), (False, False), (True, True)):
        ro, li, _ = run_finalize(f, two_shot=two_shot, split=split)
        assert_bits_equal(ro, ro_ref, f"residual_out two_shot={two_shot} split={split}")
        assert_within_ulp(li, li_ref, 1, f"layer_input two_shot={two_shot} split={split}")


@pytest.mark.parametrize("case", [(300, 4, 8, True, 0.0, True), (260, 3, 12, False, 0.2, False),
                                  (257, 1, 1, True, 0.0, True), (290, 8, 16, False, 0.1, True),
                                  (2048, 2, 5, False, 0.3, False), (1030, 4, 8, False, 0.125, True)],
                         ids=lambda c: f"M{c[0]}-tp{c[1]}-k{c[2]}-mx{int(c[5])}")
def test_finalize_balanced_form(case):
    """MoE finalize at H=5120 on 257 to 2048 unsplit tokens (eight balanced
    waves, ranks computed one at a time, routes in blocks of eight): the
    range's ends, mixed rank counts, top_k up to 16, per-rank routing with
    dropped routes, and the MXFP8 epilogue, against the oracle (codes and
    scales too)."""
    M, tp, k, replicated, drop, mxfp8 = case
    f = synth.moe_finalize(M, H=5120, tp=tp, top_k=k, replicated_routing=replicated,
                           drop_fraction=drop)
    print(f"[gpu] {f.name} M={M} tp={tp} top_k={k} mxfp8={mxfp8}", flush=True)
    ro, li, mx = run_finalize(f, mxfp8=mxfp8, split=False)
    ro_ref, li_ref, _ = oracle.finalize(f.gemm2, f.weights, f.idx, f.shared, f.residual, f.post,
                                        f.comb, f.pre, f.gamma, f.norm_eps,
                                        replicated_routing=replicated, threads=8)
    assert_bits_equal(ro, ro_ref, "residual_out")
    assert_within_ulp(li, li_ref, 1, "layer_input")
    if mxfp8:
        v_q, s_q = oracle.quant_mxfp8(li)          # the oracle quantizes the GPU's BF16 output
        assert_bits_equal(mx[0], v_q, "mxfp8 values")
        assert_bits_equal(mx[1], s_q, "mxfp8 scales")
    ro2, li2, _ = run_finalize(f, two_shot=True)
    assert_bits_equal(ro2, ro, "two-shot residual_out")
    assert_bits_equal(li2, li, "two-shot layer_input")


# ---------------------------------------------------------------------------
# GLM boundary of an MoE sublayer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", [(16, 2048, 4, 8, True, 0.0, False, 1.0),
                                  (37, 6144, 8, 8, False, 0.125, True, 2.5),
                                  (3, 512, 2, 1, True, 0.0, False, 1.0),
                                  (130, 1024, 4, 16, False, 0.3, False, 0.7),
                                  (64, 6144, 4, 8, True, 0.0, True, 1.0),
                                  (1100, 256, 2, 4, False, 0.2, True, 1.5),
                                  (24, 1024, 8, 32, False, 0.1, False, 1.0),
                                  (10, 1024, 3, 6, False, 0.2, True, 1.0)],
                         ids=lambda c: f"M{c[0]}-H{c[1]}-tp{c[2]}-k{c[3]}-bf16w{int(c[6])}")
def test_glm_moe_matches_oracle(case):
    """mhcb_finalize_glm: residual_out bit-exact, raw mixes within 1e-5
    relative and the layer input within the GLM band; replicated and
    per-rank routing with dropped routes, FP32 and BF16 weights, routed
    scaling factors, more tokens than one launch takes.  Up to 128 routes a
    token the stream pass computes the contributions itself; beyond (tp=8,
    top_k=32) they are published first, and the published contributions
    are bit-equal to the oracle's."""
    M, H, tp, k, replicated, drop, bf16w, rsf = case
    f = synth.moe_finalize(M, H=H, tp=tp, top_k=k, replicated_routing=replicated,
                           drop_fraction=drop)
    g = synth.glm(M, H=H, tp=tp)
    w = synth.to_bf16_bits(f.weights) if bf16w else f.weights
    print(f"[gpu] glm moe M={M} H={H} tp={tp} top_k={k} replicated={replicated} bf16w={bf16w}",
          flush=True)
    ro = torch.full((M, 4, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    mixes = torch.full((M, 24), float("nan"), dtype=torch.float32, device="cuda")
    li = torch.full((M, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    need = mhc.mhcb_finalize_glm_workspace_bytes(M, H, tp)
    ws = mhc.new_workspace(need, "cuda")
    rows = f.gemm2.shape[1]
    per_rank = 0 if replicated else M * k
    mhc.mhcb_finalize_glm(dev(f.gemm2), rows * H, rows, dev(w), per_rank, bf16w, rsf, dev(f.idx),
                          per_rank, dev(f.shared), M * H, dev(g.residual), dev(g.post),
                          dev(g.comb), dev(g.fn), dev(g.scale), dev(g.base), dev(g.gamma), ro,
                          mixes, li, ws, need, M, H, 4, tp, k, g.rms_eps, g.hc_eps, g.norm_eps)
    torch.cuda.synchronize()
    contrib_ref = oracle.finalize_contributions(f.gemm2, w, f.idx, f.shared,
                                                replicated_routing=replicated,
                                                routed_scaling_factor=rsf, threads=8)
    if tp * k > 128:
        off = need - tp * M * H * 2
        contrib = ws[off:need].view(torch.int16).cpu().numpy().view(np.uint16).reshape(tp, M, H)
        assert_bits_equal(contrib, contrib_ref, "published contributions")
    ro_ref, mix_ref, li_ref, pre_ref = oracle.boundary_glm_moe(
        f.gemm2, w, f.idx, f.shared, g.residual, g.post, g.comb, g.fn, g.scale, g.base, g.gamma,
        g.rms_eps, g.hc_eps, g.norm_eps, replicated_routing=replicated,
        routed_scaling_factor=rsf, threads=8)
    check_glm_outputs("glm moe", u16(ro), host(mixes), u16(li), ro_ref, mix_ref, li_ref, pre_ref,
                      g.scale, g.base, g.gamma, g.hc_eps, g.norm_eps)


def test_glm_moe_python_helper_matches_entry_point():
    """finalize_glm (outputs and workspace allocated by the binding) gives
    the same bits as the C entry point on a fresh workspace."""
    f = synth.moe_finalize(20, H=1024, tp=4, top_k=8)
    g = synth.glm(20, H=1024, tp=4)
    ro, mixes, li = mhc.finalize_glm(dev(f.gemm2), dev(f.weights), dev(f.idx), dev(f.shared),
                                     dev(g.residual), dev(g.post), dev(g.comb), dev(g.fn),
                                     dev(g.scale), dev(g.base), dev(g.gamma), g.rms_eps, g.hc_eps,
                                     g.norm_eps)
    torch.cuda.synchronize()
    ro_ref, mix_ref, li_ref, pre_ref = oracle.boundary_glm_moe(
        f.gemm2, f.weights, f.idx, f.shared, g.residual, g.post, g.comb, g.fn, g.scale, g.base,
        g.gamma, g.rms_eps, g.hc_eps, g.norm_eps, threads=8)
    check_glm_outputs("glm moe helper", u16(ro), host(mixes), u16(li), ro_ref, mix_ref, li_ref,
                      pre_ref, g.scale, g.base, g.gamma, g.hc_eps, g.norm_eps)


@pytest.mark.parametrize("M", [16, 300])
def test_glm_auto_with_sync_only_workspace(M):
    """A workspace that holds only the sync state (no two-pass scratch): the
    automatic choice falls back to the exchanging forms (one token per
    workgroup below M = 256, 16-token tiles from there) and still matches
    the oracle."""
    g = synth.glm(M)
    sync_only = mhc.mhcb_workspace_bytes(0, 0, 1, 0) - (8 << 20)  # less the 8 MiB scratch
    ws = mhc.new_workspace(sync_only, "cuda")
    ro = torch.full((M, 4, g.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    mixes = torch.full((M, 24), float("nan"), dtype=torch.float32, device="cuda")
    li = torch.full((M, g.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    print(f"[gpu] {g.name} automatic, sync-only workspace of {sync_only} bytes", flush=True)
    mhc.mhcb_boundary_glm(dev(g.partials), M * g.H, dev(g.residual), dev(g.post), dev(g.comb),
                          dev(g.fn), dev(g.scale), dev(g.base), dev(g.gamma), ro, mixes, li, ws,
                          sync_only, M, g.H, 4, g.tp, g.rms_eps, g.hc_eps, g.norm_eps, 0)
    torch.cuda.synchronize()
    assert mhc.workspace_status(ws) == mhc.MHCB_OK
    toks = np.arange(M)
    ro_ref, mix_ref, li_ref, pre_ref = oracle.boundary_glm(
        g.partials[:, toks], g.residual[toks], g.post[toks], g.comb[toks], g.fn, g.scale, g.base,
        g.gamma, g.rms_eps, g.hc_eps, g.norm_eps, threads=8)
    check_glm_outputs(f"sync-only workspace M={M}", u16(ro)[toks], host(mixes)[toks],
                      u16(li)[toks], ro_ref, mix_ref, li_ref, pre_ref, g.scale, g.base, g.gamma,
                      g.hc_eps, g.norm_eps)


# ---------------------------------------------------------------------------
# DSA indexer projection
# ---------------------------------------------------------------------------

def run_indexer(ix, workspace=None):
    """One projection; `workspace` None runs without one, "cached" with the
    binding's zeroed per-stream workspace, else the given tensor."""
    M, K = ix.M, ix.K
    key = torch.full((M, ix.key), float("nan"), dtype=torch.bfloat16, device="cuda")
    heads = torch.full((M, ix.heads), float("nan"), dtype=torch.float32, device="cuda")
    gate = torch.full((M, ix.gate), float("nan"), dtype=torch.bfloat16, device="cuda")
    nbytes = 0
    if workspace is not None:
        nbytes = mhc.mhcb_indexer_workspace_bytes(M, K, ix.key, ix.heads, ix.gate)
        if isinstance(workspace, str):
            workspace = mhc.indexer_workspace(nbytes) if nbytes else None
        else:
            nbytes = workspace.numel()
    mhc.mhcb_indexer_projection(dev(ix.x), dev(ix.w), key, heads, gate, workspace, nbytes, M, K,
                                ix.key, ix.heads, ix.gate)
    torch.cuda.synchronize()
    return u16(key), host(heads), u16(gate)


def check_indexer(ix, got):
    """The projection's outputs against the oracle's exact dot products s
    (binary64, rounded once): the FP32 head weights within 1e-5 (|s| + 1)
    and 1e-5 norm-wise per token; each BF16 key and gate output a correct
    rounding of a value within that same FP32 tolerance of s (so within 1
    BF16 ulp of the oracle's BF16 value unless the sum cancels to near
    zero)."""
    key, heads, gate = ix.key, ix.heads, ix.gate
    k_got, h_got, g_got = got
    k_ref, h_ref, g_ref = oracle.indexer_projection(ix.x, ix.w, key, heads, gate)
    rows = key + heads + gate
    _, s_all, _ = oracle.indexer_projection(ix.x, ix.w, 0, rows, 0)   # every row in FP32
    s_all = s_all.astype(np.float64)
    tol = 1e-5 * (np.abs(s_all) + 1)
    for name, g, ref, cols in (("key", k_got, k_ref, slice(0, key)),
                               ("gate", g_got, g_ref, slice(key + heads, rows))):
        if g.size == 0:
            continue
        s = s_all[:, cols]
        # half a BF16 ulp of the value: a binary32 ulp is 2^-16 of a BF16 one
        half_ulp = np.spacing((np.abs(s) + tol[:, cols]).astype(np.float32)).astype(np.float64) * 2.0 ** 15
        d = np.abs(bf16_value(g).astype(np.float64) - s)
        assert (d <= tol[:, cols] + half_ulp).all(), f"indexer {name}: max excess {(d - tol[:, cols] - half_ulp).max():.3g}"
        diff = bf16_ulp_distance(g, ref)
        far = diff > 2
        print(f"[gpu]   {name}: {int((diff > 0).sum())} of {g.size} differ from the oracle's BF16 "
              f"(max {int(diff.max())} ulps, at |s| = {np.abs(s.reshape(-1)[np.argmax(diff)]):.2e}); "
              f"{int(far.sum())} more than 2 ulps away, largest |s| among them "
              f"{(np.abs(s)[far].max() if far.any() else 0.0):.2e}", flush=True)
    if heads:
        err = np.abs(h_got.astype(np.float64) - h_ref)
        assert (err <= 1e-5 * (np.abs(h_ref) + 1)).all(), f"head weights: max err {err.max()}"
        rel = np.linalg.norm(err, axis=1) / np.maximum(np.linalg.norm(h_ref, axis=1), 1e-30)
        assert rel.max() <= 1e-5, f"head weights: norm-wise {rel.max():.2e}"
        print(f"[gpu]   head weights max abs {err.max():.2e}, norm-wise {rel.max():.2e}", flush=True)


@pytest.mark.parametrize("M,K,key,heads,gate,workspace",
                         [(1, 6144, 128, 32, 128, True), (16, 6144, 128, 32, 128, True),
                          (64, 6144, 128, 32, 128, True), (256, 6144, 128, 32, 128, True),
                          (300, 6144, 128, 32, 128, True), (5, 6144, 128, 32, 128, True),
                          (1, 6144, 128, 32, 128, False), (256, 6144, 128, 32, 128, False),
                          (33, 1024, 16, 8, 24, True), (1100, 2048, 128, 32, 128, True),
                          (7, 128, 8, 0, 8, True), (3, 65536, 8, 4, 4, True),
                          (4, 2048, 128, 32, 128, True), (9, 6144, 128, 32, 128, True),
                          (4, 6144, 128, 32, 128, True), (8, 6144, 128, 32, 128, True),
                          (6, 6144, 128, 32, 128, True), (17, 128, 4000, 64, 32, True),
                          (2500, 1024, 128, 32, 128, True), (2048, 2048, 128, 32, 128, True),
                          (4100, 1024, 128, 32, 128, True), (4096, 1024, 128, 32, 128, False)],
                         ids=lambda v: str(v))
def test_indexer_projection_matches_oracle(M, K, key, heads, gate, workspace):
    """mhcb_indexer_projection against the oracle (bars in check_indexer).
    The one-workgroup-per-row form (M <= 4 and 5 .. 6) and the matrix-core
    form (M >= 7) with K split over workgroups
    (workspace) or summed by one workgroup (none, or K too short to split),
    every output block shape (M=64, 256, 300: 1x1, 2x2, 4x2 tiles; 2048,
    2500: 4x3; 4100: 4x6), ragged token and row tiles,
    the largest K and the most rows (4096), an empty part; results repeat
    bit for bit."""
    ix = synth.indexer(M, K, key, heads, gate)
    print(f"[gpu] {ix.name} workspace={workspace}", flush=True)
    got = run_indexer(ix, "cached" if workspace else None)
    check_indexer(ix, got)
    again = run_indexer(ix, "cached" if workspace else None)
    assert all(np.array_equal(p, q) for p, q in zip(again, got)), "not repeatable"


def test_indexer_projection_object_matches_the_entry_point():
    """mhc.IndexerProjection (the page's class: the three weight parts held
    concatenated, called on x) gives the bits of mhcb_indexer_projection on
    the concatenated weight, in both forms (M = 3 and 40)."""
    for M in (3, 40):
        ix = synth.indexer(M, K=2048)
        w = dev(ix.w)
        proj = mhc.IndexerProjection(w[:ix.key], w[ix.key:ix.key + ix.heads], w[ix.key + ix.heads:])
        print(f"[gpu] {ix.name} through IndexerProjection", flush=True)
        got = proj(dev(ix.x))
        torch.cuda.synchronize()
        want = run_indexer(ix, "cached")
        assert np.array_equal(u16(got[0]), want[0]) and np.array_equal(host(got[1]), want[1])
        assert np.array_equal(u16(got[2]), want[2])


def test_indexer_workspace_reused_across_sizes():
    """One workspace, zeroed once, serves calls of different M in a row (the
    kernels leave its counters at zero, and no call's partials overlap the
    counters of another launch shape: M=300 writes partials where M=1100
    would keep counters 64..161 if the counter area followed the call's
    block count): each call matches a call on a fresh workspace bit for bit,
    and the oracle."""
    sizes = [1, 256, 16, 300, 1100, 1, 64]
    need = max(mhc.mhcb_indexer_workspace_bytes(M, 6144, 128, 32, 128) for M in sizes)
    shared = torch.empty(need, dtype=torch.uint8, device="cuda")
    mhc.mhcb_indexer_workspace_init(shared, need)
    for M in sizes:
        ix = synth.indexer(M)
        print(f"[gpu] {ix.name} on the shared workspace", flush=True)
        got = run_indexer(ix, shared)
        nbytes = max(mhc.mhcb_indexer_workspace_bytes(M, 6144, 128, 32, 128), 256)
        fresh = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        mhc.mhcb_indexer_workspace_init(fresh, nbytes)
        ref = run_indexer(ix, fresh)
        assert all(np.array_equal(p, q) for p, q in zip(got, ref)), f"M={M}: shared differs from fresh"
        check_indexer(ix, got)
