"""ctypes binding of libmhcb (include/mhcb.h).

Argument marshalling only: every step of the boundary runs in the library's
gfx950 kernels.  Torch tensors supply device memory and streams; a missing
library raises at import, and there is no fallback path.

The functions named ``mhcb_*`` mirror the C entry points one to one (tensor
or None for each pointer, the torch stream for ``hipStream_t``).  Above them,
``boundary``, ``boundary_glm``, ``finalize``, ``mixes`` and ``quant_mxfp8``
allocate outputs, and ``Mailbox`` / ``GlmBoundary`` hold the state the pages'
``AllReduceMHC`` / ``AllReduceMhcBoundary`` keep between calls.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libmhcb.so")

if not os.path.exists(LIBRARY_PATH):
    raise ImportError(
        f"{LIBRARY_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "(or python tp_reduce_mhc_amd/build.py)")

_lib = ctypes.CDLL(LIBRARY_PATH)

MHCB_OK, MHCB_EINVAL, MHCB_EALIGN, MHCB_EUNSUPPORTED, MHCB_ELAUNCH, MHCB_ETIMEOUT = range(6)
_NAMES = {1: "EINVAL", 2: "EALIGN", 3: "EUNSUPPORTED", 4: "ELAUNCH", 5: "ETIMEOUT"}


class MhcbError(RuntimeError):
    """A libmhcb call returned an error; ``code`` is the mhcb_status value."""

    def __init__(self, code: int, message: str):
        super().__init__(f"{_NAMES.get(code, code)}: {message}")
        self.code = code


class mhcb_mailbox(ctypes.Structure):
    _fields_ = [
        ("slots", ctypes.c_void_p),
        ("stage_state", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
        ("generations", ctypes.c_int),
        ("tp", ctypes.c_int),
        ("capacity", ctypes.c_int),
        ("hidden_size", ctypes.c_int),
        ("spin_limit", ctypes.c_int64),
    ]


_P, _I, _I64, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
_MB = ctypes.POINTER(mhcb_mailbox)

_SIGNATURES = {
    "mhcb_last_error": (ctypes.c_char_p, []),
    "mhcb_version": (ctypes.c_char_p, []),
    "mhcb_mxfp8_scale_bytes": (_I64, [_I64, _I64]),
    "mhcb_workspace_bytes": (_I64, [_I, _I, _I, _I]),
    "mhcb_finalize_workspace_bytes": (_I64, [_I, _I, _I, _I]),
    "mhcb_workspace_init": (_I, [_P, _I64, _P]),
    "mhcb_workspace_set_spin_limit": (_I, [_P, _I64, _P]),
    "mhcb_workspace_status": (_I, [_P, _P, _P]),
    "mhcb_set_token_slices": (_I, [_I]),
    "mhcb_boundary": (_I, [_P, _I64, _MB, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64,
                           _I, _I, _I, _I, _F, _P]),
    "mhcb_boundary_glm": (_I, [_P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64,
                               _I, _I, _I, _I, _F, _F, _F, _I, _P]),
    "mhcb_boundary_glm_noalloc": (_I, [_P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I,
                                       _I, _I, _F, _F, _F, _P]),
    "mhcb_mixes": (_I, [_P, _P, _P, _P, _P, _I, _I, _F, _F, _I, _P]),
    "mhcb_finalize": (_I, [_P, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _P, _P, _P, _P, _P,
                           _P, _P, _P, _I, _P, _I64, _I, _I, _I, _I, _I, _F, _P]),
    "mhcb_finalize_ex": (_I, [_P, _I64, _I64, _P, _I64, _I, _F, _P, _I64, _P, _I64, _P, _P, _P, _P,
                              _P, _P, _P, _P, _P, _I, _P, _I64, _I, _I, _I, _I, _I, _F, _P]),
    "mhcb_finalize_glm_workspace_bytes": (_I64, [_I, _I, _I]),
    "mhcb_finalize_glm": (_I, [_P, _I64, _I64, _P, _I64, _I, _F, _P, _I64, _P, _I64, _P, _P, _P,
                               _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _I, _F, _F,
                               _F, _P]),
    "mhcb_quant_mxfp8": (_I, [_P, _P, _P, _I, _I, _P]),
    "mhcb_indexer_workspace_bytes": (_I64, [_I, _I, _I, _I, _I]),
    "mhcb_indexer_workspace_init": (_I, [_P, _I64, _P]),
    "mhcb_indexer_projection": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _I, _P]),
    "mhcb_mailbox_init": (_I, [_MB, _P]),
    "mhcb_publish": (_I, [_MB, _P, _I64, _I, _I, _I, _P]),
    "mhcb_mailbox_status": (_I, [_MB, _P, _P]),
}

for _name, (_res, _args) in _SIGNATURES.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGNATURES)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int) -> None:
    if rc != MHCB_OK:
        raise MhcbError(rc, mhcb_last_error())


def _mb(mailbox):
    if mailbox is None:
        return None
    return ctypes.byref(mailbox.struct if isinstance(mailbox, Mailbox) else mailbox)


# ---------------------------------------------------------------------------
# One-to-one entry points
# ---------------------------------------------------------------------------

def mhcb_last_error() -> str:
    return _lib.mhcb_last_error().decode()


def mhcb_version() -> str:
    return _lib.mhcb_version().decode()


def mhcb_mxfp8_scale_bytes(M: int, hidden_size: int) -> int:
    return _lib.mhcb_mxfp8_scale_bytes(M, hidden_size)


def mhcb_workspace_bytes(M: int, hidden_size: int, tp: int, two_shot: int) -> int:
    return _lib.mhcb_workspace_bytes(M, hidden_size, tp, int(two_shot))


def mhcb_finalize_workspace_bytes(M: int, hidden_size: int, tp: int, two_shot: int) -> int:
    return _lib.mhcb_finalize_workspace_bytes(M, hidden_size, tp, int(two_shot))


def mhcb_workspace_init(workspace, workspace_bytes, stream=None) -> None:
    _check(_lib.mhcb_workspace_init(_ptr(workspace), workspace_bytes, _stream(stream)))


def mhcb_workspace_set_spin_limit(workspace, spin_limit, stream=None) -> None:
    _check(_lib.mhcb_workspace_set_spin_limit(_ptr(workspace), spin_limit, _stream(stream)))


def mhcb_workspace_status(workspace, status_out, stream=None) -> None:
    """Enqueues a copy of the workspace's time-out count into status_out
    (a one-element int32/uint32 device tensor); never synchronizes."""
    _check(_lib.mhcb_workspace_status(_ptr(workspace), _ptr(status_out), _stream(stream)))


def workspace_status(workspace, stream=None) -> int:
    """MHCB_OK, or raises MhcbError(ETIMEOUT) when a cross-workgroup wait of
    a call on `workspace` gave up.  Waits for `stream` (the helper reads the
    copied word on the host)."""
    out = torch.zeros(1, dtype=torch.int32, device=workspace.device)
    mhcb_workspace_status(workspace, out, stream)
    n = int(out.item())
    if n:
        raise MhcbError(MHCB_ETIMEOUT, f"{n} cross-workgroup wait(s) gave up")
    return MHCB_OK


def mhcb_set_token_slices(slices: int) -> int:
    """Per calling thread (the library keeps the setting thread-local)."""
    return _lib.mhcb_set_token_slices(slices)


def mhcb_boundary(partials, rank_stride, mailbox, residual, post, comb, pre, norm_weight,
                  residual_out, layer_input, mxfp8_values, mxfp8_scales, workspace, workspace_bytes,
                  M, hidden_size, hc_mult, tp, norm_eps, stream=None) -> None:
    _check(_lib.mhcb_boundary(_ptr(partials), rank_stride, _mb(mailbox), _ptr(residual), _ptr(post),
                              _ptr(comb), _ptr(pre), _ptr(norm_weight), _ptr(residual_out),
                              _ptr(layer_input), _ptr(mxfp8_values), _ptr(mxfp8_scales),
                              _ptr(workspace), workspace_bytes, M, hidden_size, hc_mult, tp,
                              norm_eps, _stream(stream)))


def mhcb_boundary_glm(partials, rank_stride, residual, post, comb, hc_fn, scale, base, norm_weight,
                      residual_out, mixes_out, layer_input, workspace, workspace_bytes, M,
                      hidden_size, hc_mult, tp, rms_eps, hc_eps, norm_eps, tokens_per_wg=0,
                      stream=None) -> None:
    _check(_lib.mhcb_boundary_glm(_ptr(partials), rank_stride, _ptr(residual), _ptr(post), _ptr(comb),
                                  _ptr(hc_fn), _ptr(scale), _ptr(base), _ptr(norm_weight),
                                  _ptr(residual_out), _ptr(mixes_out), _ptr(layer_input),
                                  _ptr(workspace), workspace_bytes, M, hidden_size, hc_mult, tp,
                                  rms_eps, hc_eps, norm_eps, tokens_per_wg, _stream(stream)))


def mhcb_boundary_glm_noalloc(partials, rank_stride, residual, post, comb, hc_fn, scale, base,
                              norm_weight, residual_out, mixes_out, layer_input, M, hidden_size,
                              hc_mult, tp, rms_eps, hc_eps, norm_eps, stream=None) -> None:
    _check(_lib.mhcb_boundary_glm_noalloc(_ptr(partials), rank_stride, _ptr(residual), _ptr(post),
                                          _ptr(comb), _ptr(hc_fn), _ptr(scale), _ptr(base),
                                          _ptr(norm_weight), _ptr(residual_out), _ptr(mixes_out),
                                          _ptr(layer_input), M, hidden_size, hc_mult, tp, rms_eps,
                                          hc_eps, norm_eps, _stream(stream)))


def mhcb_mixes(mixes, scale, base, post_out, comb_out, M, hc_mult, hc_eps, post_mult,
               sinkhorn_repeat, stream=None) -> None:
    _check(_lib.mhcb_mixes(_ptr(mixes), _ptr(scale), _ptr(base), _ptr(post_out), _ptr(comb_out), M,
                           hc_mult, hc_eps, post_mult, sinkhorn_repeat, _stream(stream)))


def mhcb_finalize(gemm2_permuted, gemm2_rank_stride, rows, expert_weights, weights_rank_stride,
                  permuted_idx, idx_rank_stride, shared_output, shared_rank_stride, residual, post,
                  comb, pre, norm_weight, residual_out, layer_input, mxfp8_values, mxfp8_scales,
                  two_shot, workspace, workspace_bytes, M, hidden_size, hc_mult, tp, top_k,
                  norm_eps, stream=None) -> None:
    _check(_lib.mhcb_finalize(_ptr(gemm2_permuted), gemm2_rank_stride, rows, _ptr(expert_weights),
                              weights_rank_stride, _ptr(permuted_idx), idx_rank_stride,
                              _ptr(shared_output), shared_rank_stride, _ptr(residual), _ptr(post),
                              _ptr(comb), _ptr(pre), _ptr(norm_weight), _ptr(residual_out),
                              _ptr(layer_input), _ptr(mxfp8_values), _ptr(mxfp8_scales),
                              int(two_shot), _ptr(workspace), workspace_bytes, M, hidden_size,
                              hc_mult, tp, top_k, norm_eps, _stream(stream)))

def mhcb_finalize_ex(gemm2_permuted, gemm2_rank_stride, rows, expert_weights, weights_rank_stride,
                     weights_bf16, routed_scaling_factor, permuted_idx, idx_rank_stride,
                     shared_output, shared_rank_stride, residual, post, comb, pre, norm_weight,
                     residual_out, layer_input, mxfp8_values, mxfp8_scales, two_shot, workspace,
                     workspace_bytes, M, hidden_size, hc_mult, tp, top_k, norm_eps,
                     stream=None) -> None:
    _check(_lib.mhcb_finalize_ex(_ptr(gemm2_permuted), gemm2_rank_stride, rows,
                                 _ptr(expert_weights), weights_rank_stride, int(weights_bf16),
                                 routed_scaling_factor, _ptr(permuted_idx), idx_rank_stride,
                                 _ptr(shared_output), shared_rank_stride, _ptr(residual),
                                 _ptr(post), _ptr(comb), _ptr(pre), _ptr(norm_weight),
                                 _ptr(residual_out), _ptr(layer_input), _ptr(mxfp8_values),
                                 _ptr(mxfp8_scales), int(two_shot), _ptr(workspace),
                                 workspace_bytes, M, hidden_size, hc_mult, tp, top_k, norm_eps,
                                 _stream(stream)))


def mhcb_quant_mxfp8(x, values, scales, M, hidden_size, stream=None) -> None:
    _check(_lib.mhcb_quant_mxfp8(_ptr(x), _ptr(values), _ptr(scales), M, hidden_size,
                                 _stream(stream)))


def mhcb_indexer_workspace_bytes(M: int, K: int, key_rows: int, heads: int, gate_rows: int) -> int:
    n = _lib.mhcb_indexer_workspace_bytes(M, K, key_rows, heads, gate_rows)
    if n < 0:
        raise MhcbError(MHCB_EINVAL, mhcb_last_error())
    return n


def mhcb_indexer_workspace_init(workspace, nbytes: int, stream=None) -> None:
    _check(_lib.mhcb_indexer_workspace_init(_ptr(workspace), nbytes, _stream(stream)))


def mhcb_indexer_projection(x, weight, key_out, heads_out, gate_out, workspace, workspace_bytes,
                            M, K, key_rows, heads, gate_rows, stream=None) -> None:
    _check(_lib.mhcb_indexer_projection(_ptr(x), _ptr(weight), _ptr(key_out), _ptr(heads_out),
                                        _ptr(gate_out), _ptr(workspace), workspace_bytes, M, K,
                                        key_rows, heads, gate_rows, _stream(stream)))


_indexer_workspaces: dict = {}


def indexer_workspace(nbytes: int, device=None, stream=None):
    """The zeroed indexer workspace of (device, stream), grown to the
    largest size asked for so far (a new one is zeroed on `stream`; the
    kernels leave the counters at zero).  Growth keeps the replaced buffer
    alive, as ``workspace`` does."""
    dev = torch.device(device if device is not None else "cuda")
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())

    def make(size):
        ws = _alloc_on(size, dev, stream)
        mhcb_indexer_workspace_init(ws, ws.numel(), stream)
        return ws

    return _cached(_indexer_workspaces, (dev.index, _stream(stream) or 0), max(nbytes, 256), make)


def indexer_projection(x, weight, key_rows: int, heads: int, gate_rows: int, *, stream=None):
    """DSA indexer projection of x [M, K] (BF16) with weight [key_rows + heads
    + gate_rows, K] (BF16); returns (key [M, key_rows] BF16, head weights
    [M, heads] FP32, gate [M, gate_rows] BF16)."""
    M, K = x.shape
    dev = x.device
    key = _bf16_empty((M, key_rows), dev)
    w = torch.empty((M, heads), dtype=torch.float32, device=dev)
    gate = _bf16_empty((M, gate_rows), dev)
    nbytes = mhcb_indexer_workspace_bytes(M, K, key_rows, heads, gate_rows)
    ws = indexer_workspace(nbytes, dev, stream) if nbytes > 0 else None
    mhcb_indexer_projection(x, weight, key, w, gate, ws, nbytes, M, K, key_rows, heads, gate_rows,
                            stream)
    return key, w, gate


def mhcb_mailbox_init(mailbox, stream=None) -> None:
    _check(_lib.mhcb_mailbox_init(_mb(mailbox), _stream(stream)))


def mhcb_publish(mailbox, partials, rank_stride, rank_begin, rank_count, M, stream=None) -> None:
    _check(_lib.mhcb_publish(_mb(mailbox), _ptr(partials), rank_stride, rank_begin, rank_count, M,
                             _stream(stream)))


def mhcb_mailbox_status(mailbox, status_out, stream=None) -> None:
    """Enqueues a copy of the mailbox's two status words (poll time-outs,
    late fragments) into status_out (two int32 on the device)."""
    _check(_lib.mhcb_mailbox_status(_mb(mailbox), _ptr(status_out), _stream(stream)))


def mailbox_status(mailbox, stream=None):
    """(poll time-outs, late fragments) since mhcb_mailbox_init; waits for
    `stream`."""
    m = mailbox.struct if isinstance(mailbox, Mailbox) else mailbox
    device = mailbox.status.device if isinstance(mailbox, Mailbox) else "cuda"
    out = torch.zeros(2, dtype=torch.int32, device=device)
    _check(_lib.mhcb_mailbox_status(ctypes.byref(m), _ptr(out), _stream(stream)))
    timeouts, late = (int(v) for v in out.tolist())
    return timeouts, late


# ---------------------------------------------------------------------------
# Allocating helpers (outputs are fresh tensors, as on the pages)
# ---------------------------------------------------------------------------

def _bf16_empty(shape, device):
    return torch.empty(shape, dtype=torch.bfloat16, device=device)


_WORKSPACES = {}
# Buffers a cache has replaced: a graph captured with one, or a call still
# queued on another stream, keeps using it, so it is never handed back to
# torch's allocator.  Growth at least doubles, so together they are never
# larger than the buffer that replaced them.
_RETIRED: list = []


def _alloc_on(nbytes: int, device, stream) -> torch.Tensor:
    """nbytes of device memory allocated for `stream` (torch's allocator
    then orders its reuse after the work queued there)."""
    if stream is not None and not isinstance(stream, int):
        with torch.cuda.stream(stream):
            return torch.empty(nbytes, dtype=torch.uint8, device=device)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _cached(cache: dict, key, need: int, make) -> torch.Tensor:
    ws = cache.get(key)
    if ws is None or ws.numel() < need:
        if ws is not None:
            need = max(need, 2 * ws.numel())
            _RETIRED.append(ws)
        ws = make(need)
        cache[key] = ws
    return ws


def workspace(device=None, *, M: int = 0, hidden_size: int = 0, tp: int = 1,
              two_shot: bool = False, nbytes: int = 0, stream=None) -> torch.Tensor:
    """An initialized workspace of at least the size the arguments ask for
    (mhcb_workspace_bytes, or nbytes if larger), one per (device, stream):
    calls on one stream are ordered, so they may share it, and calls on
    different streams get different ones.  The cached workspace only grows:
    a larger request replaces it with one at least twice its size
    (allocated and initialized on `stream`); the replaced one stays
    allocated, so memory stays within twice the largest call's."""
    device = torch.device(device if device is not None else "cuda")
    if device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    need = max(mhcb_workspace_bytes(M, hidden_size, tp, int(two_shot)), nbytes)
    return _cached(_WORKSPACES, (device.index, _stream(stream) or 0), need,
                   lambda size: new_workspace(size, device, stream))


def new_workspace(nbytes: int, device, stream=None) -> torch.Tensor:
    """A fresh workspace of `nbytes` (256-byte aligned by torch), allocated
    for and initialized by mhcb_workspace_init on `stream` (the current
    stream by default)."""
    ws = _alloc_on(nbytes, device, stream)
    mhcb_workspace_init(ws, nbytes, stream)
    return ws


def boundary(partials: torch.Tensor, residual, post, comb, pre, norm_weight, norm_eps: float,
             *, mxfp8: bool = False, split: bool = True, stream=None):
    """Delayed-mHC boundary on resident partials [tp, M, H] (BF16).  With
    split (default) the cached workspace lets small-M calls spread tokens
    over several workgroups.

    residual [M, hc, H] with hc = 1, 2, 4 or 8.
    Returns (residual_out [M,hc,H], layer_input [M,H] or None,
    (values [M,H] u8, scales u8) or None)."""
    tp, M, H = partials.shape
    hc = residual.shape[1]
    dev = partials.device
    ws = workspace(dev, stream=stream) if split else None
    residual_out = _bf16_empty((M, hc, H), dev)
    layer_input = None if pre is None else _bf16_empty((M, H), dev)
    values = scales = None
    if mxfp8:
        values = torch.empty((M, H), dtype=torch.uint8, device=dev)
        scales = torch.empty(mhcb_mxfp8_scale_bytes(M, H), dtype=torch.uint8, device=dev)
    mhcb_boundary(partials, M * H if tp > 1 else 0, None, residual, post, comb, pre, norm_weight,
                  residual_out, layer_input, values, scales, ws, ws.numel() if ws is not None else 0,
                  M, H, hc, tp, norm_eps, stream)
    return residual_out, layer_input, ((values, scales) if mxfp8 else None)


def boundary_glm(partials, residual, post, comb, hc_fn, scale, base, norm_weight, rms_eps, hc_eps,
                 norm_eps, *, tokens_per_wg: int = 0, stream=None):
    """GLM boundary; returns (residual_out, mixes [M,24] FP32, layer_input)."""
    tp, M, H = partials.shape
    dev = partials.device
    residual_out = _bf16_empty((M, 4, H), dev)
    mixes = torch.empty((M, 24), dtype=torch.float32, device=dev)
    layer_input = _bf16_empty((M, H), dev)
    ws = workspace(dev, stream=stream)
    mhcb_boundary_glm(partials, M * H if tp > 1 else 0, residual, post, comb, hc_fn, scale, base,
                      norm_weight, residual_out, mixes, layer_input, ws, ws.numel(), M, H, 4, tp,
                      rms_eps, hc_eps, norm_eps, tokens_per_wg, stream)
    return residual_out, mixes, layer_input


def mhcb_finalize_glm_workspace_bytes(M: int, hidden_size: int, tp: int) -> int:
    return _lib.mhcb_finalize_glm_workspace_bytes(M, hidden_size, tp)


def mhcb_finalize_glm(gemm2_permuted, gemm2_rank_stride, rows, expert_weights, weights_rank_stride,
                      weights_bf16, routed_scaling_factor, permuted_idx, idx_rank_stride,
                      shared_output, shared_rank_stride, residual, post, comb, hc_fn, scale, base,
                      norm_weight, residual_out, mixes_out, layer_input, workspace,
                      workspace_bytes, M, hidden_size, hc_mult, tp, top_k, rms_eps, hc_eps,
                      norm_eps, stream=None) -> None:
    _check(_lib.mhcb_finalize_glm(_ptr(gemm2_permuted), gemm2_rank_stride, rows,
                                  _ptr(expert_weights), weights_rank_stride, int(weights_bf16),
                                  routed_scaling_factor, _ptr(permuted_idx), idx_rank_stride,
                                  _ptr(shared_output), shared_rank_stride, _ptr(residual),
                                  _ptr(post), _ptr(comb), _ptr(hc_fn), _ptr(scale), _ptr(base),
                                  _ptr(norm_weight), _ptr(residual_out), _ptr(mixes_out),
                                  _ptr(layer_input), _ptr(workspace), workspace_bytes, M,
                                  hidden_size, hc_mult, tp, top_k, rms_eps, hc_eps, norm_eps,
                                  _stream(stream)))


def finalize_glm(gemm2, weights, idx, shared, residual, post, comb, hc_fn, scale, base,
                 norm_weight, rms_eps, hc_eps, norm_eps, *, routed_scaling_factor: float = 1.0,
                 stream=None):
    """GLM boundary of an MoE sublayer.  gemm2 [tp, rows, H]; shared
    [tp, M, H]; weights (FP32 or BF16) / idx [M, top_k] (replicated) or
    [tp, M, top_k]; the rest as boundary_glm.  Returns (residual_out
    [M,4,H], raw mixes [M,24], layer_input [M,H])."""
    tp, rows, H = gemm2.shape
    M = shared.shape[1]
    top_k = weights.shape[-1]
    dev = gemm2.device
    per_rank = weights.dim() == 3
    residual_out = _bf16_empty((M, 4, H), dev)
    mixes_out = torch.empty((M, 24), dtype=torch.float32, device=dev)
    layer_input = _bf16_empty((M, H), dev)
    ws = workspace(dev, nbytes=mhcb_finalize_glm_workspace_bytes(M, H, tp), stream=stream)
    mhcb_finalize_glm(gemm2, rows * H, rows, weights, M * top_k if per_rank else 0,
                      weights.dtype == torch.bfloat16, routed_scaling_factor, idx,
                      M * top_k if per_rank else 0, shared, M * H, residual, post, comb, hc_fn,
                      scale, base, norm_weight, residual_out, mixes_out, layer_input, ws,
                      ws.numel(), M, H, 4, tp, top_k, rms_eps, hc_eps, norm_eps, stream)
    return residual_out, mixes_out, layer_input


def mixes(raw_mixes, scale, base, hc_eps, post_mult, sinkhorn_repeat, *, stream=None):
    """Side-stream mixes; returns (post [M,4,1], comb [M,4,4]) FP32."""
    M = raw_mixes.shape[0]
    dev = raw_mixes.device
    post = torch.empty((M, 4, 1), dtype=torch.float32, device=dev)
    comb = torch.empty((M, 4, 4), dtype=torch.float32, device=dev)
    mhcb_mixes(raw_mixes, scale, base, post, comb, M, 4, hc_eps, post_mult, sinkhorn_repeat, stream)
    return post, comb


def finalize(gemm2, weights, idx, shared, residual, post, comb, pre, norm_weight, norm_eps, *,
             two_shot: bool = False, mxfp8: bool = False, split: bool = True,
             routed_scaling_factor: float = 1.0, stream=None):
    """MoE finalize boundary.  gemm2 [tp, rows, H]; shared [tp, M, H];
    weights (FP32 or BF16) / idx [M, top_k] (replicated) or [tp, M, top_k];
    residual [M, hc, H] (hc = 1, 2, 4 or 8)."""
    tp, rows, H = gemm2.shape
    M = shared.shape[1]
    hc = residual.shape[1]
    top_k = weights.shape[-1]
    dev = gemm2.device
    per_rank = weights.dim() == 3
    residual_out = _bf16_empty((M, hc, H), dev)
    layer_input = None if pre is None else _bf16_empty((M, H), dev)
    values = scales = None
    if mxfp8:
        values = torch.empty((M, H), dtype=torch.uint8, device=dev)
        scales = torch.empty(mhcb_mxfp8_scale_bytes(M, H), dtype=torch.uint8, device=dev)
    ws = (workspace(dev, M=M, hidden_size=H, tp=tp, two_shot=two_shot, stream=stream)
          if (two_shot or split) else None)
    mhcb_finalize_ex(gemm2, rows * H, rows, weights, M * top_k if per_rank else 0,
                     weights.dtype == torch.bfloat16, routed_scaling_factor, idx,
                     M * top_k if per_rank else 0, shared, M * H, residual, post, comb, pre,
                     norm_weight, residual_out, layer_input, values, scales, two_shot, ws,
                     ws.numel() if ws is not None else 0, M, H, hc, tp, top_k, norm_eps, stream)
    return residual_out, layer_input, ((values, scales) if mxfp8 else None)


def quant_mxfp8(x, *, stream=None):
    M, H = x.shape
    values = torch.empty((M, H), dtype=torch.uint8, device=x.device)
    scales = torch.empty(mhcb_mxfp8_scale_bytes(M, H), dtype=torch.uint8, device=x.device)
    mhcb_quant_mxfp8(x, values, scales, M, H, stream)
    return values, scales


class Mailbox:
    """A three-generation Lamport mailbox in device memory (slots, stage
    state, status) with its mhcb_mailbox descriptor."""

    def __init__(self, tp: int, capacity: int, hidden_size: int, device, spin_limit: int = 0):
        self.slots = torch.empty((3, tp, capacity, hidden_size), dtype=torch.bfloat16, device=device)
        self.stage_state = torch.zeros(2, dtype=torch.int32, device=device)
        self.status = torch.zeros(2, dtype=torch.int32, device=device)
        self.struct = mhcb_mailbox(self.slots.data_ptr(), self.stage_state.data_ptr(),
                                   self.status.data_ptr(), 3, tp, capacity, hidden_size, spin_limit)
        self.tp, self.capacity, self.hidden_size = tp, capacity, hidden_size

    def init(self, stream=None) -> None:
        mhcb_mailbox_init(self, stream)

    def publish(self, partials: torch.Tensor, rank_begin: int = 0, stream=None) -> None:
        """Publishes ranks [rank_begin, rank_begin + n) from partials [n, M, H]."""
        n, M, H = partials.shape
        mhcb_publish(self, partials, M * H, rank_begin, n, M, stream)

    def boundary(self, M, residual, post, comb, pre, norm_weight, norm_eps, *, mxfp8=False,
                 stream=None):
        """The consumer: the delayed-mHC boundary fed from this mailbox
        (residual [M, hc, H], hc = 1, 2, 4 or 8)."""
        H, hc = self.hidden_size, residual.shape[1]
        dev = residual.device
        residual_out = _bf16_empty((M, hc, H), dev)
        layer_input = None if pre is None else _bf16_empty((M, H), dev)
        values = scales = None
        if mxfp8:
            values = torch.empty((M, H), dtype=torch.uint8, device=dev)
            scales = torch.empty(mhcb_mxfp8_scale_bytes(M, H), dtype=torch.uint8, device=dev)
        ws = workspace(dev, stream=stream)
        mhcb_boundary(None, 0, self, residual, post, comb, pre, norm_weight, residual_out,
                      layer_input, values, scales, ws, ws.numel(), M, H, hc, self.tp, norm_eps,
                      stream)
        return residual_out, layer_input, ((values, scales) if mxfp8 else None)

    def peer_view(self) -> "Mailbox":
        """A second descriptor of the same slots with its own stage state and
        status words: the view a peer rank publishes through (on the pages
        each rank advances its own stage state)."""
        peer = Mailbox.__new__(Mailbox)
        peer.slots = self.slots
        peer.stage_state = torch.zeros_like(self.stage_state)
        peer.status = torch.zeros_like(self.status)
        peer.struct = mhcb_mailbox(self.slots.data_ptr(), peer.stage_state.data_ptr(),
                                   peer.status.data_ptr(), 3, self.tp, self.capacity,
                                   self.hidden_size, self.struct.spin_limit)
        peer.tp, peer.capacity, peer.hidden_size = self.tp, self.capacity, self.hidden_size
        return peer

    def status_ok(self, stream=None) -> bool:
        """True when no consumer poll of this mailbox gave up; waits for `stream`."""
        return mailbox_status(self, stream)[0] == 0


class IndexerProjection:
    """The DSA indexer projection over fixed weights (the indexer page's
    IndexerProjection): the key rows [key_rows, K], the head-weight rows
    [heads, K] and the kpool gate rows [gate_rows, K] (BF16) held as one
    concatenated [key_rows + heads + gate_rows, K] matrix; calling it on the
    layer input x [M, K] returns (key [M, key_rows] BF16, head weights
    [M, heads] FP32, gate [M, gate_rows] BF16)."""

    def __init__(self, key_weight, head_weight, gate_weight):
        parts = (key_weight, head_weight, gate_weight)
        if any(w.dtype != torch.bfloat16 or w.dim() != 2 for w in parts):
            raise ValueError("indexer weights must be 2-D BF16 tensors")
        K = key_weight.shape[1]
        if any(w.shape[1] != K for w in parts):
            raise ValueError("indexer weights must share K")
        self.key, self.heads, self.gate = (w.shape[0] for w in parts)
        self.weight = torch.cat(parts).contiguous()

    def __call__(self, x, *, stream=None):
        if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != self.weight.shape[1]:
            raise ValueError("x must be a BF16 [M, K] tensor with the weights' K")
        return indexer_projection(x.contiguous(), self.weight, self.key, self.heads, self.gate,
                                  stream=stream)


class GlmBoundary:
    """The GLM boundary with its side stream: each call runs the boundary on
    the current stream and the post/Sinkhorn mixes on a side stream; `join`
    makes the current stream wait for the last mixes (AllReduceMhcBoundary
    .__call__ / .join on the GLM page)."""

    def __init__(self, *, rms_eps: float, hc_eps: float, post_mult: float, sinkhorn_repeat: int,
                 norm_eps: float, device):
        self.rms_eps, self.hc_eps, self.norm_eps = rms_eps, hc_eps, norm_eps
        self.post_mult, self.sinkhorn_repeat = post_mult, sinkhorn_repeat
        self._side = torch.cuda.Stream(device)
        self._pending = None
        self._in_flight = None

    def join(self) -> None:
        if self._pending is not None:
            torch.cuda.current_stream().wait_event(self._pending)
            self._pending = self._in_flight = None

    def __call__(self, partials, residual, post, comb, hc_fn, scale, base, norm_weight,
                 tokens_per_wg: int = 0):
        self.join()
        residual_out, raw, layer_input = boundary_glm(
            partials, residual, post, comb, hc_fn, scale, base, norm_weight, self.rms_eps,
            self.hc_eps, self.norm_eps, tokens_per_wg=tokens_per_wg)
        M = raw.shape[0]
        # Outputs are allocated on the current stream (their consumer's), and
        # the raw mixes are kept alive until the side kernel is joined.
        post_next = torch.empty((M, 4, 1), dtype=torch.float32, device=raw.device)
        comb_next = torch.empty((M, 4, 4), dtype=torch.float32, device=raw.device)
        self._side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(self._side):
            mhcb_mixes(raw, scale, base, post_next, comb_next, M, 4, self.hc_eps, self.post_mult,
                       self.sinkhorn_repeat)
            self._pending = torch.cuda.Event()
            self._pending.record()
        self._in_flight = raw
        return residual_out, post_next, comb_next, layer_input, raw
