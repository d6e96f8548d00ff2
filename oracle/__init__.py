"""The oracle: a plain CPU implementation of the fused TP-reduce + mHC +
RMSNorm sublayer boundary, used to check the HIP path.

TEST INFRASTRUCTURE, NOT THE PRODUCT.  Only the test suite, the smoke check
(``__graft_entry__.smoke``) and the benchmark's ``cpu_baseline`` leg may
import this package.  It shares no code with ``tp_reduce_mhc_amd`` and never
imports it.  The arithmetic lives in ``mhcb_oracle.c`` (built by
``oracle/build.py`` into ``liboracle.so``); this module only marshals numpy
arrays.  BF16 arrays are ``numpy.uint16`` bit patterns.

Sources (web pages, cited by title and section in ``mhcb_oracle.c``):
  vllm.models.glm5next.nvidia.specialized_decode.all_reduce_mhc        (GLM)
  vllm.models.deepseek_v41.nvidia.ops.cute_dsl.all_reduce_mhc          (DSV4.1)
  vllm.models.glm5next.nvidia.specialized_decode.indexer               (indexer)

Every function here is pinned by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MHCB_ORACLE_LIB points the checker at another build of mhcb_oracle.c (the
# mutation test loads deliberately broken copies this way, on the CPU).
_LIB_PATH = os.environ.get("MHCB_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float

_SIGNATURES = {
    "oracle_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
    "oracle_f32_to_bf16": (ctypes.c_uint16, [_F]),
    "oracle_rcp": (_F, [_F]),
    "oracle_exp": (_F, [_F]),
    "oracle_sigmoid": (_F, [_F]),
    "oracle_rank_sum": (ctypes.c_uint16, [_P, _I64, _I, _I64]),
    "oracle_e4m3_value": (ctypes.c_double, [ctypes.c_uint8]),
    "oracle_e4m3_rne_sat": (ctypes.c_uint8, [_F]),
    "oracle_ue8m0_round_up": (ctypes.c_uint8, [_F]),
    "oracle_sf_index": (_I64, [_I64, _I64, _I64]),
    "oracle_mxfp8_scale_bytes": (_I64, [_I64, _I64]),
    "oracle_boundary": (_I, [_P, _I64, _I, _P, _P, _P, _P, _P, _F, _I, _I, _I, _P, _P, _P, _P, _I]),
    "oracle_finalize_element": (ctypes.c_uint16, [_P, _I64, _P, _P, _P, _I, _I64, _I, _I]),
    "oracle_finalize_contributions": (
        _I, [_P, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _I, _I, _I, _I, _P, _I]),
    "oracle_two_shot_publish": (None, [_P, _I, _I, _I, _P]),
    "oracle_owner_reduce": (None, [_P, _I, _I, _I, _P]),
    "oracle_finalize": (
        _I, [_P, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _I, _I,
             _P, _P, _P, _P, _P, _F, _I, _I, _I, _I, _P, _P, _P, _P, _I]),
    "oracle_glm_mixes_token": (None, [_P, _P, _P, _P, _I, _F, _F, _P, _P]),
    "oracle_glm_pre": (None, [_P, _P, _P, _F, _P]),
    "oracle_glm_collapse_rmsnorm": (_I, [_P, _P, _P, _I, _F, _P]),
    "oracle_boundary_glm": (
        _I, [_P, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _F, _F, _F, _I, _I, _P, _P, _P, _P, _I]),
    "oracle_sinkhorn": (None, [_P, _F, _I, _P]),
    "oracle_side_mixes": (_I, [_P, _P, _P, _I, _F, _F, _I, _P, _P]),
    "oracle_quant_mxfp8": (_I, [_P, _I, _I, _P, _P]),
    "oracle_indexer_projection": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P]),
}


def lib():
    """Loads liboracle.so (building it with gcc if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def default_threads() -> int:
    """Threads for the token-parallel composites: OMP_NUM_THREADS if set,
    else every host core."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return os.cpu_count() or 1


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what}: oracle rejected the arguments (status {rc})")


# ---------------------------------------------------------------------------
# Scalars and element-wise helpers
# ---------------------------------------------------------------------------

def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widens BF16 bit patterns to float32 (exact)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x) -> np.ndarray:
    """Rounds float32 values to BF16 (nearest, ties to even), element by element."""
    x = np.asarray(x, dtype=np.float32)
    f = lib().oracle_f32_to_bf16
    out = np.fromiter((f(float(v)) for v in x.ravel()), dtype=np.uint16, count=x.size)
    return out.reshape(x.shape)


def e4m3_rne_sat(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    f = lib().oracle_e4m3_rne_sat
    return np.fromiter((f(float(v)) for v in x.ravel()), dtype=np.uint8, count=x.size).reshape(x.shape)


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(code)


def ue8m0_round_up(v: float) -> int:
    return lib().oracle_ue8m0_round_up(v)


def sf_index(r: int, k: int, K: int) -> int:
    return lib().oracle_sf_index(r, k, K)


def mxfp8_scale_bytes(M: int, H: int) -> int:
    return lib().oracle_mxfp8_scale_bytes(M, H)


def sigmoid(x: float) -> float:
    return lib().oracle_sigmoid(x)


def rank_sum_element(partials: np.ndarray, element: int) -> int:
    """a1 for one flattened element of a [tp, ...] BF16 stack."""
    p = _c(partials, np.uint16)
    tp = p.shape[0]
    stride = p[0].size
    return lib().oracle_rank_sum(_ptr(p), stride, tp, element)


# ---------------------------------------------------------------------------
# Composite steps
# ---------------------------------------------------------------------------

def boundary(partials, residual, post, comb, pre, gamma, norm_eps, *, mxfp8=False,
             threads=1):
    """Delayed-mHC boundary (a1, a2, a4, optional a8).

    partials [tp, M, H] u16; residual [M, hc, H] u16 (hc = 1..8, from its
    shape); post, pre [M, hc] f32; comb [M, hc, hc] f32 [source, target];
    gamma [H] u16.  pre=None and gamma=None select the residual-only variant.
    Returns (residual_out, layer_input or None, (values, scales) or None).
    """
    partials = _c(partials, np.uint16)
    tp, M, H = partials.shape
    residual = _c(residual, np.uint16).reshape(M, -1, H)
    hc = residual.shape[1]
    post = _c(post, np.float32).reshape(M, hc)
    comb = _c(comb, np.float32).reshape(M, hc, hc)
    pre = None if pre is None else _c(pre, np.float32).reshape(M, hc)
    gamma = None if gamma is None else _c(gamma, np.uint16).reshape(H)
    res_out = np.empty((M, hc, H), np.uint16)
    layer = None if pre is None else np.empty((M, H), np.uint16)
    values = scales = None
    if mxfp8:
        values = np.empty((M, H), np.uint8)
        scales = np.full(mxfp8_scale_bytes(M, H), 0xAA, np.uint8)
    rc = lib().oracle_boundary(_ptr(partials), M * H, tp, _ptr(residual), _ptr(post), _ptr(comb),
                               _ptr(pre), _ptr(gamma), norm_eps, M, H, hc, _ptr(res_out),
                               _ptr(layer), _ptr(values), _ptr(scales), threads)
    _check(rc, "boundary")
    return res_out, layer, (None if not mxfp8 else (values, scales))


def routing_weights(weights, routed_scaling_factor=1.0) -> np.ndarray:
    """[DSV41] _QuadFinalizePublishDeviceKernel (the routing-weight load; the
    module compiles one kernel per routing-weight dtype, AllReduceMHC.__init__):
    each route's weight is read as FP32, or as BF16 widened to FP32; when the
    routed scaling factor is not 1 it is then multiplied by that factor (an
    FP32 product, one rounding).  A route whose row index is -1 is skipped by
    the contribution itself.

    weights: float32 values, or uint16 BF16 bit patterns.  Returns float32."""
    w = np.asarray(weights)
    if w.dtype == np.uint16:
        w32 = bf16_to_f32(w)
    elif w.dtype == np.float32:
        w32 = w.copy()
    else:
        raise TypeError(f"routing weights must be float32 or BF16 bits (uint16), not {w.dtype}")
    if float(routed_scaling_factor) != 1.0:
        w32 = (w32 * np.float32(routed_scaling_factor)).astype(np.float32)
    return w32


def finalize_contributions(gemm2, weights, idx, shared, *, replicated_routing=True,
                           routed_scaling_factor=1.0, threads=1):
    """a6 contributions of every rank.

    gemm2 [tp, rows, H] u16; shared [tp, M, H] u16; weights [M, top_k] (f32,
    or u16 BF16 bits: routing_weights) and idx [M, top_k] i32 when
    replicated_routing, else [tp, M, top_k].  Returns [tp, M, H] u16.
    """
    gemm2 = _c(gemm2, np.uint16)
    shared = _c(shared, np.uint16)
    tp, rows, H = gemm2.shape
    M = shared.shape[1]
    weights = np.ascontiguousarray(routing_weights(weights, routed_scaling_factor))
    idx = _c(idx, np.int32)
    top_k = weights.shape[-1]
    ws = 0 if replicated_routing else M * top_k
    out = np.empty((tp, M, H), np.uint16)
    rc = lib().oracle_finalize_contributions(_ptr(gemm2), rows * H, rows, _ptr(weights), ws, _ptr(idx),
                                             ws, _ptr(shared), M * H, tp, top_k, M, H, _ptr(out),
                                             threads)
    _check(rc, "finalize_contributions")
    return out


def finalize(gemm2, weights, idx, shared, residual, post, comb, pre, gamma, norm_eps, *,
             two_shot=False, replicated_routing=True, routed_scaling_factor=1.0, mxfp8=False,
             threads=1):
    """MoE finalize boundary (a6 + a1/a7 + a2 + a4 [+ a8]); shapes as in
    finalize_contributions and boundary."""
    gemm2 = _c(gemm2, np.uint16)
    shared = _c(shared, np.uint16)
    tp, rows, H = gemm2.shape
    M = shared.shape[1]
    weights = np.ascontiguousarray(routing_weights(weights, routed_scaling_factor))
    idx = _c(idx, np.int32)
    top_k = weights.shape[-1]
    ws = 0 if replicated_routing else M * top_k
    residual = _c(residual, np.uint16).reshape(M, -1, H)
    hc = residual.shape[1]
    post = _c(post, np.float32).reshape(M, hc)
    comb = _c(comb, np.float32).reshape(M, hc, hc)
    pre = None if pre is None else _c(pre, np.float32).reshape(M, hc)
    gamma = None if gamma is None else _c(gamma, np.uint16).reshape(H)
    res_out = np.empty((M, hc, H), np.uint16)
    layer = None if pre is None else np.empty((M, H), np.uint16)
    values = scales = None
    if mxfp8:
        values = np.empty((M, H), np.uint8)
        scales = np.full(mxfp8_scale_bytes(M, H), 0xAA, np.uint8)
    rc = lib().oracle_finalize(_ptr(gemm2), rows * H, rows, _ptr(weights), ws, _ptr(idx), ws,
                               _ptr(shared), M * H, tp, top_k, _ptr(residual), _ptr(post),
                               _ptr(comb), _ptr(pre), _ptr(gamma), norm_eps, M, H, hc,
                               int(two_shot),
                               _ptr(res_out), _ptr(layer), _ptr(values), _ptr(scales), threads)
    _check(rc, "finalize")
    return res_out, layer, (None if not mxfp8 else (values, scales))


def two_shot_publish(contrib):
    """a7: owner mailboxes own[owner, source, slot, H] from contributions [tp, M, H]."""
    contrib = _c(contrib, np.uint16)
    tp, M, H = contrib.shape
    slots = -(-M // tp)
    own = np.zeros((tp, tp, slots, H), np.uint16)
    lib().oracle_two_shot_publish(_ptr(contrib), tp, M, H, _ptr(own))
    return own


def owner_reduce(own, M):
    """a7: reduced [M, H] from the owner mailboxes."""
    own = _c(own, np.uint16)
    tp, _, _, H = own.shape
    reduced = np.empty((M, H), np.uint16)
    lib().oracle_owner_reduce(_ptr(own), tp, M, H, _ptr(reduced))
    return reduced


def glm_mixes_token(y, fn, scale, base, rms_eps, hc_eps):
    """a3 for one token: y [4, H] u16, fn [24, 4H] u16 -> (mixes [24], pre [4])."""
    y = _c(y, np.uint16)
    H = y.shape[-1]
    fn = _c(fn, np.uint16)
    scale = _c(scale, np.float32)
    base = _c(base, np.float32)
    mixes = np.empty(24, np.float32)
    pre = np.empty(4, np.float32)
    lib().oracle_glm_mixes_token(_ptr(y), _ptr(fn), _ptr(scale), _ptr(base), H, rms_eps, hc_eps,
                                 _ptr(mixes), _ptr(pre))
    return mixes, pre


def glm_pre(mixes, scale, base, hc_eps):
    """[GLM] _BoundaryDeviceKernel.kernel: pre [M, 4] from raw mixes [M, 24]
    (only columns 0..3 are read): sigmoid(mixes_j * scale[0] + base[j]) + hc_eps."""
    mixes = _c(mixes, np.float32).reshape(-1, 24)
    scale = _c(scale, np.float32).reshape(3)
    base = _c(base, np.float32).reshape(24)
    pre = np.empty((mixes.shape[0], 4), np.float32)
    f = lib().oracle_glm_pre
    for t in range(mixes.shape[0]):
        f(_ptr(mixes[t]), _ptr(scale), _ptr(base), hc_eps, _ptr(pre[t]))
    return pre


def glm_collapse_rmsnorm(y, pre, gamma, norm_eps):
    """[GLM] _BoundaryDeviceKernel.kernel, the last steps: y [M, 4, H] u16
    (the new streams), pre [M, 4] f32 -> layer input [M, H] u16, with the
    pairwise collapse (q0+q1)+(q2+q3) and RMSNorm over H."""
    y = _c(y, np.uint16)
    M, _, H = y.shape
    pre = _c(pre, np.float32).reshape(M, 4)
    gamma = _c(gamma, np.uint16).reshape(H)
    out = np.empty((M, H), np.uint16)
    f = lib().oracle_glm_collapse_rmsnorm
    for t in range(M):
        _check(f(_ptr(y[t]), _ptr(pre[t]), _ptr(gamma), H, norm_eps, _ptr(out[t])),
               "glm_collapse_rmsnorm")
    return out


def boundary_glm(partials, residual, post, comb, fn, scale, base, gamma, rms_eps, hc_eps,
                 norm_eps, *, threads=1):
    """GLM boundary (a1, a2, a3, a4).

    Returns (residual_out [M,4,H], mixes [M,24], layer_input [M,H], pre [M,4]).
    """
    partials = _c(partials, np.uint16)
    tp, M, H = partials.shape
    residual = _c(residual, np.uint16).reshape(M, 4, H)
    post = _c(post, np.float32).reshape(M, 4)
    comb = _c(comb, np.float32).reshape(M, 4, 4)
    fn = _c(fn, np.uint16).reshape(24, 4 * H)
    scale = _c(scale, np.float32).reshape(3)
    base = _c(base, np.float32).reshape(24)
    gamma = _c(gamma, np.uint16).reshape(H)
    res_out = np.empty((M, 4, H), np.uint16)
    mixes = np.empty((M, 24), np.float32)
    layer = np.empty((M, H), np.uint16)
    pre = np.empty((M, 4), np.float32)
    rc = lib().oracle_boundary_glm(_ptr(partials), M * H, tp, _ptr(residual), _ptr(post),
                                   _ptr(comb), _ptr(fn), _ptr(scale), _ptr(base), _ptr(gamma),
                                   rms_eps, hc_eps, norm_eps, M, H, _ptr(res_out), _ptr(mixes),
                                   _ptr(layer), _ptr(pre), threads)
    _check(rc, "boundary_glm")
    return res_out, mixes, layer, pre


def boundary_glm_moe(gemm2, weights, idx, shared, residual, post, comb, fn, scale, base, gamma,
                     rms_eps, hc_eps, norm_eps, *, replicated_routing=True,
                     routed_scaling_factor=1.0, threads=1):
    """GLM boundary of an MoE sublayer ([GLM] AllReduceMhcBoundary.__call__,
    MoE branch): every rank publishes its contribution (a6, routing weights
    FP32 or BF16 with the routed scaling factor), and the GLM boundary
    (a1, a2, a3, a4) reads the published contributions as its rank partials.
    Shapes as in finalize_contributions and boundary_glm."""
    contrib = finalize_contributions(gemm2, weights, idx, shared,
                                     replicated_routing=replicated_routing,
                                     routed_scaling_factor=routed_scaling_factor, threads=threads)
    return boundary_glm(contrib, residual, post, comb, fn, scale, base, gamma, rms_eps, hc_eps,
                        norm_eps, threads=threads)


def sinkhorn(logits, eps, repeat):
    """The page's Sinkhorn on one 4x4 logit matrix (row-major 16 floats)."""
    logits = _c(logits, np.float32).reshape(16)
    out = np.empty(16, np.float32)
    lib().oracle_sinkhorn(_ptr(logits), eps, repeat, _ptr(out))
    return out.reshape(4, 4)


def side_mixes(mixes, scale, base, hc_eps, post_mult, repeat):
    """a5: (post' [M,4], comb' [M,4,4]) from raw mixes [M,24]."""
    mixes = _c(mixes, np.float32).reshape(-1, 24)
    M = mixes.shape[0]
    scale = _c(scale, np.float32).reshape(3)
    base = _c(base, np.float32).reshape(24)
    post = np.empty((M, 4), np.float32)
    comb = np.empty((M, 4, 4), np.float32)
    rc = lib().oracle_side_mixes(_ptr(mixes), _ptr(scale), _ptr(base), M, hc_eps, post_mult, repeat,
                                 _ptr(post), _ptr(comb))
    _check(rc, "side_mixes")
    return post, comb


def quant_mxfp8(x):
    """a8 standalone: (values [M,H] u8, scales [scale_bytes] u8) of BF16 x [M,H]."""
    x = _c(x, np.uint16)
    M, H = x.shape
    values = np.empty((M, H), np.uint8)
    scales = np.full(mxfp8_scale_bytes(M, H), 0xAA, np.uint8)
    rc = lib().oracle_quant_mxfp8(_ptr(x), M, H, _ptr(values), _ptr(scales))
    _check(rc, "quant_mxfp8")
    return values, scales


def indexer_projection(x, w, key, heads, gate):
    """[indexer] IndexerProjection.__call__: x [M, K] u16 (BF16), w [key +
    heads + gate, K] u16 -> (key [M, key] u16, head weights [M, heads] f32,
    gate [M, gate] u16); each output the binary64 dot product rounded to
    binary32, then to BF16 for the key and gate parts."""
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    M, K = x.shape
    assert w.shape == (key + heads + gate, K)
    key_out = np.empty((M, key), np.uint16)
    heads_out = np.empty((M, heads), np.float32)
    gate_out = np.empty((M, gate), np.uint16)
    _check(lib().oracle_indexer_projection(_ptr(x), _ptr(w), M, K, key, heads, gate,
                                           _ptr(key_out), _ptr(heads_out), _ptr(gate_out)),
           "indexer_projection")
    return key_out, heads_out, gate_out
