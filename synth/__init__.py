"""Seeded synthetic inputs for the sublayer-boundary workloads.

This module only draws random numbers and shapes them; it holds none of the
boundary's arithmetic.  Both the HIP path's tests/benchmark and the oracle's
tests take their inputs from here, and neither is imported by it.

Draws use numpy's PCG64 generator (``numpy.random.default_rng``).  FP32 draws
are stored as BF16 by round-to-nearest-even through torch's CPU conversion.
The delayed-boundary and GLM workloads draw each token's rows (partials,
residual streams, mixes) from a generator seeded by (workload, shape, token)
and the weights (norm weight, hc_fn, scale, base) from one seeded by
(workload, shape): a workload at M tokens is the first M tokens of the same
workload at any larger M, so an M sweep takes prefixes.  The MoE workload
keeps one generator per (workload, M), because its row indices are a
permutation of all M * top_k rows.  The same call gives the same bits on any
machine with this numpy.

The residual mix ``comb`` is a doubly stochastic 4x4 matrix per token:
exp of N(0,1) logits followed by 20 rounds of textbook Sinkhorn-Knopp (row,
then column normalization) in float64, stored as float32.  That is an input
recipe only; the method's own Sinkhorn (with its eps and order of
operations) is a separate step that both sides implement independently.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

HC = 4
MIX = 24


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rng(workload: int, m: int) -> np.random.Generator:
    return np.random.default_rng([workload, m])


def _normal_bf16(rng, shape, std):
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def _token_rng(workload: int, shape: tuple, t: int) -> np.random.Generator:
    return np.random.default_rng([workload, *shape, t])


def _token_rows(workload, shape, M, tp, H, hc, partial_std, post_pre=True):
    """Per-token draws: partials [tp, M, H] and residual [M, hc, H] as BF16
    bits, post / pre [M, hc] U(0,1) (pre only with post_pre) and the
    Sinkhorn logits of comb [M, hc, hc] N(0,1), token t from its own
    generator."""
    partials = np.empty((tp, M, H), np.float32)
    residual = np.empty((M, hc, H), np.float32)
    post = np.empty((M, hc), np.float32)
    pre = np.empty((M, hc), np.float32)
    logits = np.empty((M, hc, hc))
    for t in range(M):
        rng = _token_rng(workload, shape, t)
        partials[:, t] = rng.standard_normal((tp, H), dtype=np.float32) * np.float32(partial_std)
        residual[t] = rng.standard_normal((hc, H), dtype=np.float32)
        post[t] = rng.uniform(0.0, 1.0, hc)
        if post_pre:
            pre[t] = rng.uniform(0.0, 1.0, hc)
        logits[t] = rng.standard_normal((hc, hc))
    return (to_bf16_bits(partials), to_bf16_bits(residual), post, pre,
            sinkhorn_knopp(np.exp(logits)))


def sinkhorn_knopp(a: np.ndarray, rounds: int = 20) -> np.ndarray:
    """[m, hc, hc] positive float64 -> float32, textbook Sinkhorn-Knopp
    (row, then column normalization, `rounds` times): an input recipe."""
    for _ in range(rounds):
        a = a / a.sum(axis=2, keepdims=True)
        a = a / a.sum(axis=1, keepdims=True)
    return a.astype(np.float32)


def doubly_stochastic(rng, m: int, rounds: int = 20, hc: int = HC) -> np.ndarray:
    """[m, hc, hc] float32: Sinkhorn-Knopp (textbook, float64) of exp(N(0,1))."""
    return sinkhorn_knopp(np.exp(rng.standard_normal((m, hc, hc))), rounds)


@dataclass
class Boundary:
    """Inputs of a delayed-mHC boundary call (DSV4.1 shape)."""
    name: str
    M: int
    H: int
    tp: int
    partials: np.ndarray        # [tp, M, H] u16
    residual: np.ndarray        # [M, hc, H] u16
    post: np.ndarray            # [M, hc] f32
    comb: np.ndarray            # [M, hc, hc] f32, [source, target]
    pre: np.ndarray             # [M, hc] f32
    gamma: np.ndarray           # [H] u16
    norm_eps: float = 1e-6


@dataclass
class Glm:
    """Inputs of a GLM boundary call (pre-mix derived in-kernel)."""
    name: str
    M: int
    H: int
    tp: int
    partials: np.ndarray        # [tp, M, H] u16
    residual: np.ndarray        # [M, 4, H] u16
    post: np.ndarray            # [M, 4] f32
    comb: np.ndarray            # [M, 4, 4] f32
    fn: np.ndarray              # [24, 4H] u16, column j*H + c
    scale: np.ndarray           # [3] f32
    base: np.ndarray            # [24] f32
    gamma: np.ndarray           # [H] u16
    rms_eps: float = 1e-6
    hc_eps: float = 1e-6
    norm_eps: float = 1e-6
    post_mult: float = 2.0
    sinkhorn_repeat: int = 20


@dataclass
class Finalize:
    """Inputs of a MoE-finalize boundary call."""
    name: str
    M: int
    H: int
    tp: int
    top_k: int
    gemm2: np.ndarray           # [tp, rows, H] u16 (rows = M * top_k)
    weights: np.ndarray         # [M, top_k] f32 (replicated) or [tp, M, top_k]
    idx: np.ndarray             # [M, top_k] i32 (replicated) or [tp, M, top_k]
    shared: np.ndarray          # [tp, M, H] u16
    residual: np.ndarray
    post: np.ndarray
    comb: np.ndarray
    pre: np.ndarray
    gamma: np.ndarray
    norm_eps: float = 1e-6
    replicated_routing: bool = True


def _mixes(rng, m, hc=HC):
    post = rng.uniform(0.0, 1.0, (m, hc)).astype(np.float32)
    pre = rng.uniform(0.0, 1.0, (m, hc)).astype(np.float32)
    comb = doubly_stochastic(rng, m, hc=hc)
    return post, comb, pre


def _gamma(rng, h):
    return to_bf16_bits(1.0 + 0.1 * rng.standard_normal(h).astype(np.float32))


def boundary(workload: int, M: int, H: int, tp: int, partial_std: float,
             name: str = "", hc: int = HC) -> Boundary:
    """hc residual streams (4 unless given); token t's rows depend only on
    (workload, H, tp, hc, t), so smaller M are prefixes of larger ones."""
    shape = (H, tp, hc)
    partials, residual, post, pre, comb = _token_rows(workload, shape, M, tp, H, hc, partial_std)
    gamma = _gamma(np.random.default_rng([workload, *shape]), H)
    return Boundary(name or f"boundary-H{H}-tp{tp}-M{M}", M, H, tp, partials, residual,
                    post, comb, pre, gamma)


def tiny_delayed() -> Boundary:
    """Tiny delayed-mHC boundary: M=4, H=512, tp=2, partials N(0,1)."""
    return boundary(0, 4, 512, 2, 1.0, "tiny-delayed-H512-tp2-M4")


def dsv41_delayed(M: int, hc: int = HC) -> Boundary:
    """DSV4.1-shaped delayed boundary: H=5120, tp=8, partials N(0,0.5);
    hc residual streams (4 unless given)."""
    if hc == HC:
        return boundary(1, M, 5120, 8, 0.5, f"dsv41-delayed-H5120-tp8-M{M}")
    return boundary(1, M, 5120, 8, 0.5, f"dsv41-delayed-H5120-tp8-hc{hc}-M{M}", hc)


def large_m_delayed(M: int = 8192) -> Boundary:
    """Large-M boundary (MXFP8 epilogue / mailbox workload), H=5120, tp=8."""
    return boundary(4, M, 5120, 8, 0.5, f"large-delayed-H5120-tp8-M{M}")


def glm(M: int, H: int = 6144, tp: int = 8, name: str = "") -> Glm:
    """GLM-style boundary: hc_fn N(0,0.02), scale U(0.1,0.4), base N(0,1);
    token t's rows depend only on (H, tp, t), the weights on H."""
    partials, residual, post, _, comb = _token_rows(3, (H, tp), M, tp, H, HC, 0.5, post_pre=False)
    rng = np.random.default_rng([3, H])
    fn = _normal_bf16(rng, (MIX, HC * H), 0.02)
    scale = rng.uniform(0.1, 0.4, 3).astype(np.float32)
    base = rng.standard_normal(MIX).astype(np.float32)
    gamma = _gamma(rng, H)
    return Glm(name or f"glm-H{H}-tp{tp}-M{M}", M, H, tp, partials, residual, post, comb, fn,
               scale, base, gamma)


def moe_finalize(M: int, H: int = 5120, tp: int = 4, top_k: int = 8,
                 replicated_routing: bool = True, drop_fraction: float = 0.0,
                 name: str = "") -> Finalize:
    """MoE finalize: per rank gemm2 [M*top_k, H] and shared [M, H] N(0,0.5);
    routing weights softmax(N(0,1)) over top_k; row indices a permutation of
    0..M*top_k-1.  With per-rank routing, drop_fraction of each rank's routes
    get index -1 (expert not held by that rank)."""
    rng = _rng(2, M * 1000 + top_k)
    rows = M * top_k
    gemm2 = _normal_bf16(rng, (tp, rows, H), 0.5)
    shared = _normal_bf16(rng, (tp, M, H), 0.5)
    lead = () if replicated_routing else (tp,)
    logits = rng.standard_normal(lead + (M, top_k))
    w = np.exp(logits - logits.max(axis=-1, keepdims=True))
    weights = (w / w.sum(axis=-1, keepdims=True)).astype(np.float32)
    if replicated_routing:
        idx = rng.permutation(rows).astype(np.int32).reshape(M, top_k)
    else:
        idx = np.stack([rng.permutation(rows).astype(np.int32).reshape(M, top_k)
                        for _ in range(tp)])
        if drop_fraction > 0:
            idx[rng.uniform(size=idx.shape) < drop_fraction] = -1
    residual = _normal_bf16(rng, (M, HC, H), 1.0)
    post, comb, pre = _mixes(rng, M)
    gamma = _gamma(rng, H)
    return Finalize(name or f"moe-finalize-H{H}-tp{tp}-k{top_k}-M{M}", M, H, tp, top_k, gemm2,
                    weights, idx, shared, residual, post, comb, pre, gamma,
                    replicated_routing=replicated_routing)


def raw_mixes(M: int, seed: int = 5):
    """Raw GLM mixes [M, 24] ~ N(0,1), scale [3] U(0.1,0.4), base [24] N(0,1)."""
    rng = _rng(seed, M)
    mixes = rng.standard_normal((M, MIX)).astype(np.float32)
    scale = rng.uniform(0.1, 0.4, 3).astype(np.float32)
    base = rng.standard_normal(MIX).astype(np.float32)
    return mixes, scale, base


def bf16_matrix(M: int, H: int, std: float = 1.0, seed: int = 6) -> np.ndarray:
    """[M, H] BF16 bits ~ N(0, std): input of the standalone MXFP8 quantizer."""
    return _normal_bf16(_rng(seed, M * 100000 + H), (M, H), std)


@dataclass
class Indexer:
    """Inputs of the DSA indexer projection: x [M, K] (the layer input) and
    the concatenated weight rows [key + heads + gate, K]."""
    name: str
    M: int
    K: int
    key: int
    heads: int
    gate: int
    x: np.ndarray               # [M, K] u16
    w: np.ndarray               # [key + heads + gate, K] u16


def indexer(M: int, K: int = 6144, key: int = 128, heads: int = 32, gate: int = 128,
            name: str = "") -> Indexer:
    """Indexer projection: x ~ N(0,1) per token (token t's row from its own
    generator, so smaller M are prefixes), weight rows ~ N(0, 0.02)."""
    x = np.empty((M, K), np.float32)
    for t in range(M):
        x[t] = _token_rng(7, (K,), t).standard_normal(K, dtype=np.float32)
    rows = key + heads + gate
    w = _normal_bf16(np.random.default_rng([7, K, key, heads, gate]), (rows, K), 0.02)
    return Indexer(name or f"indexer-K{K}-k{key}-h{heads}-g{gate}-M{M}", M, K, key, heads, gate,
                   to_bf16_bits(x), w)
