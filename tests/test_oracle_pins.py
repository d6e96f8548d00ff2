"""Pins of the oracle against what the pages and the mathematics fix.

Each test checks the oracle (``oracle/``) against something other than
itself: exact rational arithmetic, closed forms, invariants, special cases
that reduce to a library routine (torch's BF16 and FP8 conversions, numpy
float64 linear algebra), or brute force on tiny inputs.  They are chosen so
that a plausible slip (a dropped term, a wrong sign or index, a transposed
operand, a wrong rounding) fails at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.numerics import (bf16_bits_of, bf16_ulp_distance, bf16_value, exact, f32,
                            f32_ulp_distance)

RNG = np.random.default_rng(1234)
ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
FINITE_BF16 = ALL_BF16[(ALL_BF16 & 0x7F80) != 0x7F80]


def torch_bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rand_bf16(shape, std=1.0, rng=RNG):
    return torch_bf16(rng.standard_normal(shape).astype(np.float32) * np.float32(std))


# ---------------------------------------------------------------------------
# BF16 rounding
# ---------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_including_ties():
    """oracle RNE == torch's CPU float32 -> bfloat16 conversion (a library
    routine), on random values, exact ties of both parities, subnormals and
    values that round up into the next binade or to infinity."""
    hi = RNG.integers(0, 0x7F7F, 4000).astype(np.uint32)
    low = np.concatenate([RNG.integers(0, 0x10000, 2000), np.full(1000, 0x8000),
                          np.full(500, 0x7FFF), np.full(500, 0x8001)]).astype(np.uint32)
    bits = (hi << 16) | low
    sign = (RNG.integers(0, 2, bits.size).astype(np.uint32) << 31)
    x = (bits | sign).view(np.float32)
    extra = np.array([0.0, -0.0, 1e-40, -1e-40, 3.3895314e38, 3.4e38, -3.4e38, 1.0, -1.0],
                     np.float32)
    x = np.concatenate([x, extra])
    assert np.array_equal(oracle.f32_to_bf16(x), torch_bf16(x))


def test_bf16_widening_is_exact():
    x = oracle.bf16_to_f32(FINITE_BF16)
    assert np.array_equal(torch_bf16(x), FINITE_BF16)


# ---------------------------------------------------------------------------
# a1 rank sum
# ---------------------------------------------------------------------------

def test_rank_sum_tp1_is_identity_exhaustive():
    """tp = 1: 0 + x rounded to BF16 is x for every finite BF16 (and -0 -> +0)."""
    x = FINITE_BF16.reshape(1, -1)
    got = np.fromiter((oracle.rank_sum_element(x, i) for i in range(x.shape[1])), np.uint16)
    want = np.where(FINITE_BF16 == 0x8000, 0, FINITE_BF16)
    assert np.array_equal(got, want)


def _edge_bf16_pairs(n):
    vals = []
    for _ in range(n):
        kind = RNG.integers(0, 5)
        a = rand_bf16(1)[0]
        if kind == 0:      # large exponent gap
            b = torch_bf16([bf16_value(a) * np.float32(2.0 ** -RNG.integers(8, 30))])[0]
        elif kind == 1:    # cancellation
            b = a ^ 0x8000
        elif kind == 2:    # near-cancellation
            b = (a ^ 0x8000) + np.uint16(RNG.integers(1, 4))
        elif kind == 3:    # extreme magnitudes
            a = np.uint16(0x7F7F - RNG.integers(0, 3))
            b = np.uint16(RNG.integers(0x7F00, 0x7F7F))
        else:
            b = rand_bf16(1)[0]
        vals.append((a, b))
    return vals


def test_rank_sum_brute_force_exact_rationals():
    """tp = 2 and 3: s = ((0 + x0) + x1) + x2 in binary32, then BF16, computed
    with exact rationals and an explicit RNE step per operation."""
    for a, b in _edge_bf16_pairs(300):
        x = np.array([[a], [b]], np.uint16)
        s = f32(exact(bf16_value(a)) + exact(bf16_value(b)))
        want = (0x7F80 if s > 0 else 0xFF80) if np.isinf(s) else bf16_bits_of(exact(s))
        assert oracle.rank_sum_element(x, 0) == want
    for _ in range(300):
        x = rand_bf16((3, 1), std=float(2.0 ** RNG.integers(-10, 10)))
        v = [exact(bf16_value(x[r, 0])) for r in range(3)]
        s = f32(v[0])
        s = f32(exact(s) + v[1])
        s = f32(exact(s) + v[2])
        assert oracle.rank_sum_element(x, 0) == bf16_bits_of(exact(s))


def test_rank_sum_order_designed_case():
    """Ranks (1, 2^-8, 2^-24, 2^-24): adding from rank 0 keeps 1 + 2^-8 (each
    2^-24 is a tie that rounds to even), a BF16 tie that rounds to 1.0; summed
    pairwise or from the last rank the small terms survive and BF16 gives
    1 + 2^-7."""
    x = np.array([[0x3F80], [0x3B80], [0x3380], [0x3380]], np.uint16)
    assert oracle.rank_sum_element(x, 0) == 0x3F80
    assert oracle.rank_sum_element(x[::-1].copy(), 0) == 0x3F81


# ---------------------------------------------------------------------------
# a2 post-mix, a4 collapse + RMSNorm (delayed boundary)
# ---------------------------------------------------------------------------

def _delayed_case(M=3, H=256, tp=3, seed=7):
    rng = np.random.default_rng(seed)
    partials = rand_bf16((tp, M, H), 0.5, rng)
    residual = rand_bf16((M, 4, H), 1.0, rng)
    post = rng.uniform(0, 1, (M, 4)).astype(np.float32)
    comb = synth.doubly_stochastic(rng, M)
    pre = rng.uniform(0, 1, (M, 4)).astype(np.float32)
    gamma = torch_bf16(1 + 0.1 * rng.standard_normal(H))
    return partials, residual, post, comb, pre, gamma


def test_post_mix_identity_leaves_streams_unchanged():
    """comb = I and post = 0 leave the streams bit-identical."""
    partials, residual, post, comb, pre, gamma = _delayed_case()
    M = residual.shape[0]
    comb = np.broadcast_to(np.eye(4, dtype=np.float32), (M, 4, 4)).copy()
    post = np.zeros_like(post)
    ro, _, _ = oracle.boundary(partials, residual, post, comb, pre, gamma, 1e-6)
    assert np.array_equal(ro, residual)


def test_post_mix_permutation_pins_source_target_order():
    """comb = a non-symmetric permutation (source s -> target pi(s)), post = 0:
    new stream pi(s) is old stream s.  A transposed comb fails."""
    partials, residual, post, comb, pre, gamma = _delayed_case()
    M = residual.shape[0]
    pi = [1, 2, 3, 0]
    P = np.zeros((4, 4), np.float32)
    for s, j in enumerate(pi):
        P[s, j] = 1.0
    comb = np.broadcast_to(P, (M, 4, 4)).copy()
    ro, _, _ = oracle.boundary(partials, residual, np.zeros_like(post), comb, pre, gamma, 1e-6)
    for s, j in enumerate(pi):
        assert np.array_equal(ro[:, j], residual[:, s])


def test_post_mix_probe_exposes_the_bf16_sum():
    """post = 1 and comb = 0 make every new stream equal to the BF16 rank sum,
    which is checked against exact rationals."""
    partials, residual, post, comb, pre, gamma = _delayed_case(M=2, H=64, tp=3)
    M, H = 2, 64
    ro, _, _ = oracle.boundary(partials, residual, np.ones_like(post), np.zeros_like(comb), pre,
                               gamma, 1e-6)
    for t in range(M):
        for c in range(H):
            s = 0.0
            for r in range(3):
                s = f32(exact(s) + exact(bf16_value(partials[r, t, c])))
            want = bf16_bits_of(exact(s))
            for j in range(4):
                assert ro[t, j, c] == want


def test_post_mix_single_terms_closed_form():
    """comb = 0: y_j = bf16(fl(x * post_j)); comb with one entry c at
    [s, j] and post = 0: y_j = bf16(fl(res_s * c))."""
    partials, residual, post, comb, pre, gamma = _delayed_case(M=2, H=128, tp=1)
    ro, _, _ = oracle.boundary(partials, residual, post, np.zeros_like(comb), pre, gamma, 1e-6)
    x = bf16_value(partials[0])
    for j in range(4):
        want = torch_bf16((x * post[:, j:j + 1]).astype(np.float32))
        assert np.array_equal(ro[:, j], want)
    c = np.zeros_like(comb)
    c[:, 2, 1] = np.float32(0.3)
    ro, _, _ = oracle.boundary(partials, residual, np.zeros_like(post), c, pre, gamma, 1e-6)
    want = torch_bf16(bf16_value(residual[:, 2]) * np.float32(0.3))
    assert np.array_equal(ro[:, 1], want)


def test_post_mix_and_collapse_fma_chains_brute_force():
    """Tiny case with exact rationals: y_j = bf16(chain) with
    a = fl(x * post_j), then a = fl(res_s * comb[s, j] + a) for s = 0..3 (one
    rounding per fused step), and z = fl(y_j * pre_j + z) from 0 for the
    collapse.  Unfused products or a different order fail."""
    partials, residual, post, comb, pre, gamma = _delayed_case(M=2, H=24, tp=2, seed=21)
    ro, li, _ = oracle.boundary(partials, residual, post, comb, pre, gamma, 1e-6)
    M, H = 2, 24
    p_bits = np.zeros((M, H), np.uint16)
    for t in range(M):
        for c in range(H):
            s = f32(exact(bf16_value(partials[0, t, c])))
            s = f32(exact(s) + exact(bf16_value(partials[1, t, c])))
            x = exact(bf16_value(bf16_bits_of(exact(s))))
            ys = []
            for j in range(4):
                a = f32(x * exact(post[t, j]))
                for src_ in range(4):
                    a = f32(exact(bf16_value(residual[t, src_, c])) * exact(comb[t, src_, j]) + exact(a))
                yb = bf16_bits_of(exact(a))
                assert ro[t, j, c] == yb
                ys.append(yb)
            z = 0.0
            for j in range(4):
                z = f32(exact(bf16_value(ys[j])) * exact(pre[t, j]) + exact(z))
            p_bits[t, c] = bf16_bits_of(exact(z))
    # The layer input is RMSNorm of exactly these p (float64 textbook, 1 ulp).
    p = bf16_value(p_bits).astype(np.float64)
    ref = p / np.sqrt((p ** 2).mean(axis=1, keepdims=True) + 1e-6) * bf16_value(gamma)
    assert bf16_ulp_distance(li, torch_bf16(ref)).max() <= 1


# ---------------------------------------------------------------------------
# General hc_mult (the DSV4.1 consumer is compiled for the module's hc)
# ---------------------------------------------------------------------------

def _hc_case(hc, M=3, H=16, tp=2, seed=50):
    rng = np.random.default_rng(seed)
    partials = rand_bf16((tp, M, H), 0.5, rng)
    residual = rand_bf16((M, hc, H), 1.0, rng)
    post = rng.uniform(0, 1, (M, hc)).astype(np.float32)
    comb = rng.uniform(0, 0.5, (M, hc, hc)).astype(np.float32)
    pre = rng.uniform(0, 1, (M, hc)).astype(np.float32)
    gamma = torch_bf16(1 + 0.1 * rng.standard_normal(H))
    return partials, residual, post, comb, pre, gamma


@pytest.mark.parametrize("hc", [1, 2, 3, 8])
def test_general_hc_identity_and_permutation(hc):
    """comb = I with post = 0 leaves the hc streams unchanged; comb = the
    cyclic permutation s -> s + 1 moves stream s to s + 1 (source-major
    [s, j] indexing at every hc)."""
    partials, residual, post, comb, pre, gamma = _hc_case(hc)
    M = residual.shape[0]
    eye = np.broadcast_to(np.eye(hc, dtype=np.float32), (M, hc, hc)).copy()
    ro, _, _ = oracle.boundary(partials, residual, np.zeros_like(post), eye, pre, gamma, 1e-6)
    assert np.array_equal(ro, residual)
    P = np.zeros((hc, hc), np.float32)
    for s_ in range(hc):
        P[s_, (s_ + 1) % hc] = 1.0
    ro, _, _ = oracle.boundary(partials, residual, np.zeros_like(post),
                               np.broadcast_to(P, (M, hc, hc)).copy(), pre, gamma, 1e-6)
    for s_ in range(hc):
        assert np.array_equal(ro[:, (s_ + 1) % hc], residual[:, s_])


@pytest.mark.parametrize("hc", [1, 2, 8])
def test_general_hc_fma_chains_brute_force(hc):
    """The post-mix FMA chain over hc sources and the collapse chain over hc
    streams, checked with exact rationals (one rounding per fused step)."""
    partials, residual, post, comb, pre, gamma = _hc_case(hc, M=2, H=8, seed=51 + hc)
    ro, li, _ = oracle.boundary(partials, residual, post, comb, pre, gamma, 1e-6)
    M, H = 2, 8
    p_bits = np.zeros((M, H), np.uint16)
    for t in range(M):
        for c in range(H):
            s_ = f32(exact(bf16_value(partials[0, t, c])))
            s_ = f32(exact(s_) + exact(bf16_value(partials[1, t, c])))
            x = exact(bf16_value(bf16_bits_of(exact(s_))))
            ys = []
            for j in range(hc):
                a = f32(x * exact(post[t, j]))
                for src_ in range(hc):
                    a = f32(exact(bf16_value(residual[t, src_, c])) * exact(comb[t, src_, j]) + exact(a))
                yb = bf16_bits_of(exact(a))
                assert ro[t, j, c] == yb
                ys.append(yb)
            z = 0.0
            for j in range(hc):
                z = f32(exact(bf16_value(ys[j])) * exact(pre[t, j]) + exact(z))
            p_bits[t, c] = bf16_bits_of(exact(z))
    p = bf16_value(p_bits).astype(np.float64)
    ref = p / np.sqrt((p ** 2).mean(axis=1, keepdims=True) + 1e-6) * bf16_value(gamma)
    assert bf16_ulp_distance(li, torch_bf16(ref)).max() <= 1


def test_general_hc_finalize_equals_boundary_on_contributions():
    f = synth.moe_finalize(4, H=128, tp=2, top_k=3)
    rng = np.random.default_rng(55)
    for hc in (2, 8):
        residual = rand_bf16((4, hc, 128), 1.0, rng)
        post = rng.uniform(0, 1, (4, hc)).astype(np.float32)
        comb = rng.uniform(0, 0.5, (4, hc, hc)).astype(np.float32)
        pre = rng.uniform(0, 1, (4, hc)).astype(np.float32)
        contrib = oracle.finalize_contributions(f.gemm2, f.weights, f.idx, f.shared)
        a = oracle.finalize(f.gemm2, f.weights, f.idx, f.shared, residual, post, comb, pre,
                            f.gamma, 1e-6)
        b = oracle.boundary(contrib, residual, post, comb, pre, f.gamma, 1e-6)
        c = oracle.finalize(f.gemm2, f.weights, f.idx, f.shared, residual, post, comb, pre,
                            f.gamma, 1e-6, two_shot=True)
        for x, y, z in ((a[0], b[0], c[0]), (a[1], b[1], c[1])):
            assert np.array_equal(x, y) and np.array_equal(x, z)


# 3.0 * C is 2^-8 + 2^-24 + (a little): 1 + 3*C rounds in one step to
# 1 + 2^-8 + 2^-23 (BF16 then rounds up to 0x3F81), while rounding 3*C first
# gives exactly the midpoint 1 + 2^-8 + 2^-24 -> 1 + 2^-8 -> BF16 tie -> 0x3F80.
FMA_C = np.array([0x3AAAAB56], np.uint32).view(np.float32)[0]


def test_fma_readings_designed_cases():
    """The FMA reading of every `acc + a * b` step: post-mix, collapse and
    finalize, each on an input where fused and unfused binary32 arithmetic
    end on different BF16 values."""
    H = 2
    partials = np.full((1, 1, H), 0x3F80, np.uint16)                 # x = 1
    residual = np.zeros((1, 4, H), np.uint16)
    residual[0, 0, :] = 0x4040                                        # res_0 = 3
    post = np.ones((1, 4), np.float32)
    comb = np.zeros((1, 4, 4), np.float32)
    comb[0, 0, :] = FMA_C
    pre = np.full((1, 4), 0.25, np.float32)
    gamma = np.full(H, 0x3F80, np.uint16)
    ro, _, _ = oracle.boundary(partials, residual, post, comb, pre, gamma, 1e-6)
    assert (ro == 0x3F81).all()                                       # post-mix fused

    residual = np.zeros((1, 4, H), np.uint16)
    residual[0, 0, 0], residual[0, 1, 0] = 0x3F80, 0x4040             # column 0: y = (1, 3, 0, 0)
    residual[0, 0, 1] = 0x4280                                        # column 1: y = (64, 0, 0, 0)
    eye = np.eye(4, dtype=np.float32)[None]
    pre = np.array([[1.0, FMA_C, 0.0, 0.0]], np.float32)
    _, li, _ = oracle.boundary(np.zeros((1, 1, H), np.uint16), residual,
                               np.zeros((1, 4), np.float32), eye, pre, gamma, 1e-6)
    p = np.array([1.0078125, 64.0], np.float64)                       # p0 = 0x3F81 when fused
    inv = np.float32(1 / np.sqrt(np.float64(np.float32((p ** 2).sum())) / H + np.float64(np.float32(1e-6))))
    want = torch_bf16((p.astype(np.float32) * inv).astype(np.float32))
    assert np.array_equal(li[0], want)

    gemm2 = np.zeros((1, 2, H), np.uint16)
    gemm2[0, 0], gemm2[0, 1] = 0x3F80, 0x4040
    w = np.array([[1.0, FMA_C]], np.float32)
    idx = np.array([[0, 1]], np.int32)
    c = oracle.finalize_contributions(gemm2, w, idx, np.zeros((1, 1, H), np.uint16))
    assert (c == 0x3F81).all()


def test_rmsnorm_multiplies_left_to_right_designed_case():
    """out = bf16((p * inv) * gamma), not p * (inv * gamma): on this row
    (p = (0x3F95, 0x4292), gamma_0 = 0x3FF6) the orders give 0x3D31 / 0x3D32."""
    H = 2
    residual = np.zeros((1, 4, H), np.uint16)
    residual[0, 0] = [0x3F95, 0x4292]
    pre = np.array([[1.0, 0.0, 0.0, 0.0]], np.float32)
    gamma = np.array([0x3FF6, 0x3F80], np.uint16)
    _, li, _ = oracle.boundary(np.zeros((1, 1, H), np.uint16), residual,
                               np.zeros((1, 4), np.float32), np.eye(4, dtype=np.float32)[None],
                               pre, gamma, 1e-6)
    assert li[0, 0] == 0x3D31


def test_rmsnorm_gamma_after_the_normalizer_designed_case():
    """out = bf16((p * inv) * gamma), with gamma applied last: on the row
    p = (0xBD70, 0xBEC5), gamma_0 = 0x3F76 that order gives 0xBE51, while
    (p * gamma) * inv and p * (inv * gamma) give 0xBE52 (all three checked
    here with exact rationals; inv = fl(1/sqrt(fl(ss)/H + eps)) with the
    exact sum of squares of two BF16 values)."""
    import math
    H = 2
    p = np.array([0xBD70, 0xBEC5], np.uint16)
    gamma = np.array([0x3F76, 0x3F86], np.uint16)
    residual = np.zeros((1, 4, H), np.uint16)
    residual[0, 0] = p
    pre = np.array([[1.0, 0.0, 0.0, 0.0]], np.float32)
    _, li, _ = oracle.boundary(np.zeros((1, 1, H), np.uint16), residual,
                               np.zeros((1, 4), np.float32), np.eye(4, dtype=np.float32)[None],
                               pre, gamma, 1e-6)
    ss = sum(exact(bf16_value(v)) ** 2 for v in p)
    inv = exact(np.float32(1.0 / math.sqrt(f32(ss) / H + float(np.float32(1e-6)))))
    p0, g0 = exact(bf16_value(p[0])), exact(bf16_value(gamma[0]))
    left = bf16_bits_of(exact(f32(exact(f32(p0 * inv)) * g0)))
    gamma_first = bf16_bits_of(exact(f32(exact(f32(p0 * g0)) * inv)))
    inv_gamma = bf16_bits_of(exact(f32(p0 * exact(f32(inv * g0)))))
    assert (left, gamma_first, inv_gamma) == (0xBE51, 0xBE52, 0xBE52)
    assert li[0, 0] == left


def test_sinkhorn_first_round_brute_force():
    """repeat = 1: the first step (rows of fma(exp(c - rowmax), 1/sum, eps))
    followed by one column step only, c <- fl(c * fl(1/fl(s + eps))) with s
    the column's (c0 + c1) + (c2 + c3); no row step in the first round.
    With eps = 1e-3 a row step there would scale every entry by about
    1/(1 + 5 eps), far above the rounding checked here exactly."""
    import math
    eps = np.float32(1e-3)
    for _ in range(30):
        logits = RNG.standard_normal(16).astype(np.float32)
        got = oracle.sinkhorn(logits, float(eps), 1).reshape(16)
        c = [0.0] * 16
        for r in range(4):
            row = logits[4 * r:4 * r + 4]
            peak = max(row)
            e = [np.float32(math.exp(float(np.float32(v - peak)))) for v in row]
            s = np.float32(np.float32(e[0] + e[1]) + np.float32(e[2] + e[3]))
            inv = np.float32(1.0 / float(s))
            for k in range(4):
                c[4 * r + k] = f32(exact(e[k]) * exact(inv) + exact(eps))
        for k in range(4):
            s = f32(exact(f32(exact(c[k]) + exact(c[4 + k]))) + exact(f32(exact(c[8 + k]) + exact(c[12 + k]))))
            inv = f32(1 / exact(f32(exact(s) + exact(eps))))
            for r in range(4):
                assert got[4 * r + k] == np.float32(f32(exact(c[4 * r + k]) * exact(inv)))


def test_sinkhorn_first_step_brute_force():
    """repeat = 0 leaves the first step alone: rows of exp(c - rowmax), each
    scaled by the rounded reciprocal of (q0+q1)+(q2+q3) and offset by eps in
    one fused step; checked with exact rationals and libm exp."""
    import math
    eps = np.float32(1e-3)
    for _ in range(30):
        logits = RNG.standard_normal(16).astype(np.float32)
        got = oracle.sinkhorn(logits, float(eps), 0).reshape(16)
        for r in range(4):
            row = logits[4 * r:4 * r + 4]
            peak = max(row)
            e = [np.float32(math.exp(float(np.float32(v - peak)))) for v in row]
            s = np.float32(np.float32(e[0] + e[1]) + np.float32(e[2] + e[3]))
            inv = np.float32(1.0 / float(s))
            for k in range(4):
                want = f32(exact(e[k]) * exact(inv) + exact(eps))
                assert got[4 * r + k] == np.float32(want)


def test_delayed_boundary_close_to_float64_definition():
    """Every output within 1 BF16 ulp of the float64 evaluation of the
    definition (each BF16 rounding of the method kept): catches dropped
    terms, sign slips and wrong operands in the post-mix and the collapse."""
    partials, residual, post, comb, pre, gamma = _delayed_case(M=4, H=512, tp=4)
    ro, li, _ = oracle.boundary(partials, residual, post, comb, pre, gamma, 1e-6)
    xr = torch_bf16(bf16_value(partials).astype(np.float64).sum(0))
    y_ref = (bf16_value(xr)[:, None, :].astype(np.float64) * post[:, :, None]
             + np.einsum("tsc,tsj->tjc", bf16_value(residual).astype(np.float64), comb))
    assert bf16_ulp_distance(ro, torch_bf16(y_ref)).max() <= 1
    p_ref = np.einsum("tjc,tj->tc", bf16_value(ro).astype(np.float64), pre)
    p_bf = bf16_value(torch_bf16(p_ref)).astype(np.float64)
    inv = 1.0 / np.sqrt((p_bf ** 2).mean(axis=1, keepdims=True) + 1e-6)
    li_ref = torch_bf16(p_bf * inv * bf16_value(gamma))
    assert bf16_ulp_distance(li, li_ref).max() <= 1


def test_collapse_one_hot_pre_and_textbook_rmsnorm():
    """pre = e_j: the collapse is y_j exactly, and the layer input is the
    textbook RMSNorm of y_j (float64) within 1 BF16 ulp."""
    partials, residual, post, comb, pre, gamma = _delayed_case(M=3, H=384, tp=2)
    for j in range(4):
        onehot = np.zeros_like(pre)
        onehot[:, j] = 1.0
        ro, li, _ = oracle.boundary(partials, residual, post, comb, onehot, gamma, 1e-6)
        y = bf16_value(ro[:, j]).astype(np.float64)
        ref = y / np.sqrt((y ** 2).mean(axis=1, keepdims=True) + 1e-6) * bf16_value(gamma)
        assert bf16_ulp_distance(li, torch_bf16(ref)).max() <= 1


def test_rmsnorm_constant_row_closed_form():
    """Constant p = a and gamma = 1: out = bf16(fl(a * fl(1/sqrt(a^2 + eps))))."""
    M, H = 2, 256
    a = np.uint16(0x3FC0)  # 1.5
    residual = np.full((M, 4, H), a, np.uint16)
    partials = np.zeros((1, M, H), np.uint16)
    comb = np.broadcast_to(np.eye(4, dtype=np.float32), (M, 4, 4)).copy()
    pre = np.zeros((M, 4), np.float32)
    pre[:, 0] = 1
    gamma = np.full(H, 0x3F80, np.uint16)
    eps = 1e-3
    _, li, _ = oracle.boundary(partials, residual, np.zeros((M, 4), np.float32), comb, pre, gamma,
                               eps)
    inv = np.float32(1.0 / np.sqrt(np.float64(np.float32(1.5 * 1.5 * H)) / H + np.float64(np.float32(eps))))
    want = torch_bf16(np.float32(1.5) * inv)
    assert (li == want).all()


def test_rmsnorm_scale_invariance_eps0():
    """With eps = 0, doubling every stream (a power of two, exact everywhere)
    leaves the normalized output bit-identical."""
    partials, residual, post, comb, pre, gamma = _delayed_case(M=2, H=256, tp=2)
    _, li, _ = oracle.boundary(partials, residual, post, comb, pre, gamma, 0.0)
    double = lambda b: torch_bf16(bf16_value(b) * np.float32(2.0))
    _, li2, _ = oracle.boundary(double(partials), double(residual), post, comb, pre, gamma, 0.0)
    assert np.array_equal(li, li2)


def test_collapse_order_glm_pairwise_vs_delayed_sequential():
    """Streams (2, 2^-23, 2^-23, -2) with pre = 0.5 each: GLM's pairwise
    collapse (q0+q1)+(q2+q3) gives 2^-24, the delayed variant's sequential FMA
    chain gives 0.  With norm_eps = 0 and gamma = 1 the GLM layer input is
    then exactly 1.0 and the delayed one exactly 0."""
    H = 8
    col = np.array([0x4000, 0x3400, 0x3400, 0xC000], np.uint16)   # 2, 2^-23, 2^-23, -2
    residual = np.broadcast_to(col[None, :, None], (1, 4, H)).copy()
    partials = np.zeros((1, 1, H), np.uint16)
    eye = np.eye(4, dtype=np.float32)[None]
    zero_post = np.zeros((1, 4), np.float32)
    gamma = np.full(H, 0x3F80, np.uint16)
    fn = np.zeros((24, 4 * H), np.uint16)
    scale = np.ones(3, np.float32)
    base = np.zeros(24, np.float32)
    ro, mixes, li, pre = oracle.boundary_glm(partials, residual, zero_post, eye, fn, scale, base,
                                             gamma, 1e-6, 0.0, 0.0)
    assert np.array_equal(ro, residual) and (pre == 0.5).all() and (mixes == 0).all()
    assert (li == 0x3F80).all()
    _, li_d, _ = oracle.boundary(partials, residual, zero_post, eye, np.full((1, 4), 0.5, np.float32),
                                 gamma, 1e-6)
    assert (li_d == 0).all()


# ---------------------------------------------------------------------------
# a3 GLM mixes
# ---------------------------------------------------------------------------

def test_glm_mixes_one_hot_rows_and_zero_fn():
    """fn row k = indicator of one (stream, column): mixes_k = y[that] * rstd,
    rstd from the float64 textbook formula; fn = 0: mixes = 0 and
    pre = sigmoid(base) + hc_eps."""
    H = 64
    rng = np.random.default_rng(3)
    y = rand_bf16((4, H), 1.0, rng)
    fn = np.zeros((24, 4 * H), np.uint16)
    picks = [(k % 4, (7 * k) % H) for k in range(24)]
    for k, (j, c) in enumerate(picks):
        fn[k, j * H + c] = 0x3F80
    scale = np.array([0.3, 0.2, 0.1], np.float32)
    base = rng.standard_normal(24).astype(np.float32)
    mixes, pre = oracle.glm_mixes_token(y, fn, scale, base, 1e-6, 1e-6)
    yv = bf16_value(y).astype(np.float64)
    rstd = 1.0 / np.sqrt((yv ** 2).mean() + 1e-6)
    want = np.array([yv[j, c] * rstd for j, c in picks])
    assert np.abs(mixes - want).max() <= 2e-7 * np.abs(want).max()
    mixes0, pre0 = oracle.glm_mixes_token(y, np.zeros_like(fn), scale, base, 1e-6, 1e-6)
    assert (mixes0 == 0).all()
    assert np.allclose(pre0, 1 / (1 + np.exp(-base[:4].astype(np.float64))) + 1e-6, rtol=1e-7)


def test_glm_mixes_match_float64_matvec():
    """mixes = (fn @ y) * rstd with numpy float64 (library matvec); the
    pre-mix = sigmoid(mixes * scale0 + base) + eps."""
    H = 256
    rng = np.random.default_rng(4)
    y = rand_bf16((4, H), 1.0, rng)
    fn = rand_bf16((24, 4 * H), 0.02, rng)
    scale = np.array([0.25, 0.3, 0.15], np.float32)
    base = rng.standard_normal(24).astype(np.float32)
    mixes, pre = oracle.glm_mixes_token(y, fn, scale, base, 1e-6, 1e-6)
    yv = bf16_value(y).astype(np.float64).reshape(-1)
    g = bf16_value(fn).astype(np.float64) @ yv
    rstd = 1.0 / np.sqrt((yv ** 2).mean() + 1e-6)
    assert np.abs(mixes - g * rstd).max() <= 1e-6 * (np.abs(g * rstd).max() + 1)
    pre_ref = 1 / (1 + np.exp(-(g[:4] * rstd * 0.25 + base[:4]))) + 1e-6
    assert np.abs(pre - pre_ref).max() <= 1e-6


def test_glm_boundary_uses_its_own_pre_mix():
    """The GLM layer input equals a delayed boundary fed the GLM pre-mix,
    except that GLM collapses pairwise: within 1 BF16 ulp, streams identical."""
    g = synth.glm(3, H=256, tp=3)
    ro, mixes, li, pre = oracle.boundary_glm(g.partials, g.residual, g.post, g.comb, g.fn, g.scale,
                                             g.base, g.gamma, g.rms_eps, g.hc_eps, g.norm_eps)
    ro2, li2, _ = oracle.boundary(g.partials, g.residual, g.post, g.comb, pre, g.gamma, g.norm_eps)
    assert np.array_equal(ro, ro2)
    assert bf16_ulp_distance(li, li2).max() <= 1
    m2, p2 = oracle.glm_mixes_token(ro[1], g.fn, g.scale, g.base, g.rms_eps, g.hc_eps)
    assert np.array_equal(m2, mixes[1]) and np.array_equal(p2, pre[1])


def test_glm_pre_from_mixes_closed_forms_and_slices():
    """pre_j = sigmoid(mixes_j * scale[0] + base[j]) + hc_eps.  Arguments that
    are exactly 0 give 1/2 + eps; sigma(x) + sigma(-x) = 1; only mixes[0:4],
    scale[0] and base[0:4] are read; against float64 with the argument formed
    from exact rationals and rounded once (the fused product-sum)."""
    eps = 2.0 ** -10
    mixes = np.zeros((1, 24), np.float32)
    mixes[0, :4] = [2.0, -4.0, 0.5, 8.0]
    scale = np.array([0.25, 9.0, 9.0], np.float32)
    base = np.full(24, 7.0, np.float32)
    base[:4] = [-0.5, 1.0, -0.125, -2.0]
    assert (oracle.glm_pre(mixes, scale, base, eps) == np.float32(0.5 + eps)).all()

    rng = np.random.default_rng(21)
    mixes = (rng.standard_normal((40, 24)) * 3).astype(np.float32)
    scale = rng.uniform(0.1, 0.4, 3).astype(np.float32)
    base = rng.standard_normal(24).astype(np.float32)
    pre = oracle.glm_pre(mixes, scale, base, 0.0)
    neg = oracle.glm_pre(-mixes, scale, -base, 0.0)
    assert np.abs(pre.astype(np.float64) + neg - 1.0).max() <= 2.0 ** -23
    m2, s2, b2 = mixes.copy(), scale.copy(), base.copy()
    m2[:, 4:] += 1.0
    s2[1:] += 1.0
    b2[4:] += 1.0
    assert np.array_equal(oracle.glm_pre(m2, s2, b2, 0.0), pre)
    for t in range(mixes.shape[0]):
        for j in range(4):
            x = f32(exact(mixes[t, j]) * exact(scale[0]) + exact(base[j]))
            want = np.float32(1.0 / (1.0 + np.exp(-x)))
            assert f32_ulp_distance(pre[t, j], want) <= 1


def test_glm_collapse_rmsnorm_one_hot_pre_is_textbook_rmsnorm():
    """pre = e_j: the pairwise collapse is y_j exactly (the other products
    are zeros), and the layer input is the float64 textbook RMSNorm of y_j
    times gamma within 1 BF16 ulp."""
    rng = np.random.default_rng(22)
    M, H = 3, 384
    y = rand_bf16((M, 4, H), 1.0, rng)
    gamma = rand_bf16(H, 1.0, rng)
    for j in range(4):
        pre = np.zeros((M, 4), np.float32)
        pre[:, j] = 1.0
        out = oracle.glm_collapse_rmsnorm(y, pre, gamma, 1e-6)
        v = bf16_value(y[:, j]).astype(np.float64)
        ref = v / np.sqrt((v ** 2).mean(axis=1, keepdims=True) + 1e-6) * bf16_value(gamma)
        assert bf16_ulp_distance(out, torch_bf16(ref)).max() <= 1


def test_glm_collapse_pairwise_designed_case():
    """Streams (2, 2^-23, 2^-23, -2), pre 1/2: (q0+q1)+(q2+q3) = 2^-24, so
    with eps = 0 and gamma = 1 every output is exactly 1.0; a sequential sum
    (or FMA chain) would give 0 and a NaN output."""
    H = 16
    col = np.array([0x4000, 0x3400, 0x3400, 0xC000], np.uint16)
    y = np.broadcast_to(col[None, :, None], (2, 4, H)).copy()
    out = oracle.glm_collapse_rmsnorm(y, np.full((2, 4), 0.5, np.float32),
                                      np.full(H, 0x3F80, np.uint16), 0.0)
    assert (out == 0x3F80).all()


def test_glm_collapse_exact_rational_and_textbook_rmsnorm():
    """Random streams and pre-mixes: the collapse p = bf16((q0+q1)+(q2+q3)),
    q_j = fl(y_j * pre_j), evaluated with exact rationals rounded at each
    step, then the float64 textbook RMSNorm of p: within 1 BF16 ulp."""
    rng = np.random.default_rng(23)
    M, H = 2, 96
    y = rand_bf16((M, 4, H), 1.0, rng)
    pre = rng.uniform(0.0, 1.0, (M, 4)).astype(np.float32)
    gamma = rand_bf16(H, 1.0, rng)
    out = oracle.glm_collapse_rmsnorm(y, pre, gamma, 1e-6)
    p = np.empty((M, H), np.float64)
    for t in range(M):
        for c in range(H):
            q = [f32(exact(bf16_value(y[t, j, c])) * exact(pre[t, j])) for j in range(4)]
            z = f32(exact(f32(exact(q[0]) + exact(q[1]))) + exact(f32(exact(q[2]) + exact(q[3]))))
            p[t, c] = bf16_value(bf16_bits_of(exact(z)))
    ref = p / np.sqrt((p ** 2).mean(axis=1, keepdims=True) + 1e-6) * bf16_value(gamma)
    assert bf16_ulp_distance(out, torch_bf16(ref)).max() <= 1


def test_glm_collapse_rmsnorm_is_the_last_step_of_boundary_glm():
    """Fed the oracle's own streams and raw mixes, glm_pre and
    glm_collapse_rmsnorm give the GLM boundary's pre-mix and layer input."""
    g = synth.glm(3, H=256, tp=3)
    ro, mixes, li, pre = oracle.boundary_glm(g.partials, g.residual, g.post, g.comb, g.fn, g.scale,
                                             g.base, g.gamma, g.rms_eps, g.hc_eps, g.norm_eps)
    assert np.array_equal(oracle.glm_pre(mixes, g.scale, g.base, g.hc_eps), pre)
    assert np.array_equal(oracle.glm_collapse_rmsnorm(ro, pre, g.gamma, g.norm_eps), li)


# ---------------------------------------------------------------------------
# a5 sigmoid, post', Sinkhorn
# ---------------------------------------------------------------------------

def test_sigmoid_closed_forms():
    assert oracle.sigmoid(0.0) == 0.5
    xs = RNG.standard_normal(200).astype(np.float32) * 4
    got = np.array([oracle.sigmoid(float(x)) for x in xs], np.float32)
    ref = (1 / (1 + np.exp(-xs.astype(np.float64)))).astype(np.float32)
    assert f32_ulp_distance(got, ref).max() == 0


def test_side_post_zero_mix_closed_form():
    """mixes = 0: post'_j = sigmoid(base[4+j]) * post_mult."""
    base = RNG.standard_normal(24).astype(np.float32)
    post, _ = oracle.side_mixes(np.zeros((2, 24), np.float32), np.array([1, 1, 1], np.float32),
                                base, 1e-6, 2.0, 20)
    ref = (1 / (1 + np.exp(-base[4:8].astype(np.float64)))).astype(np.float32) * np.float32(2.0)
    assert np.array_equal(post[0], ref) and np.array_equal(post[1], ref)


def test_sinkhorn_equal_logits_eps0_is_exactly_quarter():
    c = oracle.sinkhorn(np.full(16, 0.7, np.float32), 0.0, 20)
    assert (c == 0.25).all()


def test_sinkhorn_equal_logits_closed_form_with_eps():
    """Equal logits stay equal; the value follows the scalar recurrence
    v0 = 1/4 + eps, then per round: row step (not the first round)
    v <- v / (4v + eps), column step v <- v / (4v + eps)."""
    eps, repeat = 1e-3, 5
    c = oracle.sinkhorn(np.zeros(16, np.float32), eps, repeat)
    v = 0.25 + eps
    for it in range(repeat):
        if it > 0:
            v = v / (4 * v + eps)
        v = v / (4 * v + eps)
    assert np.allclose(c, v, rtol=3e-7, atol=0)


def textbook_sinkhorn_knopp(logits, rounds):
    a = np.exp(logits.astype(np.float64) - logits.max(axis=1, keepdims=True))
    a = a / a.sum(axis=1, keepdims=True)
    for it in range(rounds):
        if it > 0:
            a = a / a.sum(axis=1, keepdims=True)
        a = a / a.sum(axis=0, keepdims=True)
    return a


def test_sinkhorn_eps0_matches_textbook_sinkhorn_knopp():
    for _ in range(50):
        logits = RNG.standard_normal((4, 4)).astype(np.float32)
        c = oracle.sinkhorn(logits, 0.0, 20)
        ref = textbook_sinkhorn_knopp(logits, 20)
        assert np.abs(c - ref).max() <= 2e-6


def test_sinkhorn_column_and_row_sums():
    """The last step normalizes columns: each column sums to s/(s+eps) ~ 1 - eps.
    At 200 rounds the rows have converged to the same bound."""
    eps = 1e-6
    for _ in range(100):
        logits = RNG.standard_normal(16).astype(np.float32)
        c = oracle.sinkhorn(logits, eps, 20).astype(np.float64)
        assert np.abs(c.sum(axis=0) - 1).max() <= eps + 2 ** -20
        c = oracle.sinkhorn(logits, eps, 200).astype(np.float64)
        assert np.abs(c.sum(axis=1) - 1).max() <= eps + 2 ** -20


def test_side_mixes_use_the_right_slices_of_mixes_scale_base():
    """post' reads mixes[4:8], scale[1], base[4:8]; comb' reads mixes[8:24],
    scale[2], base[8:24] (row-major 4x4): perturbing other slices changes
    nothing."""
    mixes, scale, base = synth.raw_mixes(3)
    post, comb = oracle.side_mixes(mixes, scale, base, 1e-6, 2.0, 20)
    m2 = mixes.copy()
    m2[:, :4] += 1.0
    s2 = scale.copy()
    s2[0] += 1.0
    b2 = base.copy()
    b2[:4] += 1.0
    post2, comb2 = oracle.side_mixes(m2, s2, b2, 1e-6, 2.0, 20)
    assert np.array_equal(post, post2) and np.array_equal(comb, comb2)
    for t in range(3):
        logits = np.array([f32(exact(m) * exact(scale[2]) + exact(b))
                           for m, b in zip(mixes[t, 8:], base[8:])], np.float32)
        ref = oracle.sinkhorn(logits, 1e-6, 20)
        assert np.array_equal(comb[t], ref)
        pref = 2.0 / (1 + np.exp(-(mixes[t, 4:8].astype(np.float64) * scale[1] + base[4:8])))
        assert np.abs(post[t] - pref).max() <= 1e-6


# ---------------------------------------------------------------------------
# a6 finalize, a7 two-shot
# ---------------------------------------------------------------------------

def test_finalize_single_route_unit_weight_is_the_row():
    M, H, tp = 3, 64, 2
    rng = np.random.default_rng(9)
    gemm2 = rand_bf16((tp, M, H), 0.5, rng)
    idx = np.arange(M, dtype=np.int32)[:, None][::-1].copy()
    w = np.ones((M, 1), np.float32)
    shared = np.zeros((tp, M, H), np.uint16)
    c = oracle.finalize_contributions(gemm2, w, idx, shared)
    want = np.where(gemm2[:, idx[:, 0]] == 0x8000, 0, gemm2[:, idx[:, 0]])
    assert np.array_equal(c, want)


def test_finalize_never_publishes_negative_zero():
    """A contribution that rounds to BF16 negative zero is published as +0
    (negative zero is the mailbox's empty marker): the route row -2^-126
    (0x8080) times the weight 2^-20 is the binary32 subnormal -2^-146, which
    rounds to BF16 -0; the oracle returns 0x0000."""
    H = 8
    gemm2 = np.full((1, 1, H), 0x8080, np.uint16)
    w = np.array([[2.0 ** -20]], np.float32)
    idx = np.zeros((1, 1), np.int32)
    c = oracle.finalize_contributions(gemm2, w, idx, np.zeros((1, 1, H), np.uint16))
    # the exact product -2^-146 rounds to a BF16 zero
    assert bf16_bits_of(exact(bf16_value(np.uint16(0x8080))) * exact(w[0, 0])) == 0x0000
    assert (c == 0x0000).all()


def test_finalize_dropped_routes_leave_the_shared_expert():
    M, H, tp, k = 4, 64, 2, 3
    rng = np.random.default_rng(10)
    gemm2 = rand_bf16((tp, M * k, H), 0.5, rng)
    shared = rand_bf16((tp, M, H), 0.5, rng)
    idx = np.full((M, k), -1, np.int32)
    w = rng.uniform(0, 1, (M, k)).astype(np.float32)
    c = oracle.finalize_contributions(gemm2, w, idx, shared)
    assert np.array_equal(c, np.where(shared == 0x8000, 0, shared))
    idx = np.arange(M * k, dtype=np.int32).reshape(M, k)
    c0 = oracle.finalize_contributions(gemm2, np.zeros_like(w), idx, shared)
    assert np.array_equal(c0, np.where(shared == 0x8000, 0, shared))


def test_finalize_brute_force_exact_rationals():
    """acc = fma(row_k, w_k, acc) over k (one rounding per step), + shared,
    BF16, negative zero -> +0: checked with exact rationals."""
    M, H, tp, k = 2, 16, 2, 4
    rng = np.random.default_rng(11)
    gemm2 = rand_bf16((tp, M * k, H), 0.5, rng)
    shared = rand_bf16((tp, M, H), 0.5, rng)
    idx = np.stack([rng.permutation(M * k).astype(np.int32).reshape(M, k) for _ in range(tp)])
    idx[0, 1, 2] = -1
    w = rng.uniform(0, 1, (tp, M, k)).astype(np.float32)
    c = oracle.finalize_contributions(gemm2, w, idx, shared, replicated_routing=False)
    for r in range(tp):
        for t in range(M):
            for col in range(H):
                acc = 0.0
                for kk in range(k):
                    row = idx[r, t, kk]
                    if row == -1:
                        continue
                    acc = f32(exact(bf16_value(gemm2[r, row, col])) * exact(w[r, t, kk]) + exact(acc))
                want = bf16_bits_of(exact(f32(exact(acc) + exact(bf16_value(shared[r, t, col])))))
                assert c[r, t, col] == want


def test_routing_weights_bf16_values_from_the_format():
    """BF16 routing weights widen exactly: sign, 8-bit exponent, 7-bit
    fraction (1.0, -3.0, 0.25, +-0, the smallest normal, 2^-133)."""
    bits = np.array([0x3F80, 0xC040, 0x3E80, 0x0000, 0x8000, 0x0080, 0x0001], np.uint16)
    got = oracle.routing_weights(bits)
    want = np.array([1.0, -3.0, 0.25, 0.0, -0.0, 2.0 ** -126, 2.0 ** -133], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_routing_weights_scale_is_one_fp32_product():
    """A factor of 1 leaves the bits alone (-0 and subnormals included);
    otherwise each weight is the correctly rounded FP32 product."""
    rng = np.random.default_rng(40)
    w = np.concatenate([rng.uniform(-2, 2, 64).astype(np.float32),
                        np.array([-0.0, 1e-42, 1 + 2.0 ** -23], np.float32)])
    assert np.array_equal(oracle.routing_weights(w, 1.0).view(np.uint32), w.view(np.uint32))
    for scale in (2.5, 1 + 2.0 ** -23, 0.3):
        got = oracle.routing_weights(w, scale)
        s32 = float(np.float32(scale))
        for g, x in zip(got, w):
            assert g == np.float32(f32(exact(x) * exact(s32))), (x, scale)
    # 1 + 2^-23 squared is 1 + 2^-22 + 2^-46: one rounding gives 1 + 2^-22.
    assert oracle.routing_weights(np.array([1 + 2.0 ** -23], np.float32), 1 + 2.0 ** -23)[0] == \
        np.float32(1 + 2.0 ** -22)


def test_finalize_bf16_scaled_weights_brute_force():
    """BF16 routing weights times a routed scale of 0.3, each route's weight
    scaled before its FMA (not the sum afterwards): exact rationals."""
    M, H, tp, k = 2, 8, 2, 3
    rng = np.random.default_rng(41)
    gemm2 = rand_bf16((tp, M * k, H), 0.5, rng)
    shared = rand_bf16((tp, M, H), 0.5, rng)
    idx = np.stack([rng.permutation(M * k).astype(np.int32).reshape(M, k) for _ in range(tp)])
    idx[1, 0, 1] = -1
    wb = rand_bf16((tp, M, k), 0.5, rng)
    c = oracle.finalize_contributions(gemm2, wb, idx, shared, replicated_routing=False,
                                      routed_scaling_factor=0.3)
    s32 = float(np.float32(0.3))
    for r in range(tp):
        for t in range(M):
            for col in range(H):
                acc = 0.0
                for kk in range(k):
                    row = idx[r, t, kk]
                    if row == -1:
                        continue
                    w = f32(exact(bf16_value(wb[r, t, kk])) * exact(s32))
                    acc = f32(exact(bf16_value(gemm2[r, row, col])) * exact(w) + exact(acc))
                want = bf16_bits_of(exact(f32(exact(acc) + exact(bf16_value(shared[r, t, col])))))
                assert c[r, t, col] == want


def test_two_shot_owner_layout_and_bit_equality():
    """Token t sits in owner t % tp, slot t // tp; the owner reduce gives the
    same bits as the direct sum (the pages' claim), here with -0 and
    cancellations injected."""
    f = synth.moe_finalize(10, H=128, tp=4, top_k=3, replicated_routing=False, drop_fraction=0.2)
    contrib = oracle.finalize_contributions(f.gemm2, f.weights, f.idx, f.shared,
                                            replicated_routing=False)
    own = oracle.two_shot_publish(contrib)
    for t in range(10):
        for r in range(4):
            assert np.array_equal(own[t % 4, r, t // 4], contrib[r, t])
    reduced = oracle.owner_reduce(own, 10)
    direct = np.array([[oracle.rank_sum_element(contrib, t * 128 + c) for c in range(128)]
                       for t in range(10)], np.uint16)
    assert np.array_equal(reduced, direct)
    args = (f.gemm2, f.weights, f.idx, f.shared, f.residual, f.post, f.comb, f.pre, f.gamma, 1e-6)
    a = oracle.finalize(*args, two_shot=False, replicated_routing=False, mxfp8=True)
    b = oracle.finalize(*args, two_shot=True, replicated_routing=False, mxfp8=True)
    for x, y in zip((a[0], a[1], *a[2]), (b[0], b[1], *b[2])):
        assert np.array_equal(x, y)


def test_owner_reduce_order_designed_case():
    """The owner adds contributions from rank 0 like the one-shot consumer:
    on ranks (1, 2^-8, 2^-24, 2^-24) only that order gives 1.0."""
    contrib = np.zeros((4, 5, 8), np.uint16)
    contrib[:, 3, 2] = [0x3F80, 0x3B80, 0x3380, 0x3380]
    reduced = oracle.owner_reduce(oracle.two_shot_publish(contrib), 5)
    assert reduced[3, 2] == 0x3F80
    reduced = oracle.owner_reduce(oracle.two_shot_publish(contrib[::-1].copy()), 5)
    assert reduced[3, 2] == 0x3F81


def test_finalize_equals_boundary_on_contributions():
    f = synth.moe_finalize(5, H=256, tp=2, top_k=4)
    contrib = oracle.finalize_contributions(f.gemm2, f.weights, f.idx, f.shared)
    a = oracle.finalize(f.gemm2, f.weights, f.idx, f.shared, f.residual, f.post, f.comb, f.pre,
                        f.gamma, 1e-6)
    b = oracle.boundary(contrib, f.residual, f.post, f.comb, f.pre, f.gamma, 1e-6)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _glm_moe_inputs(M, H, tp, top_k):
    f = synth.moe_finalize(M, H=H, tp=tp, top_k=top_k, replicated_routing=False)
    g = synth.glm(M, H=H, tp=tp)
    return f, g


def test_glm_moe_with_every_route_dropped_is_the_glm_boundary_on_shared():
    """No rank holds any routed expert: each contribution is the rank's
    shared-expert output with -0 made +0, so the MoE GLM boundary is the GLM
    boundary on those shared outputs."""
    f, g = _glm_moe_inputs(3, 256, 2, 2)
    idx = np.full_like(f.idx, -1)
    shared = f.shared.copy()
    shared[0, 1, :5] = 0x8000
    shared[1, 2, 7] = 0x8000
    got = oracle.boundary_glm_moe(f.gemm2, f.weights, idx, shared, g.residual, g.post, g.comb,
                                  g.fn, g.scale, g.base, g.gamma, 1e-6, 1e-6, 1e-6,
                                  replicated_routing=False)
    plain = np.where(shared == 0x8000, np.uint16(0), shared)
    want = oracle.boundary_glm(plain, g.residual, g.post, g.comb, g.fn, g.scale, g.base, g.gamma,
                               1e-6, 1e-6, 1e-6)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)


def test_glm_moe_single_unit_route_is_the_glm_boundary_on_the_rows():
    """tp = 1, top_k = 1, weight 1, shared zero: the contribution is the
    routed row itself, so the MoE GLM boundary is the GLM boundary on the
    rows in route order."""
    f, g = _glm_moe_inputs(4, 256, 1, 1)
    weights = np.ones((4, 1), np.float32)
    idx = np.array([[2], [0], [3], [1]], np.int32)
    shared = np.zeros_like(f.shared)
    got = oracle.boundary_glm_moe(f.gemm2, weights, idx, shared, g.residual, g.post, g.comb,
                                  g.fn, g.scale, g.base, g.gamma, 1e-6, 1e-6, 1e-6)
    rows = f.gemm2[:, idx[:, 0]]
    rows = np.where(rows == 0x8000, np.uint16(0), rows)
    want = oracle.boundary_glm(rows, g.residual, g.post, g.comb, g.fn, g.scale, g.base, g.gamma,
                               1e-6, 1e-6, 1e-6)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# a8 MXFP8
# ---------------------------------------------------------------------------

def test_e4m3_code_values_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(int(c)) for c in codes])
    finite = (codes & 0x7F) != 0x7F
    assert np.array_equal(got[finite], ref[finite])


def test_e4m3_conversion_matches_torch_rne():
    """|x| <= 448: nearest-even E4M3 == torch's float32 -> float8_e4m3fn
    conversion, on random values, every midpoint between adjacent codes and
    the subnormal range."""
    vals = [RNG.uniform(-448, 448, 3000), RNG.standard_normal(2000) * 2.0 ** -7,
            RNG.standard_normal(1000) * 2.0 ** -10]
    pos = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids = (pos[:-1] + pos[1:]) / 2
    vals += [mids, -mids, pos, -pos]
    x = np.concatenate(vals).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_rne_sat(x), ref)


def test_e4m3_saturates_finite():
    x = np.array([448.0, 449.0, 464.0, 480.0, 1e6, np.inf, -450.0, -np.inf], np.float32)
    assert list(oracle.e4m3_rne_sat(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_ue8m0_exhaustive_over_bf16_block_maxima():
    """For every finite non-negative BF16 block max a: e = the smallest e with
    2^(e-127) >= fl(a * fl(1/448)), computed with exact rationals."""
    inv448 = np.float32(1.0 / 448.0)
    a = bf16_value(FINITE_BF16[FINITE_BF16 < 0x8000])
    v = (a * inv448).astype(np.float32)
    for vv in v[:: 1]:
        q = exact(vv)
        e = 0
        while e < 254 and Fraction(2) ** (e - 127) < q:
            e += 1
        assert oracle.ue8m0_round_up(float(vv)) == e


def test_mxfp8_zero_block_and_roundtrip_bounds():
    """A zero block has scale 0 and codes 0.  Dequantized codes are within
    half an E4M3 step of the input at the block's scale, and requantizing the
    dequantized values at the same scale returns the same codes."""
    M, H = 6, 512
    x = rand_bf16((M, H), 1.0)
    for t in range(M):                      # the block max at every lane position once
        for b in range(H // 32):
            lane = (t * 16 + b) % 32
            x[t, b * 32 + lane] = torch_bf16([8.0 * (1 + b % 3)])[0] ^ (0x8000 * (b % 2))
    x[1, 32:64] = 0
    values, scales = oracle.quant_mxfp8(x)
    K = H // 32
    assert scales[oracle.sf_index(1, 1, K)] == 0 and (values[1, 32:64] == 0).all()
    table = np.array([oracle.e4m3_value(c) for c in range(256)])
    xv = bf16_value(x).astype(np.float64)
    for t in range(M):
        for b in range(K):
            e = int(scales[oracle.sf_index(t, b, K)])
            s = 2.0 ** (e - 127)
            deq = table[values[t, b * 32:(b + 1) * 32]] * s
            blk = xv[t, b * 32:(b + 1) * 32]
            step = np.where(np.abs(blk) >= 2.0 ** -6 * s,
                            2.0 ** (np.floor(np.log2(np.maximum(np.abs(blk), 1e-300))) - 3),
                            2.0 ** -9 * s)
            assert (np.abs(deq - blk) <= step / 2 + 1e-30).all()
            amax = np.abs(blk).max()
            assert amax == 0 or 224 < amax / s <= 448    # the smallest such power of two
            re = oracle.e4m3_rne_sat((deq / s).astype(np.float32))
            assert np.array_equal(re, values[t, b * 32:(b + 1) * 32])


def test_swizzled_scale_layout_is_a_bijection_and_matches_tile_transpose():
    """The 128x4 swizzle: a bijection onto [0, padded_rows * K), equal to
    cutting the [rows, K] scale matrix into 128x4 tiles (row-major over
    tiles), each stored as [32 lines][4 row groups][4 columns]."""
    for M, H in ((1, 128), (100, 512), (256, 1024), (300, 5120)):
        K = H // 32
        Mp = -(-M // 128) * 128
        idx = np.array([[oracle.sf_index(r, k, K) for k in range(K)] for r in range(Mp)])
        assert sorted(idx.ravel().tolist()) == list(range(Mp * K))
        assert oracle.mxfp8_scale_bytes(M, H) == Mp * K
        lin = np.arange(Mp * K).reshape(Mp, K)
        tiles = lin.reshape(Mp // 128, 4, 32, K // 4, 4)          # [rt, rgroup, line, kt, col]
        tiles = tiles.transpose(0, 3, 2, 1, 4).reshape(-1)        # [rt, kt, line, rgroup, col]
        flat = np.empty(Mp * K, np.int64)
        flat[np.arange(Mp * K)] = tiles                           # storage order -> linear id
        pos = np.empty(Mp * K, np.int64)
        pos[flat] = np.arange(Mp * K)                             # linear id -> storage offset
        assert np.array_equal(pos.reshape(Mp, K), idx)


def test_mxfp8_padding_rows_scales_zero():
    x = rand_bf16((100, 256), 1.0)
    _, scales = oracle.quant_mxfp8(x)
    K = 8
    pad = [oracle.sf_index(r, k, K) for r in range(100, 128) for k in range(K)]
    assert (scales[pad] == 0).all()


def test_golden_format_constants():
    """Values fixed by the OCP 8-bit floating point specification and the
    BF16 format, stored as a cited text fixture."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "format_constants.txt")
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        kind, a, b = line.split()
        if kind == "e4m3":
            assert oracle.e4m3_value(int(a, 16)) == float(b)
        elif kind == "e4m3_of":
            assert oracle.e4m3_rne_sat(np.float32(float(a))) == int(b, 16)
        elif kind == "bf16_of":
            assert oracle.f32_to_bf16(np.float32(float(a))) == int(b, 16)
        elif kind == "ue8m0_of":
            assert oracle.ue8m0_round_up(float(a)) == int(b)


# ---------------------------------------------------------------------------
# Structure: token independence, threads, residual-only
# ---------------------------------------------------------------------------

def test_tokens_are_independent_and_threads_do_not_change_bits():
    b = synth.boundary(9, 6, 256, 3, 0.5)
    full = oracle.boundary(b.partials, b.residual, b.post, b.comb, b.pre, b.gamma, 1e-6,
                           mxfp8=True, threads=3)
    part = oracle.boundary(b.partials[:, :4], b.residual[:4], b.post[:4], b.comb[:4], b.pre[:4],
                           b.gamma, 1e-6, mxfp8=True, threads=1)
    assert np.array_equal(full[0][:4], part[0]) and np.array_equal(full[1][:4], part[1])
    assert np.array_equal(full[2][0][:4], part[2][0])


def test_residual_only_variant_writes_the_same_streams():
    b = synth.tiny_delayed()
    a = oracle.boundary(b.partials, b.residual, b.post, b.comb, b.pre, b.gamma, 1e-6)
    r = oracle.boundary(b.partials, b.residual, b.post, b.comb, None, None, 1e-6)
    assert np.array_equal(a[0], r[0]) and r[1] is None
    with pytest.raises(ValueError):
        oracle.boundary(b.partials, b.residual, b.post, b.comb, b.pre, None, 1e-6)


def test_mailbox_model_cycles_and_resets():
    from oracle.mailbox_model import MailboxModel
    mb = MailboxModel(2, 8, 16)
    x = rand_bf16((2, 5, 16))
    x[0, 0, 0] = 0x8000
    for g in (0, 1, 2, 0):
        mb.publish(x)
        assert mb.stage[0] == g
        got = mb.consume(5)
        assert got[0, 0, 0] == 0 and np.array_equal(got[1], x[1])
        assert mb.stage[1] == (g + 1) % 3
        assert (mb.slots == 0x8000).all()


# ---------------------------------------------------------------------------
# DSA indexer projection
# ---------------------------------------------------------------------------

def test_indexer_one_hot_rows_pick_input_columns():
    """Weight row r = 1.0 at one column c_r: every output is x[t, c_r], exact
    in each part's type, so the part boundaries and the row order (key rows,
    then head rows, then gate rows) are pinned."""
    rng = np.random.default_rng(31)
    M, K, key, heads, gate = 5, 256, 16, 8, 24
    x = rand_bf16((M, K), 1.0, rng)
    cols = rng.permutation(K)[:key + heads + gate]
    w = np.zeros((key + heads + gate, K), np.uint16)
    w[np.arange(len(cols)), cols] = 0x3F80
    k_out, h_out, g_out = oracle.indexer_projection(x, w, key, heads, gate)
    assert np.array_equal(k_out, x[:, cols[:key]])
    assert np.array_equal(h_out, bf16_value(x[:, cols[key:key + heads]]))
    assert np.array_equal(g_out, x[:, cols[key + heads:]])


def test_indexer_matches_float64_matmul():
    """Against numpy's float64 product (a library routine): the head weights
    within one binary32 ulp, the BF16 parts within one BF16 ulp."""
    rng = np.random.default_rng(32)
    M, K, key, heads, gate = 3, 1024, 16, 8, 16
    x = rand_bf16((M, K), 1.0, rng)
    w = rand_bf16((key + heads + gate, K), 0.02, rng)
    k_out, h_out, g_out = oracle.indexer_projection(x, w, key, heads, gate)
    ref = bf16_value(x).astype(np.float64) @ bf16_value(w).astype(np.float64).T
    assert f32_ulp_distance(h_out, ref[:, key:key + heads].astype(np.float32)).max() <= 1
    assert bf16_ulp_distance(k_out, torch_bf16(ref[:, :key].astype(np.float32))).max() <= 1
    assert bf16_ulp_distance(g_out, torch_bf16(ref[:, key + heads:].astype(np.float32))).max() <= 1


def test_indexer_sum_is_rounded_once():
    """A row whose products cancel except for a tiny term: 1 + 2^-30 - 1
    summed exactly gives 2^-30 (a rounding per addition would lose it)."""
    K = 8
    x = np.zeros((1, K), np.uint16)
    x[0, :3] = [0x3F80, 0x3080, 0xBF80]          # 1, 2^-30, -1
    w = np.zeros((1, K), np.uint16)
    w[0, :3] = 0x3F80
    _, h_out, _ = oracle.indexer_projection(x, w, 0, 1, 0)
    assert h_out[0, 0] == np.float32(2.0 ** -30)
