"""The GPU tests' comparison helpers, checked on the CPU.

The GLM layer-input rule must admit whatever the kernel's arithmetic gives
for a pre-mix within its error, including several ulps where the collapse
cancels, and reject results outside that; the ulp distance must be a true
BF16 ulp count.  The kernel's arithmetic for a given pre-mix is restated
here (FP32 products and sums, BF16 roundings, binary64 sum of squares), so
a result "from a perturbed pre-mix" is what the GPU would give."""
import numpy as np
import pytest

from tests.gpu_util import bf16_ulp_distance, glm_layer_input_check


def _bf16_bits(x):
    """float32 values -> BF16 bit patterns, ties to even (finite inputs)."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def _bf16_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _collapse_norm(y, pre, gamma, eps):
    """[M, 4, H] BF16 streams, [M, 4] pre-mix, [H] BF16 gamma -> [M, H] BF16
    layer input: p = bf16((q0+q1)+(q2+q3)), q_j = y_j * pre_j in FP32; inv =
    1/sqrt(sum p^2 / H + eps) (binary64 sum, FP32 factor); bf16((p*inv)*gamma)."""
    yv = _bf16_f32(y)
    q = yv * pre.astype(np.float32)[:, :, None]
    p = _bf16_f32(_bf16_bits((q[:, 0] + q[:, 1]) + (q[:, 2] + q[:, 3])))
    H = p.shape[1]
    pss = (p.astype(np.float64) ** 2).sum(axis=1)
    inv = (1.0 / np.sqrt(pss.astype(np.float32).astype(np.float64) / H + eps)).astype(np.float32)
    return _bf16_bits((p * inv[:, None]) * _bf16_f32(gamma))


def _token_with_cancellation(rng, H=8):
    # Element 0: terms of about 0.16 that cancel to about 7e-7, where one FP32
    # ulp of a term is about four BF16 ulps of the sum; the rest ordinary.
    y = _bf16_bits(rng.normal(0.0, 0.5, (1, 4, H)))
    y[0, :, 0] = _bf16_bits([-0.22265625, 0.3828125, 0.0145874, -0.04101562])
    pre = np.array([[0.7058807, 0.40444183, 0.69123423, 0.18872504]], np.float32)
    gamma = _bf16_bits(1.0 + 0.1 * rng.normal(size=H))
    return y, pre, gamma


def test_bf16_ulp_distance_counts_steps_across_zero_and_binades():
    a = np.array([0x3F80, 0x3F80, 0x0001, 0x8001, 0x3F7F], np.uint16)
    b = np.array([0x3F81, 0x3F82, 0x8001, 0x0001, 0x3F80], np.uint16)
    assert bf16_ulp_distance(a, b).tolist() == [1, 2, 2, 2, 1]


def test_cancelling_collapse_admits_the_ulps_a_pre_ulp_moves():
    rng = np.random.default_rng(1)
    y, pre, gamma = _token_with_cancellation(rng)
    ref = _collapse_norm(y, pre, gamma, 1e-6)
    pre_got = pre.copy()
    pre_got[0, 0] = np.nextafter(pre[0, 0], np.float32(1))  # one FP32 ulp
    got = _collapse_norm(y, pre_got, gamma, 1e-6)
    d = bf16_ulp_distance(got, ref)
    assert d[0, 0] >= 3, "the case should move the cancelling element by several ulps"
    one, more = glm_layer_input_check(got, ref, y, pre.astype(np.float64),
                                      pre_got.astype(np.float64), gamma, 1e-6)
    assert more >= 1


def test_results_outside_the_band_fail():
    rng = np.random.default_rng(2)
    y, pre, gamma = _token_with_cancellation(rng)
    ref = _collapse_norm(y, pre, gamma, 1e-6)
    pre64 = pre.astype(np.float64)
    # The band is then one FP32 rounding of each term: about 15 BF16 ulps of
    # the cancelling element, a small fraction of one for an ordinary one.
    for col, k in ((0, 40), (3, 2)):
        bad = ref.copy()
        bad[0, col] += k
        with pytest.raises(AssertionError, match="outside"):
            glm_layer_input_check(bad, ref, y, pre64, pre64, gamma, 1e-6)


def test_results_from_slightly_different_pre_mixes_pass():
    # What the GPU can give: the same arithmetic on pre-mixes a few FP32 ulps
    # away, over tokens whose four terms often cancel.
    rng = np.random.default_rng(3)
    M, H = 64, 256
    y = _bf16_bits(rng.normal(0.0, 0.5, (M, 4, H)))
    y[:, 3] = _bf16_bits(-(_bf16_f32(y[:, 0]) + _bf16_f32(y[:, 1]) + _bf16_f32(y[:, 2]))
                         + rng.normal(0.0, 1e-3, (M, H)))
    pre = np.full((M, 4), 1.0, np.float32) + rng.uniform(-1e-3, 1e-3, (M, 4)).astype(np.float32)
    gamma = _bf16_bits(1.0 + 0.1 * rng.normal(size=H))
    ref = _collapse_norm(y, pre, gamma, 1e-6)
    pre_got = (pre * (1 + rng.uniform(-3e-7, 3e-7, (M, 4)))).astype(np.float32)
    got = _collapse_norm(y, pre_got, gamma, 1e-6)
    one, more = glm_layer_input_check(got, ref, y, pre.astype(np.float64),
                                      pre_got.astype(np.float64), gamma, 1e-6)
    assert one + more > 0, "the perturbation should change some roundings"
