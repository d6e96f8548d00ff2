"""The GPU tests' comparison helpers, checked on the CPU: the tie-aware GLM
layer-input rule admits a 2-ulp difference only where the oracle's FP32
collapse can round either way, and the ulp distance is a true BF16 ulp count."""
import numpy as np
import pytest

from tests.gpu_util import bf16_ulp_distance, glm_layer_input_check


def _bits(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_bf16_ulp_distance_counts_steps_across_zero_and_binades():
    a = np.array([0x3F80, 0x3F80, 0x0001, 0x8001, 0x3F7F], np.uint16)
    b = np.array([0x3F81, 0x3F82, 0x8001, 0x0001, 0x3F80], np.uint16)
    assert bf16_ulp_distance(a, b).tolist() == [1, 2, 2, 2, 1]


def test_cancelling_collapse_near_a_midpoint_admits_two_ulps():
    # q ~ [0.333, 0.069, -0.331, -0.072]: z ~ 3.16e-5 sits 0.13 BF16 steps from
    # a midpoint, inside the rounding of the 0.33-sized terms.
    y = _bits([0.51171875, 0.07373047, -0.35351562, -0.23144531]).reshape(1, 4, 1)
    pre_ref = np.array([[0.6516359, 0.93727237, 0.93519026, 0.31075954]], np.float32).astype(np.float64)
    pre_got = np.array([[0.65163584, 0.93727235, 0.93519024, 0.31075956]])
    one, two = glm_layer_input_check(np.array([[0x3770]], np.uint16), np.array([[0x3772]], np.uint16),
                                     y, pre_ref, pre_got)
    assert (one, two) == (0, 1)


def test_two_ulps_away_from_any_midpoint_fail():
    # Terms of the same size as z: the band is a few FP32 ulps, far from the
    # BF16 midpoint distance.
    y = _bits([1.0, 0.5, 0.25, 0.125]).reshape(1, 4, 1)
    pre = np.array([[0.3, 0.3, 0.3, 0.3]])
    with pytest.raises(AssertionError, match="near tie: False"):
        glm_layer_input_check(np.array([[0x3F80]], np.uint16), np.array([[0x3F82]], np.uint16),
                              y, pre, pre)
    with pytest.raises(AssertionError):
        glm_layer_input_check(np.array([[0x3F80]], np.uint16), np.array([[0x3F83]], np.uint16),
                              y, pre, pre)
