"""Helpers of the GPU parity tests: host <-> device transfer of BF16 bit
patterns, and the tie-aware comparison of GLM layer inputs."""
from __future__ import annotations

import numpy as np
import torch

from tests.numerics import bf16_ulp_distance, bf16_value


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> cuda tensor; uint16 arrays become BF16 tensors (same bits)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a).copy()).cuda()


def u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str) -> None:
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"{what}: {len(bad)} of {got.size} elements differ, first at "
                             f"{tuple(bad[0])}: got {got[tuple(bad[0])]:#x} want {want[tuple(bad[0])]:#x}")


def assert_within_ulp(got: np.ndarray, want: np.ndarray, ulps: int, what: str) -> int:
    d = bf16_ulp_distance(got, want)
    if d.max() > ulps:
        i = np.unravel_index(np.argmax(d), d.shape)
        raise AssertionError(f"{what}: max {d.max()} BF16 ulps at {i} (allowed {ulps})")
    return int((d > 0).sum())


def glm_pre(mixes: np.ndarray, scale: np.ndarray, base: np.ndarray, hc_eps: float) -> np.ndarray:
    """pre_j = sigmoid(mixes_j * scale0 + base_j) + hc_eps in float64."""
    x = mixes[:, :4].astype(np.float64) * float(scale[0]) + base[:4].astype(np.float64)
    return 1.0 / (1.0 + np.exp(-x)) + hc_eps


def _ulp32(v: np.ndarray) -> np.ndarray:
    return np.spacing(np.abs(v).astype(np.float32)).astype(np.float64)


def glm_layer_input_check(got_li, ref_li, y, pre_ref, pre_got):
    """The GLM layer input within 1 BF16 ulp of the oracle, except <= 2 where
    the oracle's FP32 collapse (q0+q1)+(q2+q3), q_j = y_j * pre_j, lies within
    the pre-mix error band of a BF16 rounding midpoint (the pre-mix is derived
    in-kernel, so an FP32-ulp difference there can flip the collapse's BF16
    rounding).  The band bounds how far the GPU's FP32 collapse can be from
    the oracle's: sum_j (|y_j| |pre_got_j - pre_ref_j| + ulp(q_j)) +
    ulp(q0+q1) + ulp(q2+q3) + ulp(z) -- a changed pre can move every rounded
    term by one ulp, which under cancellation is many ulps of z.
    Returns (elements off by 1, elements off by 2)."""
    d = bf16_ulp_distance(got_li, ref_li)
    yv = bf16_value(y).astype(np.float32)                          # [M, 4, H]
    pre32 = pre_ref.astype(np.float32)[:, :, None]
    q = yv * pre32                                                 # FP32 products
    s01, s23 = q[:, 0] + q[:, 1], q[:, 2] + q[:, 3]
    z = (s01 + s23).astype(np.float64)                             # the oracle's FP32 collapse
    band = (np.abs(yv.astype(np.float64)) * np.abs(pre_got - pre_ref)[:, :, None]).sum(axis=1)
    band += _ulp32(q).sum(axis=1) + _ulp32(s01) + _ulp32(s23) + _ulp32(z)
    # distance from z to the nearest BF16 rounding midpoint
    zb = np.abs(z).astype(np.float32)
    e = np.floor(np.log2(np.maximum(zb, 1e-38)))
    step = np.exp2(e - 7)                                          # BF16 spacing at |z|
    mid_dist = np.abs((np.abs(z) / step) % 1.0 - 0.5) * step
    near = mid_dist <= band
    if (d > 2).any() or ((d == 2) & ~near).any():
        i = np.unravel_index(np.argmax(np.where(near, d - 1, d)), d.shape)
        raise AssertionError(f"GLM layer_input: {d[i]} ulps at {i} (near tie: {near[i]})")
    return int((d == 1).sum()), int((d == 2).sum())
