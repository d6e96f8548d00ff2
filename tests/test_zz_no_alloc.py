"""mhcb_boundary_glm_noalloc (the GLM boundary for callers that cannot
allocate) through the C ABI: bit-identical to mhcb_boundary_glm with a
workspace on the same inputs, on two calls in a row, the second smaller, and
within the GLM bars of the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import assert_bits_equal, check_glm_outputs, dev, host, u16

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import tp_reduce_mhc_amd as mhc


def _outputs(M, H):
    return (torch.full((M, 4, H), float("nan"), dtype=torch.bfloat16, device="cuda"),
            torch.full((M, 24), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((M, H), float("nan"), dtype=torch.bfloat16, device="cuda"))


def _run(g, noalloc):
    M, H = g.M, g.H
    ro, mixes, li = _outputs(M, H)
    args = (dev(g.partials), M * H, dev(g.residual), dev(g.post), dev(g.comb), dev(g.fn),
            dev(g.scale), dev(g.base), dev(g.gamma), ro, mixes, li)
    if noalloc:
        mhc.mhcb_boundary_glm_noalloc(*args, M, H, 4, g.tp, g.rms_eps, g.hc_eps, g.norm_eps)
    else:
        ws = mhc.new_workspace(mhc.mhcb_workspace_bytes(M, H, g.tp, 0), "cuda")
        mhc.mhcb_boundary_glm(*args, ws, ws.numel(), M, H, 4, g.tp, g.rms_eps, g.hc_eps,
                              g.norm_eps, -16)
    torch.cuda.synchronize()
    return u16(ro), host(mixes), u16(li)


def test_glm_noalloc_matches_the_workspace_entry_point_twice():
    for g in (synth.glm(300), synth.glm(17, H=2048, tp=4)):
        print(f"[gpu] no-alloc {g.name}", flush=True)
        got = _run(g, True)
        want = _run(g, False)
        assert_bits_equal(got[0], want[0], f"{g.name} residual_out")
        assert np.array_equal(got[1], want[1]), f"{g.name} mixes"
        assert_bits_equal(got[2], want[2], f"{g.name} layer_input")
        ro_ref, mix_ref, li_ref, pre_ref = oracle.boundary_glm(
            g.partials, g.residual, g.post, g.comb, g.fn, g.scale, g.base, g.gamma, g.rms_eps,
            g.hc_eps, g.norm_eps, threads=oracle.default_threads())
        check_glm_outputs(f"no-alloc {g.name}", got[0], got[1], got[2], ro_ref, mix_ref, li_ref,
                          pre_ref, g.scale, g.base, g.gamma, g.hc_eps, g.norm_eps)
