"""Benchmark of the fused TP-reduce + mHC + RMSNorm sublayer boundary on one
MI355X.

Headline step: one delayed-mHC boundary call (TP partial sum, post-mix,
collapse, RMSNorm) on the DSV4.1-shaped workload, hidden 5120, tp 8, M = 128
decode tokens, all inputs resident in HBM.  Buffers rotate over > 3x the
256 MB Infinity Cache so every call streams from HBM; the K timed calls are
replayed from a captured HIP graph and bracketed by synchronizations.

One JSON line on stdout: the metric, value (achieved HBM GB/s of algorithmic
bytes), ms_per_step, the roofline of the boundary kernel, the oracle's CPU
baseline, the M sweep (us/call at M = 1 and 64), and the other workloads
(MoE finalize, GLM, MXFP8 at M = 8192, mailbox-fed).

  python bench.py [--steps K] [--warmup W] [--quick] [--only headline|...]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused reduce+mHC+RMSNorm: achieved HBM GB/s, tokens/s; µs/call at M=1,64"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "boundary_dsv41_M128_traffic.txt")
TRACE_FILE = os.path.join(ROOT, "profiles", "boundary_dsv41_M128_trace.txt")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Algorithmic bytes (each tensor counted once; weights once per call)
# ---------------------------------------------------------------------------

def bytes_delayed(M, H, tp, mxfp8=False, hc=4):
    # partials, hc residual streams in and out, the layer input; post, comb, pre
    per_token = (tp + 2 * hc + 1) * 2 * H + 4 * (2 * hc + hc * hc)
    if mxfp8:
        per_token += H + H // 32
    pad = ((M + 127) // 128 * 128 - M) * (H // 32) if mxfp8 else 0
    return M * per_token + 2 * H + pad


def bytes_mailbox_extra(M, H, tp):
    # producer reads the partials and writes the slots; the consumer resets them
    return M * 3 * tp * 2 * H


def bytes_finalize(M, H, tp, top_k, weight_bytes=4):
    return M * (tp * (top_k + 1) * 2 * H + top_k * (4 + weight_bytes) + 9 * 2 * H + 96) + 2 * H


def bytes_glm(M, H, tp):
    return M * (tp * 2 * H + 9 * 2 * H + 80 + 96) + 24 * 4 * H * 2 + 2 * H + 27 * 4


# The files the headline kernel (boundary_balanced_kernel, eight waves) is
# compiled from: a change to any of them invalidates the committed counter
# summary.
HEADLINE_SOURCES = ("boundary.hip", "device.h", "kernels.h", "sync.h", "finalize.h")


def source_hash():
    h = hashlib.sha256()
    for name in HEADLINE_SOURCES:
        h.update(open(os.path.join(ROOT, "tp_reduce_mhc_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def profile_fields(path):
    """The `key: value` lines of a committed rocprofv3 summary, if it was
    taken on the current kernel sources (its source_hash matches)."""
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    return fields if fields.get("source_hash") == source_hash() else None


def measured_traffic():
    """HBM bytes per launch of the headline kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    fields = profile_fields(TRAFFIC_FILE)
    try:
        return float(fields["hbm_bytes_per_launch"]) if fields else None
    except (KeyError, ValueError):
        return None


def traced_kernel_us():
    """(mean, median) duration in us of the headline kernel from the
    committed rocprofv3 kernel trace, if it was taken on the current source."""
    fields = profile_fields(TRACE_FILE)
    try:
        return (float(fields["kernel_mean_us"]), float(fields["kernel_median_us"])) if fields else None
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

USE_GRAPH = True


class Timed:
    """Times `steps` calls of fn(i) (i = rotation index), captured in a HIP
    graph when possible, with HIP events on the launching stream."""

    def __init__(self, torch, fn, steps, warmup, use_graph=None):
        self.torch = torch
        self.fn, self.steps, self.warmup = fn, steps, warmup
        self.graph = None
        self.use_graph = USE_GRAPH if use_graph is None else use_graph

    def run(self):
        torch = self.torch
        for i in range(self.warmup):
            self.fn(i)
        torch.cuda.synchronize()
        if self.use_graph:
            try:
                s = torch.cuda.Stream()
                s.wait_stream(torch.cuda.current_stream())
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    for i in range(self.steps):
                        self.fn(i)
                torch.cuda.synchronize()
                g.replay()               # untimed replay
                torch.cuda.synchronize()
                self.graph = g
            except Exception as e:  # capture unsupported: time eagerly
                log(f"graph capture failed ({e}); timing eager launches")
                self.graph = None
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        if self.graph is not None:
            self.graph.replay()
        else:
            for i in range(self.steps):
                self.fn(i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / self.steps  # ms per call


def rotations(per_set_bytes, minimum=4):
    return max(minimum, int(np.ceil(3.2 * MALL_BYTES / max(per_set_bytes, 1))))


def make_sets(torch, tensors, count):
    """`count` copies of the input tensors in distinct HBM."""
    sets = [tensors]
    for _ in range(count - 1):
        sets.append({k: v.clone() for k, v in tensors.items()})
    torch.cuda.synchronize()
    return sets


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

def dev(torch, a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a).copy()).cuda()


def delayed_sets(torch, b, count):
    t = dict(partials=dev(torch, b.partials), residual=dev(torch, b.residual),
             post=dev(torch, b.post), comb=dev(torch, b.comb), pre=dev(torch, b.pre),
             gamma=dev(torch, b.gamma))
    sets = make_sets(torch, t, count)
    for s in sets:
        s["residual_out"] = torch.empty(b.residual.shape, dtype=torch.bfloat16, device="cuda")
        s["layer_input"] = torch.empty((b.M, b.H), dtype=torch.bfloat16, device="cuda")
    return sets


def bench_delayed(torch, mhc, b, steps, warmup, mxfp8=False, check=False):
    hc = b.residual.shape[1]
    per_set = bytes_delayed(b.M, b.H, b.tp, mxfp8, hc)
    sets = delayed_sets(torch, b, rotations(per_set))
    if mxfp8:
        for s in sets:
            s["values"] = torch.empty((b.M, b.H), dtype=torch.uint8, device="cuda")
            s["scales"] = torch.empty(mhc.mhcb_mxfp8_scale_bytes(b.M, b.H), dtype=torch.uint8,
                                      device="cuda")

    ws = mhc.workspace(torch.device("cuda", torch.cuda.current_device()))

    def call(i):
        s = sets[i % len(sets)]
        mhc.mhcb_boundary(s["partials"], b.M * b.H, None, s["residual"], s["post"], s["comb"],
                          s["pre"], s["gamma"], s["residual_out"], s["layer_input"],
                          s.get("values"), s.get("scales"), ws, ws.numel(), b.M, b.H, hc, b.tp,
                          b.norm_eps)

    ms = Timed(torch, call, steps, warmup).run()
    mhc.workspace_status(ws)
    if check:
        # Every rotation set's output of the graph replay equals an eager call.
        for s in sets[:3]:
            ro, li = s["residual_out"].clone(), s["layer_input"].clone()
            mhc.mhcb_boundary(s["partials"], b.M * b.H, None, s["residual"], s["post"], s["comb"],
                              s["pre"], s["gamma"], s["residual_out"], s["layer_input"],
                              s.get("values"), s.get("scales"), ws, ws.numel(), b.M, b.H, hc, b.tp,
                              b.norm_eps)
            torch.cuda.synchronize()
            assert torch.equal(ro.view(torch.int16), s["residual_out"].view(torch.int16))
            assert torch.equal(li.view(torch.int16), s["layer_input"].view(torch.int16))
    return ms, per_set, len(sets)


def bench_mailbox(torch, mhc, b, steps, warmup, mxfp8=True):
    """Producer (publish of all tp partials) + mailbox-fed consumer (with the
    MXFP8 epilogue when `mxfp8`), per step, over rotating input sets."""
    mb = mhc.Mailbox(b.tp, b.M, b.H, "cuda")
    mb.init()
    nbytes = bytes_delayed(b.M, b.H, b.tp, mxfp8) + bytes_mailbox_extra(b.M, b.H, b.tp)
    sets = delayed_sets(torch, b, rotations(nbytes, minimum=2))
    for s in sets:
        s["values"] = torch.empty((b.M, b.H), dtype=torch.uint8, device="cuda") if mxfp8 else None
        s["scales"] = (torch.empty(mhc.mhcb_mxfp8_scale_bytes(b.M, b.H), dtype=torch.uint8,
                                   device="cuda") if mxfp8 else None)

    ws = mhc.workspace(torch.device("cuda", torch.cuda.current_device()))

    def call(i):
        s = sets[i % len(sets)]
        mhc.mhcb_publish(mb, s["partials"], b.M * b.H, 0, b.tp, b.M)
        mhc.mhcb_boundary(None, 0, mb, s["residual"], s["post"], s["comb"], s["pre"], s["gamma"],
                          s["residual_out"], s["layer_input"], s["values"], s["scales"], ws,
                          ws.numel(), b.M, b.H, 4, b.tp, b.norm_eps)

    ms = Timed(torch, call, steps, warmup).run()
    assert mb.status_ok()
    return ms, nbytes


def bench_finalize(torch, mhc, f, steps, warmup, two_shot=False, bf16_weights=False, scale=1.0):
    """MoE finalize; with bf16_weights the routing weights are BF16 (their
    bit patterns from the generator's rounding) and `scale` is the routed
    scaling factor (mhcb_finalize_ex)."""
    import synth
    weights = synth.to_bf16_bits(f.weights) if bf16_weights else f.weights
    per_set = bytes_finalize(f.M, f.H, f.tp, f.top_k, 2 if bf16_weights else 4)
    t = dict(gemm2=dev(torch, f.gemm2), weights=dev(torch, weights), idx=dev(torch, f.idx),
             shared=dev(torch, f.shared), residual=dev(torch, f.residual), post=dev(torch, f.post),
             comb=dev(torch, f.comb), pre=dev(torch, f.pre), gamma=dev(torch, f.gamma))
    sets = make_sets(torch, t, rotations(per_set, minimum=2))
    rows = f.gemm2.shape[1]
    ws = mhc.new_workspace(mhc.mhcb_workspace_bytes(f.M, f.H, f.tp, int(two_shot)), "cuda")
    for s in sets:
        s["residual_out"] = torch.empty((f.M, 4, f.H), dtype=torch.bfloat16, device="cuda")
        s["layer_input"] = torch.empty((f.M, f.H), dtype=torch.bfloat16, device="cuda")

    def call(i):
        s = sets[i % len(sets)]
        mhc.mhcb_finalize_ex(s["gemm2"], rows * f.H, rows, s["weights"], 0, int(bf16_weights),
                             scale, s["idx"], 0, s["shared"], f.M * f.H, s["residual"], s["post"],
                             s["comb"], s["pre"], s["gamma"], s["residual_out"], s["layer_input"],
                             None, None, int(two_shot), ws, ws.numel(), f.M, f.H, 4, f.tp, f.top_k,
                             f.norm_eps)

    ms = Timed(torch, call, steps, warmup).run()
    extra = f.M * (2 * f.tp * 2 * f.H + 2 * 2 * f.H) if two_shot else 0
    return ms, per_set + extra


def bytes_glm_moe(M, H, tp, top_k):
    """GLM boundary of an MoE sublayer: the ranks' expert rows and shared
    rows, routes (FP32 weight + int32 index), residual, post/comb in, the
    streams, raw mixes and layer input out, hc_fn and gamma once."""
    return (M * (tp * (top_k + 1) * 2 * H + top_k * 8 + 9 * 2 * H + 80 + 96)
            + 24 * 4 * H * 2 + 2 * H + 27 * 4)


def bench_glm_moe(torch, mhc, M, H, tp, top_k, steps, warmup):
    import synth
    f = synth.moe_finalize(M, H=H, tp=tp, top_k=top_k)
    g = synth.glm(M, H=H, tp=tp)
    per_set = bytes_glm_moe(M, H, tp, top_k)
    t = dict(gemm2=dev(torch, f.gemm2), weights=dev(torch, f.weights), idx=dev(torch, f.idx),
             shared=dev(torch, f.shared), residual=dev(torch, g.residual), post=dev(torch, g.post),
             comb=dev(torch, g.comb))
    sets = make_sets(torch, t, rotations(per_set, minimum=2))
    fn, scale, base, gamma = (dev(torch, g.fn), dev(torch, g.scale), dev(torch, g.base),
                              dev(torch, g.gamma))
    rows = f.gemm2.shape[1]
    need = mhc.mhcb_finalize_glm_workspace_bytes(M, H, tp)
    ws = mhc.new_workspace(need, "cuda")
    for s in sets:
        s["residual_out"] = torch.empty((M, 4, H), dtype=torch.bfloat16, device="cuda")
        s["layer_input"] = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
        s["mixes"] = torch.empty((M, 24), dtype=torch.float32, device="cuda")

    def call(i):
        s = sets[i % len(sets)]
        mhc.mhcb_finalize_glm(s["gemm2"], rows * H, rows, s["weights"], 0, 0, 1.0, s["idx"], 0,
                              s["shared"], M * H, s["residual"], s["post"], s["comb"], fn, scale,
                              base, gamma, s["residual_out"], s["mixes"], s["layer_input"], ws,
                              need, M, H, 4, tp, top_k, g.rms_eps, g.hc_eps, g.norm_eps)

    return Timed(torch, call, steps, warmup).run(), per_set


def bench_glm(torch, mhc, g, steps, warmup, tokens_per_wg=0):
    per_set = bytes_glm(g.M, g.H, g.tp)
    t = dict(partials=dev(torch, g.partials), residual=dev(torch, g.residual),
             post=dev(torch, g.post), comb=dev(torch, g.comb))
    sets = make_sets(torch, t, rotations(per_set))
    fn, scale, base, gamma = (dev(torch, g.fn), dev(torch, g.scale), dev(torch, g.base),
                              dev(torch, g.gamma))
    for s in sets:
        s["residual_out"] = torch.empty((g.M, 4, g.H), dtype=torch.bfloat16, device="cuda")
        s["layer_input"] = torch.empty((g.M, g.H), dtype=torch.bfloat16, device="cuda")
        s["mixes"] = torch.empty((g.M, 24), dtype=torch.float32, device="cuda")

    ws = mhc.workspace(torch.device("cuda", torch.cuda.current_device()))

    def call(i):
        s = sets[i % len(sets)]
        mhc.mhcb_boundary_glm(s["partials"], g.M * g.H, s["residual"], s["post"], s["comb"], fn,
                              scale, base, gamma, s["residual_out"], s["mixes"], s["layer_input"],
                              ws, ws.numel(), g.M, g.H, 4, g.tp, g.rms_eps, g.hc_eps, g.norm_eps,
                              tokens_per_wg)

    ms = Timed(torch, call, steps, warmup).run()
    return ms, per_set


def bytes_mixes(M):
    """Side mixes: raw mixes in (96 B), post' and comb' out (16 + 64 B) per
    token, scale and base once."""
    return M * (96 + 16 + 64) + 27 * 4


def bench_mixes(torch, mhc, M, steps, warmup):
    import synth
    raw, scale, base = synth.raw_mixes(M)
    per_set = bytes_mixes(M)
    sets = make_sets(torch, {"raw": dev(torch, raw)}, rotations(per_set, minimum=8))
    scale, base = dev(torch, scale), dev(torch, base)
    for s in sets:
        s["post"] = torch.empty((M, 4, 1), dtype=torch.float32, device="cuda")
        s["comb"] = torch.empty((M, 4, 4), dtype=torch.float32, device="cuda")

    def call(i):
        s = sets[i % len(sets)]
        mhc.mhcb_mixes(s["raw"], scale, base, s["post"], s["comb"], M, 4, 1e-6, 2.0, 20)

    return Timed(torch, call, steps, warmup).run(), per_set


def bench_glm_with_side_mixes(torch, mhc, g, steps, warmup):
    """The GLM boundary on the launching stream and the side mixes on a
    second stream, each call joining the previous call's mixes first (the
    GLM page's __call__ / join), all captured in one graph."""
    per_set = bytes_glm(g.M, g.H, g.tp) + bytes_mixes(g.M) - g.M * 96 - 27 * 4
    t = dict(partials=dev(torch, g.partials), residual=dev(torch, g.residual),
             post=dev(torch, g.post), comb=dev(torch, g.comb))
    sets = make_sets(torch, t, rotations(per_set))
    fn, scale, base, gamma = (dev(torch, g.fn), dev(torch, g.scale), dev(torch, g.base),
                              dev(torch, g.gamma))
    for s in sets:
        s["residual_out"] = torch.empty((g.M, 4, g.H), dtype=torch.bfloat16, device="cuda")
        s["layer_input"] = torch.empty((g.M, g.H), dtype=torch.bfloat16, device="cuda")
        s["mixes"] = torch.empty((g.M, 24), dtype=torch.float32, device="cuda")
        s["post_next"] = torch.empty((g.M, 4, 1), dtype=torch.float32, device="cuda")
        s["comb_next"] = torch.empty((g.M, 4, 4), dtype=torch.float32, device="cuda")
    ws = mhc.workspace(torch.device("cuda", torch.cuda.current_device()))
    side = torch.cuda.Stream()

    def call(i):
        s = sets[i % len(sets)]
        cur = torch.cuda.current_stream()
        if i > 0:
            cur.wait_stream(side)  # join the previous call's mixes (none before the first)
        mhc.mhcb_boundary_glm(s["partials"], g.M * g.H, s["residual"], s["post"], s["comb"], fn,
                              scale, base, gamma, s["residual_out"], s["mixes"], s["layer_input"],
                              ws, ws.numel(), g.M, g.H, 4, g.tp, g.rms_eps, g.hc_eps, g.norm_eps, 0)
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            mhc.mhcb_mixes(s["mixes"], scale, base, s["post_next"], s["comb_next"], g.M, 4,
                           g.hc_eps, g.post_mult, g.sinkhorn_repeat)
        if i == steps - 1:
            cur.wait_stream(side)  # the last call's mixes rejoin before the capture ends

    return Timed(torch, call, steps, warmup).run(), per_set


def bytes_indexer(M, K, key, heads, gate):
    """The weight rows once, the tokens' inputs, the three outputs."""
    return (key + heads + gate) * K * 2 + M * (K * 2 + key * 2 + heads * 4 + gate * 2)


def bench_indexer(torch, mhc, ix, steps, warmup, torch_matmul=False):
    """The DSA indexer projection over rotating input sets; with
    `torch_matmul`, torch's x @ w.T (hipBLASLt) on the same sets, timed the
    same way, as the library GEMM to compare with."""
    per_set = bytes_indexer(ix.M, ix.K, ix.key, ix.heads, ix.gate)
    sets = make_sets(torch, {"x": dev(torch, ix.x), "w": dev(torch, ix.w)},
                     rotations(per_set, minimum=4))
    for s in sets:
        s["key"] = torch.empty((ix.M, ix.key), dtype=torch.bfloat16, device="cuda")
        s["heads"] = torch.empty((ix.M, ix.heads), dtype=torch.float32, device="cuda")
        s["gate"] = torch.empty((ix.M, ix.gate), dtype=torch.bfloat16, device="cuda")
    nbytes = mhc.mhcb_indexer_workspace_bytes(ix.M, ix.K, ix.key, ix.heads, ix.gate)
    ws = mhc.indexer_workspace(nbytes) if nbytes else None

    def call(i):
        s = sets[i % len(sets)]
        if torch_matmul:
            torch.matmul(s["x"], s["w"].t())
        else:
            mhc.mhcb_indexer_projection(s["x"], s["w"], s["key"], s["heads"], s["gate"], ws,
                                        nbytes, ix.M, ix.K, ix.key, ix.heads, ix.gate)

    return Timed(torch, call, steps, warmup).run(), per_set


def copy_bandwidth(torch, nbytes=1 << 30, reps=20):
    """Achieved GB/s (read + write bytes) of a plain device-to-device copy
    of `nbytes`: the practical HBM ceiling next to the 8 TB/s peak."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    del src, dst
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def entry(ms, nbytes, M):
    return {"us_per_call": round(ms * 1e3, 3), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tokens_per_s": round(M / (ms * 1e-3), 1), "algorithmic_bytes": int(nbytes)}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the headline workload
# ---------------------------------------------------------------------------

def cpu_baseline(b, cpu_seconds=12.0, wall_cap_s=20.0):
    """The oracle on the host's cores, repeated on the headline workload until
    about `cpu_seconds` of CPU work (wall time x threads) has been spent."""
    import oracle
    threads = oracle.default_threads()
    oracle.boundary(b.partials[:, :2], b.residual[:2], b.post[:2], b.comb[:2], b.pre[:2], b.gamma,
                    b.norm_eps, threads=1)  # load + warm
    reps, times = 0, []
    start = time.perf_counter()
    while reps < 3 or (sum(times) * threads < cpu_seconds and time.perf_counter() - start < wall_cap_s):
        t0 = time.perf_counter()
        oracle.boundary(b.partials, b.residual, b.post, b.comb, b.pre, b.gamma, b.norm_eps,
                        threads=threads)
        times.append(time.perf_counter() - t0)
        reps += 1
    sec = float(np.median(times))
    nbytes = bytes_delayed(b.M, b.H, b.tp)
    return {"value": round(nbytes / sec / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "tokens_per_s": round(b.M / sec, 1),
            "us_per_call": round(sec * 1e6, 1), "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count(),
            "sample": f"{reps} calls of the same workload ({b.name}), median wall time, "
                      f"{threads} threads, about {sum(times) * threads:.0f} s of CPU work"}


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), as lscpu reports it."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline only, no extra workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma-separated workloads to run alone for profiling (headline, sweep, "
                         "finalize, glm, mixes, glm_moe, indexer, mxfp8, mailbox, copy); prints no "
                         "JSON")
    ap.add_argument("--slices", type=int, default=0,
                    help="workgroups per token for small-M calls (0 = the library's choice)")
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed calls one by one instead of replaying a HIP graph")
    args = ap.parse_args()
    global USE_GRAPH
    USE_GRAPH = not args.eager
    only = set(filter(None, args.only.split(",")))

    def want(name):
        return not only or name in only
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (libmhcb has no "
              "multi-GPU path; the boundary would shard over tokens)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import tp_reduce_mhc_amd as mhc
    torch.cuda.set_device(0)
    mhc.mhcb_set_token_slices(args.slices)
    K, W = args.steps, args.warmup
    result = {}

    if want("headline"):
        b = synth.dsv41_delayed(128)
        log(f"headline {b.name}: {K} steps, {W} warmup")
        ms, nbytes, nsets = bench_delayed(torch, mhc, b, K, W, check=True)
        gbps = nbytes / (ms * 1e-3) / 1e9
        traffic = measured_traffic()
        traced = traced_kernel_us()
        result.update({
            "metric": METRIC, "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
            "warmup": W, "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "storage": "bf16", "data": "synthetic",
            "config": {"workload": b.name, "hidden_size": b.H, "tp": b.tp, "hc_mult": 4, "M": b.M,
                       "rotating_input_sets": nsets, "timing": "HIP graph of K calls, HIP events"},
            "tokens_per_s": round(b.M / (ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBS, 4),
                         "traffic": traffic,
                         "kernel": "boundary_balanced_kernel<1, 512, Source 0> (delayed mHC, tp 8, eight waves)",
                         "algorithmic_bytes_per_launch": int(nbytes),
                         # The same fraction from the committed kernel trace
                         # (profiles/, mean launch duration under rocprofv3),
                         # while it matches the current sources; else null.
                         "frac_from_trace": (round(nbytes / (traced[0] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                             if traced else None),
                         "trace_mean_us": traced[0] if traced else None,
                         "trace_median_us": traced[1] if traced else None},
        })
        if not only:
            result["roofline"]["measured_copy_GBps"] = copy_bandwidth(torch)
            log(f"device copy: {result['roofline']['measured_copy_GBps']} GB/s")
        if not args.no_cpu_baseline and not only:
            log("cpu baseline (oracle)")
            result["cpu_baseline"] = cpu_baseline(b)
        if only:
            log(f"headline: {ms * 1e3:.2f} us/call, {gbps:.0f} GB/s")

    if want("sweep") and not args.quick:
        sweep = {}
        for M in (1, 8, 32, 64, 128, 256, 512, 1024, 2048, 4096):
            b = synth.dsv41_delayed(M)
            ms, nbytes, _ = bench_delayed(torch, mhc, b, min(K, 200 if M <= 512 else 50), W)
            sweep[f"M{M}"] = entry(ms, nbytes, M)
            log(f"sweep M={M}: {sweep[f'M{M}']}")
        result["sweep_dsv41_delayed"] = sweep
        result["us_per_call"] = {"M1": sweep["M1"]["us_per_call"], "M64": sweep["M64"]["us_per_call"]}
        for hc in (1, 2, 8):
            b = synth.dsv41_delayed(128, hc)
            ms, nbytes, _ = bench_delayed(torch, mhc, b, min(K, 200), W)
            sweep[f"hc{hc}_M128"] = entry(ms, nbytes, 128)
            log(f"sweep hc={hc} M=128: {sweep[f'hc{hc}_M128']}")

    extra = {}
    if want("finalize") and not args.quick:
        for M in (64, 512, 4096):
            f = synth.moe_finalize(M)
            steps = max(10, min(K, 100 if M <= 512 else 20))
            ms, nbytes = bench_finalize(torch, mhc, f, steps, min(W, 5))
            extra[f"moe_finalize_M{M}"] = entry(ms, nbytes, M)
            log(f"finalize M={M}: {extra[f'moe_finalize_M{M}']}")
            if M == 512:
                ms, nbytes = bench_finalize(torch, mhc, f, steps, min(W, 5), two_shot=True)
                extra[f"moe_finalize_two_shot_M{M}"] = entry(ms, nbytes, M)
                ms, nbytes = bench_finalize(torch, mhc, f, steps, min(W, 5), bf16_weights=True,
                                            scale=2.5)
                extra[f"moe_finalize_bf16_weights_scale2.5_M{M}"] = entry(ms, nbytes, M)
                log(f"finalize M={M} BF16 weights, scale 2.5: "
                    f"{extra[f'moe_finalize_bf16_weights_scale2.5_M{M}']}")
            del f
    if want("glm") and not args.quick:
        for M in (1, 16, 64, 256, 512):
            g = synth.glm(M)
            ms, nbytes = bench_glm(torch, mhc, g, min(K, 100), min(W, 5))
            extra[f"glm_M{M}"] = entry(ms, nbytes, M)
            log(f"glm M={M}: {extra[f'glm_M{M}']}")
            if M == 64:  # the tokens-per-workgroup choices at one size
                for G in (1, 2, 4, 16, -16):
                    name = f"glm_M64_tokens_per_wg{G}" if G > 0 else "glm_M64_two_pass_tiles"
                    ms, nbytes = bench_glm(torch, mhc, g, min(K, 100), min(W, 5), G)
                    extra[name] = entry(ms, nbytes, M)
                    log(f"glm M=64 tokens_per_wg={G}: {extra[name]}")
    if want("mixes") and not args.quick:
        for M in (64, 512):  # a5: the side-stream mixes, alone and beside the boundary
            ms, nbytes = bench_mixes(torch, mhc, M, min(K, 100), min(W, 5))
            extra[f"glm_side_mixes_M{M}"] = entry(ms, nbytes, M)
            log(f"side mixes M={M}: {extra[f'glm_side_mixes_M{M}']}")
            g = synth.glm(M)
            ms, nbytes = bench_glm_with_side_mixes(torch, mhc, g, min(K, 100), min(W, 5))
            extra[f"glm_M{M}_with_side_mixes"] = entry(ms, nbytes, M)
            log(f"glm M={M} + side mixes on a second stream: {extra[f'glm_M{M}_with_side_mixes']}")
    if want("glm_moe") and not args.quick:
        for M in (64, 512):  # the GLM boundary of an MoE sublayer, H=6144 tp=4 top_k=8
            ms, nbytes = bench_glm_moe(torch, mhc, M, 6144, 4, 8, min(K, 100), min(W, 5))
            extra[f"glm_moe_tp4_k8_M{M}"] = entry(ms, nbytes, M)
            log(f"glm moe M={M}: {extra[f'glm_moe_tp4_k8_M{M}']}")
    if want("indexer") and not args.quick:
        for M in (1, 4, 6, 8, 16, 64, 256, 1024, 2048, 4096):  # K=6144, 128 + 32 + 128 rows
            ix = synth.indexer(M)
            ms, nbytes = bench_indexer(torch, mhc, ix, min(K, 100), min(W, 5))
            extra[f"indexer_projection_M{M}"] = entry(ms, nbytes, M)
            log(f"indexer M={M}: {extra[f'indexer_projection_M{M}']}")
            ms, nbytes = bench_indexer(torch, mhc, ix, min(K, 100), min(W, 5), torch_matmul=True)
            extra[f"indexer_projection_M{M}_torch_matmul"] = entry(ms, nbytes, M)
            log(f"indexer M={M}, torch x @ w.T: {extra[f'indexer_projection_M{M}_torch_matmul']}")
            del ix
    if (want("mxfp8") or want("mailbox")) and not args.quick:
        b = synth.large_m_delayed(8192)
        if want("mxfp8"):
            ms, nbytes, _ = bench_delayed(torch, mhc, b, 20, 3, mxfp8=True)
            extra["mxfp8_M8192"] = entry(ms, nbytes, 8192)
            log(f"mxfp8 M=8192: {extra['mxfp8_M8192']}")
        if want("mailbox"):
            ms, nbytes = bench_mailbox(torch, mhc, b, 10, 2)
            extra["mailbox_mxfp8_M8192"] = entry(ms, nbytes, 8192)
            log(f"mailbox M=8192: {extra['mailbox_mxfp8_M8192']}")
            for M in (1, 8, 32, 64):  # publish + consume at decode sizes (H=5120, tp=8)
                bm = synth.dsv41_delayed(M)
                ms, nbytes = bench_mailbox(torch, mhc, bm, min(K, 200), W, mxfp8=False)
                extra[f"mailbox_publish_consume_M{M}"] = entry(ms, nbytes, M)
                log(f"mailbox publish + consume M={M}: {extra[f'mailbox_publish_consume_M{M}']}")
    if "copy" in only:
        # Calibration for the HBM byte counters: a plain device copy of a
        # known size (read n bytes, write n bytes), launched `steps` times.
        n = 512 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy: {args.steps} copies of {n} bytes")
    if extra:
        result["other_workloads"] = extra

    if not only:
        print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
