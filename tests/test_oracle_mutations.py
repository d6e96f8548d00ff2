"""Mutation record of the oracle's pins (CPU only).

Each entry below plants one plausible slip in a copy of
``oracle/mhcb_oracle.c``: a dropped term, a wrong sign or index, a
transposed operand, another rounding or summation order.  The copy is built
with the oracle's own flags and ``tests/test_oracle_pins.py`` runs against
it in a child process (``MHCB_ORACLE_LIB``).  Every mutant must make at
least one pin fail: a slip that no pin notices would pass through the
oracle into every parity claim.  The mutants never write out of bounds, so
a failure is always a failed assertion, never a crash.
"""
import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from oracle import build as oracle_build  # noqa: E402

SOURCE = os.path.join(ROOT, "oracle", "mhcb_oracle.c")

# (name, text in mhcb_oracle.c (must occur once), replacement)
MUTANTS = [
    ("bf16: ties away from zero", "(dropped == 0x8000u && (kept & 1u) != 0u)", "(dropped == 0x8000u)"),
    ("bf16: truncation", "kept += 1u; /* a carry", "kept += 0u; /* a carry"),
    ("sigmoid: sign of the exponent", "exp(-(double)x)", "exp((double)x)"),
    ("rms: eps dropped", "(double)sum_sq / count + (double)eps", "(double)sum_sq / count"),
    ("rank sum: last rank first",
     "for (int r = 0; r < tp; ++r) s = s + bf(partials[",
     "for (int r = tp - 1; r >= 0; --r) s = s + bf(partials["),
    ("post-mix: comb transposed", "comb[s * hc + j], a)", "comb[j * hc + s], a)"),
    ("post-mix: unfused multiply-add",
     "a = fmaf(bf(res[s]), comb[s * hc + j], a);", "a = a + bf(res[s]) * comb[s * hc + j];"),
    ("delayed collapse: unfused", "z = fmaf(bf(y[j]), pre[j], z);", "z = z + bf(y[j]) * pre[j];"),
    ("delayed collapse: last stream dropped",
     "for (int j = 0; j < hc; ++j) z = fmaf(", "for (int j = 0; j < hc - 1; ++j) z = fmaf("),
    ("glm collapse: sequential instead of pairwise",
     "return tobf((q[0] + q[1]) + (q[2] + q[3]));", "return tobf(((q[0] + q[1]) + q[2]) + q[3]);"),
    ("rmsnorm: gamma before the normalizer",
     "tobf((bf(p[c]) * inv) * bf(gamma[c]))", "tobf((bf(p[c]) * bf(gamma[c])) * inv)"),
    ("rmsnorm: mean over H + 1", "inv_rms((float)ss, (double)H, eps)", "inv_rms((float)ss, (double)(H + 1), eps)"),
    ("e4m3: ties to the odd code", "(err == best_err && (code & 1) == 0)", "(err == best_err && (code & 1) == 1)"),
    ("ue8m0: strict comparison", "if (ldexp(1.0, e - 127) >= (double)v)", "if (ldexp(1.0, e - 127) > (double)v)"),
    ("swizzle: line and word strides swapped",
     "(r % 32) * 16 + ((r % 128) / 32) * 4", "(r % 32) * 4 + ((r % 128) / 32) * 16"),
    ("mxfp8: 1/256 instead of 1/448", "(float)(1.0 / 448.0)", "(float)(1.0 / 256.0)"),
    ("mxfp8: amax of signed values", "float a = fabsf(bf(x[b * 32 + i]));", "float a = bf(x[b * 32 + i]);"),
    ("mxfp8: padding scales left as they were",
     "for (int64_t k = 0; k < K; ++k) scales[oracle_sf_index(r, k, K)] = 0;",
     "for (int64_t k = 0; k < K; ++k) scales[oracle_sf_index(r, k, K)] |= 0;"),
    ("finalize: shared expert dropped",
     "return sanitize(tobf(acc + bf(shared[t * H + c])));", "return sanitize(tobf(acc));"),
    ("finalize: negative zero kept", "return b == 0x8000u ? 0u : b;", "return b;"),
    ("finalize: row 0 skipped", "if (row < 0 || row >= rows) continue;", "if (row <= 0 || row >= rows) continue;"),
    ("two-shot: owner by t / tp",
     "int owner = t % tp;\n      int64_t slot = t / tp;\n      memcpy",
     "int owner = (t / tp) % tp;\n      int64_t slot = t / tp;\n      memcpy"),
    ("owner reduce: last rank first",
     "for (int r = 0; r < tp; ++r) s = s + bf(own[", "for (int r = tp - 1; r >= 0; --r) s = s + bf(own["),
    ("glm pre: hc_eps dropped",
     "pre[j] = oracle_sigmoid(fmaf(mixes[j], scale[0], base[j])) + hc_eps;",
     "pre[j] = oracle_sigmoid(fmaf(mixes[j], scale[0], base[j]));"),
    ("glm pre: scale[1] instead of scale[0]",
     "fmaf(mixes[j], scale[0], base[j])", "fmaf(mixes[j], scale[1], base[j])"),
    ("glm mixes: rstd over H instead of 4H",
     "inv_rms((float)g[NMIX], 4.0 * H, rms_eps)", "inv_rms((float)g[NMIX], (double)H, rms_eps)"),
    ("glm mixes: hc_fn column order transposed",
     "fn[(int64_t)k * NSTREAM * H + (int64_t)j * H + c]",
     "fn[(int64_t)k * NSTREAM * H + (int64_t)c * NSTREAM + j]"),
    ("side mixes: post_mult dropped", "base[NSTREAM + j])) * post_mult;", "base[NSTREAM + j]));"),
    ("side mixes: scale[1] for the comb logits",
     "fmaf(row[8 + i], scale[2], base[8 + i])", "fmaf(row[8 + i], scale[1], base[8 + i])"),
    ("sinkhorn: rows normalized in the first round too", "if (round > 0)", "if (round >= 0)"),
    ("sinkhorn: eps dropped from the normalizer",
     "float inv = oracle_rcp(pair_sum4(c, first, stride) + eps);",
     "float inv = oracle_rcp(pair_sum4(c, first, stride));"),
    ("sinkhorn: softmax eps not fused",
     "row[k] = fmaf(row[k], inv, eps);", "row[k] = row[k] * inv + eps;"),
    ("indexer: head weights rounded to BF16",
     "heads_out[(int64_t)t * heads + (r - key)] = f;", "heads_out[(int64_t)t * heads + (r - key)] = bf(tobf(f));"),
    ("indexer: FP32 sum",
     "      double s = 0.0;\n      for (int k = 0; k < K; ++k)\n        s += (double)bf(x[(int64_t)t * K + k]) * (double)bf(w[(int64_t)r * K + k]);",
     "      float s = 0.0f;\n      for (int k = 0; k < K; ++k)\n        s += bf(x[(int64_t)t * K + k]) * bf(w[(int64_t)r * K + k]);"),
    ("indexer: weight indexed column-major",
     "(double)bf(w[(int64_t)r * K + k]);", "(double)bf(w[(int64_t)k * rows + r]);"),
    ("indexer: last K column dropped", "      for (int k = 0; k < K; ++k)\n        s += (double)",
     "      for (int k = 0; k < K - 1; ++k)\n        s += (double)"),
]


def _plant(text, old, new):
    assert text.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    return text.replace(old, new)


def _run_mutant(args):
    name, old, new, tmp, text = args
    slug = re.sub(r"[^a-z0-9]+", "_", name.lower()).strip("_")
    src = os.path.join(tmp, f"{slug}.c")
    lib = os.path.join(tmp, f"{slug}.so")
    with open(src, "w") as f:
        f.write(_plant(text, old, new))
    subprocess.run(["gcc", *oracle_build.FLAGS, src, "-o", lib, "-lm"], check=True,
                   capture_output=True)
    env = dict(os.environ, MHCB_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    failed = re.findall(r"^FAILED (\S+)", r.stdout, re.M)
    return name, r.returncode, failed[0] if failed else r.stdout[-300:]


def test_every_mutant_fails_a_pin():
    text = open(SOURCE).read()
    for _, old, _ in MUTANTS:
        assert text.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
            results = list(pool.map(_run_mutant, [(n, o, w, tmp, text) for n, o, w in MUTANTS]))
    survivors = []
    for name, rc, caught_by in results:
        print(f"[mutant] {name}: {'caught by ' + caught_by if rc == 1 else f'rc={rc} {caught_by}'}")
        if rc != 1:  # 1 = tests ran and some failed; 0 = all passed (survivor)
            survivors.append((name, rc))
    assert not survivors, f"mutants no pin catches (or runs that did not complete): {survivors}"
