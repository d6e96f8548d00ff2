/*
 * mhcb_oracle.c -- plain CPU oracle of the fused TP-reduce + mHC + RMSNorm
 * sublayer boundary.
 *
 * TEST INFRASTRUCTURE, NOT THE PRODUCT.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg load this file's library.  It shares no
 * code, header, table or constant with the HIP path, and the HIP path never
 * loads it.
 *
 * Sources, cited by page title and section (class / method) below:
 *   [GLM]   vllm.models.glm5next.nvidia.specialized_decode.all_reduce_mhc
 *           (GLM-5.3-Flash boundary with the in-kernel prenorm GEMV)
 *   [DSV41] vllm.models.deepseek_v41.nvidia.ops.cute_dsl.all_reduce_mhc
 *           (DSV4.1 delayed-mHC boundary, MoE finalize, two-shot, MXFP8)
 *   [IDX]   vllm.models.glm5next.nvidia.specialized_decode.indexer
 *           (the DSA indexer's fused input projection)
 *
 * Precision.  The pages store BF16 and compute in FP32 in a stated order.
 * This file follows that order with IEEE binary32 operations; it is built
 * with -ffp-contract=off, so an FMA happens only where fmaf() is written.
 * Where the pages leave an order to a hardware reduction tree (sums of
 * squares, the 24-row GEMV) the sum is accumulated in binary64 and rounded
 * to binary32 once.  exp, 1/x and 1/sqrt are evaluated in binary64 and
 * rounded once.
 *
 * All arrays are row-major and dense unless a stride is passed.  BF16 values
 * are uint16_t bit patterns.  Work is split over tokens across `threads`
 * POSIX threads; no step reorders any arithmetic.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { NSTREAM = 4, MAXSTREAM = 8, NMIX = 24 };

/* ------------------------------------------------------------------------ */
/* BF16 <-> FP32                                                             */
/* ------------------------------------------------------------------------ */

/* BF16 is the upper half of a binary32; widening is exact. */
float oracle_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Round a binary32 to BF16, nearest with ties to even, by looking at the
 * 16 bits that are dropped ([DSV41] and [GLM] round with .to(BFloat16);
 * the mode is not printed, round-to-nearest-even is the reading). */
uint16_t oracle_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u)
    return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
  uint32_t kept = u >> 16;
  uint32_t dropped = u & 0xffffu;
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u) != 0u))
    kept += 1u; /* a carry into the exponent is the correct rounding */
  return (uint16_t)kept;
}

static float bf(uint16_t b) { return oracle_bf16_to_f32(b); }
static uint16_t tobf(float f) { return oracle_f32_to_bf16(f); }

/* The Lamport sentinel is BF16 negative zero; a published value never
 * carries it ([DSV41] _QuadFinalizePublishDeviceKernel.kernel sanitizes). */
static uint16_t sanitize(uint16_t b) { return b == 0x8000u ? 0u : b; }

/* ------------------------------------------------------------------------ */
/* Scalar functions: 1/x, exp, sigmoid, 1/sqrt                               */
/* ------------------------------------------------------------------------ */

float oracle_rcp(float x) { return (float)(1.0 / (double)x); }
float oracle_exp(float x) { return (float)exp((double)x); }
/* sigmoid(x) = 1 / (1 + e^-x) */
float oracle_sigmoid(float x) { return (float)(1.0 / (1.0 + exp(-(double)x))); }

/* 1 / sqrt(sum_sq / count + eps), the RMS normalizer. */
static float inv_rms(float sum_sq, double count, float eps) {
  return (float)(1.0 / sqrt((double)sum_sq / count + (double)eps));
}

/* ------------------------------------------------------------------------ */
/* a1  TP partial sum                                                        */
/* ------------------------------------------------------------------------ */

/* [DSV41] _LamportMHCDeviceKernel.kernel: the sum starts at 0.0 and adds
 * each rank's FP32-widened fragment in rank order; the result is rounded to
 * BF16 "as the collective returns it".  The module text states that the
 * two-shot owner sums in the same order, so both protocols agree bit for bit. */
uint16_t oracle_rank_sum(const uint16_t *partials, int64_t rank_stride, int tp,
                         int64_t element) {
  float s = 0.0f;
  for (int r = 0; r < tp; ++r) s = s + bf(partials[(int64_t)r * rank_stride + element]);
  return tobf(s);
}

/* ------------------------------------------------------------------------ */
/* a2  post-mix                                                              */
/* ------------------------------------------------------------------------ */

/* [DSV41] _LamportMHCDeviceKernel.kernel (and [GLM] _BoundaryDeviceKernel
 * .kernel): new stream j = x * post_j, then the hc old streams (four for GLM)
 * are added in source order, each times comb[source][j]; the sum of a
 * product is an FMA (reading).  Rounded to BF16. */
static uint16_t post_mix(float x, const uint16_t *res, const float *post, const float *comb,
                         int j, int hc) {
  float a = x * post[j];
  for (int s = 0; s < hc; ++s) a = fmaf(bf(res[s]), comb[s * hc + j], a);
  return tobf(a);
}

/* ------------------------------------------------------------------------ */
/* a4  collapse and RMSNorm                                                   */
/* ------------------------------------------------------------------------ */

/* [DSV41] _LamportMHCDeviceKernel.kernel: the collapse starts at 0.0 and adds
 * y_j * pre_j over the hc streams in order (FMA reading). */
static uint16_t collapse_delayed(const uint16_t *y, const float *pre, int hc) {
  float z = 0.0f;
  for (int j = 0; j < hc; ++j) z = fmaf(bf(y[j]), pre[j], z);
  return tobf(z);
}

/* [GLM] _BoundaryDeviceKernel.kernel: lane j forms y_j * pre_j, and two
 * butterfly steps add lanes one apart, then two apart: (q0+q1)+(q2+q3). */
static uint16_t collapse_glm(const uint16_t y[NSTREAM], const float *pre) {
  float q[NSTREAM];
  for (int j = 0; j < NSTREAM; ++j) q[j] = bf(y[j]) * pre[j];
  return tobf((q[0] + q[1]) + (q[2] + q[3]));
}

/* RMSNorm of one token ([DSV41] _LamportMHCDeviceKernel.kernel, [GLM]
 * _BoundaryDeviceKernel.kernel): inv = 1/sqrt(sum p^2 / H + eps), then
 * out = bf16((p * inv) * gamma). */
static void rmsnorm_token(const uint16_t *p, const uint16_t *gamma, int H, float eps,
                          uint16_t *out) {
  double ss = 0.0;
  for (int c = 0; c < H; ++c) {
    double v = bf(p[c]);
    ss += v * v;
  }
  float inv = inv_rms((float)ss, (double)H, eps);
  for (int c = 0; c < H; ++c) out[c] = tobf((bf(p[c]) * inv) * bf(gamma[c]));
}

/* ------------------------------------------------------------------------ */
/* a8  MXFP8: E4M3 codes, UE8M0 scales, swizzled 128x4 scale layout          */
/* ------------------------------------------------------------------------ */

/* OCP FP8 E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0
 * holds subnormals m * 2^-9; 0x7f / 0xff are NaN, so the largest finite
 * magnitude is code 0x7e = 1.75 * 2^8 = 448. */
double oracle_e4m3_value(uint8_t code) {
  int e = (code >> 3) & 0xf, m = code & 7;
  double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return (code & 0x80) ? -v : v;
}

/* Nearest E4M3 code, ties to the even code, magnitudes past 448 saturate to
 * 448 (the "rn.satfinite" reading), sign kept (so -0 -> 0x80).  Written as a
 * search over the 127 non-negative finite codes. */
uint8_t oracle_e4m3_rne_sat(float x) {
  if (isnan(x)) return 0x7f;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (a >= 448.0) return (uint8_t)(sign | 0x7e);
  int best = 0;
  double best_err = a;
  for (int code = 1; code <= 0x7e; ++code) {
    double err = fabs(a - oracle_e4m3_value((uint8_t)code));
    if (err < best_err || (err == best_err && (code & 1) == 0)) {
      best = code;
      best_err = err;
    }
  }
  return (uint8_t)(sign | best);
}

/* UE8M0 scale: the power of two 2^(e-127), e in [0, 254], rounded up: the
 * smallest e with 2^(e-127) >= v; past 2^127 it saturates at 254 and v <= 0
 * gives 0 (reading of float_to_ue8m0_fast in [DSV41]). */
uint8_t oracle_ue8m0_round_up(float v) {
  if (isnan(v)) return 0xff;
  for (int e = 0; e <= 254; ++e)
    if (ldexp(1.0, e - 127) >= (double)v) return (uint8_t)e;
  return 254;
}

/* Byte offset of scale (row r, scale column k) with K scale columns in the
 * swizzled 128x4 layout: 128-row x 4-column tiles of 512 bytes, tiles row-major
 * over (r / 128, k / 4); inside a tile, row r sits in 16-byte line r % 32,
 * 4-byte word (r % 128) / 32, byte k % 4. */
int64_t oracle_sf_index(int64_t r, int64_t k, int64_t K) {
  int64_t tile = (r / 128) * (K / 4) + k / 4;
  return tile * 512 + (r % 32) * 16 + ((r % 128) / 32) * 4 + (k % 4);
}

/* Bytes of the scale array: rows padded to a multiple of 128, H / 32 columns. */
int64_t oracle_mxfp8_scale_bytes(int64_t M, int64_t H) {
  return (M + 127) / 128 * 128 * (H / 32);
}

/* [DSV41] _LamportMHCDeviceKernel.kernel, quantize branch: per block of 32
 * columns, amax = max |x|, e = UE8M0(amax * fl(1/448)), codes = E4M3(x *
 * 2^(127-e)).  Scales of rows M .. padded M are zero. */
static const float INV_E4M3_MAX = (float)(1.0 / 448.0);

static void quant_token(const uint16_t *x, int64_t t, int H, uint8_t *values,
                        uint8_t *scales) {
  int64_t K = H / 32;
  for (int b = 0; b < H / 32; ++b) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
      float a = fabsf(bf(x[b * 32 + i]));
      if (a > amax) amax = a;
    }
    uint8_t e = oracle_ue8m0_round_up(amax * INV_E4M3_MAX);
    float inv = ldexpf(1.0f, 127 - (int)e);
    for (int i = 0; i < 32; ++i)
      values[t * H + b * 32 + i] = oracle_e4m3_rne_sat(bf(x[b * 32 + i]) * inv);
    scales[oracle_sf_index(t, b, K)] = e;
  }
}

static void zero_padding_scales(int64_t M, int H, uint8_t *scales) {
  int64_t K = H / 32, padded = (M + 127) / 128 * 128;
  for (int64_t r = M; r < padded; ++r)
    for (int64_t k = 0; k < K; ++k) scales[oracle_sf_index(r, k, K)] = 0;
}

/* ------------------------------------------------------------------------ */
/* Token-parallel driver                                                     */
/* ------------------------------------------------------------------------ */

typedef void (*token_fn)(void *ctx, int t0, int t1);
typedef struct {
  token_fn fn;
  void *ctx;
  int t0, t1;
} slice_t;

static void *run_slice(void *arg) {
  slice_t *s = (slice_t *)arg;
  s->fn(s->ctx, s->t0, s->t1);
  return NULL;
}

/* Runs fn over tokens [0, M) in `threads` contiguous slices. */
static int parallel_tokens(int M, int threads, token_fn fn, void *ctx) {
  if (threads < 1) threads = 1;
  if (threads > M) threads = M > 0 ? M : 1;
  if (threads == 1) {
    fn(ctx, 0, M);
    return 0;
  }
  pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof *tid);
  slice_t *sl = (slice_t *)calloc((size_t)threads, sizeof *sl);
  if (!tid || !sl) {
    free(tid);
    free(sl);
    return -1;
  }
  int started = 0;
  for (int i = 0; i < threads; ++i) {
    sl[i].fn = fn;
    sl[i].ctx = ctx;
    sl[i].t0 = (int)((int64_t)M * i / threads);
    sl[i].t1 = (int)((int64_t)M * (i + 1) / threads);
    if (pthread_create(&tid[i], NULL, run_slice, &sl[i]) != 0) break;
    ++started;
  }
  for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
  /* A thread that could not be started runs its slice here. */
  for (int i = started; i < threads; ++i) run_slice(&sl[i]);
  free(tid);
  free(sl);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Delayed-mHC boundary: a1 + a2 + a4 (+ a8)                                 */
/* ------------------------------------------------------------------------ */

typedef struct {
  const uint16_t *partials;
  int64_t rank_stride;
  int tp;
  const uint16_t *residual;
  const float *post, *comb, *pre;
  const uint16_t *gamma;
  float norm_eps;
  int H, hc;
  uint16_t *residual_out, *layer_input;
  uint8_t *mx_values, *mx_scales;
} boundary_ctx;

static void boundary_tokens(void *arg, int t0, int t1) {
  boundary_ctx *a = (boundary_ctx *)arg;
  int H = a->H;
  uint16_t *p = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)H);
  uint16_t *out = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)H);
  const int hc = a->hc;
  for (int t = t0; t < t1; ++t) {
    const float *post = a->post + (int64_t)t * hc;
    const float *comb = a->comb + (int64_t)t * hc * hc;
    for (int c = 0; c < H; ++c) {
      float x = bf(oracle_rank_sum(a->partials, a->rank_stride, a->tp, (int64_t)t * H + c));
      uint16_t res[MAXSTREAM], y[MAXSTREAM];
      for (int s = 0; s < hc; ++s) res[s] = a->residual[((int64_t)t * hc + s) * H + c];
      for (int j = 0; j < hc; ++j) {
        y[j] = post_mix(x, res, post, comb, j, hc);
        a->residual_out[((int64_t)t * hc + j) * H + c] = y[j];
      }
      if (a->pre) p[c] = collapse_delayed(y, a->pre + (int64_t)t * hc, hc);
    }
    if (!a->pre) continue; /* residual-only variant */
    rmsnorm_token(p, a->gamma, H, a->norm_eps, out);
    memcpy(a->layer_input + (int64_t)t * H, out, sizeof(uint16_t) * (size_t)H);
    if (a->mx_values) quant_token(out, t, H, a->mx_values, a->mx_scales);
  }
  free(p);
  free(out);
}

/* [DSV41] AllReduceMHC.__call__ with _LamportMHCDeviceKernel (compiled for
 * the module's hc_mult): partials are tp BF16 [M, H] arrays `rank_stride`
 * elements apart; residual [M, hc, H]; post, pre [M, hc] FP32; comb
 * [M, hc, hc] FP32 indexed [source][target]; gamma [H]; 1 <= hc <= 8.
 * pre == NULL selects the residual-only variant (layer_input, gamma and the
 * MXFP8 outputs unused).  mx_values [M, H] / mx_scales (scale_bytes) optional. */
int oracle_boundary(const uint16_t *partials, int64_t rank_stride, int tp,
                    const uint16_t *residual, const float *post, const float *comb,
                    const float *pre, const uint16_t *gamma, float norm_eps, int M, int H, int hc,
                    uint16_t *residual_out, uint16_t *layer_input, uint8_t *mx_values,
                    uint8_t *mx_scales, int threads) {
  if (M < 0 || H <= 0 || tp < 1 || hc < 1 || hc > MAXSTREAM) return 1;
  if ((pre == NULL) != (gamma == NULL) || (pre == NULL && mx_values != NULL)) return 1;
  if (mx_values && H % 128) return 1;
  boundary_ctx a = {partials, rank_stride, tp, residual, post, comb, pre, gamma,
                    norm_eps, H, hc, residual_out, layer_input, mx_values, mx_scales};
  if (parallel_tokens(M, threads, boundary_tokens, &a)) return 2;
  if (mx_values) zero_padding_scales(M, H, mx_scales);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* a6  MoE finalize contributions and a7 two-shot owner reduce                */
/* ------------------------------------------------------------------------ */

/* [DSV41] _QuadFinalizePublishDeviceKernel.kernel: one rank's contribution to
 * token t, column c: the accumulator starts at 0.0; for k ascending, a route
 * whose row index is -1 (expert not on this rank) is skipped, otherwise
 * acc = fma(row[idx][c], w[k], acc); then the shared-expert value is added,
 * the sum is rounded to BF16 and negative zero becomes +0.  (Reading: a row
 * index outside [0, rows) is treated like -1.) */
uint16_t oracle_finalize_element(const uint16_t *gemm2, int64_t rows, const float *w,
                                 const int32_t *idx, const uint16_t *shared, int top_k,
                                 int64_t t, int H, int c) {
  float acc = 0.0f;
  for (int k = 0; k < top_k; ++k) {
    int32_t row = idx[t * top_k + k];
    if (row < 0 || row >= rows) continue;
    acc = fmaf(bf(gemm2[(int64_t)row * H + c]), w[t * top_k + k], acc);
  }
  return sanitize(tobf(acc + bf(shared[t * H + c])));
}

typedef struct {
  const uint16_t *gemm2;
  int64_t g_stride, rows;
  const float *w;
  int64_t w_stride;
  const int32_t *idx;
  int64_t i_stride;
  const uint16_t *shared;
  int64_t s_stride;
  int tp, top_k, M, H;
  uint16_t *contrib; /* [tp][M][H] */
} contrib_ctx;

static void contrib_tokens(void *arg, int t0, int t1) {
  contrib_ctx *a = (contrib_ctx *)arg;
  for (int r = 0; r < a->tp; ++r)
    for (int t = t0; t < t1; ++t)
      for (int c = 0; c < a->H; ++c)
        a->contrib[((int64_t)r * a->M + t) * a->H + c] = oracle_finalize_element(
            a->gemm2 + r * a->g_stride, a->rows, a->w + r * a->w_stride,
            a->idx + r * a->i_stride, a->shared + r * a->s_stride, a->top_k, t, a->H, c);
}

/* All tp ranks' contributions [tp][M][H] (each rank's inputs `*_stride`
 * elements apart; stride 0 = replicated). */
int oracle_finalize_contributions(const uint16_t *gemm2, int64_t g_stride, int64_t rows,
                                  const float *w, int64_t w_stride, const int32_t *idx,
                                  int64_t i_stride, const uint16_t *shared, int64_t s_stride,
                                  int tp, int top_k, int M, int H, uint16_t *contrib,
                                  int threads) {
  if (M < 0 || H <= 0 || tp < 1 || top_k < 1) return 1;
  contrib_ctx a = {gemm2, g_stride, rows, w, w_stride, idx, i_stride, shared, s_stride,
                   tp, top_k, M, H, contrib};
  return parallel_tokens(M, threads, contrib_tokens, &a) ? 2 : 0;
}

/* [DSV41] module text and _SharedOnlyPublishDeviceKernel /
 * _OwnerReduceMulticastDeviceKernel: in the two-shot protocol token t belongs
 * to rank t % tp and occupies slot t / tp of that owner's mailbox
 * [source rank][owned token][H].  Every owner's mailbox is emulated in one
 * array own[owner][source][slot][H] with ceil(M/tp) slots. */
void oracle_two_shot_publish(const uint16_t *contrib, int tp, int M, int H, uint16_t *own) {
  int64_t slots = (M + tp - 1) / tp;
  for (int r = 0; r < tp; ++r)
    for (int t = 0; t < M; ++t) {
      int owner = t % tp;
      int64_t slot = t / tp;
      memcpy(own + (((int64_t)owner * tp + r) * slots + slot) * H,
             contrib + ((int64_t)r * M + t) * H, sizeof(uint16_t) * (size_t)H);
    }
}

/* [DSV41] _OwnerReduceMulticastDeviceKernel.kernel: the owner sums its
 * token's tp contributions in FP32 from rank 0, rounds to BF16 and sanitizes
 * negative zero; the result is the token's reduced value. */
void oracle_owner_reduce(const uint16_t *own, int tp, int M, int H, uint16_t *reduced) {
  int64_t slots = (M + tp - 1) / tp;
  for (int t = 0; t < M; ++t) {
    int owner = t % tp;
    int64_t slot = t / tp;
    for (int c = 0; c < H; ++c) {
      float s = 0.0f;
      for (int r = 0; r < tp; ++r) s = s + bf(own[(((int64_t)owner * tp + r) * slots + slot) * H + c]);
      reduced[(int64_t)t * H + c] = sanitize(tobf(s));
    }
  }
}

/* [DSV41] AllReduceMHC.finalize: contributions, then either the direct sum
 * (one-shot) or the two-shot emulation whose consumer reads the one reduced
 * value per token, then the same mHC consumer as oracle_boundary. */
int oracle_finalize(const uint16_t *gemm2, int64_t g_stride, int64_t rows, const float *w,
                    int64_t w_stride, const int32_t *idx, int64_t i_stride,
                    const uint16_t *shared, int64_t s_stride, int tp, int top_k,
                    const uint16_t *residual, const float *post, const float *comb,
                    const float *pre, const uint16_t *gamma, float norm_eps, int M, int H,
                    int hc, int two_shot, uint16_t *residual_out, uint16_t *layer_input,
                    uint8_t *mx_values, uint8_t *mx_scales, int threads) {
  if (M < 0 || H <= 0 || tp < 1 || top_k < 1) return 1;
  uint16_t *contrib = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)tp * (size_t)M * (size_t)H + 2);
  if (!contrib) return 2;
  int rc = oracle_finalize_contributions(gemm2, g_stride, rows, w, w_stride, idx, i_stride,
                                         shared, s_stride, tp, top_k, M, H, contrib, threads);
  if (rc == 0 && !two_shot) {
    rc = oracle_boundary(contrib, (int64_t)M * H, tp, residual, post, comb, pre, gamma,
                         norm_eps, M, H, hc, residual_out, layer_input, mx_values, mx_scales,
                         threads);
  } else if (rc == 0) {
    int64_t slots = (M + tp - 1) / tp;
    uint16_t *own = (uint16_t *)calloc((size_t)tp * (size_t)tp * (size_t)slots * (size_t)H + 2, sizeof(uint16_t));
    uint16_t *reduced = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)M * (size_t)H + 2);
    if (!own || !reduced) {
      rc = 2;
    } else {
      oracle_two_shot_publish(contrib, tp, M, H, own);
      oracle_owner_reduce(own, tp, M, H, reduced);
      rc = oracle_boundary(reduced, 0, 1, residual, post, comb, pre, gamma, norm_eps, M, H, hc,
                           residual_out, layer_input, mx_values, mx_scales, threads);
    }
    free(own);
    free(reduced);
  }
  free(contrib);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* GLM boundary: a1 + a2 + a3 + a4                                           */
/* ------------------------------------------------------------------------ */

typedef struct {
  const uint16_t *partials;
  int64_t rank_stride;
  int tp;
  const uint16_t *residual;
  const float *post, *comb;
  const uint16_t *fn;
  const float *scale, *base;
  const uint16_t *gamma;
  float rms_eps, hc_eps, norm_eps;
  int H;
  uint16_t *residual_out;
  float *mixes_out, *pre_out;
  uint16_t *layer_input;
} glm_ctx;

/* [GLM] _BoundaryDeviceKernel.kernel: the pre-mix of one token from its
 * raw mixes, pre_j = sigmoid(mixes_j * scale[0] + base[j]) + hc_eps for the
 * four streams (the product-sum is one FMA, reading R3). */
void oracle_glm_pre(const float mixes[NMIX], const float *scale, const float *base,
                    float hc_eps, float pre[NSTREAM]) {
  for (int j = 0; j < NSTREAM; ++j)
    pre[j] = oracle_sigmoid(fmaf(mixes[j], scale[0], base[j])) + hc_eps;
}

/* [GLM] _BoundaryDeviceKernel.kernel, after the post-mix of token t (y holds
 * its 4 x H new streams):
 *   g_k  = sum over j, c of fn[k][j*H + c] * y_j[c]      (k < 24)
 *   g_24 = sum over j, c of y_j[c]^2
 *   rstd = 1 / sqrt(g_24 / (4H) + rms_eps);  mixes_k = g_k * rstd
 *   pre  = oracle_glm_pre(mixes)
 * The products of BF16 values are exact in binary64; the sums are binary64,
 * rounded to binary32 once. */
void oracle_glm_mixes_token(const uint16_t *y, const uint16_t *fn, const float *scale,
                            const float *base, int H, float rms_eps, float hc_eps,
                            float mixes[NMIX], float pre[NSTREAM]) {
  double g[NMIX + 1];
  for (int k = 0; k <= NMIX; ++k) g[k] = 0.0;
  for (int j = 0; j < NSTREAM; ++j)
    for (int c = 0; c < H; ++c) {
      double v = bf(y[(int64_t)j * H + c]);
      for (int k = 0; k < NMIX; ++k)
        g[k] += (double)bf(fn[(int64_t)k * NSTREAM * H + (int64_t)j * H + c]) * v;
      g[NMIX] += v * v;
    }
  float rstd = inv_rms((float)g[NMIX], 4.0 * H, rms_eps);
  for (int k = 0; k < NMIX; ++k) mixes[k] = (float)g[k] * rstd;
  oracle_glm_pre(mixes, scale, base, hc_eps, pre);
}

/* [GLM] _BoundaryDeviceKernel.kernel, last steps of a token: its four new
 * streams y [4][H] collapse with the pre-mix, p = bf16((q0+q1)+(q2+q3)),
 * q_j = y_j * pre_j (collapse_glm), then RMSNorm over H with norm_weight
 * (rmsnorm_token): out [H].  0 on success, 2 when out of memory. */
int oracle_glm_collapse_rmsnorm(const uint16_t *y, const float pre[NSTREAM],
                                const uint16_t *gamma, int H, float norm_eps, uint16_t *out) {
  uint16_t *p = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)H);
  if (!p) return 2;
  for (int c = 0; c < H; ++c) {
    uint16_t yc[NSTREAM];
    for (int j = 0; j < NSTREAM; ++j) yc[j] = y[(int64_t)j * H + c];
    p[c] = collapse_glm(yc, pre);
  }
  rmsnorm_token(p, gamma, H, norm_eps, out);
  free(p);
  return 0;
}

static void glm_tokens(void *arg, int t0, int t1) {
  glm_ctx *a = (glm_ctx *)arg;
  int H = a->H;
  uint16_t *y = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)NSTREAM * (size_t)H);
  for (int t = t0; t < t1; ++t) {
    const float *post = a->post + (int64_t)t * NSTREAM;
    const float *comb = a->comb + (int64_t)t * NSTREAM * NSTREAM;
    for (int c = 0; c < H; ++c) {
      float x = bf(oracle_rank_sum(a->partials, a->rank_stride, a->tp, (int64_t)t * H + c));
      uint16_t res[NSTREAM];
      for (int s = 0; s < NSTREAM; ++s) res[s] = a->residual[((int64_t)t * NSTREAM + s) * H + c];
      for (int j = 0; j < NSTREAM; ++j) y[(int64_t)j * H + c] = post_mix(x, res, post, comb, j, NSTREAM);
    }
    memcpy(a->residual_out + (int64_t)t * NSTREAM * H, y, sizeof(uint16_t) * (size_t)NSTREAM * (size_t)H);
    float mixes[NMIX], pre[NSTREAM];
    oracle_glm_mixes_token(y, a->fn, a->scale, a->base, H, a->rms_eps, a->hc_eps, mixes, pre);
    memcpy(a->mixes_out + (int64_t)t * NMIX, mixes, sizeof mixes);
    if (a->pre_out) memcpy(a->pre_out + (int64_t)t * NSTREAM, pre, sizeof pre);
    oracle_glm_collapse_rmsnorm(y, pre, a->gamma, H, a->norm_eps, a->layer_input + (int64_t)t * H);
  }
  free(y);
}

/* [GLM] AllReduceMhcBoundary.__call__ with _BoundaryDeviceKernel: as
 * oracle_boundary, but the pre-mix comes from the new streams through hc_fn
 * [24, 4H] (column j*H + c), scale [3] and base [24]; the raw mixes [M, 24]
 * are written for the side kernel; pre_out [M, 4] (optional) receives the
 * pre-mix used by the collapse. */
int oracle_boundary_glm(const uint16_t *partials, int64_t rank_stride, int tp,
                        const uint16_t *residual, const float *post, const float *comb,
                        const uint16_t *fn, const float *scale, const float *base,
                        const uint16_t *gamma, float rms_eps, float hc_eps, float norm_eps,
                        int M, int H, uint16_t *residual_out, float *mixes_out,
                        uint16_t *layer_input, float *pre_out, int threads) {
  if (M < 0 || H <= 0 || tp < 1) return 1;
  glm_ctx a = {partials, rank_stride, tp, residual, post, comb, fn, scale, base, gamma,
               rms_eps, hc_eps, norm_eps, H, residual_out, mixes_out, pre_out, layer_input};
  return parallel_tokens(M, threads, glm_tokens, &a) ? 2 : 0;
}

/* ------------------------------------------------------------------------ */
/* a5  side-stream mixes: post-mix and Sinkhorn residual mix                 */
/* ------------------------------------------------------------------------ */

/* Sinkhorn-Knopp on a 4x4 matrix with an eps floor ([GLM]
 * _MixesDeviceKernel._sinkhorn).  Mathematically: make every row a softmax
 * of its logits (offset by eps), then alternately scale the columns and the
 * rows so that each sums to one.  What the bits depend on, and is kept from
 * the page: four entries are always added as (a + b) + (c + d); the softmax
 * takes exp(x - rowmax), multiplies by the reciprocal of the row sum and
 * adds eps in one fused step; every later normalization multiplies by the
 * reciprocal of (sum + eps); the first round scales only the columns, each
 * later round the rows and then the columns.  `repeat` counts the column
 * steps (0: the softmax alone). */

/* (a + b) + (c + d) over entries first, first + stride, ... of c. */
static float pair_sum4(const float *c, int first, int stride) {
  return (c[first] + c[first + stride]) + (c[first + 2 * stride] + c[first + 3 * stride]);
}

/* Scales the four entries first, first + stride, ... by 1/(their sum + eps). */
static void normalize4(float *c, int first, int stride, float eps) {
  float inv = oracle_rcp(pair_sum4(c, first, stride) + eps);
  for (int i = 0; i < 4; ++i) c[first + i * stride] = c[first + i * stride] * inv;
}

/* Row r of the logits becomes fma(exp(x - max), 1/sum, eps). */
static void softmax_row_eps(float *c, int r, float eps) {
  float *row = c + 4 * r;
  float peak = fmaxf(fmaxf(row[0], row[1]), fmaxf(row[2], row[3]));
  for (int k = 0; k < 4; ++k) row[k] = oracle_exp(row[k] - peak);
  float inv = oracle_rcp(pair_sum4(row, 0, 1));
  for (int k = 0; k < 4; ++k) row[k] = fmaf(row[k], inv, eps);
}

void oracle_sinkhorn(const float logits[16], float eps, int repeat, float c[16]) {
  for (int i = 0; i < 16; ++i) c[i] = logits[i];
  for (int r = 0; r < 4; ++r) softmax_row_eps(c, r, eps);
  for (int round = 0; round < repeat; ++round) {
    if (round > 0)
      for (int r = 0; r < 4; ++r) normalize4(c, 4 * r, 1, eps);  /* rows    */
    for (int k = 0; k < 4; ++k) normalize4(c, k, 4, eps);        /* columns */
  }
}

/* [GLM] _MixesDeviceKernel.kernel, per token: post'_j = sigmoid(mixes[4+j] *
 * scale[1] + base[4+j]) * post_mult; comb' = Sinkhorn(mixes[8+i] * scale[2] +
 * base[8+i]) with eps = hc_eps.  post_out [M, 4], comb_out [M, 4, 4]. */
int oracle_side_mixes(const float *mixes, const float *scale, const float *base, int M,
                      float hc_eps, float post_mult, int repeat, float *post_out,
                      float *comb_out) {
  if (M < 0 || repeat < 0) return 1;
  for (int t = 0; t < M; ++t) {
    const float *row = mixes + (int64_t)t * NMIX;
    for (int j = 0; j < NSTREAM; ++j)
      post_out[(int64_t)t * NSTREAM + j] =
          oracle_sigmoid(fmaf(row[NSTREAM + j], scale[1], base[NSTREAM + j])) * post_mult;
    float logits[16];
    for (int i = 0; i < 16; ++i) logits[i] = fmaf(row[8 + i], scale[2], base[8 + i]);
    oracle_sinkhorn(logits, hc_eps, repeat, comb_out + (int64_t)t * 16);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* DSA indexer projection                                                    */
/* ------------------------------------------------------------------------ */

/* [IDX] vllm.models.glm5next.nvidia.specialized_decode.indexer,
 * IndexerProjection.__call__: one product of the layer input x [M, K] with
 * the concatenated weight rows w [key + heads + gate, K] (the indexer key
 * rows, the head-weight rows, the kpool gate rows, in that order), each
 * part written in its own type: key [M, key] BF16, head weights [M, heads]
 * FP32, gate [M, gate] BF16.  The products of BF16 values are exact and the
 * page leaves the order of the sum open: the sum is taken in binary64 and
 * rounded to binary32 once, then to BF16 for the key and gate parts. */
int oracle_indexer_projection(const uint16_t *x, const uint16_t *w, int M, int K, int key,
                              int heads, int gate, uint16_t *key_out, float *heads_out,
                              uint16_t *gate_out) {
  if (M < 0 || K <= 0 || key < 0 || heads < 0 || gate < 0) return 1;
  const int rows = key + heads + gate;
  for (int t = 0; t < M; ++t)
    for (int r = 0; r < rows; ++r) {
      double s = 0.0;
      for (int k = 0; k < K; ++k)
        s += (double)bf(x[(int64_t)t * K + k]) * (double)bf(w[(int64_t)r * K + k]);
      const float f = (float)s;
      if (r < key) key_out[(int64_t)t * key + r] = tobf(f);
      else if (r < key + heads) heads_out[(int64_t)t * heads + (r - key)] = f;
      else gate_out[(int64_t)t * gate + (r - key - heads)] = tobf(f);
    }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* a8 standalone: MXFP8 of a BF16 [M, H] array                               */
/* ------------------------------------------------------------------------ */

int oracle_quant_mxfp8(const uint16_t *x, int M, int H, uint8_t *values, uint8_t *scales) {
  if (M < 0 || H <= 0 || H % 128) return 1;
  for (int t = 0; t < M; ++t) quant_token(x + (int64_t)t * H, t, H, values, scales);
  zero_padding_scales(M, H, scales);
  return 0;
}
