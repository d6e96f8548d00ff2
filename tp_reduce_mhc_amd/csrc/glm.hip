// GLM-style boundary for gfx950: the pre-mix is derived in-kernel from the
// new residual through the 24-row prenorm GEMV, and a small side-stream
// kernel finishes the post-mix and the Sinkhorn residual mix for the next
// boundary.
//
// Arithmetic follows the page
//   vllm.models.glm5next.nvidia.specialized_decode.all_reduce_mhc
//     (_BoundaryDeviceKernel.kernel, _GroupBoundaryDeviceKernel.kernel,
//      _MixesDeviceKernel.kernel, _MixesDeviceKernel._sinkhorn)
// with the rank sum taken from rank 0 in order as the DSV4.1 page does (the
// GLM page's lane butterfly assumes tp = 4).
//
// gfx950 design: one workgroup takes G tokens (1, 2 or 4) with one 16-byte
// fragment per thread; each hc_fn fragment is read once per workgroup and
// applied to all G tokens with v_dot2c_f32_bf16 (BF16 products are exact in
// FP32); the 24 x G partial dot products are reduce-scattered across the
// wave (each lane ends with one total) and the waves are added through LDS
// in fixed order, in place of the page's cluster-wide DSMEM reduction.
#include "device.h"
#include "kernels.h"
#include "sync.h"
#include "finalize.h"

#include <type_traits>

namespace mhcb {
namespace {

constexpr int kGlmWideThreads = 768;  // G = 4 workgroups: hidden <= 6144

// Wave64 reduce-scatter of N (32 or 64) values per lane: returns on every
// lane the wave total of value index (N == 64 ? lane : lane / 2).  Each
// halving step keeps the half selected by the lane bit and adds the
// partner's copy of it; the steps are unrolled by template recursion so
// every index is a compile-time constant (the values stay in VGPRs).
template <int N, int O>
struct HalvingStep {
  static __device__ __forceinline__ void run(float *v, int lane) {
    const bool upper = (lane & O) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float send = upper ? v[i] : v[i + N / 2];
      const float keep = upper ? v[i + N / 2] : v[i];
      v[i] = keep + __shfl_xor(send, O, kWave);
    }
    HalvingStep<N / 2, O / 2>::run(v, lane);
  }
};
template <int O>
struct HalvingStep<1, O> {
  static __device__ __forceinline__ void run(float *, int) {}
};

template <int N>
__device__ __forceinline__ float reduce_scatter(float (&v)[N]) {
  static_assert(N == 32 || N == 64, "32 or 64 values");
  const int lane = threadIdx.x & (kWave - 1);
  HalvingStep<N, kWave / 2>::run(v, lane);
  float r = v[0];
  if constexpr (N == 32) r += __shfl_xor(r, 1, kWave);
  return r;
}

__device__ __forceinline__ float sigmoid(float x) {
  return (float)(1.0 / (1.0 + exp(-(double)x)));
}

// Offsets in a token's exchange area (kernels.h): the binary64 sums of
// exchange 0 and 1, and the GEMV rows, stored two FP32 rows per 8-byte word.
constexpr int kSum1 = kCopySum1, kSum2 = kCopySum2;
constexpr int kPairs = kMix / 2;

// The GEMV rows a workgroup of slice s (of S) needs after exchange 0: the
// pre-mix rows 0..3, and the rows k >= 4 with k % S == s.  Row k's raw mix
// is written by slice k % S, so each slice gathers a few rows instead of 24.
// Row j of the list is needed_row(j); the list has `count` rows (at most
// 24).  No integer division: the values are uniform and tiny, loops suffice.
struct RowList {
  int first, count;  // first own row >= 4; rows in the list
};
__device__ __forceinline__ RowList row_list(int S, int s) {
  int m = s - kStreams;
  while (m < 0) m += S;
  RowList l = {kStreams + m, kStreams};
  for (int k = l.first; k < kMix; k += S) ++l.count;
  return l;
}
__device__ __forceinline__ int needed_row(const RowList &l, int S, int j) {
  return j < kStreams ? j : l.first + (j - kStreams) * S;
}
// Whether row k (a row of the list) is this slice's to write: k % S == s.
__device__ __forceinline__ bool own_row(int S, int s, int k) {
  if (k >= kStreams) return true;  // rows >= 4 are in the list only if owned
  const int d = k - s;             // k < 4: owned iff d is 0, S, 2S or 3S
  return d == 0 || d == S || d == 2 * S || d == 3 * S;
}
// The 8-byte row pairs that hold the list's rows: pairs 0 and 1 (rows 0..3),
// then the pair of each own row (distinct for S >= 2; all 12 for S = 1).
__device__ __forceinline__ int pair_count(const RowList &l, int S) {
  return S == 1 ? kPairs : 2 + (l.count - kStreams);
}
__device__ __forceinline__ int needed_pair(const RowList &l, int S, int j) {
  return S == 1 || j < 2 ? j : needed_row(l, S, j + 2) >> 1;
}

// Stores one 8-byte value into token t's exchange area of this call (from
// its slot's epoch word), unless the slot is broken.
__device__ __forceinline__ void call_store(const GlmArgs &a, int t, uint64_t callw, int offset,
                                           uint64_t v) {
  const SlotCall c = unpack_call(callw);
  if (!c.broken) slot_store_u64(token_slot(a.sync, t) + copy_offset(c.epoch), offset, v);
}

template <int G>
struct GlmShared {
  uint64_t callw[G];                    // split: each token slot's epoch word
  float part[kMaxThreads / kWave][64];  // per-wave reduce-scatter results
  float mix[G][kMix];                   // GEMV totals of each token
  float pre[G][kStreams];
  double tot[G];
  double red[(kMaxThreads / kWave) * G];
};

// Exchanges the per-slice partials of the G tokens of a split workgroup:
// the GEMV rows sh.mix (FP32, with `rows`) and one binary64 sum per token
// (`sums`, at `sum` in the exchange area).  Afterwards every slice holds the
// slice-ordered totals of the sums and of the rows in its row_list.
// Exchange 0 is the rows and sum 1, exchange 1 is sum 2.  Contains
// barriers: every thread of the workgroup calls it.
template <int G>
__device__ void exchange(const GlmArgs &a, GlmShared<G> &sh, int t0, int s, double (&sums)[G],
                         int sum, bool rows) {
  const int tid = threadIdx.x, S = a.slices;
  if (rows) {
    for (int i = tid; i < G * kPairs; i += blockDim.x) {
      const int g = i / kPairs, p = i % kPairs;
      if (t0 + g < a.M) {
        const uint64_t w = (uint64_t)__builtin_bit_cast(uint32_t, sh.mix[g][2 * p]) |
                           ((uint64_t)__builtin_bit_cast(uint32_t, sh.mix[g][2 * p + 1]) << 32);
        call_store(a, t0 + g, sh.callw[g], kCopyRows + kRowsEntry * s + 8 * p, w);
      }
    }
  }
  if (tid < G && t0 + tid < a.M) {
    double v = 0.0;  // sums[tid], without indexing a register array at run time
#pragma unroll
    for (int g = 0; g < G; ++g) v = g == tid ? sums[g] : v;
    call_store(a, t0 + tid, sh.callw[tid], sum + 8 * s, __builtin_bit_cast(uint64_t, v));
  }
  if (rows) {
    const RowList l = row_list(S, s);
    for (int i = tid; i < G * 32; i += blockDim.x) {
      const int g = i >> 5, j = i & 31;
      if (j >= pair_count(l, S) || t0 + g >= a.M) continue;
      const int p = needed_pair(l, S, j);
      uint64_t w[kMaxSlices];
      gather64(a.sync, token_slot(a.sync, t0 + g), unpack_call(sh.callw[g]), kCopyRows + 8 * p,
               kRowsEntry, S, w);
      float lo = 0.0f, hi = 0.0f;
#pragma unroll
      for (int q = 0; q < kMaxSlices; ++q) {
        if (q >= S) break;
        lo += __builtin_bit_cast(float, (uint32_t)w[q]);
        hi += __builtin_bit_cast(float, (uint32_t)(w[q] >> 32));
      }
      sh.mix[g][2 * p] = lo;
      sh.mix[g][2 * p + 1] = hi;
    }
  }
  if (tid < G)
    sh.tot[tid] = t0 + tid < a.M ? gather_sum64(a.sync, token_slot(a.sync, t0 + tid),
                                                unpack_call(sh.callw[tid]), sum, S)
                                 : 0.0;
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) sums[g] = sh.tot[g];
  __syncthreads();
}

// When the call exchanges (`exchanges`), thread i < tokens reads the epoch
// word of token t0 + i's slot (0 for other threads and tokens past M).
__device__ __forceinline__ uint64_t read_call_word(const GlmArgs &a, bool exchanges, int t0,
                                                   int tokens, int i) {
  if (!exchanges || i >= tokens || t0 + i >= a.M) return 0u;
  return slot_call_word(token_slot(a.sync, t0 + i));
}

// After a slice's last read of the call's exchanges: thread i < tokens
// advances token t0 + i's epoch, and the slices share the clearing of the
// copies the previous calls used (sync.h), one (token, word) item per
// worker (the worker index interleaves the slices).  Every thread calls it.
__device__ void finish_exchanges(const GlmArgs &a, const uint64_t *callw, int t0, int tokens, int s) {
  const int tid = threadIdx.x, nt = blockDim.x, S = a.slices;
  if (tid < tokens && t0 + tid < a.M)
    advance_epoch(token_slot(a.sync, t0 + tid), unpack_call(callw[tid]), S);
  for (int f = tid * S + s; f < tokens * kClearWords; f += nt * S) {
    const int g = f / kClearWords;
    if (t0 + g < a.M) clear_previous_word(token_slot(a.sync, t0 + g), unpack_call(callw[g]), f % kClearWords);
  }
}

// KB = hc_fn rows per pass (24 for G <= 2; 12 for G = 4 to bound registers);
// MAXT = the workgroup size bound (768 for G = 4 leaves 168 VGPRs a lane).
// Grid (slices, ceil(M/G)) when split, else (ceil(M/G)): workgroup (s, grp)
// covers fragments [s * slice_frags, (s + 1) * slice_frags) of tokens
// grp*G .. grp*G + G - 1; the slices exchange their partial GEMV rows and
// sums of squares through the workspace.
template <int G, int KB, int MAXT>
__global__ void __launch_bounds__(MAXT)
glm_kernel(const GlmArgs a) {
  static_assert(kMix % KB == 0, "rows per pass must divide 24");
  constexpr int V = G * KB;                  // values reduced per pass
  constexpr int N = V <= 32 ? 32 : 64;
  static_assert(V <= 64, "too many values per pass");
  __shared__ GlmShared<G> sh;

  const int H = a.H, F = H / kFrag, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave, waves = blockDim.x / kWave;
  const int s = a.slices > 1 ? blockIdx.x : 0;
  const int grp = a.slices > 1 ? blockIdx.y : blockIdx.x;
  const int t0 = grp * G;
  const int first = a.slices > 1 ? s * a.slice_frags : 0;
  const int last = a.slices > 1 ? min(F, first + a.slice_frags) : F;
  const bool valid = first + tid < last;
  const int64_t col = valid ? (int64_t)(first + tid) * kFrag : 0;
  // Split: each token slot's epoch word, in flight with the streams.
  const uint64_t callw = read_call_word(a, a.slices > 1, t0, G, tid);

  // a1 + a2 for the G tokens: y[g][j] packed BF16, sum of y^2 per token.
  u32x4 y[G][kStreams];
  double ssy[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int t = t0 + g;
    const bool live = valid && t < a.M;
    const int tt = t < a.M ? t : a.M - 1;
    u32x4 res[kStreams];
#pragma unroll
    for (int q = 0; q < kStreams; ++q)
      res[q] = load_stream(a.residual + ((int64_t)tt * kStreams + q) * H + col);
    float s8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s8[e] = 0.0f;
    const uint16_t *src = a.partials + (int64_t)tt * H + col;
    for (int r0 = 0; r0 < a.tp; r0 += 8) {
      u32x4 w[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        w[q] = r0 + q < a.tp ? load_stream(src + (r0 + q) * a.rank_stride) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (r0 + q >= a.tp) break;
        float v[8];
        unpack8(w[q], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) s8[e] = s8[e] + v[e];
      }
    }
    float x[8];
    unpack8(pack8(s8), x);
    const float *post = a.post + tt * kStreams;
    const float *comb = a.comb + tt * kStreams * kStreams;
    float r4[kStreams][8];
#pragma unroll
    for (int q = 0; q < kStreams; ++q) unpack8(res[q], r4[q]);
    ssy[g] = 0.0;
#pragma unroll
    for (int j = 0; j < kStreams; ++j) {
      float acc[8];
      const float pj = post[j];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = x[e] * pj;
#pragma unroll
        for (int q = 0; q < kStreams; ++q) v = __builtin_fmaf(r4[q][e], comb[q * kStreams + j], v);
        acc[e] = v;
      }
      y[g][j] = pack8(acc);
      if (live) {
        store_stream(a.residual_out + ((int64_t)t * kStreams + j) * H + col, y[g][j]);
        float yv[8];
        unpack8(y[g][j], yv);
#pragma unroll
        for (int e = 0; e < 8; ++e) ssy[g] += (double)yv[e] * (double)yv[e];
      }
    }
    if (!valid) {
#pragma unroll
      for (int j = 0; j < kStreams; ++j) y[g][j] = u32x4{0, 0, 0, 0};
    }
  }

  // a3: g_k = sum_{j,c} fn[k][j*H + c] * y_j[c], KB rows per pass.
#pragma unroll
  for (int pass = 0; pass < kMix / KB; ++pass) {
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.0f;
    if (valid) {
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const int k = pass * KB + kk;
#pragma unroll
        for (int j = 0; j < kStreams; ++j) {
          const u32x4 w = load_cached(a.fn + (int64_t)k * kStreams * H + (int64_t)j * H + col);
#pragma unroll
          for (int g = 0; g < G; ++g) acc[g * KB + kk] = dot8(w, y[g][j], acc[g * KB + kk]);
        }
      }
    }
    const float total = reduce_scatter<N>(acc);
    const int idx = N == 64 ? lane : lane >> 1;
    if ((N == 64 || (lane & 1) == 0) && idx < V) sh.part[wave][idx] = total;
    __syncthreads();
    if (tid < V) {
      float v = 0.0f;
      for (int w = 0; w < waves; ++w) v += sh.part[w][tid];
      sh.mix[tid / KB][pass * KB + tid % KB] = v;
    }
    __syncthreads();
  }

  // g_24 and rstd; raw mixes out; pre_j = sigmoid(mix_j * scale0 + base_j) + hc_eps.
  if (a.slices > 1 && tid < G) sh.callw[tid] = callw;  // read after block_sum's barriers
  block_sum<double, G>(ssy, sh.red);
  if (a.slices > 1) exchange<G>(a, sh, t0, s, ssy, kSum1, true);
  // (Unsplit: S = 1, every row here.)
  const int S = a.slices;
  const RowList rl = row_list(S, s);
  for (int i = tid; i < G * 32; i += blockDim.x) {  // a workgroup may have fewer threads
    const int g = i >> 5, j = i & 31, k = needed_row(rl, S, j), t = t0 + g;
    if (j >= rl.count) continue;
    double total = 0.0;
#pragma unroll
    for (int q = 0; q < G; ++q) total = q == g ? ssy[q] : total;
    const float rstd = (float)(1.0 / __builtin_sqrt((double)(float)total / (4.0 * H) + (double)a.rms_eps));
    const float mix = sh.mix[g][k] * rstd;
    if (t < a.M && own_row(S, s, k)) a.mixes_out[(int64_t)t * kMix + k] = mix;
    if (k < kStreams) sh.pre[g][k] = sigmoid(__builtin_fmaf(mix, a.scale[0], a.base[k])) + a.hc_eps;
  }
  __syncthreads();

  // a4: p = bf16((q0+q1)+(q2+q3)), q_j = y_j * pre_j; RMSNorm over H.
  u32x4 p[G];
  double pss[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float q[kStreams][8];
#pragma unroll
    for (int j = 0; j < kStreams; ++j) {
      float yv[8];
      unpack8(y[g][j], yv);
      const float pj = sh.pre[g][j];
#pragma unroll
      for (int e = 0; e < 8; ++e) q[j][e] = yv[e] * pj;
    }
    float z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (q[0][e] + q[1][e]) + (q[2][e] + q[3][e]);
    p[g] = pack8(z);
    pss[g] = 0.0;
    if (valid) {
      float pv[8];
      unpack8(p[g], pv);
#pragma unroll
      for (int e = 0; e < 8; ++e) pss[g] += (double)pv[e] * (double)pv[e];
    }
  }
  block_sum<double, G>(pss, sh.red);
  if (a.slices > 1) {
    exchange<G>(a, sh, t0, s, pss, kSum2, false);
    finish_exchanges(a, sh.callw, t0, G, s);
  }
  float gam[8];
  unpack8(load_cached(a.gamma + col), gam);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int t = t0 + g;
    const float inv = (float)(1.0 / __builtin_sqrt((double)(float)pss[g] / (double)H + (double)a.norm_eps));
    float pv[8], o[8];
    unpack8(p[g], pv);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (pv[e] * inv) * gam[e];
    if (valid && t < a.M) store_stream(a.layer_input + (int64_t)t * H + col, pack8(o));
  }
}

// ---------------------------------------------------------------------------
// Token tiles: the prenorm GEMV of 16 tokens on the matrix cores.
//
// Workgroup (s, grp) takes tokens grp*16 .. grp*16+15 over the fragments
// [s * sf, (s + 1) * sf) of their columns (sf = slice_frags).  The
// streaming steps (rank sum, post-mix, residual_out, collapse, layer_input)
// put consecutive threads on consecutive fragments of a token, so every
// load and store is a contiguous run.  The post-mixed streams also go to
// LDS, from where the GEMV reads them as the A operand of
// v_mfma_f32_16x16x32_bf16: a wave step covers 16 tokens (rows) x 4
// fragments (32 columns, K) of one stream, lane l taking token l % 16 at
// fragment l / 16.  The B operand is hc_fn: lane l loads row l % 16 (and
// 16 + l % 16 for the tile of rows 16..23) at the same fragment, so each
// hc_fn fragment is read once per 16 tokens.  The 16 x 24 partial GEMV and
// the sums of squares are added across waves in LDS and across slices
// through the workspace, with one cross-workgroup barrier per tile (the
// slot of its first token) for the mixes and one for the RMSNorm sum.
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;              // tokens per tile
constexpr int kTileThreads = 512;      // at most
constexpr int kTileWaves = kTileThreads / kWave;
constexpr int kTileMaxFrags = 96;      // fragments per slice

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

struct TileShared {
  uint64_t callw[kTile];                // each token slot's epoch word
  float post[kTile][kStreams];
  float comb[kTile][kStreams * kStreams];
  float part[kTileWaves][kTile][kMix];  // per-wave GEMV partials
  float mix[kTile][kMix];
  float pre[kTile][kStreams];
  double tot[kTile];
};

// Dynamic LDS of a tile workgroup: the post-mixed streams [tok][j*sf + f]
// (token rows padded by 16 bytes so that the 16 rows of an MFMA read fall in
// distinct banks), then the per-fragment sums of squares [tok][f].
__host__ __device__ inline int tile_row_words(int sf) { return kStreams * sf + 1; }
__host__ __device__ inline size_t tile_ys_bytes(int sf) {
  return (size_t)kTile * tile_row_words(sf) * 16;
}
__host__ __device__ inline size_t tile_dyn_bytes(int sf) {
  return tile_ys_bytes(sf) + (size_t)kTile * sf * 8;
}

// Publishes this slice's per-token sums sh.tot (at `sum` in the exchange
// area; with `rows`, also the GEMV partials in sh.mix) and leaves the
// slice-ordered totals in sh.tot (and, of the rows in its row_list, in
// sh.mix).  A thread reads all the slices' values of its (token, row pair)
// or token sum as they land and adds them in slice order.  Every thread
// calls it.
__device__ void tile_exchange(const GlmArgs &a, TileShared &sh, int t0, int s, int sum, bool rows) {
  const int tid = threadIdx.x, nt = blockDim.x, S = a.slices;
  const int valid = min(kTile, a.M - t0);
  if (rows) {
    for (int e = tid; e < valid * kPairs; e += nt) {
      const int tok = e / kPairs, p = e % kPairs;
      const uint64_t w = (uint64_t)__builtin_bit_cast(uint32_t, sh.mix[tok][2 * p]) |
                         ((uint64_t)__builtin_bit_cast(uint32_t, sh.mix[tok][2 * p + 1]) << 32);
      call_store(a, t0 + tok, sh.callw[tok], kCopyRows + kRowsEntry * s + 8 * p, w);
    }
  }
  if (tid < valid)
    call_store(a, t0 + tid, sh.callw[tid], sum + 8 * s, __builtin_bit_cast(uint64_t, sh.tot[tid]));
  __syncthreads();  // every thread has read its own sh values before they are replaced
  // Work items: the row pairs this slice needs of each token (with rows; a
  // stride of 12 per token keeps them within one pass), then the sums.
  const RowList l = row_list(S, s);
  const int np = pair_count(l, S), row_items = rows ? valid * kPairs : 0;
  for (int e = tid; e < row_items + valid; e += nt) {
    if (e < row_items) {
      const int tok = e / kPairs, j = e % kPairs;
      if (j >= np) continue;
      const int p = needed_pair(l, S, j);
      uint64_t w[kMaxSlices];
      gather64(a.sync, token_slot(a.sync, t0 + tok), unpack_call(sh.callw[tok]), kCopyRows + 8 * p,
               kRowsEntry, S, w);
      float lo = 0.0f, hi = 0.0f;
#pragma unroll
      for (int q = 0; q < kMaxSlices; ++q) {
        if (q >= S) break;
        lo += __builtin_bit_cast(float, (uint32_t)w[q]);
        hi += __builtin_bit_cast(float, (uint32_t)(w[q] >> 32));
      }
      sh.mix[tok][2 * p] = lo;
      sh.mix[tok][2 * p + 1] = hi;
    } else {
      const int tok = e - row_items;
      sh.tot[tok] = gather_sum64(a.sync, token_slot(a.sync, t0 + tok), unpack_call(sh.callw[tok]),
                                 sum, S);
    }
  }
  __syncthreads();
}

// sh.tot[tok] = sum over f < sf of item[tok][f], in fragment order.
__device__ __forceinline__ void tile_item_sums(TileShared &sh, const double *item, int sf) {
  __syncthreads();
  if (threadIdx.x < kTile) {
    double v = 0.0;
    for (int f = 0; f < sf; ++f) v += item[threadIdx.x * sf + f];
    sh.tot[threadIdx.x] = v;
  }
  __syncthreads();
}

// hc_fn B operands of one 4-fragment chunk for lane (i, q): rows i and
// 16 + i (zero for rows past 24 or fragments past the slice) of each stream.
struct FnChunk {
  u32x4 b1[kStreams], b2[kStreams];
};
__device__ __forceinline__ void load_fn_chunk(const GlmArgs &a, int i, int f, bool ok, FnChunk &c) {
  const int64_t H = a.H, col = ok ? (int64_t)f * kFrag : 0;
#pragma unroll
  for (int j = 0; j < kStreams; ++j) {
    c.b1[j] = ok ? load_cached(a.fn + (int64_t)i * kStreams * H + j * H + col) : u32x4{0, 0, 0, 0};
    c.b2[j] = ok && i < kMix - kTile
                  ? load_cached(a.fn + (int64_t)(kTile + i) * kStreams * H + j * H + col)
                  : u32x4{0, 0, 0, 0};
  }
}

// U = (token, fragment) items per thread, and also 4-fragment GEMV chunks
// per wave; TP = fixed rank count, or 0 for the runtime count.
template <int U, int TP>
__global__ void __launch_bounds__(kTileThreads, 1)
glm_tile_kernel(const GlmArgs a) {
  __shared__ TileShared sh;
  extern __shared__ __align__(16) char dyn[];
  const int H = a.H, F = H / kFrag, tid = threadIdx.x, nt = blockDim.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave, waves = nt / kWave;
  const int s = blockIdx.x, t0 = blockIdx.y * kTile;
  const int sf = a.slice_frags, first = s * sf, last = min(F, first + sf);
  const int valid = min(kTile, a.M - t0);
  const int tp = TP > 0 ? TP : a.tp;
  const int rw = tile_row_words(sf);
  u32x4 *ys = reinterpret_cast<u32x4 *>(dyn);
  double *item = reinterpret_cast<double *>(dyn + tile_ys_bytes(sf));
  const int mi = lane & (kTile - 1), mq = lane >> 4;  // MFMA row, K chunk

  // Each token slot's epoch word (thread i < 16: token t0 + i), first in the
  // queue: loads return in order, and it is needed only at the exchanges.
  const uint64_t callw = read_call_word(a, true, t0, kTile, tid);
  // The tile's post and comb (20 floats a token) and this wave's first
  // hc_fn chunk, loaded before the streams.
  constexpr int kMixVals = kTile * 20, kMixPerThread = kMixVals / kWave;
  float mv[kMixPerThread];
#pragma unroll
  for (int u = 0; u < kMixPerThread; ++u) {
    const int e = tid + u * nt, tok = e / 20, k = e % 20, tt = t0 + tok;
    mv[u] = e < kMixVals && tok < valid
                ? (k < kStreams ? a.post[(int64_t)tt * kStreams + k] : a.comb[(int64_t)tt * 16 + (k - kStreams)])
                : 0.0f;
  }
  FnChunk fc[U];
  load_fn_chunk(a, mi, first + 4 * wave + mq, 4 * wave < sf && first + 4 * wave + mq < last, fc[0]);

  // Items: idx = tid + u * nt -> token idx / sf, fragment first + idx % sf.
  int tok[U];
  int64_t col[U];
  bool live[U];
  u32x4 part[U][TP > 0 ? TP : 1], res[U][kStreams], gam[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int idx = tid + u * nt;
    tok[u] = idx / sf;
    const int f = first + idx % sf;
    live[u] = tok[u] < valid && f < last;
    col[u] = live[u] ? (int64_t)f * kFrag : 0;
    const int64_t t = t0 + (live[u] ? tok[u] : 0);
#pragma unroll
    for (int r = 0; r < kStreams; ++r)
      res[u][r] = live[u] ? load_stream(a.residual + (t * kStreams + r) * H + col[u]) : u32x4{0, 0, 0, 0};
    if constexpr (TP > 0) {
#pragma unroll
      for (int r = 0; r < TP; ++r)
        part[u][r] = live[u] ? load_stream(a.partials + r * a.rank_stride + t * H + col[u]) : u32x4{0, 0, 0, 0};
    }
    gam[u] = live[u] ? load_cached(a.gamma + col[u]) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int u = 0; u < kMixPerThread; ++u) {
    const int e = tid + u * nt, tk = e / 20, k = e % 20;
    if (e < kMixVals) {
      if (k < kStreams) sh.post[tk][k] = mv[u];
      else sh.comb[tk][k - kStreams] = mv[u];
    }
  }
  __syncthreads();

  // a1 + a2 per item; y to LDS (the GEMV's A operand, and the collapse's).
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float sum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] = 0.0f;
    const int64_t t = t0 + (live[u] ? tok[u] : 0);
    if constexpr (TP > 0) {
#pragma unroll
      for (int r = 0; r < TP; ++r) {
        float v[8];
        unpack8(part[u][r], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[e] = sum[e] + v[e];
      }
    } else {
      const uint16_t *src = a.partials + t * H + col[u];
      for (int r0 = 0; r0 < tp; r0 += 8) {
        u32x4 w[8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
          w[r] = live[u] && r0 + r < tp ? load_stream(src + (r0 + r) * a.rank_stride) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if (r0 + r >= tp) break;
          float v[8];
          unpack8(w[r], v);
#pragma unroll
          for (int e = 0; e < 8; ++e) sum[e] = sum[e] + v[e];
        }
      }
    }
    float x[8];
    unpack8(pack8(sum), x);
    float r4[kStreams][8];
#pragma unroll
    for (int r = 0; r < kStreams; ++r) unpack8(res[u][r], r4[r]);
    const int tk = live[u] ? tok[u] : 0;
    const int idx = tid + u * nt;
    double ysq = 0.0;
#pragma unroll
    for (int j = 0; j < kStreams; ++j) {
      const float pj = sh.post[tk][j];
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = x[e] * pj;
#pragma unroll
        for (int r = 0; r < kStreams; ++r) v = __builtin_fmaf(r4[r][e], sh.comb[tk][r * kStreams + j], v);
        acc[e] = v;
      }
      const u32x4 yj = live[u] ? pack8(acc) : u32x4{0, 0, 0, 0};
      if (live[u]) {
        store_stream(a.residual_out + (t * kStreams + j) * H + col[u], yj);
        ysq += (double)dot8(yj, yj, 0.0f);  // FP32 within the fragment
      }
      if (idx < kTile * sf) ys[(idx / sf) * rw + j * sf + idx % sf] = yj;
    }
    if (idx < kTile * sf) item[idx] = ysq;  // [tok][f]
  }
  // The wave's remaining hc_fn chunks, in flight across the barrier.
#pragma unroll
  for (int m = 1; m < U; ++m) {
    const int c = wave + m * waves, f = first + 4 * c + mq;
    load_fn_chunk(a, mi, f, 4 * c < sf && f < last, fc[m]);
  }
  if (tid < kTile) sh.callw[tid] = callw;
  __syncthreads();

  // a3: the GEMV on the matrix cores, wave w taking 4-fragment chunks
  // w, w + waves, ...
  {
    f32x4 c1 = {0.0f, 0.0f, 0.0f, 0.0f}, c2 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < U; ++m) {
      const int c = wave + m * waves;
      if (4 * c >= sf) break;
#pragma unroll
      for (int j = 0; j < kStreams; ++j) {
        const u32x4 av = ys[mi * rw + j * sf + 4 * c + mq];
        c1 = mfma_bf16(av, fc[m].b1[j], c1);
        c2 = mfma_bf16(av, fc[m].b2[j], c2);
      }
    }
    // Lane l holds rows l % 16 and 16 + l % 16 of tokens 4*(l/16) .. +3.
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sh.part[wave][4 * mq + e][mi] = c1[e];
      if (mi < kMix - kTile) sh.part[wave][4 * mq + e][kTile + mi] = c2[e];
    }
  }
  tile_item_sums(sh, item, sf);  // (its first barrier also publishes sh.part)
  for (int e = tid; e < kTile * kMix; e += nt) {
    float v = 0.0f;
    for (int w = 0; w < waves; ++w) v += sh.part[w][e / kMix][e % kMix];
    sh.mix[e / kMix][e % kMix] = v;
  }
  __syncthreads();
  tile_exchange(a, sh, t0, s, kSum1, true);

  // rstd over 4H; raw mixes out (row k by slice k % S); pre_j.
  const int S = a.slices;
  const RowList rl = row_list(S, s);
  for (int e = tid; e < valid * 32; e += nt) {
    const int tk = e >> 5, j = e & 31, k = needed_row(rl, S, j), tt = t0 + tk;
    if (j >= rl.count) continue;
    const float rstd = (float)(1.0 / __builtin_sqrt((double)(float)sh.tot[tk] / (4.0 * H) + (double)a.rms_eps));
    const float mix = sh.mix[tk][k] * rstd;
    if (own_row(S, s, k)) a.mixes_out[(int64_t)tt * kMix + k] = mix;
    if (k < kStreams) sh.pre[tk][k] = sigmoid(__builtin_fmaf(mix, a.scale[0], a.base[k])) + a.hc_eps;
  }
  __syncthreads();

  // a4: p = bf16((q0+q1)+(q2+q3)), q_j = y_j * pre_j; RMSNorm over H.
  u32x4 p[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int idx = tid + u * nt;
    const int tk = live[u] ? tok[u] : 0;
    float qv[kStreams][8];
#pragma unroll
    for (int j = 0; j < kStreams; ++j) {
      float yv[8];
      unpack8(live[u] ? ys[tk * rw + j * sf + idx % sf] : u32x4{0, 0, 0, 0}, yv);
      const float pj = sh.pre[tk][j];
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[j][e] = yv[e] * pj;
    }
    float z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (qv[0][e] + qv[1][e]) + (qv[2][e] + qv[3][e]);
    p[u] = pack8(z);
    double pss = 0.0;
    if (live[u]) pss = (double)dot8(p[u], p[u], 0.0f);
    if (idx < kTile * sf) item[idx] = pss;
  }
  tile_item_sums(sh, item, sf);
  tile_exchange(a, sh, t0, s, kSum2, false);
  finish_exchanges(a, sh.callw, t0, kTile, s);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!live[u]) continue;
    const float inv = (float)(1.0 / __builtin_sqrt((double)(float)sh.tot[tok[u]] / (double)H + (double)a.norm_eps));
    float pv[8], g[8], o[8];
    unpack8(p[u], pv);
    unpack8(gam[u], g);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (pv[e] * inv) * g[e];
    store_stream(a.layer_input + (int64_t)(t0 + tok[u]) * H + col[u], pack8(o));
  }
}

// ---------------------------------------------------------------------------
// Two-pass tiles: the same 16-token matrix-core GEMV without any
// cross-workgroup exchange.
//
// Pass 1, glm_stream_kernel: workgroup (s, grp) takes tokens grp*16 ..
// grp*16+15 over the fragments [s * sf, (s + 1) * sf), one (token,
// fragment) item per thread (16 * sf threads).  It streams the ranks (for
// an MoE sublayer: computes each rank's contribution from the tile's routes)
// and the residual streams, writes residual_out, and leaves the slice's 24
// partial GEMV rows and its sum of squares of the token's streams in the
// scratch area.  Workgroups are small (sf = 16 or 32 fragments), several to
// a compute unit.
//
// Pass 2, glm_finish_kernel: one workgroup per token, one fragment per
// thread.  It adds the slices' partials in slice order, writes the raw
// mixes, derives the pre-mix and takes the collapse and RMSNorm over the
// residual_out rows the first pass just wrote.
// ---------------------------------------------------------------------------

constexpr int kStreamMaxThreads = 1024;

struct StreamShared {
  float post[kTile][kStreams];
  float comb[kTile][kStreams * kStreams];
};

// Dynamic LDS of a stream workgroup: the tile's post-mixed streams (as in
// the exchanging tiles), the per-item sums of squares, then the per-wave
// GEMV partials [wave][token][row].
__host__ __device__ inline size_t stream_dyn_bytes(int sf) {
  return tile_dyn_bytes(sf) + (size_t)(sf / 4) * kTile * kMix * 4;
}

// The tile's MoE routes (FIN): [token][rank][k] rows and weights, as the
// per-token kernels stage them (stage_routes): weights widened from BF16
// when so given, times the routed scaling factor when not 1, and 0 for a
// route whose row is -1.
struct TileRoutes {
  int32_t row[kTile * kGlmTileRoutes];
  float w[kTile * kGlmTileRoutes];
};
struct NoRoutes {};

__device__ __forceinline__ void stage_tile_routes(const FinalizeView &f, int tp, int t0, int valid,
                                                  TileRoutes &rt) {
  const int per = tp * f.top_k;
  for (int i = threadIdx.x; i < valid * per; i += blockDim.x) {
    const int tok = i / per, rem = i % per, r = rem / f.top_k, k = rem % f.top_k;
    const int64_t t = t0 + tok;
    const int64_t e = r * f.w_stride + t * f.top_k + k;
    const int32_t row = f.idx[r * f.i_stride + t * f.top_k + k];
    float w = f.w_bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t *>(f.weights)[e] << 16)
                       : static_cast<const float *>(f.weights)[e];
    if (f.w_scale != 1.0f) w = w * f.w_scale;
    rt.row[i] = row;
    rt.w[i] = row == -1 ? 0.0f : w;
  }
}

// TP = fixed rank count of the partials (0: runtime); FIN = the ranks'
// contributions are MoE finalize outputs computed from a.fin (TP = 0: one
// rank's gathers at a time; TP = 2: two ranks' at a time, top_k <= 8, in
// workgroups of at most kStreamPairThreads).
constexpr int kStreamPairThreads = 256;

template <int TP, bool FIN>
__global__ void __launch_bounds__(FIN && TP == 2 ? kStreamPairThreads : kStreamMaxThreads)
glm_stream_kernel(const GlmArgs a) {
  __shared__ StreamShared sh;
  __shared__ std::conditional_t<FIN, TileRoutes, NoRoutes> routes;
  extern __shared__ __align__(16) char dyn[];
  const int H = a.H, F = H / kFrag, tid = threadIdx.x, nt = blockDim.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave, waves = nt / kWave;
  const int s = blockIdx.x, t0 = blockIdx.y * kTile, S = a.slices;
  const int sf = a.slice_frags, first = s * sf, last = min(F, first + sf);
  const int valid = min(kTile, a.M - t0);
  constexpr int kHeld = FIN ? 0 : TP;  // partials held in registers (FIN: TP picks the gather form)
  const int tp = kHeld > 0 ? kHeld : a.tp;
  const int rw = tile_row_words(sf);
  u32x4 *ys = reinterpret_cast<u32x4 *>(dyn);
  double *item = reinterpret_cast<double *>(dyn + tile_ys_bytes(sf));
  float *wpart = reinterpret_cast<float *>(dyn + tile_dyn_bytes(sf));  // [wave][tok][row]
  const int mi = lane & (kTile - 1), mq = lane >> 4;  // MFMA row, K chunk

  // The tile's post and comb (20 floats a token; at least 256 threads).
  constexpr int kMixVals = kTile * 20;
  float mv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + u * nt, tok = e / 20, k = e % 20, tt = t0 + tok;
    mv[u] = e < kMixVals && tok < valid
                ? (k < kStreams ? a.post[(int64_t)tt * kStreams + k] : a.comb[(int64_t)tt * 16 + (k - kStreams)])
                : 0.0f;
  }
  // This wave's hc_fn chunk (fragments first + 4*wave .. +3; sf / 4 waves,
  // one chunk each), first in the queue: it is needed only after the
  // streams.  (Loading it after the streams halves the registers, to 68,
  // but measured no faster.)
  FnChunk fc;
  load_fn_chunk(a, mi, first + 4 * wave + mq, first + 4 * wave + mq < last, fc);

  // The thread's item: token tid / sf, fragment first + tid % sf.
  const int tok = tid / sf, fl = tid % sf, f = first + fl;
  const bool live = tok < valid && f < last;
  const int64_t col = live ? (int64_t)f * kFrag : 0;
  const int64_t t = t0 + (live ? tok : 0);
  u32x4 res[kStreams], part[kHeld > 0 ? kHeld : 1];
#pragma unroll
  for (int r = 0; r < kStreams; ++r)
    res[r] = live ? load_stream(a.residual + (t * kStreams + r) * H + col) : u32x4{0, 0, 0, 0};
  if constexpr (kHeld > 0) {
#pragma unroll
    for (int r = 0; r < kHeld; ++r)
      part[r] = live ? load_stream(a.partials + r * a.rank_stride + t * H + col) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + u * nt, tk = e / 20, k = e % 20;
    if (e < kMixVals) {
      if (k < kStreams) sh.post[tk][k] = mv[u];
      else sh.comb[tk][k - kStreams] = mv[u];
    }
  }
  if constexpr (FIN) stage_tile_routes(a.fin, tp, t0, valid, routes);
  __syncthreads();

  // a1 + a2: rank sum, post-mix, residual_out; y to LDS.
  float sum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sum[e] = 0.0f;
  if constexpr (FIN && TP == 2) {
    // a6 then a1, two ranks' gathers in flight at a time (top_k <= 8): the
    // same contributions as finalize_fragment, added in rank order.
    const int per = tp * a.fin.top_k, K = a.fin.top_k;
    for (int r0 = 0; r0 < tp; r0 += 2) {
      if (!live) break;
      u32x4 rows[2][8], shv[2];
      bool ok[2][8];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int r = r0 + q, o = tok * per + r * K;
        const bool have = r < tp;
        const uint16_t *g = a.fin.gemm2 + r * a.fin.g_stride + col;
        shv[q] = have ? load_stream(a.fin.shared + r * a.fin.s_stride + t * H + col) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int32_t row = have && k < K ? routes.row[o + k] : -1;
          ok[q][k] = row >= 0 && row < a.fin.rows;
          rows[q][k] = ok[q][k] ? load_stream(g + (int64_t)row * H) : u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (r0 + q >= tp) break;
        const int o = tok * per + (r0 + q) * K;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (!ok[q][k]) continue;
          const float w = routes.w[o + k];
          float v[8];
          unpack8(rows[q][k], v);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(v[e], w, acc[e]);
        }
        float sv[8];
        unpack8(shv[q], sv);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] + sv[e];
        float v[8];
        unpack8(sanitize4(pack8(acc)), v);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[e] = sum[e] + v[e];
      }
    }
  } else if constexpr (FIN) {
    // a6 then a1: each rank's contribution (BF16, sanitized), added in rank
    // order.
    const int per = tp * a.fin.top_k;
    for (int r = 0; r < tp; ++r) {
      if (!live) break;
      const int o = tok * per + r * a.fin.top_k;
      float v[8];
      unpack8(finalize_fragment(a.fin, routes.row + o, routes.w + o, r, (int)t, H, col), v);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] = sum[e] + v[e];
    }
  } else if constexpr (kHeld > 0) {
#pragma unroll
    for (int r = 0; r < kHeld; ++r) {
      float v[8];
      unpack8(part[r], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] = sum[e] + v[e];
    }
  } else {
    const uint16_t *src = a.partials + t * H + col;
    for (int r0 = 0; r0 < tp; r0 += 8) {
      u32x4 w[8];
#pragma unroll
      for (int r = 0; r < 8; ++r)
        w[r] = live && r0 + r < tp ? load_stream(src + (r0 + r) * a.rank_stride) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if (r0 + r >= tp) break;
        float v[8];
        unpack8(w[r], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[e] = sum[e] + v[e];
      }
    }
  }
  float x[8];
  unpack8(pack8(sum), x);
  float r4[kStreams][8];
#pragma unroll
  for (int r = 0; r < kStreams; ++r) unpack8(res[r], r4[r]);
  const int tk = live ? tok : 0;
  double ysq = 0.0;
#pragma unroll
  for (int j = 0; j < kStreams; ++j) {
    const float pj = sh.post[tk][j];
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = x[e] * pj;
#pragma unroll
      for (int r = 0; r < kStreams; ++r) v = __builtin_fmaf(r4[r][e], sh.comb[tk][r * kStreams + j], v);
      acc[e] = v;
    }
    const u32x4 yj = live ? pack8(acc) : u32x4{0, 0, 0, 0};
    if (live) {
      // A plain store: the finish pass reads these rows back.
      *reinterpret_cast<u32x4 *>(a.residual_out + (t * kStreams + j) * H + col) = yj;
      ysq += (double)dot8(yj, yj, 0.0f);  // FP32 within the fragment
    }
    ys[tok * rw + j * sf + fl] = yj;
  }
  item[tid] = ysq;  // [tok][fl]
  __syncthreads();

  // a3 (partial): this wave's 4-fragment chunk of the 16 x 24 GEMV.
  {
    f32x4 c1 = {0.0f, 0.0f, 0.0f, 0.0f}, c2 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < kStreams; ++j) {
      const u32x4 av = ys[mi * rw + j * sf + 4 * wave + mq];
      c1 = mfma_bf16(av, fc.b1[j], c1);
      c2 = mfma_bf16(av, fc.b2[j], c2);
    }
    // Lane l holds rows l % 16 and 16 + l % 16 of tokens 4*(l/16) .. +3.
    float *wp = wpart + wave * kTile * kMix;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wp[(4 * mq + e) * kMix + mi] = c1[e];
      if (mi < kMix - kTile) wp[(4 * mq + e) * kMix + kTile + mi] = c2[e];
    }
  }
  __syncthreads();
  // The slice's partials: rows summed over the waves in order, the sum of
  // squares over the fragments in order.
  for (int e = tid; e < valid * kMix; e += nt) {
    const int tkn = e / kMix, k = e % kMix;
    float v = 0.0f;
    for (int w = 0; w < waves; ++w) v += wpart[(w * kTile + tkn) * kMix + k];
    a.parts[((int64_t)(t0 + tkn) * S + s) * kPartWords + k] = v;
  }
  if (tid < valid) {
    double v = 0.0;
    for (int q = 0; q < sf; ++q) v += item[tid * sf + q];
    *reinterpret_cast<double *>(a.parts + ((int64_t)(t0 + tid) * S + s) * kPartWords + kPartSum) = v;
  }
}

__global__ void __launch_bounds__(kMaxThreads)
glm_finish_kernel(const GlmArgs a) {
  __shared__ u32x4 staged[kGlmMaxParts * kPartWords / 4];  // the token's partials
  __shared__ float mix[kMix];
  __shared__ float pre[kStreams];
  __shared__ double tot;
  __shared__ double red[kMaxThreads / kWave];
  const int H = a.H, F = H / kFrag, tid = threadIdx.x, S = a.slices;
  const int64_t t = blockIdx.x;
  const bool valid = tid < F;
  const int64_t col = valid ? (int64_t)tid * kFrag : 0;  // in bounds for every thread
  // Every load is issued before the first wait: the token's residual_out
  // rows, gamma and the pre-mix's scale and bias (a thread past the last
  // fragment reads column 0 and leaves it unused), then its S x 128-byte
  // partials, staged through LDS.
  // (With the partials first, their LDS store waited for them before the
  // rows were even requested: two round trips in a row.)
  u32x4 y[kStreams];
#pragma unroll
  for (int j = 0; j < kStreams; ++j) y[j] = load_cached(a.residual_out + (t * kStreams + j) * H + col);
  const u32x4 gam = load_cached(a.gamma + col);
  const float scale0 = a.scale[0], base_j = a.base[tid < kStreams ? tid : 0];
  const u32x4 *pt = reinterpret_cast<const u32x4 *>(a.parts + t * S * kPartWords);
  for (int i = tid; i < S * (kPartWords / 4); i += blockDim.x) staged[i] = pt[i];
  __syncthreads();
  // Slice order: rows by threads 0..23, the binary64 sum by thread 24.
  const float *sp = reinterpret_cast<const float *>(staged);
  if (tid < kMix) {
    float v = 0.0f;
    for (int q = 0; q < S; ++q) v += sp[q * kPartWords + tid];
    mix[tid] = v;
  } else if (tid == kMix) {
    double v = 0.0;
    for (int q = 0; q < S; ++q) v += *reinterpret_cast<const double *>(sp + q * kPartWords + kPartSum);
    tot = v;
  }
  __syncthreads();
  // rstd over 4H; raw mixes out; pre_j = sigmoid(mix_j * scale0 + base_j) + hc_eps.
  if (tid < kMix) {
    const float rstd = (float)(1.0 / __builtin_sqrt((double)(float)tot / (4.0 * H) + (double)a.rms_eps));
    const float m = mix[tid] * rstd;
    a.mixes_out[t * kMix + tid] = m;
    if (tid < kStreams) pre[tid] = sigmoid(__builtin_fmaf(m, scale0, base_j)) + a.hc_eps;
  }
  __syncthreads();
  // a4: p = bf16((q0+q1)+(q2+q3)), q_j = y_j * pre_j; RMSNorm over H.
  float qv[kStreams][8];
#pragma unroll
  for (int j = 0; j < kStreams; ++j) {
    float yv[8];
    unpack8(y[j], yv);
    const float pj = pre[j];
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[j][e] = yv[e] * pj;
  }
  float z[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (qv[0][e] + qv[1][e]) + (qv[2][e] + qv[3][e]);
  const u32x4 p = pack8(z);
  double pss[1] = {0.0};
  float pv[8];
  unpack8(p, pv);
  if (valid) {
#pragma unroll
    for (int e = 0; e < 8; ++e) pss[0] += (double)pv[e] * (double)pv[e];
  }
  block_sum<double, 1>(pss, red);
  const float inv = (float)(1.0 / __builtin_sqrt((double)(float)pss[0] / (double)H + (double)a.norm_eps));
  float g[8], o[8];
  unpack8(gam, g);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (pv[e] * inv) * g[e];
  if (valid) store_stream(a.layer_input + t * H + col, pack8(o));
}

// ---------------------------------------------------------------------------
// Side-stream mixes: sixteen lanes per token.
// ---------------------------------------------------------------------------

// The pages' side kernel is compiled with fast math; here the reciprocal is
// the hardware's (v_rcp_f32, within 1 ulp) and exp the FP32 library one
// (within 1 ulp).  Twenty Sinkhorn rounds of binary64 divisions in one
// thread per token took about 7 us; errors of a few ulps stay far inside
// the side kernel's 1e-5 relative tolerance.
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float exp_fast(float x) { return expf(x); }
__device__ __forceinline__ float sigmoid_fast(float x) { return 1.0f / (1.0f + expf(-x)); }

// Sixteen lanes per token, lane e holding entry (e / 4, e % 4) of the 4x4
// residual mix (source row, target column).  A row's sum is two xor
// exchanges within its four lanes, a column's two exchanges at strides 4
// and 8; every lane of a row (column) then holds ((a + b) + (c + d)) in the
// page's pairing, the same bits on every lane because each addition is
// commutative.
constexpr int kMixLanes = 16;
constexpr int kMixThreads = 256;

__global__ void __launch_bounds__(kMixThreads)
mixes_kernel(const float *mixes, const float *scale, const float *base, float *post_out,
             float *comb_out, int M, float eps, float post_mult, int repeat) {
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int t = gid / kMixLanes, e = gid % kMixLanes;
  const bool live = t < M;                   // every lane takes part in the exchanges
  const float *row = mixes + (int64_t)(live ? t : M - 1) * kMix;
  if (live && e < kStreams)
    post_out[(int64_t)t * kStreams + e] =
        sigmoid_fast(__builtin_fmaf(row[kStreams + e], scale[1], base[kStreams + e])) * post_mult;

  // Sinkhorn on the 4x4 residual mix.
  float c = __builtin_fmaf(row[8 + e], scale[2], base[8 + e]);
  float peak = __builtin_fmaxf(c, row_xor<1>(c));
  peak = __builtin_fmaxf(peak, row_xor<2>(peak));
  c = exp_fast(c - peak);
  float sum = c + row_xor<1>(c);
  sum = sum + row_xor<2>(sum);
  c = __builtin_fmaf(c, rcp(sum), eps);
  for (int it = 0; it < repeat; ++it) {
    if (it > 0) {
      sum = c + row_xor<1>(c);
      sum = sum + row_xor<2>(sum);
      c = c * rcp(sum + eps);
    }
    sum = c + row_xor<4>(c);
    sum = sum + row_xor<8>(sum);
    c = c * rcp(sum + eps);
  }
  if (live) comb_out[(int64_t)t * 16 + e] = c;
}

}  // namespace

hipError_t launch_boundary_glm(const GlmArgs &a, hipStream_t stream) {
  const int F = a.slices > 1 ? a.slice_frags : a.H / kFrag;
  const int threads = (F + kWave - 1) / kWave * kWave;
  const int G = a.tokens_per_wg;
  const int groups = (a.M + G - 1) / G;
  dim3 grid = a.slices > 1 ? dim3(a.slices, groups) : dim3(groups), block(threads);
  switch (G) {
    case 1: hipLaunchKernelGGL((glm_kernel<1, 24, 1024>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((glm_kernel<2, 24, 1024>), grid, block, 0, stream, a); break;
    case 4:
      if (threads > kGlmWideThreads) return hipErrorInvalidValue;
      hipLaunchKernelGGL((glm_kernel<4, 12, kGlmWideThreads>), grid, block, 0, stream, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Tile geometry: 16 * slice_frags items, two or three per thread (at most
// 512 threads, four items); dynamic LDS sized by the slice.
hipError_t launch_boundary_glm_tile(const GlmArgs &a, hipStream_t stream) {
  const int sf = a.slice_frags;
  if (sf % 4 || sf > kTileMaxFrags || a.slices > kMaxSlices) return hipErrorInvalidValue;
  const int items = kTile * sf;
  // Two items per thread (up to 512 threads); three beyond that.  Every
  // rank load of every item is then issued before the first use (tp = 8).
  int threads = ((items + 1) / 2 + kWave - 1) / kWave * kWave;
  if (threads > kTileThreads) threads = ((items + 2) / 3 + kWave - 1) / kWave * kWave;
  threads = threads > kTileThreads ? kTileThreads : threads;
  const int U = (items + threads - 1) / threads;
  if (U > 4) return hipErrorInvalidValue;
  const dim3 grid(a.slices, (a.M + kTile - 1) / kTile), block(threads);
  const size_t lds = tile_dyn_bytes(sf);
  // Slices of more than 48 fragments take more than 64 KiB of LDS.
#define MHCB_TILE_LAUNCH(UU, TPP)                                                            \
  if (lds > 65536) {                                                                         \
    const hipError_t e = hipFuncSetAttribute((const void *)glm_tile_kernel<UU, TPP>,          \
                                             hipFuncAttributeMaxDynamicSharedMemorySize,      \
                                             (int)lds);                                      \
    if (e != hipSuccess) return e;                                                           \
  }                                                                                          \
  hipLaunchKernelGGL((glm_tile_kernel<UU, TPP>), grid, block, lds, stream, a);
#define MHCB_TILE(UU)                                                                        \
  if (a.tp == 8) {                                                                           \
    MHCB_TILE_LAUNCH(UU, 8)                                                                  \
  } else {                                                                                   \
    MHCB_TILE_LAUNCH(UU, 0)                                                                  \
  }
  switch (U) {
    case 1: MHCB_TILE(1) break;
    case 2: MHCB_TILE(2) break;
    case 3: MHCB_TILE(3) break;
    default: MHCB_TILE_LAUNCH(4, 0) break;  // four items of eight held ranks would spill
  }
#undef MHCB_TILE
#undef MHCB_TILE_LAUNCH
  return hipGetLastError();
}

// Two passes: 16 * sf threads per stream workgroup (sf a multiple of 4,
// 16..64), then one workgroup per token.
hipError_t launch_boundary_glm_two_pass(const GlmArgs &a, hipStream_t stream) {
  const int sf = a.slice_frags, F = a.H / kFrag;
  if (sf % 4 || sf < 16 || kTile * sf > kStreamMaxThreads || a.slices > kGlmMaxParts ||
      (int64_t)a.slices * sf < F || a.H > kFrag * kMaxThreads)
    return hipErrorInvalidValue;
  const dim3 grid(a.slices, (a.M + kTile - 1) / kTile), block(kTile * sf);
  const size_t lds = stream_dyn_bytes(sf);
#define MHCB_STREAM_LAUNCH(TPP, FINN)                                                        \
  if (lds > 65536) {                                                                         \
    const hipError_t e = hipFuncSetAttribute((const void *)glm_stream_kernel<TPP, FINN>,      \
                                             hipFuncAttributeMaxDynamicSharedMemorySize,      \
                                             (int)lds);                                      \
    if (e != hipSuccess) return e;                                                           \
  }                                                                                          \
  hipLaunchKernelGGL((glm_stream_kernel<TPP, FINN>), grid, block, lds, stream, a);
  if (a.fin.gemm2) {
    if (a.tp * a.fin.top_k > kGlmTileRoutes) return hipErrorInvalidValue;
    if (a.tp > 1 && a.fin.top_k <= 8 && kTile * sf <= kStreamPairThreads) {
      MHCB_STREAM_LAUNCH(2, true)
    } else {
      MHCB_STREAM_LAUNCH(0, true)
    }
  } else if (a.tp == 8) {
    MHCB_STREAM_LAUNCH(8, false)
  } else if (a.tp == 4) {
    MHCB_STREAM_LAUNCH(4, false)
  } else {
    MHCB_STREAM_LAUNCH(0, false)
  }
#undef MHCB_STREAM_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int threads = (F + kWave - 1) / kWave * kWave;
  hipLaunchKernelGGL(glm_finish_kernel, dim3(a.M), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_mixes(const float *mixes, const float *scale, const float *base, float *post_out,
                        float *comb_out, int M, float hc_eps, float post_mult, int repeat,
                        hipStream_t stream) {
  const int64_t threads = (int64_t)M * kMixLanes;
  hipLaunchKernelGGL(mixes_kernel, dim3((unsigned)((threads + kMixThreads - 1) / kMixThreads)),
                     dim3(kMixThreads), 0, stream, mixes, scale, base, post_out, comb_out, M,
                     hc_eps, post_mult, repeat);
  return hipGetLastError();
}

}  // namespace mhcb
