// Per-token sublayer-boundary kernels for gfx950: TP partial sum, mHC
// post-mix, pre-mix collapse, RMSNorm and the optional MXFP8 epilogue, fed
// from resident partials, from a Lamport mailbox, or from an unfinalized MoE
// output.  Also the mailbox producer / initializer, the two-shot owner
// reduce and the standalone MXFP8 quantizer.
//
// Arithmetic follows the pages
//   vllm.models.deepseek_v41.nvidia.ops.cute_dsl.all_reduce_mhc
//     (_LamportMHCDeviceKernel.kernel, _QuadFinalizePublishDeviceKernel.kernel,
//      _OwnerReduceMulticastDeviceKernel.kernel, _SharedOnlyPublishDeviceKernel.kernel)
//   vllm.models.glm5next.nvidia.specialized_decode.all_reduce_mhc
//     (AllReduceMhcBoundary.__init__, _PublishDeviceKernel.kernel)
// step for step: the rank sum starts at 0 and adds ranks in order; the
// post-mix is x*post_j followed by four FMAs over the source streams; the
// collapse is an FMA chain from 0 over the targets; RMSNorm multiplies
// (p * inv) * gamma.  The design is gfx950's own: one workgroup per token,
// 16-byte coalesced loads of consecutive fragments per lane, wave64
// butterflies plus an LDS step for the sum of squares (no clusters), every
// load of a token issued before its first use.
#include <type_traits>

#include "device.h"
#include "kernels.h"
#include "sync.h"
#include "finalize.h"

namespace mhcb {

// A workgroup covering `frags` fragments: 1, 2 or 4 fragments per thread,
// at most kTokenThreads threads (frags <= 2048, i.e. hidden <= 16384), or
// one fragment per thread up to `wide_threads` threads.  A token's VALU work
// is then spread over more waves: at H=5120 ten one-fragment waves put at
// most three fragments' work on a SIMD, five two-fragment waves four.
Geometry fragment_geometry(int frags, int wide_threads) {
  Geometry g;
  if (frags <= wide_threads) {
    g.trips = 1;
    g.threads = (frags + kWave - 1) / kWave * kWave;
    return g;
  }
  g.trips = frags <= kTokenThreads ? 1 : (frags <= 2 * kTokenThreads ? 2 : 4);
  const int per = (frags + g.trips - 1) / g.trips;
  g.threads = (per + kWave - 1) / kWave * kWave;
  return g;
}

namespace {

constexpr int kMaxRoutes = 1024;  // tp * top_k staged per workgroup

// A token's mixes for HC streams (post [HC], comb [HC][HC] source-major,
// pre [HC]).
template <int HC>
struct Mixes {
  float post[HC], comb[HC * HC], pre[HC];
};

template <int HC>
__device__ __forceinline__ void load_mixes(const BoundaryArgs &a, int t, Mixes<HC> &m) {
#pragma unroll
  for (int j = 0; j < HC; ++j) m.post[j] = a.post[t * HC + j];
#pragma unroll
  for (int i = 0; i < HC * HC; ++i) m.comb[i] = a.comb[t * HC * HC + i];
#pragma unroll
  for (int j = 0; j < HC; ++j) m.pre[j] = a.pre ? a.pre[t * HC + j] : 0.0f;
}

// Adds one rank's fragment to the running FP32 sum (rank order).
__device__ __forceinline__ void accumulate(float (&s)[8], u32x4 w) {
  float v[8];
  unpack8(w, v);
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = s[e] + v[e];
}

__device__ __forceinline__ bool fragment_has_sentinel(u32x4 w) {
  return has_sentinel(w[0]) || has_sentinel(w[1]) || has_sentinel(w[2]) || has_sentinel(w[3]);
}

// Waits until no element of a mailbox fragment is the sentinel, re-reading
// it at device scope at most spin_limit times.  A fragment still not all
// there then reads as BF16 NaN, so the token's results come out NaN rather
// than wrong, and the time-out is counted in status[0].  With `count`, a
// fragment that had to be re-read is counted in status[1].
__device__ __forceinline__ u32x4 poll(const uint16_t *p, u32x4 w, const MailboxView &mb,
                                      bool count) {
  if (!fragment_has_sentinel(w)) return w;
  if (count) atomicAdd(mb.status + 1, 1);
  int64_t spins = 0;
  do {
    if (++spins > mb.spin_limit) {
      atomicAdd(mb.status, 1);
      return u32x4{kPoisonBf16x2, kPoisonBf16x2, kPoisonBf16x2, kPoisonBf16x2};
    }
    __builtin_amdgcn_s_sleep(1);
    w = load_agent(p);
  } while (fragment_has_sentinel(w));
  return w;
}

// finalize_fragment for a compile-time rank count and top_k <= 8: every
// expert row of every rank is loaded before the first multiply, so the
// token waits for one round of gathers instead of one per rank.  `shared`
// holds the ranks' shared-expert fragments, loaded earlier.
template <int TP>
__device__ __forceinline__ void finalize_fixed(const FinalizeView &f, const int32_t *srow,
                                               const float *sw, const u32x4 (&shared)[TP], int H,
                                               int64_t col, float (&sum)[8]) {
  u32x4 rows[TP][8];
  bool ok[TP][8];
#pragma unroll
  for (int r = 0; r < TP; ++r) {
    const uint16_t *g = f.gemm2 + r * f.g_stride + col;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int32_t row = k < f.top_k ? srow[r * f.top_k + k] : -1;
      ok[r][k] = row >= 0 && row < f.rows;
      rows[r][k] = ok[r][k] ? load_stream(g + (int64_t)row * H) : u32x4{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int r = 0; r < TP; ++r) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (!ok[r][k]) continue;
      const float w = sw[r * f.top_k + k];
      float v[8];
      unpack8(rows[r][k], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(v[e], w, acc[e]);
    }
    float sh[8];
    unpack8(shared[r], sh);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] + sh[e];
    accumulate(sum, sanitize4(pack8(acc)));
  }
}

// Stages every rank's (row, weight) routes of token t in LDS
// (_QuadFinalizePublishDeviceKernel.kernel): the weight is read as FP32 or
// widened from BF16, multiplied by the routed scaling factor when that is
// not 1, and a route whose row is -1 gets weight 0 (it is skipped anyway).
__device__ __forceinline__ void stage_routes(const FinalizeView &f, int tp, int t, int32_t *srow,
                                             float *sw) {
  const int n = tp * f.top_k;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int r = i / f.top_k, k = i % f.top_k;
    const int64_t e = r * f.w_stride + (int64_t)t * f.top_k + k;
    const int32_t row = f.idx[r * f.i_stride + (int64_t)t * f.top_k + k];
    // (not behind the index load)
    float w = f.w_bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t *>(f.weights)[e] << 16)
                       : static_cast<const float *>(f.weights)[e];
    if (f.w_scale != 1.0f) w = w * f.w_scale;
    srow[i] = row;
    sw[i] = row == -1 ? 0.0f : w;
  }
  __syncthreads();
}

// The token's RMSNorm factor inv = (float)(1/sqrt((double)(float)ss/H +
// eps)) from each thread's binary64 sum of squares: wave xor sums, then one
// wave adds the waves in index order (and, split, publishes its slice's
// partial, adds the slices' in slice order and advances the slot's epoch:
// each square of a BF16 value is exact in binary64, and the sums round near
// 2^-53 relative, far below the binary32 rounding of inv, so the split does
// not show in the bits in practice), one thread evaluates inv and shares it
// through LDS.
// `callw` is the slot's epoch word (wave 0's).  Every thread calls it.
__device__ float token_inv(const BoundaryArgs &a, int t, int s, double ss, double *red,
                           uint64_t callw) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  if (wave == 0) {
    double total = 0.0;
    for (int w = 0; w < (int)blockDim.x / kWave; ++w) total += red[w];
    if (a.slices > 1) {
      char *slot = token_slot(a.sync, t);
      const SlotCall c = unpack_call(callw);
      if (lane == 0 && !c.broken) slot_store64(slot + copy_offset(c.epoch), kCopySum1 + 8 * s, total);
      total = wave_gather_sum64(a.sync, slot, c, kCopySum1, a.slices);  // NaN if broken
      if (lane == 0) advance_epoch(slot, c, a.slices);  // after this slice's last read
    }
    if (lane == 0)
      red[kTokenThreadsWide / kWave] =
          (double)(float)(1.0 / __builtin_sqrt((double)(float)total / (double)a.H + (double)a.norm_eps));
  }
  __syncthreads();
  return (float)red[kTokenThreadsWide / kWave];
}

// The fused boundary.  Workgroup (s, t) covers fragments
// [s * slice_frags, (s + 1) * slice_frags) of token t (all of them when
// slices == 1).  TP > 0 fixes the rank count at compile time so that every
// rank load of every trip is issued up front; TP == 0 reads it from the
// arguments.
// Threads of a one-fragment-per-thread workgroup (0: none; at most
// kTokenThreads then): eight streams hold twice the registers, and their
// mailbox variant's poll path does not fit 768 threads' registers.
template <Source SRC, int HC>
constexpr int wide_threads() {
  return HC <= kStreams ? kTokenThreadsWide : SRC == Source::kMailbox ? 0 : kTokenThreadsWide8;
}

template <int TRIPS, int TP, Source SRC, int HC>
__global__ void __launch_bounds__((TRIPS > 1 || (SRC == Source::kFinalize && TP > 0) ||
                                           wide_threads<SRC, HC>() == 0
                                       ? kTokenThreads
                                       : wide_threads<SRC, HC>()))
boundary_kernel(const BoundaryArgs a) {
  __shared__ double red[kTokenThreadsWide / kWave + 1];
  __shared__ int32_t srow[SRC == Source::kFinalize ? kMaxRoutes : 1];
  __shared__ float sw[SRC == Source::kFinalize ? kMaxRoutes : 1];

  // Split: grid (slices, M), a token's slices consecutive in dispatch order
  // (so the workgroups a wait depends on are never queued behind it).
  // Unsplit: grid (M).
  const int s = a.slices > 1 ? blockIdx.x : 0, t = a.slices > 1 ? blockIdx.y : blockIdx.x;
  const int H = a.H, F = H / kFrag, nt = blockDim.x;
  const int tid = threadIdx.x;
  const int tp = TP > 0 ? TP : a.tp;
  const bool norm = a.pre != nullptr;
  const int first = a.slices > 1 ? s * a.slice_frags : 0;
  const int last = a.slices > 1 ? min(F, first + a.slice_frags) : F;

  // Sources of the contributions.
  const uint16_t *src = nullptr;
  int64_t rs = 0;
  uint32_t gen = 0;
  if constexpr (SRC == Source::kPartials) {
    src = a.partials + (int64_t)t * H;
    rs = a.rank_stride;
  } else if constexpr (SRC == Source::kMailbox) {
    gen = (uint32_t)__hip_atomic_load(a.mailbox.stage_state, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) % 3u;  // stays inside the slots
    rs = (int64_t)a.mailbox.capacity * H;
    src = a.mailbox.slots + (int64_t)gen * tp * rs + (int64_t)t * H;
  }

  int64_t col[TRIPS];
  bool valid[TRIPS];
#pragma unroll
  for (int i = 0; i < TRIPS; ++i) {
    const int f = first + tid + i * nt;
    valid[i] = f < last;
    col[i] = valid[i] ? (int64_t)f * kFrag : 0;
  }

  // Issue the streamed loads first: residual streams, gamma, and (fixed tp)
  // the partials, for every trip.
  u32x4 res[TRIPS][HC], gam[TRIPS];
  constexpr int kHeld = TP > 0 ? TP : 1;
  u32x4 part[TRIPS][kHeld];
#pragma unroll
  for (int i = 0; i < TRIPS; ++i) {
    if constexpr (TP > 0 && SRC == Source::kFinalize) {
#pragma unroll
      for (int r = 0; r < TP; ++r)
        part[i][r] = load_stream(a.fin.shared + r * a.fin.s_stride + (int64_t)t * H + col[i]);
    } else if constexpr (TP > 0) {
#pragma unroll
      // Mailbox: a plain streaming read first; a fragment still holding the
      // sentinel is re-read at device scope by poll().  (In stream order the
      // producer's kernel boundary has already made its stores visible.)
      for (int r = 0; r < TP; ++r) part[i][r] = load_stream(src + r * rs + col[i]);
    }
#pragma unroll
    for (int q = 0; q < HC; ++q)
      res[i][q] = load_stream(a.residual + ((int64_t)t * HC + q) * H + col[i]);
    gam[i] = norm ? load_cached(a.gamma + col[i]) : u32x4{0, 0, 0, 0};
  }
  // Finalize: the routes are staged while those loads are in flight (the
  // workgroup barrier inside waits for LDS only).
  if constexpr (SRC == Source::kFinalize) stage_routes(a.fin, tp, t, srow, sw);
  // The token's mixes are scalar loads; keep them behind the vector loads so
  // that waiting for them does not delay the stream.
  __builtin_amdgcn_sched_barrier(0);
  Mixes<HC> m;
  load_mixes<HC>(a, t, m);
  // Split: the token slot's epoch word, read by wave 0 (its latency hides
  // behind the loads above).
  uint64_t callw = 0;
  if (a.slices > 1 && norm && tid < kWave) callw = slot_call_word(token_slot(a.sync, t));

  u32x4 pfrag[TRIPS];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < TRIPS; ++i) {
    // a1: s = ((0 + c_0) + c_1) + ... ; xr = bf16(s).
    float sum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] = 0.0f;
    if (valid[i]) {
      if constexpr (SRC == Source::kFinalize && TP > 0) {
        finalize_fixed<TP>(a.fin, srow, sw, part[i], H, col[i], sum);
      } else if constexpr (SRC == Source::kFinalize) {
        for (int r = 0; r < tp; ++r)
          accumulate(sum, finalize_fragment(a.fin, srow + r * a.fin.top_k, sw + r * a.fin.top_k, r,
                                            t, H, col[i]));
      } else if constexpr (TP > 0) {
        if constexpr (SRC == Source::kMailbox) {
          // Slow path only for fragments that are not all there yet; a wave
          // counts its late fragments with one atomic.
          bool dirty = false;
          int late = 0;  // the wave's late fragments (ballots: uniform over the active lanes)
#pragma unroll
          for (int r = 0; r < TP; ++r) {
            const bool d = fragment_has_sentinel(part[i][r]);
            dirty |= d;
            late += __popcll(__ballot(d));
          }
          if (late) {
            const uint64_t act = __ballot(true);
            if ((tid & (kWave - 1)) == __builtin_ctzll(act)) atomicAdd(a.mailbox.status + 1, late);
            if (dirty)
              for (int r = 0; r < TP; ++r)
                part[i][r] = poll(src + r * rs + col[i], part[i][r], a.mailbox, false);
          }
        }
#pragma unroll
        for (int r = 0; r < TP; ++r) accumulate(sum, part[i][r]);
      } else {
        for (int r = 0; r < tp; ++r) {
          const uint16_t *p = src + r * rs + col[i];
          u32x4 w = load_stream(p);
          if constexpr (SRC == Source::kMailbox) w = poll(p, w, a.mailbox, true);
          accumulate(sum, w);
        }
      }
    }
    float x[8];
    unpack8(pack8(sum), x);

    // a2: y_j = bf16(x * post_j (+) sum_s res_s * comb[s][j]), s ascending.
    float r4[HC][8];
#pragma unroll
    for (int q = 0; q < HC; ++q) unpack8(res[i][q], r4[q]);
    float y[HC][8];
#pragma unroll
    for (int j = 0; j < HC; ++j) {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = x[e] * m.post[j];
#pragma unroll
        for (int q = 0; q < HC; ++q) v = __builtin_fmaf(r4[q][e], m.comb[q * HC + j], v);
        acc[e] = v;
      }
      const u32x4 packed = pack8(acc);
      if (valid[i]) store_stream(a.residual_out + ((int64_t)t * HC + j) * H + col[i], packed);
      unpack8(packed, y[j]);
    }

    // a4 (first half): p = bf16(0 (+) y_0*pre_0 (+) ... (+) y_3*pre_3).
    float z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = 0.0f;
#pragma unroll
      for (int j = 0; j < HC; ++j) v = __builtin_fmaf(y[j][e], m.pre[j], v);
      z[e] = v;
    }
    pfrag[i] = pack8(z);
    if (valid[i] && norm) {
      float p[8];
      unpack8(pfrag[i], p);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += (double)p[e] * (double)p[e];
    }
  }

  // Mailbox: advance the generation and return the consumed slots to the
  // sentinel (the next publish of this generation is two calls away).
  if constexpr (SRC == Source::kMailbox) {
    if (t == 0 && s == 0 && tid == 0) a.mailbox.stage_state[1] = (int32_t)((gen + 1) % 3);
    const u32x4 empty = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
#pragma unroll
    for (int i = 0; i < TRIPS; ++i)
      if (valid[i])
        for (int r = 0; r < tp; ++r) store_stream(const_cast<uint16_t *>(src) + r * rs + col[i], empty);
  }

  if (!norm) return;  // residual-only variant: uniform over the grid

  // a4 (second half): inv = 1/sqrt(sum p^2 / H + eps); out = bf16((p*inv)*gamma).
  // Each square of a BF16 value is exact in binary64; the binary64 sums
  // round near 2^-53 relative, far below the binary32 rounding of inv.
  const float inv = token_inv(a, t, s, ss, red, callw);
  if (a.slices > 1 && tid < kWave)
    for (int w = tid * a.slices + s; w < kClearWords; w += kWave * a.slices)
      clear_previous_word(token_slot(a.sync, t), unpack_call(callw), w);

#pragma unroll
  for (int i = 0; i < TRIPS; ++i) {
    float p[8], g[8], o[8];
    unpack8(pfrag[i], p);
    unpack8(gam[i], g);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (p[e] * inv) * g[e];
    const u32x4 out = pack8(o);
    if (valid[i]) store_stream(a.layer_input + (int64_t)t * H + col[i], out);

    if (a.mx_values) {
      // a8: the block of 32 columns is the fragments of lanes 4q .. 4q+3.
      float ov[8];
      unpack8(out, ov);
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(ov[e]));
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, kWave));
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2, kWave));
      const uint32_t e8 = ue8m0_round_up(amax * (1.0f / 448.0f));
      const float sc = ue8m0_inverse(e8);
      u32x2 codes = {0, 0};
#pragma unroll
      for (int e = 0; e < 8; ++e) codes[e >> 2] |= e4m3_rne_sat(ov[e] * sc) << (8 * (e & 3));
      if (valid[i]) {
        store8(a.mx_values + (int64_t)t * H + col[i], codes);
        const int f = first + tid + i * nt;
        if ((f & 3) == 0) a.mx_scales[sf_offset(t, f >> 2, H / 32)] = (uint8_t)e8;
      }
    }
  }

  if (a.mx_values) {
    // Zero the scales of the padding rows M .. ceil(M/128)*128 - 1, one
    // 4-column word per store, spread over the grid.
    const int K = H / 32, words_per_row = K / 4;
    const int64_t padded = ((int64_t)a.M + 127) / 128 * 128;
    const int64_t words = (padded - a.M) * words_per_row;
    const int64_t wg = (int64_t)t * a.slices + s, wgs = (int64_t)a.M * a.slices;
    for (int64_t w = wg * nt + tid; w < words; w += wgs * nt) {
      const int64_t row = a.M + w / words_per_row;
      const int k = (int)(w % words_per_row) * 4;
      *reinterpret_cast<uint32_t *>(a.mx_scales + sf_offset(row, k, K)) = 0u;
    }
  }
}

// A chunk of a token row: a 16-byte fragment (E = 8 BF16 values) or half
// of one (E = 4).
template <int E>
struct Chunk {
  using W = std::conditional_t<E == 8, u32x4, u32x2>;
  static __device__ __forceinline__ W load(const uint16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const W *>(p));
  }
  static __device__ __forceinline__ W load_cached(const uint16_t *p) {
    return *reinterpret_cast<const W *>(p);
  }
  static __device__ __forceinline__ void store(uint16_t *p, W w) {
    __builtin_nontemporal_store(w, reinterpret_cast<W *>(p));
  }
  static __device__ __forceinline__ void unpack(W w, float (&f)[E]) {
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
      f[2 * i] = lo_bf16(w[i]);
      f[2 * i + 1] = hi_bf16(w[i]);
    }
  }
  static __device__ __forceinline__ W pack(const float (&f)[E]) {
    W w;
#pragma unroll
    for (int i = 0; i < E / 2; ++i) w[i] = pack_bf16(f[2 * i], f[2 * i + 1]);
    return w;
  }
  static __device__ __forceinline__ W filled(uint32_t v) {
    W w;
#pragma unroll
    for (int i = 0; i < E / 2; ++i) w[i] = v;
    return w;
  }
  static __device__ __forceinline__ bool sentinel(W w) {
    bool any = false;
#pragma unroll
    for (int i = 0; i < E / 2; ++i) any |= has_sentinel(w[i]);
    return any;
  }
  // A mailbox chunk read at device scope (8-byte atomic loads).
  static __device__ __forceinline__ W load_agent(const uint16_t *p) {
    if constexpr (E == 8) {
      return mhcb::load_agent(p);
    } else {
      const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      return W{(uint32_t)v, (uint32_t)(v >> 32)};
    }
  }
};

// poll() for a chunk: re-read at device scope, at most spin_limit times,
// until no element is the sentinel; a chunk still not all there reads as
// NaN and the time-out is counted in status[0].
template <int E>
__device__ __forceinline__ typename Chunk<E>::W poll_chunk(const uint16_t *p,
                                                           typename Chunk<E>::W w,
                                                           const MailboxView &mb) {
  int64_t spins = 0;
  while (Chunk<E>::sentinel(w)) {
    if (++spins > mb.spin_limit) {
      atomicAdd(mb.status, 1);
      return Chunk<E>::filled(kPoisonBf16x2);
    }
    __builtin_amdgcn_s_sleep(1);
    w = Chunk<E>::load_agent(p);
  }
  return w;
}

// The mailbox consumer's check of one chunk of every rank: a wave counts
// its late chunks with one atomic (status[1]), and a lane with a late
// chunk re-reads it (poll_chunk).  Called by whole waves.
template <int E, int TP>
__device__ __forceinline__ void settle_chunk(typename Chunk<E>::W (&part)[TP], const uint16_t *src,
                                             int64_t rs, const MailboxView &mb) {
  bool dirty = false;
  int late = 0;  // ballots: uniform over the wave
#pragma unroll
  for (int r = 0; r < TP; ++r) {
    const bool d = Chunk<E>::sentinel(part[r]);
    dirty |= d;
    late += __popcll(__ballot(d));
  }
  if (late) {
    const uint64_t act = __ballot(true);
    if ((threadIdx.x & (kWave - 1)) == __builtin_ctzll(act)) atomicAdd(mb.status + 1, late);
    if (dirty)
      for (int r = 0; r < TP; ++r) part[r] = poll_chunk<E>(src + r * rs, part[r], mb);
  }
}

// a1 for one chunk: the ranks' BF16 contributions added from 0 in rank
// order.
template <int E, int TP>
__device__ __forceinline__ void rank_sum_chunk(const typename Chunk<E>::W (&part)[TP], float (&sum)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e) sum[e] = 0.0f;
#pragma unroll
  for (int r = 0; r < TP; ++r) {
    float v[E];
    Chunk<E>::unpack(part[r], v);
#pragma unroll
    for (int e = 0; e < E; ++e) sum[e] = sum[e] + v[e];
  }
}

// The rest of one chunk of the balanced kernel below, the same steps as
// boundary_kernel: xr = bf16(rank sum), a2 post-mix (stores residual_out),
// a4 collapse; returns the BF16 collapse and adds its squares to ss.
template <int E>
__device__ __forceinline__ typename Chunk<E>::W
balanced_chunk(const float (&sum)[E], const typename Chunk<E>::W (&res)[kStreams],
               const Mixes<kStreams> &m, uint16_t *out, int64_t H, double &ss) {
  using C = Chunk<E>;
  float x[E];
  C::unpack(C::pack(sum), x);
  float r4[kStreams][E], y[kStreams][E];
#pragma unroll
  for (int q = 0; q < kStreams; ++q) C::unpack(res[q], r4[q]);
#pragma unroll
  for (int j = 0; j < kStreams; ++j) {
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float v = x[e] * m.post[j];
#pragma unroll
      for (int q = 0; q < kStreams; ++q) v = __builtin_fmaf(r4[q][e], m.comb[q * kStreams + j], v);
      acc[e] = v;
    }
    const typename C::W packed = C::pack(acc);
    C::store(out + j * H, packed);
    C::unpack(packed, y[j]);
  }
  float z[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float v = 0.0f;
#pragma unroll
    for (int j = 0; j < kStreams; ++j) v = __builtin_fmaf(y[j][e], m.pre[j], v);
    z[e] = v;
  }
  const typename C::W pz = C::pack(z);
  float p[E];
  C::unpack(pz, p);
#pragma unroll
  for (int e = 0; e < E; ++e) ss += (double)p[e] * (double)p[e];
  return pz;
}

// One rank's MoE finalize contributions (as finalize_fragment: acc = 0,
// fma(row_k, w_k, acc) for the valid routes k ascending, + shared, BF16,
// negative zero -> +0) to a thread's FF full fragments (columns
// 8 (tid + NT c)) and, with `half`, its half fragment at column hcol, each
// added to its rank sum.  Every gather of a block of eight routes is
// issued before the first product.
template <int FF, int NT>
__device__ __forceinline__ void finalize_rank(const FinalizeView &f, const int32_t *srow,
                                              const float *sw, int r, int64_t t, int64_t H,
                                              int tid, int64_t hcol, bool half,
                                              float (&sf)[FF > 0 ? FF : 1][8], float (&sh)[4]) {
  const uint16_t *g = f.gemm2 + r * f.g_stride;
  const uint16_t *shared = f.shared + r * f.s_stride + t * H;
  float af[FF > 0 ? FF : 1][8], ah[4];
  u32x4 shf[FF > 0 ? FF : 1];
  u32x2 shh = {0, 0};
#pragma unroll
  for (int c = 0; c < FF; ++c) {
    shf[c] = Chunk<8>::load(shared + (int64_t)(tid + NT * c) * kFrag);
#pragma unroll
    for (int e = 0; e < 8; ++e) af[c][e] = 0.0f;
  }
  if (half) shh = Chunk<4>::load(shared + hcol);
#pragma unroll
  for (int e = 0; e < 4; ++e) ah[e] = 0.0f;
  for (int k0 = 0; k0 < f.top_k; k0 += 8) {
    u32x4 rf[FF > 0 ? FF : 1][8];
    u32x2 rh[8];
    bool ok[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + i;
      const int32_t row = k < f.top_k ? srow[r * f.top_k + k] : -1;
      ok[i] = row >= 0 && row < f.rows;
      const uint16_t *rp = g + (int64_t)(ok[i] ? row : 0) * H;
#pragma unroll
      for (int c = 0; c < FF; ++c)
        rf[c][i] = ok[i] ? Chunk<8>::load(rp + (int64_t)(tid + NT * c) * kFrag) : u32x4{0, 0, 0, 0};
      rh[i] = ok[i] && half ? Chunk<4>::load(rp + hcol) : u32x2{0, 0};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (!ok[i]) continue;
      const float w = sw[r * f.top_k + k0 + i];
#pragma unroll
      for (int c = 0; c < FF; ++c) {
        float v[8];
        Chunk<8>::unpack(rf[c][i], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) af[c][e] = __builtin_fmaf(v[e], w, af[c][e]);
      }
    }
    if (half) {  // (uniform over each wave: the waves without one skip it)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (!ok[i]) continue;
        const float w = sw[r * f.top_k + k0 + i];
        float v[4];
        Chunk<4>::unpack(rh[i], v);
#pragma unroll
        for (int e = 0; e < 4; ++e) ah[e] = __builtin_fmaf(v[e], w, ah[e]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < FF; ++c) {
    float s[8];
    Chunk<8>::unpack(shf[c], s);
#pragma unroll
    for (int e = 0; e < 8; ++e) af[c][e] = af[c][e] + s[e];
    float v[8];
    Chunk<8>::unpack(sanitize4(Chunk<8>::pack(af[c])), v);
#pragma unroll
    for (int e = 0; e < 8; ++e) sf[c][e] = sf[c][e] + v[e];
  }
  if (half) {
    float s[4];
    Chunk<4>::unpack(shh, s);
#pragma unroll
    for (int e = 0; e < 4; ++e) ah[e] = ah[e] + s[e];
    u32x2 w = Chunk<4>::pack(ah);
    w[0] = sanitize_word(w[0]);
    w[1] = sanitize_word(w[1]);
    float v[4];
    Chunk<4>::unpack(w, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) sh[e] = sh[e] + v[e];
  }
}

// The delayed boundary for an unsplit token whose fragment count is
// NT * FF + 128 (H = 5120: FF = 2 with NT = 256 threads, FF = 1 with 512),
// from 8 ranks' resident partials or the ACTIVE generation of a mailbox,
// or from the MoE finalize contributions of any rank count (computed a
// rank at a time), four streams and a layer input (optionally with the
// MXFP8 epilogue).  boundary_kernel would give such a
// token 4 FF + 2 one-fragment waves (NT = 256), and the SIMD that gets the
// extra waves sets the VALU time.  Here every thread takes FF fragments
// and the first 256 threads one half-fragment each (the last 128
// fragments), so each SIMD carries the same work: FF + 1/2 fragments in one
// wave (NT = 256), or FF fragments in each of two waves and a half in one
// (NT = 512).  Same arithmetic per element, same results.
template <int FF, int NT, Source SRC>
__global__ void __launch_bounds__(NT) boundary_balanced_kernel(const BoundaryArgs a) {
  constexpr bool kFin = SRC == Source::kFinalize;
  constexpr int TP = kFin ? 1 : 8;  // ranks held in registers
  static_assert(NT == 256 || NT == 512, "four or eight waves");
  __shared__ double red[kTokenThreadsWide / kWave + 1];
  __shared__ int32_t srow[kFin ? kMaxRoutes : 1];
  __shared__ float sw[kFin ? kMaxRoutes : 1];
  const int t = blockIdx.x, tid = threadIdx.x;
  const bool half = NT == 256 || tid < 256;  // uniform over each wave
  const int H = a.H;
  const uint16_t *src = nullptr;
  int64_t rs = 0;
  uint32_t gen = 0;
  if constexpr (SRC == Source::kMailbox) {
    gen = (uint32_t)__hip_atomic_load(a.mailbox.stage_state, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) % 3u;  // stays inside the slots
    rs = (int64_t)a.mailbox.capacity * H;
    src = a.mailbox.slots + (int64_t)gen * TP * rs + (int64_t)t * H;
  } else if constexpr (SRC == Source::kPartials) {
    rs = a.rank_stride;
    src = a.partials + (int64_t)t * H;
  }
  const uint16_t *res_row = a.residual + (int64_t)t * kStreams * H;
  uint16_t *out_row = a.residual_out + (int64_t)t * kStreams * H;

  // Every load first: FF full fragments (columns 8 (tid + NT c)), then the
  // half fragment at column 8 NT FF + 4 tid.
  u32x4 pf[FF > 0 ? FF : 1][TP], rf[FF > 0 ? FF : 1][kStreams], gf[FF > 0 ? FF : 1];
  u32x2 ph[TP], rh[kStreams], gh = {0, 0};
#pragma unroll
  for (int c = 0; c < FF; ++c) {
    const int64_t col = (int64_t)(tid + NT * c) * kFrag;
    if constexpr (!kFin) {
#pragma unroll
      for (int r = 0; r < TP; ++r) pf[c][r] = Chunk<8>::load(src + r * rs + col);
    }
#pragma unroll
    for (int q = 0; q < kStreams; ++q) rf[c][q] = Chunk<8>::load(res_row + q * H + col);
    gf[c] = Chunk<8>::load_cached(a.gamma + col);
  }
  const int64_t hcol = (int64_t)FF * NT * kFrag + 4 * (tid & 255);
  if (half) {
    if constexpr (!kFin) {
#pragma unroll
      for (int r = 0; r < TP; ++r) ph[r] = Chunk<4>::load(src + r * rs + hcol);
    }
#pragma unroll
    for (int q = 0; q < kStreams; ++q) rh[q] = Chunk<4>::load(res_row + q * H + hcol);
    gh = Chunk<4>::load_cached(a.gamma + hcol);
  }
  // Finalize: the routes are staged while those loads are in flight.
  if constexpr (kFin) stage_routes(a.fin, a.tp, t, srow, sw);
  __builtin_amdgcn_sched_barrier(0);
  Mixes<kStreams> m;
  load_mixes<kStreams>(a, t, m);
  if constexpr (SRC == Source::kMailbox) {
    // A plain streaming read first (above); chunks still holding the
    // sentinel are re-read at device scope.
#pragma unroll
    for (int c = 0; c < FF; ++c)
      settle_chunk<8, TP>(pf[c], src + (int64_t)(tid + NT * c) * kFrag, rs, a.mailbox);
    if (half) settle_chunk<4, TP>(ph, src + hcol, rs, a.mailbox);
  }

  float sumf[FF > 0 ? FF : 1][8], sumh[4];
  if constexpr (kFin) {
#pragma unroll
    for (int c = 0; c < FF; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) sumf[c][e] = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) sumh[e] = 0.0f;
    for (int r = 0; r < a.tp; ++r)
      finalize_rank<FF, NT>(a.fin, srow, sw, r, t, H, tid, hcol, half, sumf, sumh);
  }
  double ss = 0.0;
  u32x4 pzf[FF > 0 ? FF : 1];
#pragma unroll
  for (int c = 0; c < FF; ++c) {
    const int64_t col = (int64_t)(tid + NT * c) * kFrag;
    if constexpr (!kFin) rank_sum_chunk<8, TP>(pf[c], sumf[c]);
    pzf[c] = balanced_chunk<8>(sumf[c], rf[c], m, out_row + col, H, ss);
  }
  u32x2 pzh = {0, 0};
  if (half) {
    if constexpr (!kFin) rank_sum_chunk<4, TP>(ph, sumh);
    pzh = balanced_chunk<4>(sumh, rh, m, out_row + hcol, H, ss);
  }
  if constexpr (SRC == Source::kMailbox) {
    // Advance the generation and return the consumed slots to the sentinel.
    if (t == 0 && tid == 0) a.mailbox.stage_state[1] = (int32_t)((gen + 1) % 3);
    uint16_t *slots = const_cast<uint16_t *>(src);
#pragma unroll
    for (int c = 0; c < FF; ++c)
#pragma unroll
      for (int r = 0; r < TP; ++r)
        Chunk<8>::store(slots + r * rs + (int64_t)(tid + NT * c) * kFrag, Chunk<8>::filled(0x80008000u));
    if (half)
#pragma unroll
      for (int r = 0; r < TP; ++r) Chunk<4>::store(slots + r * rs + hcol, Chunk<4>::filled(0x80008000u));
  }

  const float inv = token_inv(a, t, 0, ss, red, 0);
  // out = bf16((p * inv) * gamma); with MXFP8 also the E4M3 codes and the
  // UE8M0 scale of each 32-column block, which spans lanes 4q .. 4q+3 of a
  // full fragment and lanes 8q .. 8q+7 of a half fragment.
  uint16_t *li = a.layer_input + (int64_t)t * H;
  const int K = H / 32;
#pragma unroll
  for (int c = 0; c < FF; ++c) {
    const int f = tid + NT * c;
    float p[8], g[8], o[8];
    Chunk<8>::unpack(pzf[c], p);
    Chunk<8>::unpack(gf[c], g);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (p[e] * inv) * g[e];
    const u32x4 out = Chunk<8>::pack(o);
    Chunk<8>::store(li + (int64_t)f * kFrag, out);
    if (a.mx_values) {
      float ov[8];
      Chunk<8>::unpack(out, ov);
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(ov[e]));
      amax = __builtin_fmaxf(amax, row_xor<1>(amax));
      amax = __builtin_fmaxf(amax, row_xor<2>(amax));
      const uint32_t e8 = ue8m0_round_up(amax * (1.0f / 448.0f));
      const float sc = ue8m0_inverse(e8);
      u32x2 codes = {0, 0};
#pragma unroll
      for (int e = 0; e < 8; ++e) codes[e >> 2] |= e4m3_rne_sat(ov[e] * sc) << (8 * (e & 3));
      store8(a.mx_values + (int64_t)t * H + (int64_t)f * kFrag, codes);
      if ((f & 3) == 0) a.mx_scales[sf_offset(t, f >> 2, K)] = (uint8_t)e8;
    }
  }
  if (half) {
    float p[4], g[4], o[4];
    Chunk<4>::unpack(pzh, p);
    Chunk<4>::unpack(gh, g);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (p[e] * inv) * g[e];
    const u32x2 out = Chunk<4>::pack(o);
    Chunk<4>::store(li + hcol, out);
    if (a.mx_values) {
      float ov[4];
      Chunk<4>::unpack(out, ov);
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(ov[e]));
      amax = __builtin_fmaxf(amax, row_xor<1>(amax));
      amax = __builtin_fmaxf(amax, row_xor<2>(amax));
      amax = __builtin_fmaxf(amax, row_xor<4>(amax));
      const uint32_t e8 = ue8m0_round_up(amax * (1.0f / 448.0f));
      const float sc = ue8m0_inverse(e8);
      uint32_t codes = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) codes |= e4m3_rne_sat(ov[e] * sc) << (8 * e);
      __builtin_nontemporal_store(codes,
                                  reinterpret_cast<uint32_t *>(a.mx_values + (int64_t)t * H + hcol));
      if ((tid & 7) == 0) a.mx_scales[sf_offset(t, (int)(hcol / 32), K)] = (uint8_t)e8;
    }
  }
  if (a.mx_values) {
    // The scales of the padding rows M .. ceil(M/128)*128 - 1 are zero, one
    // 4-column word per store, spread over the grid.
    const int words_per_row = K / 4;
    const int64_t padded = ((int64_t)a.M + 127) / 128 * 128;
    const int64_t words = (padded - a.M) * words_per_row;
    for (int64_t w = (int64_t)t * NT + tid; w < words; w += (int64_t)a.M * NT) {
      const int64_t row = a.M + w / words_per_row;
      *reinterpret_cast<uint32_t *>(a.mx_scales + sf_offset(row, (int)(w % words_per_row) * 4, K)) = 0u;
    }
  }
}

// The delayed boundary for a token split over slices of 128 fragments
// (H = 5120: five slices), from 8 ranks' resident partials or the ACTIVE
// generation of a mailbox, four streams and a layer input (optionally with
// the MXFP8 epilogue).  Each of the 256 threads takes a half fragment (4
// columns): one wave per SIMD, each with half a fragment's chain.  Slices
// of 160 one-fragment lanes (192 threads) ran a whole fragment's chain on
// three SIMDs and left the fourth idle.  Same arithmetic per element, same
// results; the slices' sums of squares meet in token_inv.
template <Source SRC>
__global__ void __launch_bounds__(256) boundary_split_half_kernel(const BoundaryArgs a) {
  constexpr int TP = 8;
  static_assert(SRC == Source::kPartials || SRC == Source::kMailbox, "partials or mailbox");
  __shared__ double red[kTokenThreadsWide / kWave + 1];
  const int s = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  const int H = a.H;
  const int64_t col = (int64_t)s * a.slice_frags * kFrag + 4 * tid;
  const uint16_t *src;
  int64_t rs;
  uint32_t gen = 0;
  if constexpr (SRC == Source::kMailbox) {
    gen = (uint32_t)__hip_atomic_load(a.mailbox.stage_state, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) % 3u;  // stays inside the slots
    rs = (int64_t)a.mailbox.capacity * H;
    src = a.mailbox.slots + (int64_t)gen * TP * rs + (int64_t)t * H;
  } else {
    rs = a.rank_stride;
    src = a.partials + (int64_t)t * H;
  }
  const uint16_t *res_row = a.residual + (int64_t)t * kStreams * H;
  u32x2 ph[TP], rh[kStreams];
#pragma unroll
  for (int r = 0; r < TP; ++r) ph[r] = Chunk<4>::load(src + r * rs + col);
#pragma unroll
  for (int q = 0; q < kStreams; ++q) rh[q] = Chunk<4>::load(res_row + q * H + col);
  const u32x2 gh = Chunk<4>::load_cached(a.gamma + col);
  __builtin_amdgcn_sched_barrier(0);
  Mixes<kStreams> m;
  load_mixes<kStreams>(a, t, m);
  // The token slot's epoch word, read by wave 0 behind the loads above.
  uint64_t callw = 0;
  if (tid < kWave) callw = slot_call_word(token_slot(a.sync, t));
  if constexpr (SRC == Source::kMailbox) settle_chunk<4, TP>(ph, src + col, rs, a.mailbox);

  float sum[4];
  rank_sum_chunk<4, TP>(ph, sum);
  double ss = 0.0;
  const u32x2 pz = balanced_chunk<4>(sum, rh, m, a.residual_out + (int64_t)t * kStreams * H + col, H, ss);
  if constexpr (SRC == Source::kMailbox) {
    // Advance the generation and return the consumed slots to the sentinel.
    if (t == 0 && s == 0 && tid == 0) a.mailbox.stage_state[1] = (int32_t)((gen + 1) % 3);
    uint16_t *slots = const_cast<uint16_t *>(src);
#pragma unroll
    for (int r = 0; r < TP; ++r) Chunk<4>::store(slots + r * rs + col, Chunk<4>::filled(0x80008000u));
  }

  const float inv = token_inv(a, t, s, ss, red, callw);
  if (tid < kWave)
    for (int w = tid * a.slices + s; w < kClearWords; w += kWave * a.slices)
      clear_previous_word(token_slot(a.sync, t), unpack_call(callw), w);

  // out = bf16((p * inv) * gamma); with MXFP8 also the E4M3 codes and the
  // UE8M0 scale of each 32-column block (lanes 8q .. 8q+7).
  float p[4], g[4], o[4];
  Chunk<4>::unpack(pz, p);
  Chunk<4>::unpack(gh, g);
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = (p[e] * inv) * g[e];
  const u32x2 out = Chunk<4>::pack(o);
  Chunk<4>::store(a.layer_input + (int64_t)t * H + col, out);
  if (a.mx_values) {
    const int K = H / 32;
    float ov[4];
    Chunk<4>::unpack(out, ov);
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(ov[e]));
    amax = __builtin_fmaxf(amax, row_xor<1>(amax));
    amax = __builtin_fmaxf(amax, row_xor<2>(amax));
    amax = __builtin_fmaxf(amax, row_xor<4>(amax));
    const uint32_t e8 = ue8m0_round_up(amax * (1.0f / 448.0f));
    const float sc = ue8m0_inverse(e8);
    uint32_t codes = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) codes |= e4m3_rne_sat(ov[e] * sc) << (8 * e);
    __builtin_nontemporal_store(codes, reinterpret_cast<uint32_t *>(a.mx_values + (int64_t)t * H + col));
    if ((tid & 7) == 0) a.mx_scales[sf_offset(t, (int)(col / 32), K)] = (uint8_t)e8;
    // The scales of the padding rows M .. ceil(M/128)*128 - 1 are zero, one
    // 4-column word per store, spread over the grid.
    const int words_per_row = K / 4;
    const int64_t padded = ((int64_t)a.M + 127) / 128 * 128;
    const int64_t words = (padded - a.M) * words_per_row;
    const int64_t wg = (int64_t)t * a.slices + s, wgs = (int64_t)a.M * a.slices;
    for (int64_t w = wg * 256 + tid; w < words; w += wgs * 256) {
      const int64_t row = a.M + w / words_per_row;
      *reinterpret_cast<uint32_t *>(a.mx_scales + sf_offset(row, (int)(w % words_per_row) * 4, K)) = 0u;
    }
  }
}

template <int TRIPS, int TP, Source SRC, int HC>
void launch_one(const BoundaryArgs &a, dim3 grid, dim3 block, hipStream_t stream) {
  hipLaunchKernelGGL((boundary_kernel<TRIPS, TP, SRC, HC>), grid, block, 0, stream, a);
}

template <int TRIPS, Source SRC, int HC>
void launch_held(const BoundaryArgs &a, dim3 grid, dim3 block, hipStream_t stream) {
  // Ranks held in registers (every load issued up front) for tp = 1, 2, 4
  // and 8 with four streams; other stream counts for tp = 4 and 8 only, to
  // bound the kernel count, and eight streams in one trip, or two from
  // resident partials (more would spill).  Four trips of eight mailbox ranks
  // would spill too.  Everything else takes the runtime-rank kernel.
  constexpr bool kAll = HC == kStreams;
  constexpr bool kHold4 = HC <= kStreams || TRIPS == 1 || (TRIPS == 2 && SRC == Source::kPartials);
  constexpr bool kHold8 = kHold4 && !(TRIPS == 4 && SRC == Source::kMailbox);
  if (kAll && a.tp == 1) launch_one<TRIPS, kAll ? 1 : 0, SRC, HC>(a, grid, block, stream);
  else if (kAll && a.tp == 2) launch_one<TRIPS, kAll ? 2 : 0, SRC, HC>(a, grid, block, stream);
  else if (kHold4 && a.tp == 4) launch_one<TRIPS, kHold4 ? 4 : 0, SRC, HC>(a, grid, block, stream);
  else if (kHold8 && a.tp == 8) launch_one<TRIPS, kHold8 ? 8 : 0, SRC, HC>(a, grid, block, stream);
  else launch_one<TRIPS, 0, SRC, HC>(a, grid, block, stream);
}

template <int TRIPS, Source SRC, int HC>
hipError_t launch_tp(const BoundaryArgs &a, int threads, hipStream_t stream) {
  const dim3 grid = a.slices > 1 ? dim3(a.slices, a.M) : dim3(a.M), block(threads);
  if constexpr (SRC == Source::kFinalize) {
    // All 36 gathers in flight at once need one fragment per thread and at
    // most 512 threads (their registers).
    if (TRIPS == 1 && HC <= kStreams && a.tp == 4 && a.fin.top_k <= 8 && threads <= kTokenThreads)
      launch_one<1, HC <= kStreams ? 4 : 0, SRC, HC>(a, grid, block, stream);
    else
      launch_one<TRIPS, 0, SRC, HC>(a, grid, block, stream);
  } else {
    launch_held<TRIPS, SRC, HC>(a, grid, block, stream);
  }
  return hipGetLastError();
}

template <Source SRC, int HC>
hipError_t launch_hc(const BoundaryArgs &a, hipStream_t stream) {
  if constexpr (SRC == Source::kFinalize && HC == kStreams) {
    // Unsplit H = 5120 tokens with a layer input, 257 to 2048 of them: eight
    // balanced waves.  Measured (tp=4, top_k=8, us per call, ten waves in
    // brackets): M=192 20.5 (19.4), 256 24.1 (23.9), 320 31.1 (36.1), 384
    // 33.3 (39.0), 512 40.4-41.0 (44.3-45.5), 768 60.8 (64.0), 1024 77.0
    // (82.1), 1536 116.2 (120.3), 2048 158.4 (159.5), 3072 243.5 (241.2),
    // 4096 331.7 (321.5).  Past that, ten waves (five a SIMD against
    // four) are faster again.
    if (a.slices == 1 && a.pre && a.H / kFrag == 640 && a.M > 256 && a.M <= 2048) {
      hipLaunchKernelGGL((boundary_balanced_kernel<1, 512, Source::kFinalize>), dim3(a.M), dim3(512), 0,
                         stream, a);
      return hipGetLastError();
    }
  }
  if constexpr ((SRC == Source::kPartials || SRC == Source::kMailbox) && HC == kStreams) {
    if (a.slices > 1 && a.slice_frags == 128 && a.tp == 8 && a.pre && a.H / kFrag == 640) {
      hipLaunchKernelGGL((boundary_split_half_kernel<SRC>), dim3(a.slices, a.M), dim3(256), 0, stream, a);
      return hipGetLastError();
    }
    // Unsplit tokens of NT FF + 128 fragments, eight ranks and a layer
    // input: the balanced forms.  Measured (us per call, the ten-wave form
    // in brackets):
    //  - H = 5120, eight waves, at every M: M=128 6.64 (7.02), 160 6.99
    //    (7.48), 256 9.4 (9.8), 1024 31.2 (33.6), 4096 116 (120); with
    //    MXFP8 M=200 9.9 (10.2), 1024 34.4 (35.5), 8192 241.7 (251.2);
    //    unsplit M = 1-64 the same within 0.05.  Mailbox-fed (publish +
    //    consume): M=256 20.0 (21.6), 1024 82.6 (82.7), 8192 with MXFP8
    //    619 (623).
    //  - other widths, four waves (FF <= 3), from 129 tokens (1024 with
    //    MXFP8): at H=5120 four waves took 7.1 us at M=128 (7.0), 7.43 at
    //    160, 116.8 at 4096, and with MXFP8 21.3 at M=512 (20.6) but 246.9
    //    at 8192: one wave per SIMD hides less latency, and the MXFP8
    //    epilogue lengthens each wave's serial tail.
    const int F = a.H / kFrag, FF = F / 256;
    if (a.slices == 1 && a.tp == 8 && a.pre && F % 256 == 128 && FF <= 3) {
      const dim3 grid(a.M);
      if (F == 640) {
        hipLaunchKernelGGL((boundary_balanced_kernel<1, 512, SRC>), grid, dim3(512), 0, stream, a);
        return hipGetLastError();
      }
      if (SRC == Source::kPartials && a.M >= (a.mx_values ? 1024 : 129)) {
        switch (FF) {  // FF = 2 is H = 5120, taken above
          case 0: hipLaunchKernelGGL((boundary_balanced_kernel<0, 256, Source::kPartials>), grid, dim3(256), 0, stream, a); break;
          case 1: hipLaunchKernelGGL((boundary_balanced_kernel<1, 256, Source::kPartials>), grid, dim3(256), 0, stream, a); break;
          default: hipLaunchKernelGGL((boundary_balanced_kernel<3, 256, Source::kPartials>), grid, dim3(256), 0, stream, a); break;
        }
        return hipGetLastError();
      }
    }
  }
  const Geometry g = fragment_geometry(a.slices > 1 ? a.slice_frags : a.H / kFrag,
                                       wide_threads<SRC, HC>());
  switch (g.trips) {
    case 1: return launch_tp<1, SRC, HC>(a, g.threads, stream);
    case 2: return launch_tp<2, SRC, HC>(a, g.threads, stream);
    default: return launch_tp<4, SRC, HC>(a, g.threads, stream);
  }
}

template <Source SRC>
hipError_t launch_src(const BoundaryArgs &a, hipStream_t stream) {
  switch (a.hc) {
    case 1: return launch_hc<SRC, 1>(a, stream);
    case 2: return launch_hc<SRC, 2>(a, stream);
    case 4: return launch_hc<SRC, 4>(a, stream);
    case 8: return launch_hc<SRC, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Two-shot emulation
// ---------------------------------------------------------------------------

// Every rank's contribution of token t (blockIdx.x) into owner t % owners,
// slot t / owners: own[owner][rank][slot][H]
// (_QuadFinalizePublishDeviceKernel.kernel: the two-shot branch with
// owners = tp; with owners = 1 the one-shot publish, own[rank][t][H], the
// contributions the GLM boundary of an MoE sublayer reads as its partials).
__global__ void __launch_bounds__(kTokenThreads)
finalize_to_owners_kernel(const FinalizeView f, int tp, int owners, int M, int H, uint16_t *own) {
  __shared__ int32_t srow[kMaxRoutes];
  __shared__ float sw[kMaxRoutes];
  const int t = blockIdx.x, F = H / kFrag;
  stage_routes(f, tp, t, srow, sw);
  const int64_t slots = (M + owners - 1) / owners;
  const int owner = t % owners;
  const int64_t slot = t / owners;
  // Column chunk blockIdx.y of gridDim.y (small M spreads a token's
  // fragments over several workgroups).
  for (int fr = blockIdx.y * blockDim.x + threadIdx.x; fr < F; fr += gridDim.y * blockDim.x) {
    const int64_t col = (int64_t)fr * kFrag;
    for (int r = 0; r < tp; ++r) {
      const u32x4 c = finalize_fragment(f, srow + r * f.top_k, sw + r * f.top_k, r, t, H, col);
      store_stream(own + (((int64_t)owner * tp + r) * slots + slot) * H + col, c);
    }
  }
}

// The owners' reduce (_OwnerReduceMulticastDeviceKernel.kernel): token t's
// tp contributions summed in FP32 from rank 0, BF16, negative zero -> +0.
__global__ void __launch_bounds__(256)
owner_reduce_kernel(const uint16_t *own, int tp, int M, int H, uint16_t *reduced) {
  const int F = H / kFrag;
  const int64_t slots = (M + tp - 1) / tp;
  const int64_t n = (int64_t)M * F;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / F);
    const int64_t col = (i % F) * kFrag;
    const int owner = t % tp;
    const int64_t slot = t / tp;
    float s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.0f;
    for (int r = 0; r < tp; ++r)
      accumulate(s, load_stream(own + (((int64_t)owner * tp + r) * slots + slot) * H + col));
    store_stream(reduced + (int64_t)t * H + col, sanitize4(pack8(s)));
  }
}

// ---------------------------------------------------------------------------
// Mailbox producer and initializer
// ---------------------------------------------------------------------------

// Fills every slot with the sentinel and zeroes the stage state and status
// (AllReduceMhcBoundary.__init__).
__global__ void __launch_bounds__(256)
mailbox_init_kernel(MailboxView mb, int64_t frags) {
  const u32x4 empty = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < frags;
       i += (int64_t)gridDim.x * blockDim.x)
    store_stream(mb.slots + i * kFrag, empty);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    mb.stage_state[0] = 0;
    mb.stage_state[1] = 0;
    mb.status[0] = 0;
    mb.status[1] = 0;
  }
}

// Publishes ranks [rank_begin, rank_begin + rank_count) of token t
// (blockIdx.y) into generation NEXT: sanitized fragments, then ACTIVE = NEXT
// (_PublishDeviceKernel.kernel).  The rank loads of a fragment are issued
// together; the 16-byte stores become visible device-wide at the latest when
// the kernel ends, which a concurrent consumer's bounded poll waits out.
__global__ void __launch_bounds__(256)
publish_kernel(MailboxView mb, int tp, int H, const uint16_t *partials, int64_t rank_stride,
               int rank_begin, int rank_count) {
  const int t = blockIdx.y, F = H / kFrag;
  const int fr = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t gen = (uint32_t)__hip_atomic_load(mb.stage_state + 1, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT) % 3u;
  if (fr < F) {
    const int64_t col = (int64_t)fr * kFrag;
    for (int q0 = 0; q0 < rank_count; q0 += 8) {
      u32x4 w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (q0 + i < rank_count)
          w[i] = load_stream(partials + (q0 + i) * rank_stride + (int64_t)t * H + col);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (q0 + i >= rank_count) break;
        const int r = rank_begin + q0 + i;
        store_stream(mb.slots + (((int64_t)gen * tp + r) * mb.capacity + t) * H + col, sanitize4(w[i]));
      }
    }
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
    __hip_atomic_store(mb.stage_state, (int32_t)gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Standalone MXFP8 quantizer (same encoding as the fused epilogue)
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(kTokenThreads)
quant_kernel(const uint16_t *x, uint8_t *values, uint8_t *scales, int M, int H) {
  const int t = blockIdx.x, F = H / kFrag, K = H / 32;
  for (int f0 = 0; f0 < F; f0 += blockDim.x) {
    const int f = f0 + threadIdx.x;
    const bool valid = f < F;
    const int64_t col = valid ? (int64_t)f * kFrag : 0;
    float v[8];
    unpack8(load_stream(x + (int64_t)t * H + col), v);
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[e]));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2, kWave));
    const uint32_t e8 = ue8m0_round_up(amax * (1.0f / 448.0f));
    const float sc = ue8m0_inverse(e8);
    u32x2 codes = {0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e) codes[e >> 2] |= e4m3_rne_sat(v[e] * sc) << (8 * (e & 3));
    if (valid) {
      store8(values + (int64_t)t * H + col, codes);
      if ((f & 3) == 0) scales[sf_offset(t, f >> 2, K)] = (uint8_t)e8;
    }
  }
  const int words_per_row = K / 4;
  const int64_t padded = ((int64_t)M + 127) / 128 * 128;
  const int64_t words = (padded - M) * words_per_row;
  for (int64_t w = (int64_t)t * blockDim.x + threadIdx.x; w < words; w += (int64_t)M * blockDim.x) {
    const int64_t row = M + w / words_per_row;
    *reinterpret_cast<uint32_t *>(scales + sf_offset(row, (int)(w % words_per_row) * 4, K)) = 0u;
  }
}

__global__ void __launch_bounds__(64) copy_words_kernel(const uint32_t *src, uint32_t *dst, int count) {
  if ((int)threadIdx.x < count)
    dst[threadIdx.x] = __hip_atomic_load(src + threadIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void __launch_bounds__(64) store_word64_kernel(int64_t *dst, int64_t value) {
  if (threadIdx.x == 0) __hip_atomic_store(dst, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void __launch_bounds__(256) zero_kernel(uint32_t *p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

int grid_for(int64_t items, int block) {
  int64_t g = (items + block - 1) / block;
  if (g > 65536) g = 65536;
  return (int)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_boundary(const BoundaryArgs &a, hipStream_t stream) {
  switch (a.source) {
    case Source::kPartials: return launch_src<Source::kPartials>(a, stream);
    case Source::kMailbox: return launch_src<Source::kMailbox>(a, stream);
    case Source::kFinalize: return launch_src<Source::kFinalize>(a, stream);
  }
  return hipErrorInvalidValue;
}

// The sync state's initial contents: the header and each slot's first 128
// bytes (the epoch word) zero, every other word kSlotEmpty.
__global__ void __launch_bounds__(256) sync_init_kernel(uint32_t *p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t in_slot = (i - 64) % (kSyncSlot / 4);
    p[i] = i < 64 || in_slot < kSlotCopy0 / 4 ? 0u : kSlotEmpty;
  }
}

hipError_t launch_sync_init(void *workspace, hipStream_t stream) {
  const int64_t words = kSyncBytes / 4;
  hipLaunchKernelGGL(sync_init_kernel, dim3(grid_for(words, 256)), dim3(256), 0, stream,
                     static_cast<uint32_t *>(workspace), words);
  return hipGetLastError();
}

hipError_t launch_copy_words(const uint32_t *src, uint32_t *dst, int count, hipStream_t stream) {
  if (count < 1 || count > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_words_kernel, dim3(1), dim3(64), 0, stream, src, dst, count);
  return hipGetLastError();
}

hipError_t launch_store_word64(int64_t *dst, int64_t value, hipStream_t stream) {
  hipLaunchKernelGGL(store_word64_kernel, dim3(1), dim3(64), 0, stream, dst, value);
  return hipGetLastError();
}

hipError_t launch_zero(void *p, int64_t bytes, hipStream_t stream) {
  const int64_t words = bytes / 4;
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(words, 256)), dim3(256), 0, stream,
                     static_cast<uint32_t *>(p), words);
  return hipGetLastError();
}

hipError_t launch_finalize_to_owners(const FinalizeView &fin, int tp, int owners, int M, int H,
                                     uint16_t *own, hipStream_t stream) {
  // One workgroup per token, or below 256 tokens the token's fragments in
  // chunks of at least one wave, about 512 workgroups in all: every rank's
  // gathers of a fragment are one dependent round trip each, so the round
  // trips of many workgroups must overlap.
  const int F = H / kFrag;
  int chunks = M < 256 ? (512 + M - 1) / M : 1;
  const int max_chunks = (F + kWave - 1) / kWave;
  chunks = chunks > max_chunks ? max_chunks : chunks;
  const int wide = token_geometry(H).threads;  // at most kTokenThreads
  int threads = wide;
  if (chunks > 1) {
    threads = ((F + chunks - 1) / chunks + kWave - 1) / kWave * kWave;
    threads = threads > wide ? wide : threads;
    chunks = (F + threads - 1) / threads;  // the kernel's loop strides over any remainder
  }
  hipLaunchKernelGGL(finalize_to_owners_kernel, dim3(M, chunks), dim3(threads), 0, stream, fin, tp,
                     owners, M, H, own);
  return hipGetLastError();
}

hipError_t launch_owner_reduce(const uint16_t *own, int tp, int M, int H, uint16_t *reduced,
                               hipStream_t stream) {
  const int64_t items = (int64_t)M * (H / kFrag);
  hipLaunchKernelGGL(owner_reduce_kernel, dim3(grid_for(items, 256)), dim3(256), 0, stream, own, tp,
                     M, H, reduced);
  return hipGetLastError();
}

hipError_t launch_mailbox_init(const MailboxView &mb, int tp, int H, hipStream_t stream) {
  const int64_t frags = 3LL * tp * mb.capacity * (H / kFrag);
  hipLaunchKernelGGL(mailbox_init_kernel, dim3(grid_for(frags, 256)), dim3(256), 0, stream, mb,
                     frags);
  return hipGetLastError();
}

hipError_t launch_publish(const MailboxView &mb, int tp, int H, const uint16_t *partials,
                          int64_t rank_stride, int rank_begin, int rank_count, int M,
                          hipStream_t stream) {
  const int F = H / kFrag;
  dim3 grid((F + 255) / 256, M);
  hipLaunchKernelGGL(publish_kernel, grid, dim3(256), 0, stream, mb, tp, H, partials, rank_stride,
                     rank_begin, rank_count);
  return hipGetLastError();
}

hipError_t launch_quant_mxfp8(const uint16_t *x, uint8_t *values, uint8_t *scales, int M, int H,
                              hipStream_t stream) {
  const Geometry g = token_geometry(H);
  hipLaunchKernelGGL(quant_kernel, dim3(M), dim3(g.threads), 0, stream, x, values, scales, M, H);
  return hipGetLastError();
}

}  // namespace mhcb
