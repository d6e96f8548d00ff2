// DSA indexer input projection for gfx950 (the page
//   vllm.models.glm5next.nvidia.specialized_decode.indexer,
//   IndexerProjection.__call__ / _ProjectionKernel):
// the layer input x [M, K] times the concatenated weight rows
// w [key + heads + gate, K] (indexer key rows, head-weight rows, kpool gate
// rows), each part written in its own type: key [M, key] BF16, head weights
// [M, heads] FP32, gate [M, gate] BF16.  The products of BF16 values are
// exact in FP32; only the order of the sum is the kernel's.
//
// gfx950 design, two forms:
// - Up to kIndexerGemvMaxM (6) tokens, indexer_gemv_kernel: one workgroup
//   per weight row, v_dot2c_f32_bf16 over coalesced 16-byte chunks.
// - Otherwise indexer_kernel: v_mfma_f32_16x16x32_bf16 with tokens as the M
//   dimension (16-token tiles, a tile's missing tokens padded with the last
//   one) and weight rows as the N dimension.  A workgroup owns an output
//   block of TT token tiles x RT row tiles and one of S contiguous ranges of
//   the 32-column chunks of K; its W waves take every W-th chunk of the
//   range, loading each chunk's TT + RT operands once (16 bytes a lane,
//   straight from global memory in the MFMA operand layout) for TT * RT
//   products.  The waves' tiles are added in a fixed order through LDS.
//   (TT, RT, S, W) come from plan_indexer, a rule fitted to measurements.
//
// With S = 1 that sum is the output.  With S > 1 (a workspace, and few
// enough blocks; S = 8 puts one range on each XCD) each workgroup stores its
// block's partial sums in the workspace, and the last of the block's S
// workgroups to finish, found with a device-scope counter, adds the S
// partials in range order and writes the output; it also sets the counter
// back to zero for the next call.  Nobody waits, and each output is a sum in
// a fixed order, so results repeat bit for bit for a given (M, S).
//
// The workspace starts with a fixed area of kIndexerCounters counters (zero
// between calls), followed by the partials of the current call.  Partials
// and counters are accessed with device-scope (sc1) atomics, which
// are performed at the device's coherence point: the eight XCDs' L2 caches
// are not coherent with one another.  A workgroup's partial stores are
// complete (s_waitcnt 0 in every thread, then the barrier) before its
// counter increment, and the last workgroup's partial loads follow the
// increment's result, so they see every partial.  No device-scope fence is
// used: it would write back and invalidate the XCD's whole L2, which holds
// the operands other workgroups re-read.
#include "device.h"
#include "indexer.h"

namespace mhcb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kIdxTile = 16;  // tokens per token tile, weight rows per row tile
constexpr int kIdxFold = 4;   // LDS slots of the waves' sum

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Output row r of token t: the key part in BF16, the head weights in FP32,
// the gate part in BF16.
__device__ __forceinline__ void store_output(const IndexerArgs &a, int64_t t, int r, float v) {
  if (r < a.key) {
    a.key_out[t * a.key + r] = (uint16_t)(pack_bf16(v, 0.0f) & 0xffffu);
  } else if (r < a.key + a.heads) {
    a.heads_out[t * a.heads + (r - a.key)] = v;
  } else {
    a.gate_out[t * a.gate + (r - a.key - a.heads)] = (uint16_t)(pack_bf16(v, 0.0f) & 0xffffu);
  }
}

// A thread's E = TT * RT partial sums move as E / 2 8-byte device-scope
// words (one 4-byte word when E = 1).  Word j of thread tid sits at word
// j * 256 + tid of the block's area, so each store or load instruction of a
// wave covers one contiguous stretch of memory: device-scope stores are
// written through, and scattered 8-byte stores would each cost a partial
// sector write.
template <int E>
struct PartialWords {
  static constexpr int kWords = E > 1 ? E / 2 : 1;
  __device__ static void store(float *area, int tid, const float (&v)[E]) {
    if constexpr (E == 1) {
      __hip_atomic_store(reinterpret_cast<uint32_t *>(area) + tid,
                         __builtin_bit_cast(uint32_t, v[0]), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    } else {
#pragma unroll
      for (int j = 0; j < kWords; ++j) {
        const uint64_t w = (uint64_t)__builtin_bit_cast(uint32_t, v[2 * j]) |
                           (uint64_t)__builtin_bit_cast(uint32_t, v[2 * j + 1]) << 32;
        __hip_atomic_store(reinterpret_cast<uint64_t *>(area) + j * 256 + tid, w,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  __device__ static uint64_t load(const float *area, int tid, int j) {
    if constexpr (E == 1)
      return __hip_atomic_load(reinterpret_cast<const uint32_t *>(area) + tid, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    else
      return __hip_atomic_load(reinterpret_cast<const uint64_t *>(area) + j * 256 + tid,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ static float value(uint64_t w, int e) {
    return __builtin_bit_cast(float, (uint32_t)(E == 1 ? w : (e & 1) ? w >> 32 : w));
  }
};

// Few tokens (M <= kIndexerGemvMaxM = 6), indexer_gemv_kernel<TOK>, TOK = 4
// or 8 tokens a launch: one workgroup per weight row (288 for the 288-row
// projection), the whole row read in one coalesced pass (thread i takes the
// 16-byte chunks i, i + 256, ...).  Each token's dot product accumulates
// with v_dot2c_f32_bf16 (exact BF16 products, FP32 sums) and is added over
// the workgroup in a fixed order: a butterfly within each wave, then the
// waves in order.  There are no partials and no second pass; the tokens'
// rows are re-read from L2 by every workgroup.
// Measured on MI355X: M = 5 / 6 took 5.0 / 5.4 us against 6.2 / 6.2 with
// the matrix-core form; at M = 8 the two were within 3% and over cold
// inputs the matrix cores won (6.8 against 7.0 us); sixteen tokens in four
// groups took 16.9 us against 8.3.  TOK = 8 at M <= 4 cost 4.7 us against
// 4.3 for TOK = 4: its registers halve the waves a SIMD holds.
constexpr int kGemvWaves = 4;
constexpr int kGemvThreads = kGemvWaves * kWave;
constexpr int kGemvPiece = 4;  // 16-byte chunks per thread per round

template <int TOK>
__global__ void __launch_bounds__(kGemvThreads) indexer_gemv_kernel(const IndexerArgs a) {
  constexpr int kTok = TOK;
  __shared__ float red[kGemvWaves][kTok];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int row = blockIdx.x, K = a.K, M = a.M, chunks = K / 8;
  const uint16_t *wr = a.w + (int64_t)row * K;
  float acc[kTok];
#pragma unroll
  for (int t = 0; t < kTok; ++t) acc[t] = 0.0f;

  for (int j0 = tid; j0 < chunks; j0 += kGemvPiece * kGemvThreads) {
    u32x4 w[kGemvPiece], xv[kTok][kGemvPiece];
#pragma unroll
    for (int p = 0; p < kGemvPiece; ++p) {
      const int c = j0 + p * kGemvThreads;
      w[p] = c < chunks ? load_cached(wr + (int64_t)c * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < kTok; ++t)
        xv[t][p] = t < M && c < chunks ? load_cached(a.x + (int64_t)t * K + (int64_t)c * 8)
                                       : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int t = 0; t < kTok; ++t)
#pragma unroll
      for (int p = 0; p < kGemvPiece; ++p) acc[t] = dot8(xv[t][p], w[p], acc[t]);
  }

#pragma unroll
  for (int t = 0; t < kTok; ++t) {
    if (t >= M) break;  // uniform
    const float v = wave_sum(acc[t]);
    if (lane == 0) red[wave][t] = v;
  }
  __syncthreads();
  if (tid < M) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kGemvWaves; ++w) v += red[w][tid];
    store_output(a, tid, row, v);
  }
}

// Workgroup L of the one-dimensional grid -> (K range, output block).
// With a multiple of 8 ranges, range s runs on XCD s % 8 (workgroups are
// dealt to the eight XCDs in turn), so the operand slices of a range are
// read from memory once per XCD and re-read from its L2 by the range's
// other blocks.
__device__ __forceinline__ void decode_workgroup(int L, int blocks, int S, int &split, int &block) {
  if (S % 8 == 0) {
    split = L % 8 + 8 * (L / 8 / blocks);
    block = L / 8 % blocks;
  } else {
    split = L / blocks;
    block = L % blocks;
  }
}

// Output block (token group, row group) of TT token tiles x RT row tiles,
// over K range `split` of S, by W waves.
template <int TT, int RT, int W>
__global__ void __launch_bounds__(W * kWave)
indexer_kernel(const IndexerArgs a, const int groups, const int blocks, const int S) {
  constexpr int kTile = kIdxTile * kIdxTile;
  constexpr int E = TT * RT;               // outputs per thread
  constexpr int kThreads = W * kWave;
  static_assert(W % kIdxFold == 0 && kThreads >= kTile, "block shape");
  using Words = PartialWords<E>;
  __shared__ float red[kIdxFold][E * kTile];
  __shared__ int last;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  int split, block;
  decode_workgroup(blockIdx.x, blocks, S, split, block);
  const int group = block % groups, rgroup = block / groups;
  const int K = a.K, M = a.M, tiles = (M + kIdxTile - 1) / kIdxTile, chunks = K / 32;
  const int c0 = (int)((int64_t)split * chunks / S), c1 = (int)((int64_t)(split + 1) * chunks / S);
  const int mi = lane & (kIdxTile - 1), mq = lane >> 4;  // operand row, 8-column group

  // This lane's weight rows (zero beyond the last row) and token rows
  // (the last token again beyond it).
  const uint16_t *wp[RT];
  bool row_ok[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int row = (rgroup * RT + r) * kIdxTile + mi;
    row_ok[r] = row < a.rows;
    wp[r] = a.w + (int64_t)(row_ok[r] ? row : 0) * K + mq * 8;
  }
  const uint16_t *xp[TT];
  bool tile_ok[TT];
#pragma unroll
  for (int u = 0; u < TT; ++u) {
    const int tile = group * TT + u;
    tile_ok[u] = tile < tiles;  // uniform over the workgroup
    int t = tile * kIdxTile + mi;
    t = t < M ? t : M - 1;
    xp[u] = a.x + (int64_t)t * K + mq * 8;
  }

  f32x4 acc[TT][RT];
#pragma unroll
  for (int u = 0; u < TT; ++u)
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[u][r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Two chunks per round (c and c + W), all loads before the products.
  for (int c = c0 + wave; c < c1; c += 2 * W) {
    const bool second = c + W < c1;
    u32x4 b[2][RT], x8[2][TT];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int cc = c + h * W;
      const bool ok = h == 0 || second;
#pragma unroll
      for (int r = 0; r < RT; ++r)
        b[h][r] = ok && row_ok[r] ? load_cached(wp[r] + (int64_t)cc * 32) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < TT; ++u)
        x8[h][u] = ok && tile_ok[u] ? load_cached(xp[u] + (int64_t)cc * 32) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int u = 0; u < TT; ++u)
#pragma unroll
        for (int r = 0; r < RT; ++r)
          if (tile_ok[u]) acc[u][r] = mfma16(x8[h][u], b[h][r], acc[u][r]);
  }

  // Block element i = (u * RT + r) * 256 + m * 16 + n is (token m of
  // token tile u, row n of row tile r); lane l holds m = 4 (l / 16) + e,
  // n = l % 16 of each tile.  Waves kIdxFold * g + j (g = W / kIdxFold - 1
  // down to 1) are added into wave j in turn; then the kIdxFold sums are
  // added in wave order: a fixed order.
  auto slot = [&](int u, int r, int e) { return (u * RT + r) * kTile + (4 * mq + e) * kIdxTile + mi; };
#pragma unroll
  for (int g = W / kIdxFold - 1; g >= 1; --g) {
    if (wave / kIdxFold == g)
#pragma unroll
      for (int u = 0; u < TT; ++u)
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int e = 0; e < 4; ++e) red[wave % kIdxFold][slot(u, r, e)] = acc[u][r][e];
    __syncthreads();
    if (wave < kIdxFold)
#pragma unroll
      for (int u = 0; u < TT; ++u)
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[u][r][e] += red[wave][slot(u, r, e)];
    __syncthreads();
  }
  if (wave < kIdxFold)
#pragma unroll
    for (int u = 0; u < TT; ++u)
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave][slot(u, r, e)] = acc[u][r][e];
  __syncthreads();

  // Thread tid < 256 owns position tid (token m = tid / 16, row n = tid %
  // 16) of every tile of the block: element e = u * RT + r is that position
  // of tile (u, r).  The other threads only take part in the barriers.
  const bool owner = tid < kTile;
  const int pos = owner ? tid : 0, m = pos / kIdxTile, n = pos % kIdxTile;
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    v[e] = 0.0f;
#pragma unroll
    for (int w = 0; w < kIdxFold; ++w) v[e] += red[w][e * kTile + pos];
  }
  auto store_all = [&](const float (&o)[E]) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t t = (int64_t)(group * TT + e / RT) * kIdxTile + m;
      const int row = (rgroup * RT + e % RT) * kIdxTile + n;
      if (t < M && row < a.rows) store_output(a, t, row, o[e]);
    }
  };
  if (S == 1) {
    if (owner) store_all(v);
    return;
  }

  // Partials: [split][block][E * 256 values, word-major], read back by the
  // block's last workgroup in range order.
  const int64_t plane = (int64_t)blocks * E * kTile;
  float *area = a.parts + (int64_t)block * E * kTile;
  if (owner) Words::store(area + split * plane, tid, v);
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
  __syncthreads();
  uint32_t *counter = a.counters + block;
  if (tid == 0)
    last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (uint32_t)(S - 1);
  __syncthreads();
  if (!last) return;
  if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!owner) return;
  // Eight ranges' words in flight at a time, added in range order.
  float sum[E];
#pragma unroll
  for (int e = 0; e < E; ++e) sum[e] = 0.0f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    uint64_t w[8][Words::kWords];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int j = 0; j < Words::kWords; ++j)
        w[q][j] = s0 + q < S ? Words::load(area + (s0 + q) * plane, tid, j) : 0;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (s0 + q < S)
#pragma unroll
        for (int e = 0; e < E; ++e) sum[e] += Words::value(w[q][e / 2], e);
  }
  store_all(sum);
}

}  // namespace

IndexerPlan plan_indexer(int M, int K, int rows, int cus, bool workspace) {
  IndexerPlan p;
  if (M <= kIndexerGemvMaxM) {
    p.gemv = M <= 4 ? 4 : 8;
    p.tt = p.rt = p.groups = p.row_groups = p.splits = 1;
    p.blocks = rows;
    p.waves = kGemvWaves;
    p.counter_bytes = p.workspace_bytes = 0;
    return p;
  }
  p.gemv = 0;
  const int tiles = (M + kIdxTile - 1) / kIdxTile, row_tiles = (rows + kIdxTile - 1) / kIdxTile;
  auto shape = [&](int tt, int rt) {
    p.tt = tt;
    p.rt = rt;
    p.groups = (tiles + tt - 1) / tt;
    p.row_groups = (row_tiles + rt - 1) / rt;
    return (int64_t)p.groups * p.row_groups;
  };
  // Launch shapes measured on MI355X (K=6144, 288 rows, M = 8 .. 4096, HIP
  // graphs over cold inputs), best of blocks {1x1, 2x2, 4x2} x {1, 2, 4, 8}
  // K ranges x {4, 8, 16} waves: 1x1 blocks up to four token tiles, 2x2 up
  // to sixteen, 4x2 beyond; eight K ranges (one per XCD) while there are
  // at most 96 blocks, four up to the counter area's 1024; 8 waves at
  // M <= 16, for 2x2 blocks past eight token tiles and for 4x2 blocks with
  // eight ranges, else 4.  (M=256: 15.0 us against 21.7 with the rule this
  // replaced; M=4096: 87 against 110.)  From 128 token tiles, 4x3 and then
  // 4x6 blocks: a wave loads TT + RT operands a chunk for TT * RT matrix
  // products, and with 4x2 the loads, not the matrix cores, set the time
  // (M=2048: 40.7 us against 49.1 with 4x2; M=4096, 4x6: 72.9 against 87;
  // 4x3 at M=1024 took 36.5 against 32.6, 4x6 at 2048 61 against 49: with
  // few blocks their larger LDS fold and registers cost more).  A single
  // range (no workspace, or more blocks than counters) takes 16 waves once
  // a wave would have more than eight chunks, so that more of its loads
  // are in flight (8 for blocks of more than 8 tiles, whose 16-wave form
  // would spill registers).
  int64_t blocks;
  int64_t splits = 1;
  if (workspace) {
    blocks = tiles <= 4     ? shape(1, 1)
             : tiles <= 16  ? shape(2, 2)
             : tiles < 128  ? shape(4, 2)
             : tiles < 256  ? shape(4, 3)
                            : shape(4, 6);
    splits = blocks <= 96 ? 8 : blocks <= kIndexerCounters ? 4 : 1;
  } else {
    // Without K ranges, the largest block that still gives a workgroup per
    // compute unit.
    blocks = shape(4, 2);
    if (blocks < cus) blocks = shape(2, 2);
    if (blocks < cus) blocks = shape(1, 1);
  }
  const int by_k = K / 32 / 4;  // at least one 32-column chunk per wave of 4
  if (splits > by_k) splits = by_k;
  p.splits = splits < 1 ? 1 : (int)splits;
  p.blocks = (int)blocks;
  if (tiles <= 1) p.waves = 8;
  else if (p.tt == 2) p.waves = tiles > 8 ? 8 : 4;
  else if (p.tt == 4) p.waves = p.splits == 8 ? 8 : 4;
  else p.waves = 4;
  if (p.splits == 1 && (int64_t)K / 32 > 8 * p.waves) p.waves = p.tt * p.rt > 8 ? 8 : 16;
  p.counter_bytes = kIndexerCounters * 4;
  p.workspace_bytes =
      p.splits > 1 ? p.counter_bytes + (int64_t)p.splits * blocks * p.tt * p.rt * kIdxTile * kIdxTile * 4 : 0;
  return p;
}

namespace {
template <int TT, int RT>
void launch_shape(const IndexerArgs &a, const IndexerPlan &p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.blocks * p.splits));
  if (TT * RT <= 8 && p.waves == 16)
    hipLaunchKernelGGL((indexer_kernel<TT, RT, TT * RT <= 8 ? 16 : 8>), grid,
                       dim3((TT * RT <= 8 ? 16 : 8) * kWave), 0, stream, a, p.groups, p.blocks,
                       p.splits);
  else if (p.waves == 8)
    hipLaunchKernelGGL((indexer_kernel<TT, RT, 8>), grid, dim3(8 * kWave), 0, stream, a, p.groups,
                       p.blocks, p.splits);
  else
    hipLaunchKernelGGL((indexer_kernel<TT, RT, 4>), grid, dim3(4 * kWave), 0, stream, a, p.groups,
                       p.blocks, p.splits);
}
}  // namespace

hipError_t launch_indexer(const IndexerArgs &a, const IndexerPlan &p, hipStream_t stream) {
  if (p.gemv) {
    if (a.K % 8 || a.M > p.gemv || (p.gemv != 4 && p.gemv != 8)) return hipErrorInvalidValue;
    if (p.gemv == 4)
      hipLaunchKernelGGL(indexer_gemv_kernel<4>, dim3(a.rows), dim3(kGemvThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(indexer_gemv_kernel<8>, dim3(a.rows), dim3(kGemvThreads), 0, stream, a);
    return hipGetLastError();
  }
  if (a.K % 32 || p.splits < 1 || (p.splits > 1 && (!a.parts || !a.counters)) ||
      (p.waves != 4 && p.waves != 8 && p.waves != 16))
    return hipErrorInvalidValue;
  if (p.tt == 1 && p.rt == 1) launch_shape<1, 1>(a, p, stream);
  else if (p.tt == 2 && p.rt == 2) launch_shape<2, 2>(a, p, stream);
  else if (p.tt == 4 && p.rt == 2) launch_shape<4, 2>(a, p, stream);
  else if (p.tt == 4 && p.rt == 3) launch_shape<4, 3>(a, p, stream);
  else if (p.tt == 4 && p.rt == 6) launch_shape<4, 6>(a, p, stream);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mhcb
