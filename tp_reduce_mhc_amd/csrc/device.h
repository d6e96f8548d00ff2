// Device-side helpers for the gfx950 boundary kernels: BF16 packing and
// rounding, 16-byte global access, wave64 / workgroup reductions, and the
// MXFP8 (E4M3 + UE8M0, swizzled 128x4) encoders.
//
// Every helper is written for CDNA4 wave64 execution; nothing here is shared
// with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhcb {

constexpr int kStreams = 4;        // hc_mult, the number of residual streams
constexpr int kMix = 24;           // pre (4) + post (4) + residual mix (16)
constexpr int kFrag = 8;           // BF16 values in one 16-byte fragment
constexpr int kWave = 64;
constexpr int kMaxThreads = 1024;
constexpr int kTokenThreads = 512;  // workgroup size bound of the per-token kernels
constexpr int kTokenThreadsWide = 1024;  // the same with one fragment per thread
constexpr int kTokenThreadsWide8 = 768;  // the same for eight residual streams
constexpr uint16_t kSentinel = 0x8000;  // BF16 negative zero marks an empty slot
constexpr uint32_t kPoisonBf16x2 = 0x7FC07FC0u;  // two BF16 quiet NaNs

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// BF16 <-> FP32
// ---------------------------------------------------------------------------

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two FP32 values -> packed BF16 pair (low half = a), round to nearest even,
// in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Dot product of 8 BF16 pairs (v_dot2c_f32_bf16: exact products, FP32
// sums) added to acc.  Each word is copied to a scalar before the bit cast:
// a bit cast applied directly to an ext_vector element (a[i]) was compiled
// to read element 0 for every i by this toolchain.
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float acc) {
  const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aw[i]),
                                          __builtin_bit_cast(bf16x2, bw[i]), acc, false);
  return acc;
}

// A fragment as 8 floats (exact widening) and back.
__device__ __forceinline__ void unpack8(u32x4 w, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = lo_bf16(w[i]);
    f[2 * i + 1] = hi_bf16(w[i]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16(f[2 * i], f[2 * i + 1]);
  return w;
}

// Negative zero halves -> +0 (a published value must never look empty).
__device__ __forceinline__ uint32_t sanitize_word(uint32_t w) {
  if ((w & 0xffffu) == kSentinel) w &= 0xffff0000u;
  if ((w >> 16) == kSentinel) w &= 0x0000ffffu;
  return w;
}

__device__ __forceinline__ u32x4 sanitize4(u32x4 w) {
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = sanitize_word(w[i]);
  return w;
}

__device__ __forceinline__ bool has_sentinel(uint32_t w) {
  return (w & 0xffffu) == kSentinel || (w >> 16) == kSentinel;
}

// ---------------------------------------------------------------------------
// Global memory
// ---------------------------------------------------------------------------

// Streamed, read-once data: non-temporal 16-byte loads keep L2 for reused
// operands (gamma, hc_fn).
__device__ __forceinline__ u32x4 load_stream(const uint16_t *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x4 load_cached(const uint16_t *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void store_stream(uint16_t *p, u32x4 w) {
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void store8(uint8_t *p, u32x2 w) {
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2 *>(p));
}

// A mailbox fragment read at device (agent) scope: two 8-byte atomic loads
// that bypass the non-coherent per-XCD cache state, so a producer running
// on another XCD is seen.  Each 2-byte element is single-copy atomic, which
// is all the sentinel check needs.
__device__ __forceinline__ u32x4 load_agent(const uint16_t *p) {
  const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
  uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  u32x4 w = {(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
  return w;
}
__device__ __forceinline__ void store_agent(uint16_t *p, u32x4 w) {
  uint64_t *q = reinterpret_cast<uint64_t *>(p);
  __hip_atomic_store(q, (uint64_t)w[0] | ((uint64_t)w[1] << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, (uint64_t)w[2] | ((uint64_t)w[3] << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until every earlier vector-memory access of the wave, stores
// included, has completed: s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at
// their maxima, GFX9-family encoding).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------------------
// Reductions.  Butterfly (xor) exchanges give every lane the same bits, and
// the cross-wave step adds the waves in index order, so every sum is
// deterministic run to run.
// ---------------------------------------------------------------------------

// Lane exchanges within rows of sixteen lanes as DPP moves (a VALU operand
// modifier, no LDS crossbar): lane i reads lane i ^ X.  xor 1 and 2 are
// quad permutations, xor 8 a rotation of the row by eight, xor 4 the quad
// reversal (xor 3) followed by the half-row mirror (xor 7).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int X>
__device__ __forceinline__ uint32_t row_xor_u32(uint32_t v) {
  static_assert(X == 1 || X == 2 || X == 4 || X == 8, "within a 16-lane row");
  if constexpr (X == 1) return dpp_u32<0xB1>(v);         // quad_perm 1,0,3,2
  else if constexpr (X == 2) return dpp_u32<0x4E>(v);    // quad_perm 2,3,0,1
  else if constexpr (X == 4) return dpp_u32<0x141>(dpp_u32<0x1B>(v));
  else return dpp_u32<0x128>(v);                         // row_ror 8
}
template <int X>
__device__ __forceinline__ float row_xor(float v) {
  return __uint_as_float(row_xor_u32<X>(__float_as_uint(v)));
}
template <int X>
__device__ __forceinline__ double row_xor(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = row_xor_u32<X>((uint32_t)u), hi = row_xor_u32<X>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, lo | (hi << 32));
}

// Lane i ^ 16 and i ^ 32 through gfx950's row swaps: permlane16_swap(v, v)
// gives rows (0, 0, 2, 2) and (1, 1, 3, 3) of v, permlane32_swap(v, v) its
// lower and its upper half twice; each lane takes the one that is not its
// own.
__device__ __forceinline__ uint32_t lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}
template <int X>
__device__ __forceinline__ uint32_t cross_xor_u32(uint32_t v) {
  static_assert(X == 16 || X == 32, "across rows");
  const u32x2 s = X == 16 ? __builtin_amdgcn_permlane16_swap(v, v, false, false)
                          : __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (lane_id() & X) ? s.x : s.y;
}
template <int X>
__device__ __forceinline__ float cross_xor(float v) {
  return __uint_as_float(cross_xor_u32<X>(__float_as_uint(v)));
}
template <int X>
__device__ __forceinline__ double cross_xor(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = cross_xor_u32<X>((uint32_t)u), hi = cross_xor_u32<X>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, lo | (hi << 32));
}

// The butterfly v + (lane ^ 32), + (lane ^ 16), ..., + (lane ^ 1): every
// lane ends with the same bits.  The two cross-row steps are row swaps, the
// four within a row DPP moves; no step goes through the LDS crossbar.
// Every lane of the wave must call it.
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  v += cross_xor<32>(v);
  v += cross_xor<16>(v);
  v += row_xor<8>(v);
  v += row_xor<4>(v);
  v += row_xor<2>(v);
  v += row_xor<1>(v);
  return v;
}

// Workgroup sum of N values per thread; `scratch` holds N * waves entries.
// Returns the totals in `v` on every thread.  Contains barriers: every
// thread of the workgroup must call it.
template <typename T, int N>
__device__ __forceinline__ void block_sum(T (&v)[N], T *scratch) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int waves = blockDim.x / kWave;
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_sum(v[i]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) scratch[wave * N + i] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    T s = 0;
    for (int w = 0; w < waves; ++w) s += scratch[w * N + i];
    v[i] = s;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// MXFP8: UE8M0 scales and E4M3 codes
// ---------------------------------------------------------------------------

// The scale exponent e (scale = 2^(e-127)) rounded up: the smallest e in
// [0, 254] with 2^(e-127) >= v, for finite v >= 0.
__device__ __forceinline__ uint32_t ue8m0_round_up(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t exp = (u >> 23) & 0xffu, mant = u & 0x7fffffu;
  uint32_t e;
  if (exp == 0) e = mant > 0x400000u ? 1u : 0u;   // 2^-127 is the subnormal 0x00400000
  else e = exp + (mant != 0u ? 1u : 0u);
  return e > 254u ? 254u : e;
}

// 2^(127 - e) as a float (e in [0, 254]).
__device__ __forceinline__ float ue8m0_inverse(uint32_t e) {
  return e < 254u ? __uint_as_float((254u - e) << 23) : __uint_as_float(0x00400000u);
}

// FP32 -> OCP E4M3 (bias 7, max 448), round to nearest even, saturating to
// +-448, sign kept.  Written from the format: subnormal codes are multiples
// of 2^-9; normal codes keep 3 mantissa bits.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = __builtin_fabsf(x);
  if (!(a == a)) return sign | 0x7fu;  // NaN
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0.015625f) {                  // below 2^-6: quantum 2^-9
    float q = __builtin_rintf(a * 512.0f);  // exact scaling, ties to even
    return sign | (uint32_t)q;              // q == 8 is the smallest normal
  }
  uint32_t biased = (u >> 23) & 0xffu;      // 121 .. 135
  uint32_t keep = (u >> 20) & 7u, rest = u & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  return sign | (((biased - 120u) << 3) + keep);
}

// Byte offset of scale (row r, scale column k), K scale columns, in the
// swizzled 128x4 layout: 512-byte tiles of 128 rows x 4 columns, tiles
// row-major over (r/128, k/4); inside a tile row r lives in 16-byte line
// r%32, 4-byte word (r%128)/32, byte k%4.
__device__ __forceinline__ int64_t sf_offset(int64_t r, int k, int K) {
  return ((r >> 7) * (K >> 2) + (k >> 2)) * 512 + (r & 31) * 16 + ((r & 127) >> 5) * 4 + (k & 3);
}

}  // namespace mhcb
