// Cross-workgroup exchange of the token-split kernels, in the caller's
// workspace (slot layout in kernels.h).
//
// Every value entry of a slot holds kSlotEmpty until a slice writes it.  A
// slice stores its partials, then reads the other slices' entries, re-reading
// (bounded) while any is still empty: a value that is no longer empty has
// landed, so no barrier is needed and the wait costs about one device-scope
// round trip after the slowest slice's store.  Once a workgroup has read
// everything it needs (at the end of the kernel, off the critical path), it
// counts itself on the exchange's counter; the last of the slices resets the
// counter and writes kSlotEmpty back into the entries.  The next use of the
// slot is a later kernel launch, which the kernel boundary orders after
// those stores.
//
// Every shared word is accessed with device-scope (sc1) atomics, performed at
// the device's coherence point, because the eight XCDs' L2 caches are not
// coherent with one another.  No release/acquire fence is used: at device
// scope they write back / invalidate the XCD's whole L2.
#pragma once

#include "device.h"
#include "kernels.h"

namespace mhcb {

// A NaN payload that no arithmetic here produces: BF16 data converted to
// FP32 or FP64 carries zeros in those low mantissa bits, and the hardware's
// own NaNs are canonical.
constexpr uint32_t kSlotEmpty = 0x7FC0DEADu;
constexpr uint64_t kSlotEmpty64 = ((uint64_t)kSlotEmpty << 32) | kSlotEmpty;

__device__ __forceinline__ char *token_slot(const SyncView &sy, int t) {
  return sy.slots + (int64_t)t * kSyncSlot;
}

__device__ __forceinline__ uint64_t slot_load_u64(const char *slot, int offset) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t *>(slot + offset), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void slot_store_u64(char *slot, int offset, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t *>(slot + offset), v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t slot_load_u32(const char *slot, int offset) {
  return __hip_atomic_load(reinterpret_cast<const uint32_t *>(slot + offset), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void slot_store_u32(char *slot, int offset, uint32_t v) {
  __hip_atomic_store(reinterpret_cast<uint32_t *>(slot + offset), v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void slot_store64(char *slot, int offset, double v) {
  slot_store_u64(slot, offset, __builtin_bit_cast(uint64_t, v));
}
__device__ __forceinline__ void slot_store32(char *slot, int offset, float v) {
  slot_store_u32(slot, offset, __builtin_bit_cast(uint32_t, v));
}

// One more round of a bounded wait: false (and the time-out counted in the
// status word) once `spin_limit` rounds have passed, so every wave exits.
__device__ __forceinline__ bool spin_again(const SyncView &sy, int64_t &spins) {
  if (++spins > sy.spin_limit) {
    atomicAdd(sy.status, 1u);
    return false;
  }
  __builtin_amdgcn_s_sleep(2);
  return true;
}

// The 8-byte entries at `offset + step * q` (q < slices <= kMaxSlices) of a
// slot, once all are written: every load is issued before any is tested.
__device__ __forceinline__ void gather64(const SyncView &sy, const char *slot, int offset, int step,
                                         int slices, uint64_t (&w)[kMaxSlices]) {
  int64_t spins = 0;
  for (;;) {
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q) w[q] = q < slices ? slot_load_u64(slot, offset + step * q) : 0;
    bool missing = false;
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q) missing |= q < slices && w[q] == kSlotEmpty64;
    if (!missing || !spin_again(sy, spins)) return;
  }
}
__device__ __forceinline__ void gather32(const SyncView &sy, const char *slot, int offset, int step,
                                         int slices, uint32_t (&w)[kMaxSlices]) {
  int64_t spins = 0;
  for (;;) {
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q) w[q] = q < slices ? slot_load_u32(slot, offset + step * q) : 0;
    bool missing = false;
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q) missing |= q < slices && w[q] == kSlotEmpty;
    if (!missing || !spin_again(sy, spins)) return;
  }
}

// Binary64 entries added in slice order.
__device__ __forceinline__ double gather_sum64(const SyncView &sy, const char *slot, int offset,
                                               int slices) {
  uint64_t w[kMaxSlices];
  gather64(sy, slot, offset, 8, slices, w);
  double total = 0.0;
#pragma unroll
  for (int q = 0; q < kMaxSlices; ++q)
    if (q < slices) total += __builtin_bit_cast(double, w[q]);
  return total;
}
// FP32 entries `step` bytes apart, added in slice order.
__device__ __forceinline__ float gather_sum32(const SyncView &sy, const char *slot, int offset,
                                              int step, int slices) {
  uint32_t w[kMaxSlices];
  gather32(sy, slot, offset, step, slices, w);
  float total = 0.0f;
#pragma unroll
  for (int q = 0; q < kMaxSlices; ++q)
    if (q < slices) total += __builtin_bit_cast(float, w[q]);
  return total;
}

// This workgroup has read everything it needs of exchange e (0 or 1) whose
// counter is in token t's slot.  True for the last of `slices` workgroups,
// which has reset the counter and must write kSlotEmpty back into the
// exchange's entries.
__device__ __forceinline__ bool exchange_done(const SyncView &sy, int t, int e, int slices) {
  uint32_t *count = reinterpret_cast<uint32_t *>(token_slot(sy, t)) + e;
  const uint32_t old = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old != (uint32_t)slices - 1u) return false;
  __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

}  // namespace mhcb
