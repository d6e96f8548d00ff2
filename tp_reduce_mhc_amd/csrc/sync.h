// Cross-workgroup exchange of the token-split kernels: a per-token
// sense-reversing barrier in the caller's workspace (layout in kernels.h).
//
// Every shared word is accessed with device-scope atomics, which are
// performed at the device's coherence point; ordering them only needs the
// wave's earlier accesses to have completed (wait_vmem: s_waitcnt vmcnt(0),
// which on CDNA counts stores too), and values are read only after the
// atomic or generation load that released the wait has returned.  Device-scope
// release/acquire fences would instead write back / invalidate the XCD's
// whole L2 at every arrival and every poll.
#pragma once

#include "device.h"
#include "kernels.h"

namespace mhcb {

__device__ __forceinline__ char *token_slot(const SyncView &sy, int t) {
  return sy.slots + (int64_t)t * kSyncSlot;
}

__device__ __forceinline__ void slot_store64(char *slot, int offset, double v) {
  __hip_atomic_store(reinterpret_cast<uint64_t *>(slot + offset),
                     __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double slot_load64(const char *slot, int offset) {
  return __builtin_bit_cast(double, __hip_atomic_load(reinterpret_cast<const uint64_t *>(slot + offset),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void slot_store32(char *slot, int offset, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t *>(slot + offset), __builtin_bit_cast(uint32_t, v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float slot_load32(const char *slot, int offset) {
  return __builtin_bit_cast(float, __hip_atomic_load(reinterpret_cast<const uint32_t *>(slot + offset),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Token t's barrier.  Word 0 of the slot (8 bytes) holds the arrivals of
// the current generation in its low half and the generation in its high
// half, so an arrival is one atomic add that also returns the generation,
// and the last arrival starts the next generation (count back to zero,
// generation + 1) with a second add.  It comes in two halves so that one
// thread can take several tokens' barriers without ever waiting while it
// still owes an arrival (arrive at all of them, then wait at each).
//
// barrier_arrive: one slice's arrival.  The caller must have completed its
// stores to the slot (wait_vmem) first; that same wait also covers this
// thread's previous add on the word, so a last arrival's reset always lands
// before the same thread arrives again.  Returns true for the last of
// `slices` arrivals; otherwise false with the generation to wait on in
// *gen_seen.
__device__ __forceinline__ bool barrier_arrive(const SyncView &sy, int t, int slices,
                                               uint32_t *gen_seen) {
  uint64_t *word = reinterpret_cast<uint64_t *>(token_slot(sy, t));
  const uint64_t old = __hip_atomic_fetch_add(word, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  *gen_seen = (uint32_t)(old >> 32);
  if ((uint32_t)old != (uint32_t)slices - 1u) return false;
  __hip_atomic_fetch_add(word, (1ull << 32) - (uint64_t)slices, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// barrier_wait: waits for token t's generation to move past `g`.  Bounded:
// a time-out is counted in the status word and the caller goes on (every
// wave always exits).
__device__ __forceinline__ void barrier_wait(const SyncView &sy, int t, uint32_t g) {
  const uint32_t *gen = reinterpret_cast<const uint32_t *>(token_slot(sy, t)) + 1;
  int64_t spins = 0;
  while (__hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g) {
    if (++spins > sy.spin_limit) {
      atomicAdd(sy.status, 1u);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Both halves for a single token, after this thread's slot stores.
// Reusable any number of times per call and across calls.
__device__ __forceinline__ void token_barrier(const SyncView &sy, int t, int slices) {
  wait_vmem();
  uint32_t g;
  if (!barrier_arrive(sy, t, slices, &g)) barrier_wait(sy, t, g);
}

}  // namespace mhcb
