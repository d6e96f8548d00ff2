// Cross-workgroup exchange of the token-split kernels, in the caller's
// workspace (slot layout in kernels.h).
//
// A token slot holds an epoch word (E = split calls that used the slot, and
// the slice count of the last of them; or "broken", below) and two copies
// of the exchange area.
// A call uses copy E % 2.  At the start of that call, every word of that
// copy holds the empty marker kSlotEmpty:
//   - every slice reads the epoch word at its start, off the critical path;
//   - a slice stores its values in its entries of copy E % 2 and reads the
//     other slices' entries, re-reading (bounded) while any is still empty:
//     a value that is no longer empty has landed, so the wait costs about one
//     device-scope round trip after the slowest slice's store;
//   - after its last read it raises the epoch word to (E + 1, its slice
//     count) with an atomic maximum (every slice writes the same value; no
//     return value, no wait).
//     No slice of the call can still read the old word then: a slice stores
//     its values only after its epoch load has returned, and the others'
//     last reads saw those values;
//   - the slices also write the empty marker back into the entries the
//     previous call wrote in the other copy (its slice count is in the
//     epoch word).  Nothing reads that copy during this call, and the kernel
//     boundary orders those stores before the next call, which uses that
//     copy.
// So no workgroup waits after its last read, and nothing is reset at the
// end of a call.
//
// A wait that gives up (spin limit) breaks the invariant above: a slice of
// the same token that starts later could read an advanced epoch.  So the
// giving-up slice raises the epoch word to kSlotBroken and reads what it
// could not get as NaN; a slice that reads a broken word stores and clears
// nothing and produces NaN.  The slot stays broken until the workspace is
// initialized again, so no later call can sum stale entries.
//
// Co-residency: the slices of a token wait for one another, so they must be
// able to run at the same time.  They are consecutive in dispatch order, so
// on an otherwise idle device a wait never depends on a workgroup queued
// behind it.  A kernel running concurrently that leaves fewer free workgroup
// slots than a token's slice count can hold a slice back until the waiting
// ones give up (after the spin limit): those slices then produce NaN results
// and the time-out is counted in the workspace status.
//
// Exchanged words are accessed with device-scope (sc1) atomics, performed at
// the device's coherence point, because the eight XCDs' L2 caches are not
// coherent with one another.  No release/acquire fence is used: at device
// scope they write back / invalidate the XCD's whole L2.
#pragma once

#include "device.h"
#include "kernels.h"

namespace mhcb {

// The empty marker: no value written here has this bit pattern.  As two
// binary32 words it is a NaN payload that BF16-derived arithmetic never
// produces; as one binary64 it is the finite 2^1021 * 1.87, far above any
// sum of squares of BF16 values.  It is never used as a value: a wait that
// gives up replaces what it could not read by kPoison64.
constexpr uint32_t kSlotEmpty = 0x7FC0DEADu;
constexpr uint64_t kSlotEmpty64 = ((uint64_t)kSlotEmpty << 32) | kSlotEmpty;
// A NaN both as one binary64 and as two binary32 words.
constexpr uint64_t kPoison64 = 0x7FF800007FC00000ull;
// The epoch word of a token slot whose exchange gave up: the maximum, so the
// atomic-max advance of the other slices leaves it in place.
constexpr uint64_t kSlotBroken = ~0ull;

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
__device__ __forceinline__ void slot_store64(char *slot, int offset, double v) {
  slot_store_u64(slot, offset, __builtin_bit_cast(uint64_t, v));
}
// An atomic maximum whose result is not used (no return, no wait).
__device__ __forceinline__ void slot_max_u64(char *slot, int offset, uint64_t v) {
  __hip_atomic_fetch_max(reinterpret_cast<uint64_t *>(slot + offset), v, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
}

// The epoch word: the epoch E in bits 8..63, the slice count of the call
// that set it in bits 0..7; kSlotBroken once a wait on the slot gave up.
// Calls advance it with an atomic maximum, so a broken slot stays broken
// until mhcb_workspace_init: every later call's results for that token are
// NaN instead of sums of stale entries.
struct SlotCall {
  uint64_t epoch;
  int prev_slices;
  bool broken;
};
__device__ __forceinline__ SlotCall unpack_call(uint64_t w) {
  return SlotCall{w >> 8, (int)(w & 0xffu), w == kSlotBroken};
}
__device__ __forceinline__ uint64_t slot_call_word(const char *slot) {
  return slot_load_u64(slot, kSlotEpoch);
}
// Where copy epoch % 2 of the exchange area starts.
__device__ __forceinline__ int copy_offset(uint64_t epoch) {
  return kSlotCopy0 + (int)(epoch & 1u) * kCopyBytes;
}
// After this slice's last read of the call's exchanges.
__device__ __forceinline__ void advance_epoch(char *slot, const SlotCall &c, int slices) {
  if (!c.broken) slot_max_u64(slot, kSlotEpoch, ((c.epoch + 1u) << 8) | (uint64_t)slices);
}
__device__ __forceinline__ void mark_broken(char *slot) { slot_max_u64(slot, kSlotEpoch, kSlotBroken); }

// The 8-byte words of one slot's clearing: the entries of kMaxSlices slices
// (both sums and the rows).
constexpr int kClearWords = 2 * kMaxSlices + kMaxSlices * kRowsEntry / 8;

// Word w (< kClearWords) of a slot's clearing: the empty marker goes back
// into the entries of slices [0, c.prev_slices) of the copy the previous
// call used (nothing reads that copy in this call).  Words past those
// entries are skipped, and nothing is cleared in a broken slot.  Like every
// exchanged word, a device-scope store.
__device__ __forceinline__ void clear_previous_word(char *slot, const SlotCall &c, int w) {
  if (c.broken) return;
  const int prev = c.prev_slices, row_words = prev * (kRowsEntry / 8);
  int offset;
  if (w < prev) offset = kCopySum1 + 8 * w;
  else if (w < 2 * prev) offset = kCopySum2 + 8 * (w - prev);
  else if (w < 2 * prev + row_words) offset = kCopyRows + 8 * (w - 2 * prev);
  else return;
  slot_store_u64(slot, copy_offset(c.epoch + 1u) + offset, kSlotEmpty64);
}

// The workspace's spin limit, read only once a wait has found a value
// missing (the fast path never loads it).
__device__ __forceinline__ int64_t spin_limit_of(const SyncView &sy) {
  const int64_t v = __hip_atomic_load(sy.limit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v > 0 ? v : kDefaultSpin;
}

// One more round of a bounded wait: false once the workspace's spin limit of
// re-reads has passed, so every wave exits; then the time-out is counted in
// the status word and the token's slot is marked broken.
__device__ __forceinline__ bool spin_again(const SyncView &sy, char *slot, int64_t &spins,
                                           int64_t &limit) {
  if (spins == 0) limit = spin_limit_of(sy);
  if (++spins > limit) {
    atomicAdd(sy.status, 1u);
    mark_broken(slot);
    return false;
  }
  __builtin_amdgcn_s_sleep(2);
  return true;
}

// The 8-byte entries at `offset + step * q` (q < slices <= kMaxSlices) of
// this call's copy of the slot's exchange area, once all are written: every
// load of a round is issued before any is tested.  In a broken slot, or for
// an entry still empty when the wait gives up, the entry reads kPoison64.
__device__ __forceinline__ void gather64(const SyncView &sy, char *slot, const SlotCall &c,
                                         int offset, int step, int slices,
                                         uint64_t (&w)[kMaxSlices]) {
  const char *area = slot + copy_offset(c.epoch);
  int64_t spins = 0, limit = 0;
  for (;;) {
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q)
      w[q] = c.broken ? kPoison64 : q < slices ? slot_load_u64(area, offset + step * q) : 0;
    bool missing = false;
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q) missing |= q < slices && w[q] == kSlotEmpty64;
    if (!missing) return;
    if (!spin_again(sy, slot, spins, limit)) {
#pragma unroll
      for (int q = 0; q < kMaxSlices; ++q) w[q] = w[q] == kSlotEmpty64 ? kPoison64 : w[q];
      return;
    }
  }
}

// Binary64 entries (8 bytes apart) added in slice order.
__device__ __forceinline__ double gather_sum64(const SyncView &sy, char *slot, const SlotCall &c,
                                               int offset, int slices) {
  uint64_t w[kMaxSlices];
  gather64(sy, slot, c, offset, 8, slices, w);
  double total = 0.0;
#pragma unroll
  for (int q = 0; q < kMaxSlices; ++q)
    if (q < slices) total += __builtin_bit_cast(double, w[q]);
  return total;
}

// gather_sum64 by a whole wave, lane q reading slice q's entry (the
// registers of a one-thread gather of 16 entries would set the kernel's
// register budget); every lane returns the slice-ordered total.  Called by
// all lanes of the wave with the same arguments.
__device__ __forceinline__ double wave_gather_sum64(const SyncView &sy, char *slot,
                                                    const SlotCall &c, int offset, int slices) {
  const int lane = threadIdx.x & (kWave - 1);
  if (c.broken) return __builtin_bit_cast(double, kPoison64);
  const char *area = slot + copy_offset(c.epoch);
  uint64_t v = 0;
  int64_t spins = 0, limit = 0;
  for (;;) {
    if (lane < slices) v = slot_load_u64(area, offset + 8 * lane);
    if (!__any(lane < slices && v == kSlotEmpty64)) break;
    if (spins == 0) limit = spin_limit_of(sy);
    if (++spins > limit) {  // uniform over the wave
      if (lane == 0) {
        atomicAdd(sy.status, 1u);
        mark_broken(slot);
      }
      if (v == kSlotEmpty64) v = kPoison64;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  double total = 0.0;
  for (int q = 0; q < slices; ++q) {
    const uint32_t l = __builtin_amdgcn_readlane((int)(uint32_t)v, q);
    const uint32_t h = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), q);
    total += __builtin_bit_cast(double, ((uint64_t)h << 32) | l);
  }
  return total;
}

}  // namespace mhcb
