// Cross-workgroup exchange of the token-split kernels, in the caller's
// workspace (slot layout in kernels.h).
//
// A token slot holds an epoch word (E = split calls that used the slot, and
// the slice count of the last of them) and two copies of the exchange area.
// A call uses copy E % 2.  At the start of that call, every word of that
// copy holds the empty marker kSlotEmpty:
//   - every slice reads the epoch word at its start, off the critical path;
//   - a slice stores its values in its entries of copy E % 2 and reads the
//     other slices' entries, re-reading (bounded) while any is still empty:
//     a value that is no longer empty has landed, so the wait costs about one
//     device-scope round trip after the slowest slice's store;
//   - after its last read it stores (E + 1, its slice count) into the epoch
//     word (every slice stores the same value; no return value, no wait).
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
// Exchanged words are accessed with device-scope (sc1) atomics, performed at
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
__device__ __forceinline__ void slot_store64(char *slot, int offset, double v) {
  slot_store_u64(slot, offset, __builtin_bit_cast(uint64_t, v));
}

// The epoch word: the epoch E in the low half, the slice count of the call
// that set it in the high half.
struct SlotCall {
  uint32_t epoch;
  int prev_slices;
};
__device__ __forceinline__ SlotCall unpack_call(uint64_t w) {
  return SlotCall{(uint32_t)w, (int)(uint32_t)(w >> 32)};
}
__device__ __forceinline__ uint64_t slot_call_word(const char *slot) {
  return slot_load_u64(slot, kSlotEpoch);
}
// Where copy epoch % 2 of the exchange area starts.
__device__ __forceinline__ int copy_offset(uint32_t epoch) {
  return kSlotCopy0 + (int)(epoch & 1u) * kCopyBytes;
}
// After this slice's last read of the call's exchanges.
__device__ __forceinline__ void advance_epoch(char *slot, const SlotCall &c, int slices) {
  slot_store_u64(slot, kSlotEpoch, ((uint64_t)(uint32_t)slices << 32) | (c.epoch + 1u));
}

// The 8-byte words of one slot's clearing: the entries of kMaxSlices slices
// (both sums and the rows).
constexpr int kClearWords = 2 * kMaxSlices + kMaxSlices * kRowsEntry / 8;

// Word w (< kClearWords) of a slot's clearing: the empty marker goes back
// into the entries of slices [0, c.prev_slices) of the copy the previous
// call used (nothing reads that copy in this call).  Words past those
// entries are skipped.  Like every exchanged word, a device-scope store.
__device__ __forceinline__ void clear_previous_word(char *slot, const SlotCall &c, int w) {
  const int prev = c.prev_slices, row_words = prev * (kRowsEntry / 8);
  int offset;
  if (w < prev) offset = kCopySum1 + 8 * w;
  else if (w < 2 * prev) offset = kCopySum2 + 8 * (w - prev);
  else if (w < 2 * prev + row_words) offset = kCopyRows + 8 * (w - 2 * prev);
  else return;
  slot_store_u64(slot, copy_offset(c.epoch + 1u) + offset, kSlotEmpty64);
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

// The 8-byte entries at `offset + step * q` (q < slices <= kMaxSlices) of
// `area`, once all are written: every load of a round is issued before any
// is tested.
__device__ __forceinline__ void gather64(const SyncView &sy, const char *area, int offset, int step,
                                         int slices, uint64_t (&w)[kMaxSlices]) {
  int64_t spins = 0;
  for (;;) {
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q) w[q] = q < slices ? slot_load_u64(area, offset + step * q) : 0;
    bool missing = false;
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q) missing |= q < slices && w[q] == kSlotEmpty64;
    if (!missing || !spin_again(sy, spins)) return;
  }
}

// Binary64 entries (8 bytes apart) added in slice order.
__device__ __forceinline__ double gather_sum64(const SyncView &sy, const char *area, int offset,
                                               int slices) {
  uint64_t w[kMaxSlices];
  gather64(sy, area, offset, 8, slices, w);
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
__device__ __forceinline__ double wave_gather_sum64(const SyncView &sy, const char *area, int offset,
                                                    int slices) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t v = 0;
  int64_t spins = 0;
  for (;;) {
    if (lane < slices) v = slot_load_u64(area, offset + 8 * lane);
    if (!__any(lane < slices && v == kSlotEmpty64)) break;
    if (++spins > sy.spin_limit) {  // uniform over the wave
      if (lane == 0) atomicAdd(sy.status, 1u);
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
