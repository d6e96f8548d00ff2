// Internal launch interface of the DSA indexer projection between the
// C-ABI layer (api.hip) and indexer.hip.  Arguments are validated by the
// caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhcb {

// DSA indexer projection: x [M, K] times w [rows, K], rows = key + heads +
// gate (key rows, head-weight rows, gate rows).
struct IndexerArgs {
  const uint16_t *x, *w;
  uint16_t *key_out;     // [M, key] BF16
  float *heads_out;      // [M, heads] FP32
  uint16_t *gate_out;    // [M, gate] BF16
  float *parts;          // FP32 partials per K range and output block (splits > 1)
  uint32_t *counters;    // one per output block, zero between calls (splits > 1)
  int M, K, key, heads, gate, rows;
};
constexpr int kIndexerGemvMaxM = 6;  // tokens of the one-workgroup-per-row form, at most
constexpr int kIndexerCounters = 1024;  // output blocks of a call with K ranges, at most
// The launch shape of one projection: output blocks of tt token tiles x rt
// row tiles, K cut into `splits` ranges, and the workspace that needs.
struct IndexerPlan {
  int gemv;              // 4 or 8: one workgroup per weight row, that many tokens at most; 0: MFMA blocks
  int tt, rt, groups, row_groups, blocks, splits, waves;
  int64_t counter_bytes, workspace_bytes;
};
IndexerPlan plan_indexer(int M, int K, int rows, int cus, bool workspace);
hipError_t launch_indexer(const IndexerArgs &a, const IndexerPlan &p, hipStream_t stream);

}  // namespace mhcb
