// One rank's MoE finalize contribution to a 16-byte fragment, shared by the
// per-token boundary kernels and the GLM stream pass.  Nothing here is
// shared with the CPU oracle.
#pragma once

#include "device.h"
#include "kernels.h"

namespace mhcb {

// One rank's MoE finalize contribution to a fragment
// (_QuadFinalizePublishDeviceKernel.kernel): acc = 0; for k ascending, a
// route with a valid row adds fma(row[k], w[k], acc); then + shared; BF16;
// negative zero -> +0.  Rows outside [0, rows) (e.g. -1: expert not held by
// this rank) are skipped.
__device__ __forceinline__ u32x4 finalize_fragment(const FinalizeView &f, const int32_t *srow,
                                                   const float *sw, int r, int t, int H,
                                                   int64_t col) {
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  const uint16_t *g = f.gemm2 + r * f.g_stride + col;
  u32x4 sh = load_stream(f.shared + r * f.s_stride + (int64_t)t * H + col);
  for (int k0 = 0; k0 < f.top_k; k0 += 8) {
    u32x4 rows[8];
    bool ok[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + i;
      const int32_t row = k < f.top_k ? srow[k] : -1;
      ok[i] = row >= 0 && row < f.rows;
      rows[i] = ok[i] ? load_stream(g + (int64_t)row * H) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (!ok[i]) continue;
      const float w = sw[k0 + i];
      float v[8];
      unpack8(rows[i], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(v[e], w, acc[e]);
    }
  }
  float s[8];
  unpack8(sh, s);
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = acc[e] + s[e];
  return sanitize4(pack8(acc));
}

}  // namespace mhcb
