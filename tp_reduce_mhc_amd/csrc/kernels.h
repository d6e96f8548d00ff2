// Internal launch interface between the C-ABI layer (api.hip) and the
// kernel translation units.  Arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhcb {

// Where a token's tp contributions come from.
enum class Source : int {
  kPartials = 0,   // tp BF16 [M, H] arrays, rank_stride elements apart
  kMailbox = 1,    // the ACTIVE generation of a Lamport mailbox (polled)
  kFinalize = 2,   // MoE finalize: top-k weighted expert rows + shared expert
};

struct MailboxView {
  uint16_t *slots;       // [3][tp][capacity][H]
  int32_t *stage_state;  // [ACTIVE, NEXT]
  int32_t *status;       // [2]: polls that gave up, fragments that were re-read
  int capacity;
  int64_t spin_limit;
};

struct FinalizeView {
  const uint16_t *gemm2;  // per rank [rows, H], g_stride elements apart
  int64_t g_stride, rows;
  const void *weights;    // per rank [M, top_k], w_stride apart (0 = shared):
  int64_t w_stride;       //   FP32, or BF16 bit patterns when w_bf16
  int w_bf16;
  float w_scale;          // routed scaling factor (1 = none)
  const int32_t *idx;     // per rank [M, top_k], i_stride apart (0 = shared)
  int64_t i_stride;
  const uint16_t *shared; // per rank [M, H], s_stride apart
  int64_t s_stride;
  int top_k;
};

// Cross-workgroup state of the token-split kernels, at the start of the
// caller's workspace: a 256-byte header (status word), then one 4 KiB slot
// per token, so that different tokens' words never share a cache line.  A
// slot holds (sync.h):
//   +0     epoch word: split calls that used the slot (low 32 bits) and the
//          slice count of the last of them (high 32 bits)
//   +128   copy 0 of the exchange area, +1920 copy 1, each:
//            +0    [kMaxSlices] binary64  first partial sum per slice
//            +128  [kMaxSlices] binary64  second partial sum per slice
//            +256  [kMaxSlices][24] FP32  partial GEMV rows per slice
// mhcb_workspace_init writes the epoch words 0 and every other word of the
// slots kSlotEmpty.
constexpr int kSyncTokens = 1024;  // tokens a split call may have
constexpr int kMaxSlices = 16;     // workgroups a token may be split over
constexpr int kSyncSlot = 4096;    // bytes per token
constexpr int kSlotEpoch = 0, kSlotCopy0 = 128;
constexpr int kCopySum1 = 0, kCopySum2 = 128, kCopyRows = 256;
constexpr int kRowsEntry = 4 * 24;  // bytes per slice in the rows
constexpr int kCopyBytes = kCopyRows + kMaxSlices * kRowsEntry;  // 1792, a multiple of 128
static_assert(kCopySum2 == kCopySum1 + 8 * kMaxSlices && kCopyRows == kCopySum2 + 8 * kMaxSlices,
              "copy layout");
static_assert(kCopyBytes % 128 == 0 && kSlotCopy0 + 2 * kCopyBytes <= kSyncSlot, "slot layout");
constexpr int64_t kSyncBytes = 256 + (int64_t)kSyncSlot * kSyncTokens;

// Two-pass GLM tiles keep their per-(token, slice) partials after the sync
// state (workspace + kSyncBytes): [tokens][slices][kPartWords] FP32 words,
// the 24 GEMV rows, then the binary64 sum of squares at word 24.  The area
// is plain scratch: the first pass writes every word the second pass reads.
constexpr int kPartWords = 32;
constexpr int kPartSum = 24;        // word offset of the binary64 sum
constexpr int kGlmMaxParts = 64;    // slices of at least 16 fragments, H <= 8192
constexpr int kGlmTileRoutes = 128; // tp * top_k a two-pass MoE tile stages in LDS
constexpr int64_t kGlmPartBytes = (int64_t)kSyncTokens * kGlmMaxParts * kPartWords * 4;  // 8 MiB

// The workspace header (its first 256 bytes): the time-out count, then the
// spin limit of the cross-workgroup waits (re-reads before a wait gives up;
// 0 or less: kDefaultSpin), which mhcb_workspace_set_spin_limit writes.
constexpr int kHeaderStatus = 0, kHeaderSpinLimit = 8;
constexpr int64_t kDefaultSpin = 1 << 20;  // about a second of polling

struct SyncView {
  uint32_t *status;       // header: cross-workgroup waits that gave up
  const int64_t *limit;   // header: spin limit
  char *slots;            // [kSyncTokens][kSyncSlot]
};

struct BoundaryArgs {
  Source source;
  int slices;        // workgroups per token (1 = no cross-workgroup sync)
  int slice_frags;   // fragments per workgroup when slices > 1
  SyncView sync;
  const uint16_t *partials;
  int64_t rank_stride;
  MailboxView mailbox;
  FinalizeView fin;
  int tp;
  int hc;                    // residual streams: 1, 2, 4 or 8
  const uint16_t *residual;  // [M, hc, H]
  const float *post;         // [M, hc]
  const float *comb;         // [M, hc, hc] [source][target]
  const float *pre;          // [M, hc] or null (residual only)
  const uint16_t *gamma;     // [H] or null
  uint16_t *residual_out;    // [M, 4, H]
  uint16_t *layer_input;     // [M, H] or null
  uint8_t *mx_values;        // [M, H] or null
  uint8_t *mx_scales;        // swizzled scales or null
  int M, H;
  float norm_eps;
};

hipError_t launch_boundary(const BoundaryArgs &a, hipStream_t stream);

// Every rank's finalize contribution into own[t % owners][rank][t / owners][H]:
// the two-shot owner mailboxes (owners = tp) or the rank-major published
// contributions (owners = 1).  Then, two-shot, the owners' reduced sums.
hipError_t launch_finalize_to_owners(const FinalizeView &fin, int tp, int owners, int M, int H,
                                     uint16_t *own, hipStream_t stream);
hipError_t launch_owner_reduce(const uint16_t *own, int tp, int M, int H, uint16_t *reduced,
                               hipStream_t stream);

hipError_t launch_mailbox_init(const MailboxView &mb, int tp, int H, hipStream_t stream);
hipError_t launch_publish(const MailboxView &mb, int tp, int H, const uint16_t *partials,
                          int64_t rank_stride, int rank_begin, int rank_count, int M,
                          hipStream_t stream);

hipError_t launch_quant_mxfp8(const uint16_t *x, uint8_t *values, uint8_t *scales, int M, int H,
                              hipStream_t stream);

struct GlmArgs {
  int slices;        // workgroups per token group (1 = no cross-workgroup sync)
  int slice_frags;   // fragments per workgroup when slices > 1
  SyncView sync;
  const uint16_t *partials;
  int64_t rank_stride;
  int tp;
  const uint16_t *residual;
  const float *post, *comb;
  const uint16_t *fn;        // [24, 4H]
  const float *scale, *base; // [3], [24]
  const uint16_t *gamma;
  uint16_t *residual_out;
  float *mixes_out;          // [M, 24]
  uint16_t *layer_input;
  int M, H;
  float rms_eps, hc_eps, norm_eps;
  int tokens_per_wg;         // 1, 2 or 4
  float *parts;              // two-pass tiles: [M][slices][kPartWords] partials
  FinalizeView fin;          // two-pass tiles of an MoE sublayer (gemm2 NULL: partials)
};

hipError_t launch_boundary_glm(const GlmArgs &a, hipStream_t stream);
// 16-token tiles on the matrix cores; always split (a.slices >= 1 with a
// sync view), at most kSyncTokens tokens per launch.
constexpr int kGlmTileTokens = 16;
hipError_t launch_boundary_glm_tile(const GlmArgs &a, hipStream_t stream);
// The same tiles in two passes (stream, then finish), exchanging nothing:
// a.slices x a.slice_frags cover the hidden size, a.parts is the scratch.
hipError_t launch_boundary_glm_two_pass(const GlmArgs &a, hipStream_t stream);

hipError_t launch_mixes(const float *mixes, const float *scale, const float *base, float *post_out,
                        float *comb_out, int M, float hc_eps, float post_mult, int repeat,
                        hipStream_t stream);

// Launch geometry of a workgroup covering `frags` 16-byte fragments
// (1, 2 or 4 of them per thread, at most 512 threads; with `wide`, one per
// thread up to 1024 threads).
struct Geometry {
  int trips, threads;
};
Geometry fragment_geometry(int frags, int wide_threads = 0);
inline Geometry token_geometry(int H) { return fragment_geometry(H / 8); }

hipError_t launch_zero(void *p, int64_t bytes, hipStream_t stream);
hipError_t launch_sync_init(void *workspace, hipStream_t stream);
// Stream-ordered copy of `count` 32-bit words (status reads that never
// synchronize), and a store of one 64-bit word.
hipError_t launch_copy_words(const uint32_t *src, uint32_t *dst, int count, hipStream_t stream);
hipError_t launch_store_word64(int64_t *dst, int64_t value, hipStream_t stream);

}  // namespace mhcb
