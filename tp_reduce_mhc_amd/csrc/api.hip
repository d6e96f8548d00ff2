// The C ABI of libmhcb: argument validation (before any launch or state
// write, as AllReduceMHC._consumer on the DSV4.1 page requires) and dispatch
// to the gfx950 kernels.  Host code only.
#include <stdarg.h>
#include <stdio.h>

#include <cmath>
#include <mutex>

#include "../../include/mhcb.h"
#include "device.h"
#include "kernels.h"
#include "indexer.h"

using namespace mhcb;

// Scratch of mhcb_boundary_glm_noalloc, for callers that cannot allocate:
// a file-scope device array, one copy per GPU the library runs on, held
// until the process ends.  Host code never passes `scratch` itself to a
// kernel (on the host the name is only a stand-in): static_scratch() looks
// up each device's address once with hipGetSymbolAddress and keeps it.
constexpr int64_t kScratchBytes = mhcb::kGlmPartBytes;  // 8 MiB
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

thread_local char g_error[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_error[0] = '\0';
  return MHCB_OK;
}

int launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(MHCB_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kMaxHidden = 16384;
constexpr int kMaxHiddenGlm = 8192;
constexpr int kMaxTp = 64;
constexpr int kMaxRoutes = 1024;
constexpr int kGlmTileMinM = 256;  // automatic matrix-core tiles from this M
constexpr int kGlmTwoPassMinM = 1;  // automatic two-pass tiles from this M
constexpr int kIndexerMaxRows = 4096;
constexpr int kIndexerMaxK = 65536;

// Checks shared by the boundary variants ([DSV41] AllReduceMHC._check and
// _consumer, _LamportMHCDeviceKernel.__init__).
int check_common(const char *fn, const uint16_t *residual, const float *post, const float *comb,
                 const float *pre, const uint16_t *norm_weight, const uint16_t *residual_out,
                 const uint16_t *layer_input, const uint8_t *mx_values, const uint8_t *mx_scales,
                 int M, int H, int hc, int tp, bool any_hc) {
  if (M < 1) return fail(MHCB_EINVAL, "%s: M=%d is outside [1, capacity]", fn, M);
  if (any_hc ? (hc != 1 && hc != 2 && hc != 4 && hc != 8) : hc != kStreams)
    return fail(MHCB_EUNSUPPORTED, "%s: hc_mult=%d (%s)", fn, hc, any_hc ? "1, 2, 4 or 8" : "only 4");
  if (H <= 0 || H % kFrag) return fail(MHCB_EUNSUPPORTED, "%s: hidden_size=%d must be a positive multiple of 8", fn, H);
  if (H > kMaxHidden) return fail(MHCB_EUNSUPPORTED, "%s: hidden_size=%d exceeds %d", fn, H, kMaxHidden);
  if (tp < 1 || tp > kMaxTp) return fail(MHCB_EINVAL, "%s: tp=%d is outside [1, %d]", fn, tp, kMaxTp);
  if (!residual || !post || !comb || !residual_out)
    return fail(MHCB_EINVAL, "%s: residual, post, comb and residual_out are required", fn);
  if ((pre == nullptr) != (norm_weight == nullptr))
    return fail(MHCB_EINVAL, "%s: pre and norm_weight are both given or both NULL", fn);
  if ((pre == nullptr) != (layer_input == nullptr))
    return fail(MHCB_EINVAL, "%s: layer_input is required exactly when pre is given", fn);
  if ((mx_values == nullptr) != (mx_scales == nullptr))
    return fail(MHCB_EINVAL, "%s: mxfp8_values and mxfp8_scales are both given or both NULL", fn);
  if (mx_values && !pre) return fail(MHCB_EINVAL, "%s: a residual-only boundary has no layer input", fn);
  if (mx_values && H % 128)
    return fail(MHCB_EUNSUPPORTED, "%s: MXFP8 output needs hidden_size %% 128 == 0 (got %d)", fn, H);
  if (!aligned(residual, 16) || !aligned(residual_out, 16) || (norm_weight && !aligned(norm_weight, 16)) ||
      (layer_input && !aligned(layer_input, 16)) || (mx_values && !aligned(mx_values, 8)) ||
      (mx_scales && !aligned(mx_scales, 4)) || !aligned(post, 4) || !aligned(comb, 4) ||
      (pre && !aligned(pre, 4)))
    return fail(MHCB_EALIGN, "%s: BF16 tensors must be 16-byte aligned, FP32 4-byte", fn);
  return MHCB_OK;
}

int check_mailbox(const char *fn, const mhcb_mailbox *mb, int H, int tp, int M) {
  if (!mb->slots || !mb->stage_state || !mb->status)
    return fail(MHCB_EINVAL, "%s: mailbox slots, stage_state and status are required", fn);
  if (mb->generations != 3) return fail(MHCB_EINVAL, "%s: mailbox generations=%d (must be 3)", fn, mb->generations);
  if (mb->tp != tp) return fail(MHCB_EINVAL, "%s: mailbox tp=%d but tp=%d", fn, mb->tp, tp);
  if (mb->hidden_size != H) return fail(MHCB_EINVAL, "%s: mailbox hidden_size=%d but hidden_size=%d", fn, mb->hidden_size, H);
  if (mb->capacity < 1) return fail(MHCB_EINVAL, "%s: mailbox capacity=%d", fn, mb->capacity);
  if (M > mb->capacity) return fail(MHCB_EINVAL, "%s: M=%d is outside [1, %d]", fn, M, mb->capacity);
  if (!aligned(mb->slots, 16) || !aligned(mb->stage_state, 4) || !aligned(mb->status, 4))
    return fail(MHCB_EALIGN, "%s: mailbox slots must be 16-byte aligned", fn);
  return MHCB_OK;
}

thread_local int g_slices_override = 0;  // mhcb_set_token_slices (0 = automatic), per calling thread

// Compute units of the current device (cached per device).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Checks a workspace argument: NULL, or at least `need` bytes, 256-byte
// aligned (its first kSyncBytes hold the cross-workgroup sync state).
int check_workspace(const char *fn, const void *ws, int64_t bytes, int64_t need) {
  if (!ws) return MHCB_OK;
  if (bytes < need)
    return fail(MHCB_EINVAL, "%s: workspace_bytes=%lld < %lld (mhcb_workspace_bytes)", fn,
                (long long)bytes, (long long)need);
  if (!aligned(ws, 256)) return fail(MHCB_EALIGN, "%s: workspace must be 256-byte aligned", fn);
  return MHCB_OK;
}

SyncView sync_view(void *ws) {
  char *b = static_cast<char *>(ws);
  SyncView v;
  v.status = reinterpret_cast<uint32_t *>(b + kHeaderStatus);
  v.limit = reinterpret_cast<const int64_t *>(b + kHeaderSpinLimit);
  v.slots = b + 256;
  return v;
}

// Workgroups per token: with a workspace and few tokens, the token's
// fragments are spread over up to `max_slices` workgroups (at least one
// wave of fragments each; slices cover whole 32-column blocks) until there
// are about `target` workgroups in flight, for fewer than `split_below`
// tokens.  Measured on MI355X (H=5120, tp=8): 4 slices save 0.5-0.8 us per
// call for M <= 64 (M=1: 4.9 vs 5.7 us, M=64: 6.0 vs 6.5); at M=128, 2
// slices cost 0.3 us more than none.
void choose_slices(BoundaryArgs &a, void *ws, int target, int max_slices, int split_below = 128) {
  a.slices = 1;
  a.slice_frags = a.H / kFrag;
  if (!ws || a.M > kSyncTokens) return;
  const int F = a.H / kFrag;
  int S = g_slices_override > 0 ? g_slices_override : (a.M < split_below ? target / a.M : 1);
  if (g_slices_override <= 0 && S > max_slices) S = max_slices;
  const int cap = g_slices_override > 0 ? F / 4 : F / kWave;
  S = S < 1 ? 1 : S;
  S = S > kMaxSlices ? kMaxSlices : S;
  S = S > cap ? cap : S;
  if (S <= 1) return;
  int frags = (F + S - 1) / S;
  frags = (frags + 3) / 4 * 4;
  a.slices = (F + frags - 1) / frags;
  a.slice_frags = frags;
  if (a.slices > 1) a.sync = sync_view(ws);
}

// The per-slice partials of the two-pass GLM tiles in a workspace: after
// its sync state.
float *workspace_parts(void *workspace) {
  return reinterpret_cast<float *>(static_cast<char *>(workspace) + kSyncBytes);
}

// The two-pass GLM tiles on validated arguments: slices of sf fragments (a
// multiple of 4, 16..64), partials in `parts` (kGlmPartBytes, reused by
// every launch), launches of at most kSyncTokens tokens.
int glm_two_pass(const char *fn, const uint16_t *partials, int64_t rank_stride,
                 const uint16_t *residual, const float *post, const float *comb,
                 const uint16_t *hc_fn, const float *scale, const float *base,
                 const uint16_t *norm_weight, uint16_t *residual_out, float *mixes_out,
                 uint16_t *layer_input, float *parts, int M, int hidden_size, int tp,
                 float rms_eps, float hc_eps, float norm_eps, const FinalizeView *fin,
                 hipStream_t stream) {
  const int F = hidden_size / kFrag;
  // Slices of 16 fragments up to M = 64, 32 beyond (M=64: 12.6 vs 13.2
  // us; M=128: 14.4 vs 15.1; M=1024: 56.7 vs 60.8).
  int sf = M <= 64 ? 16 : 32;
  if (g_slices_override > 0) sf = (F + g_slices_override - 1) / g_slices_override;
  sf = (sf + 3) / 4 * 4;
  sf = sf < 16 ? 16 : sf > 64 ? 64 : sf;
  GlmArgs a = {(F + sf - 1) / sf, sf, SyncView{}, partials, rank_stride, tp, residual, post, comb,
               hc_fn, scale, base, norm_weight, residual_out, mixes_out, layer_input, M,
               hidden_size, rms_eps, hc_eps, norm_eps, kGlmTileTokens, parts};
  if (fin) a.fin = *fin;  // the ranks' contributions from MoE routes (partials unused)
  const int64_t H = hidden_size;
  for (int c = 0; c < M; c += kSyncTokens) {
    GlmArgs b = a;
    b.M = M - c < kSyncTokens ? M - c : kSyncTokens;
    b.partials = partials + c * H;
    b.residual = residual + c * kStreams * H;
    b.post = post + (int64_t)c * kStreams;
    b.comb = comb + (int64_t)c * kStreams * kStreams;
    b.residual_out = residual_out + c * kStreams * H;
    b.mixes_out = mixes_out + (int64_t)c * kMix;
    b.layer_input = layer_input + c * H;
    if (fin) {  // this launch's tokens of the routes and shared rows
      const int64_t k = fin->top_k;
      b.partials = nullptr;
      b.fin.weights = static_cast<const char *>(fin->weights) + c * k * (fin->w_bf16 ? 2 : 4);
      b.fin.idx = fin->idx + c * k;
      b.fin.shared = fin->shared + c * H;
    }
    const int rc = launched(launch_boundary_glm_two_pass(b, stream), fn);
    if (rc) return rc;
  }
  return ok();
}

// Checks the MoE routing arguments shared by the finalize entry points
// ([DSV41] AllReduceMHC.finalize) and fills the view.
int check_routes(const char *fn, const uint16_t *gemm2_permuted, int64_t gemm2_rank_stride,
                 int64_t rows, const void *expert_weights, int64_t weights_rank_stride,
                 int weights_bf16, float routed_scaling_factor, const int32_t *permuted_idx,
                 int64_t idx_rank_stride, const uint16_t *shared_output,
                 int64_t shared_rank_stride, int tp, int top_k, FinalizeView *f) {
  if (top_k < 1) return fail(MHCB_EINVAL, "%s: top_k=%d < 1", fn, top_k);
  if (weights_bf16 != 0 && weights_bf16 != 1)
    return fail(MHCB_EINVAL, "%s: weights_bf16=%d (0 = FP32, 1 = BF16)", fn, weights_bf16);
  if (!std::isfinite(routed_scaling_factor))
    return fail(MHCB_EINVAL, "%s: routed_scaling_factor must be finite", fn);
  if ((int64_t)tp * top_k > kMaxRoutes)
    return fail(MHCB_EINVAL, "%s: tp * top_k = %d exceeds %d", fn, tp * top_k, kMaxRoutes);
  if (rows < 0) return fail(MHCB_EINVAL, "%s: rows=%lld < 0", fn, (long long)rows);
  if (!gemm2_permuted || !expert_weights || !permuted_idx || !shared_output)
    return fail(MHCB_EINVAL, "%s: gemm2_permuted, expert_weights, permuted_idx and shared_output are required", fn);
  if (gemm2_rank_stride < 0 || weights_rank_stride < 0 || idx_rank_stride < 0 || shared_rank_stride < 0)
    return fail(MHCB_EINVAL, "%s: negative rank stride", fn);
  if (!aligned(gemm2_permuted, 16) || !aligned(shared_output, 16) || gemm2_rank_stride % kFrag ||
      shared_rank_stride % kFrag)
    return fail(MHCB_EALIGN, "%s: BF16 inputs must be 16-byte aligned with rank strides %% 8 == 0", fn);
  if (!aligned(expert_weights, weights_bf16 ? 2 : 4) || !aligned(permuted_idx, 4))
    return fail(MHCB_EALIGN, "%s: expert_weights must be aligned to its element (4 bytes FP32, 2 BF16), permuted_idx to 4", fn);
  *f = FinalizeView{gemm2_permuted, gemm2_rank_stride, rows, expert_weights, weights_rank_stride,
                    weights_bf16, routed_scaling_factor, permuted_idx, idx_rank_stride,
                    shared_output, shared_rank_stride, top_k};
  return MHCB_OK;
}

// Checks of the GLM boundary's arguments ([GLM] AllReduceMhcBoundary.__call__),
// shared by its entry points.
int check_glm(const char *fn, const uint16_t *partials, int64_t rank_stride,
              const uint16_t *residual, const float *post, const float *comb,
              const uint16_t *hc_fn, const float *scale, const float *base,
              const uint16_t *norm_weight, const uint16_t *residual_out, const float *mixes_out,
              const uint16_t *layer_input, int M, int hidden_size, int hc_mult, int tp) {
  if (!partials || !hc_fn || !scale || !base || !norm_weight || !mixes_out || !layer_input)
    return fail(MHCB_EINVAL, "%s: partials, hc_fn, scale, base, norm_weight, mixes_out and layer_input are required", fn);
  // The GLM pre-mix is derived in-kernel from scale/base: check the normalized path.
  int rc = check_common(fn, residual, post, comb, scale, norm_weight, residual_out, layer_input,
                        nullptr, nullptr, M, hidden_size, hc_mult, tp, false);
  if (rc) return rc;
  if (hidden_size > kMaxHiddenGlm)
    return fail(MHCB_EUNSUPPORTED, "%s: hidden_size=%d exceeds %d", fn, hidden_size, kMaxHiddenGlm);
  if (tp > 1 && rank_stride < (int64_t)M * hidden_size && rank_stride != 0)
    return fail(MHCB_EINVAL, "%s: rank_stride=%lld overlaps a rank's [M, hidden] block", fn, (long long)rank_stride);
  if (!aligned(partials, 16) || rank_stride % kFrag || !aligned(hc_fn, 16) || !aligned(base, 4) ||
      !aligned(mixes_out, 4))
    return fail(MHCB_EALIGN, "%s: partials/hc_fn must be 16-byte aligned, rank_stride %% 8 == 0", fn);
  return MHCB_OK;
}

MailboxView view_of(const mhcb_mailbox *mb) {
  MailboxView v;
  v.slots = mb->slots;
  v.stage_state = mb->stage_state;
  v.status = mb->status;
  v.capacity = mb->capacity;
  v.spin_limit = mb->spin_limit > 0 ? mb->spin_limit : kDefaultSpin;
  return v;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on its first use).
int static_scratch(const char *fn, float **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MHCB_ELAUNCH, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MHCB_EUNSUPPORTED, "%s: device %d beyond the %d the library tracks", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MHCB_ELAUNCH, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<float *>(g_scratch_ptr[dev]);
  return MHCB_OK;
}

}  // namespace

extern "C" {

const char *mhcb_last_error(void) { return g_error; }

const char *mhcb_version(void) { return "0.1.0"; }

int64_t mhcb_mxfp8_scale_bytes(int64_t M, int64_t hidden_size) {
  if (M < 0 || hidden_size < 0) return -1;
  return (M + 127) / 128 * 128 * (hidden_size / 32);
}

int64_t mhcb_workspace_bytes(int M, int hidden_size, int tp, int two_shot) {
  if (M < 0 || hidden_size < 0 || tp < 1) return -1;
  // After the sync state: the two-shot owner areas, or the two-pass GLM
  // partials (never used by the same call, so they share the space).
  int64_t scratch = kGlmPartBytes;
  if (two_shot) {
    const int64_t slots = ((int64_t)M + tp - 1) / tp;
    const int64_t own = ((int64_t)tp * tp * slots + M) * hidden_size * 2;
    scratch = own > scratch ? own : scratch;
  }
  return kSyncBytes + scratch;
}

int mhcb_workspace_init(void *workspace, int64_t workspace_bytes, hipStream_t stream) {
  const char *fn = "mhcb_workspace_init";
  if (!workspace || workspace_bytes < kSyncBytes)
    return fail(MHCB_EINVAL, "%s: a workspace of at least %lld bytes is required", fn, (long long)kSyncBytes);
  if (!aligned(workspace, 256)) return fail(MHCB_EALIGN, "%s: workspace must be 256-byte aligned", fn);
  return launched(launch_sync_init(workspace, stream), fn);
}

int64_t mhcb_finalize_workspace_bytes(int M, int hidden_size, int tp, int two_shot) {
  return mhcb_workspace_bytes(M, hidden_size, tp, two_shot);
}

int mhcb_workspace_set_spin_limit(void *workspace, int64_t spin_limit, hipStream_t stream) {
  const char *fn = "mhcb_workspace_set_spin_limit";
  if (!workspace) return fail(MHCB_EINVAL, "%s: workspace is required", fn);
  if (!aligned(workspace, 256)) return fail(MHCB_EALIGN, "%s: workspace must be 256-byte aligned", fn);
  return launched(launch_store_word64(reinterpret_cast<int64_t *>(static_cast<char *>(workspace) +
                                                                  kHeaderSpinLimit),
                                      spin_limit, stream),
                  fn);
}

int mhcb_workspace_status(const void *workspace, uint32_t *status_out, hipStream_t stream) {
  const char *fn = "mhcb_workspace_status";
  if (!workspace || !status_out) return fail(MHCB_EINVAL, "%s: workspace and status_out are required", fn);
  if (!aligned(workspace, 256) || !aligned(status_out, 4))
    return fail(MHCB_EALIGN, "%s: workspace must be 256-byte aligned, status_out 4-byte", fn);
  return launched(launch_copy_words(static_cast<const uint32_t *>(workspace) + kHeaderStatus / 4,
                                    status_out, 1, stream),
                  fn);
}

int mhcb_set_token_slices(int slices) {
  const int previous = g_slices_override;
  g_slices_override = slices < 0 ? 0 : (slices > kGlmMaxParts ? kGlmMaxParts : slices);
  return previous;
}

int mhcb_boundary(const uint16_t *partials, int64_t rank_stride, const mhcb_mailbox *mailbox,
                  const uint16_t *residual, const float *post, const float *comb, const float *pre,
                  const uint16_t *norm_weight, uint16_t *residual_out, uint16_t *layer_input,
                  uint8_t *mxfp8_values, uint8_t *mxfp8_scales, void *workspace,
                  int64_t workspace_bytes, int M, int hidden_size, int hc_mult, int tp,
                  float norm_eps, hipStream_t stream) {
  const char *fn = "mhcb_boundary";
  int rc = check_common(fn, residual, post, comb, pre, norm_weight, residual_out, layer_input,
                        mxfp8_values, mxfp8_scales, M, hidden_size, hc_mult, tp, true);
  if (rc) return rc;
  if ((rc = check_workspace(fn, workspace, workspace_bytes, kSyncBytes))) return rc;
  if ((partials == nullptr) == (mailbox == nullptr))
    return fail(MHCB_EINVAL, "%s: give exactly one of partials and mailbox", fn);
  BoundaryArgs a = {};
  if (mailbox) {
    if ((rc = check_mailbox(fn, mailbox, hidden_size, tp, M))) return rc;
    a.source = Source::kMailbox;
    a.mailbox = view_of(mailbox);
  } else {
    if (tp > 1 && (rank_stride < (int64_t)M * hidden_size && rank_stride != 0))
      return fail(MHCB_EINVAL, "%s: rank_stride=%lld overlaps a rank's [M, hidden] block", fn,
                  (long long)rank_stride);
    if (!aligned(partials, 16) || rank_stride % kFrag)
      return fail(MHCB_EALIGN, "%s: partials must be 16-byte aligned with rank_stride %% 8 == 0", fn);
    a.source = Source::kPartials;
    a.partials = partials;
    a.rank_stride = rank_stride;
  }
  a.tp = tp;
  a.hc = hc_mult;
  a.residual = residual;
  a.post = post;
  a.comb = comb;
  a.pre = pre;
  a.gamma = norm_weight;
  a.residual_out = residual_out;
  a.layer_input = layer_input;
  a.mx_values = mxfp8_values;
  a.mx_scales = mxfp8_scales;
  a.M = M;
  a.H = hidden_size;
  a.norm_eps = norm_eps;
  choose_slices(a, workspace, device_cus(), 4);
  // H = 5120 with eight ranks, four streams and a layer input:
  //  - where four slices were chosen: five slices of 128 fragments (four
  //    columns a thread) while every slice of the call has a compute unit
  //    of its own.  Per call (us, four slices in brackets): M=1 4.16-4.33
  //    (4.72-4.75), 8 4.63 (5.28), 16 4.75 (5.33), 32 4.93-5.03
  //    (5.53-5.55), 51 5.43-5.48 (5.84-5.87); at M=64, 320 workgroups, 6.21
  //    (6.08).  Ten slices of 64 fragments (two columns a thread) were no
  //    faster up to M=25;
  //  - where two were chosen (86-127 tokens): none, the eight-wave form.
  //    Per call (us, two slices in brackets): M=90 6.36-6.39 (6.70-6.73),
  //    100 6.39-6.45 (6.80-6.82), 127 6.55-6.58 (7.21-7.28); with three
  //    slices (65-85 tokens) the split still wins or ties: M=72 6.15-6.17
  //    against 6.24-6.35 unsplit, M=80 6.24 against 6.26-6.27.
  if (g_slices_override <= 0 && a.tp == 8 && a.hc == kStreams && a.pre && a.H / kFrag == 640) {
    if (a.slices == 4 && 5 * a.M <= device_cus()) {
      a.slices = 5;
      a.slice_frags = 128;
    } else if (a.slices == 2) {
      a.slices = 1;
      a.slice_frags = a.H / kFrag;
    }
  }
  return launched(launch_boundary(a, stream), fn);
}

int mhcb_boundary_glm(const uint16_t *partials, int64_t rank_stride, const uint16_t *residual,
                      const float *post, const float *comb, const uint16_t *hc_fn, const float *scale,
                      const float *base, const uint16_t *norm_weight, uint16_t *residual_out,
                      float *mixes_out, uint16_t *layer_input, void *workspace,
                      int64_t workspace_bytes, int M, int hidden_size, int hc_mult, int tp,
                      float rms_eps, float hc_eps, float norm_eps, int tokens_per_wg,
                      hipStream_t stream) {
  const char *fn = "mhcb_boundary_glm";
  int rc = check_glm(fn, partials, rank_stride, residual, post, comb, hc_fn, scale, base,
                     norm_weight, residual_out, mixes_out, layer_input, M, hidden_size, hc_mult, tp);
  if (rc) return rc;
  if ((rc = check_workspace(fn, workspace, workspace_bytes, kSyncBytes))) return rc;
  int G = tokens_per_wg;
  // Automatic: two-pass tiles whenever the workspace holds their scratch
  // (measured on MI355X, H=6144, tp=8, us per call, the previous automatic
  // one-pass choice in brackets: M=1 9.4 (11.6), 16 11.7 (12.2), 64 12.6
  // (15.0), 128 14.4 (19.3), 256 19.4-20.0 (23.5), 512 31.8-32.0 (34.0),
  // 1024 56.7-58.0 (70.2)).
  if (G == 0 && workspace && workspace_bytes >= kSyncBytes + kGlmPartBytes && M >= kGlmTwoPassMinM)
    G = -kGlmTileTokens;
  if (G == -kGlmTileTokens) {
    const int64_t need = kSyncBytes + kGlmPartBytes;
    if (!workspace || workspace_bytes < need)
      return fail(MHCB_EINVAL, "%s: tokens_per_wg=-16 needs a workspace of %lld bytes", fn, (long long)need);
    return glm_two_pass(fn, partials, rank_stride, residual, post, comb, hc_fn, scale, base,
                        norm_weight, residual_out, mixes_out, layer_input,
                        workspace_parts(workspace), M, hidden_size, tp, rms_eps, hc_eps, norm_eps,
                        nullptr, stream);
  }
  // Measured on MI355X (H=6144, tp=8): one token per workgroup below M=256
  // (M=128: 18.8 us; 16-token tiles: 22.3), 16-token tiles from M=256
  // (24.8 us; one token: 25.7, two: 28.7) and beyond (M=512: 33.2 us; one
  // token: 47.1, two: 36.5).  Without a workspace, two tokens per workgroup
  // beyond M=256.
  if (G == 0) G = workspace && M >= kGlmTileMinM ? kGlmTileTokens : (M <= 256 ? 1 : 2);
  if (G != 1 && G != 2 && G != 4 && G != kGlmTileTokens)
    return fail(MHCB_EINVAL, "%s: tokens_per_wg=%d (0, 1, 2, 4, 16 or -16)", fn, tokens_per_wg);
  if (G == 4 && hidden_size > 6144)
    return fail(MHCB_EUNSUPPORTED, "%s: tokens_per_wg=4 needs hidden_size <= 6144", fn);
  if (G == kGlmTileTokens && !workspace)
    return fail(MHCB_EINVAL, "%s: tokens_per_wg=16 needs a workspace", fn);
  GlmArgs a = {1, hidden_size / kFrag, SyncView{}, partials, rank_stride, tp, residual, post, comb,
               hc_fn, scale, base, norm_weight, residual_out, mixes_out, layer_input, M,
               hidden_size, rms_eps, hc_eps, norm_eps, G};
  if (G == kGlmTileTokens) {
    // Slices of at most 96 fragments; launches of at most kSyncTokens
    // tokens.  16 slices while that gives at most one workgroup per compute
    // unit (M <= 256 on 256 units), else 8: measured on MI355X at H=6144,
    // M=256: 25.8 us (16) vs 28.8 us (8); M=512: 38.7 us (16) vs 33.2 us (8).
    const int F = hidden_size / kFrag;
    const int tiles = ((M < kSyncTokens ? M : kSyncTokens) + kGlmTileTokens - 1) / kGlmTileTokens;
    int S = g_slices_override > 0 ? g_slices_override
                                  : (tiles * kMaxSlices <= device_cus() ? kMaxSlices : 8);
    S = S > kMaxSlices ? kMaxSlices : S;
    S = S > F / 4 ? F / 4 : S;
    S = S < (F + 95) / 96 ? (F + 95) / 96 : S;
    S = S < 1 ? 1 : S;
    int frags = (F + S - 1) / S;
    frags = (frags + 3) / 4 * 4;
    a.slices = (F + frags - 1) / frags;
    a.slice_frags = frags;
    a.sync = sync_view(workspace);
    const int64_t H = hidden_size;
    for (int c = 0; c < M; c += kSyncTokens) {
      GlmArgs b = a;
      b.M = M - c < kSyncTokens ? M - c : kSyncTokens;
      b.partials = partials + c * H;
      b.residual = residual + c * kStreams * H;
      b.post = post + (int64_t)c * kStreams;
      b.comb = comb + (int64_t)c * kStreams * kStreams;
      b.residual_out = residual_out + c * kStreams * H;
      b.mixes_out = mixes_out + (int64_t)c * kMix;
      b.layer_input = layer_input + c * H;
      if ((rc = launched(launch_boundary_glm_tile(b, stream), fn))) return rc;
    }
    return ok();
  }
  // Slices per token group: measured on MI355X (H=6144, tp=8), one-wave
  // slices save about 3 us at M=1; at M=64 4 slices break even; larger M
  // is faster unsplit.  The choice depends on M only (not on
  // tokens_per_wg), so the results do not depend on tokens_per_wg.
  if (workspace && M <= kSyncTokens) {
    const int F = hidden_size / kFrag;
    // (Requested 16, i.e. 12 slices of one wave at H=6144: M=1 11.6 us,
    // M=16 12.5 us; 8 slices: 11.8 and 13.5; 4: 12.5 and 13.3.  M=64: 4
    // slices 15.0 us, 16 requested 16.6.)
    int S = g_slices_override > 0 ? g_slices_override : (M <= 16 ? 16 : M <= 64 ? 4 : 1);
    const int cap = F / kWave;
    S = S > kMaxSlices ? kMaxSlices : S;
    S = S > cap ? cap : S;
    if (S > 1) {
      int frags = (F + S - 1) / S;
      frags = (frags + 3) / 4 * 4;
      a.slices = (F + frags - 1) / frags;
      a.slice_frags = frags;
      if (a.slices > 1) a.sync = sync_view(workspace);
      else a.slice_frags = F;
    }
  }
  return launched(launch_boundary_glm(a, stream), fn);
}

int mhcb_boundary_glm_noalloc(const uint16_t *partials, int64_t rank_stride,
                              const uint16_t *residual, const float *post, const float *comb,
                              const uint16_t *hc_fn, const float *scale, const float *base,
                              const uint16_t *norm_weight, uint16_t *residual_out,
                              float *mixes_out, uint16_t *layer_input, int M, int hidden_size,
                              int hc_mult, int tp, float rms_eps, float hc_eps, float norm_eps,
                              hipStream_t stream) {
  const char *fn = "mhcb_boundary_glm_noalloc";
  int rc = check_glm(fn, partials, rank_stride, residual, post, comb, hc_fn, scale, base,
                     norm_weight, residual_out, mixes_out, layer_input, M, hidden_size, hc_mult, tp);
  if (rc) return rc;
  // The two-pass tiles' partials of one launch: at most kSyncTokens tokens
  // x kGlmMaxParts slices of kPartWords words; hidden_size <= 8192 keeps
  // the slices within kGlmMaxParts.
  const int64_t need = (int64_t)kSyncTokens * kGlmMaxParts * kPartWords * 4;
  if (need > kScratchBytes)
    return fail(MHCB_EINVAL, "%s: needs %lld bytes of scratch, the static array holds %lld", fn,
                (long long)need, (long long)kScratchBytes);
  float *parts = nullptr;
  if ((rc = static_scratch(fn, &parts))) return rc;
  return glm_two_pass(fn, partials, rank_stride, residual, post, comb, hc_fn, scale, base,
                      norm_weight, residual_out, mixes_out, layer_input, parts, M, hidden_size, tp,
                      rms_eps, hc_eps, norm_eps, nullptr, stream);
}

int64_t mhcb_finalize_glm_workspace_bytes(int M, int hidden_size, int tp) {
  if (M < 0 || hidden_size < 0 || tp < 1) return -1;
  return kSyncBytes + kGlmPartBytes + (int64_t)tp * M * hidden_size * 2;
}

int mhcb_finalize_glm(const uint16_t *gemm2_permuted, int64_t gemm2_rank_stride, int64_t rows,
                      const void *expert_weights, int64_t weights_rank_stride, int weights_bf16,
                      float routed_scaling_factor, const int32_t *permuted_idx,
                      int64_t idx_rank_stride, const uint16_t *shared_output,
                      int64_t shared_rank_stride, const uint16_t *residual, const float *post,
                      const float *comb, const uint16_t *hc_fn, const float *scale,
                      const float *base, const uint16_t *norm_weight, uint16_t *residual_out,
                      float *mixes_out, uint16_t *layer_input, void *workspace,
                      int64_t workspace_bytes, int M, int hidden_size, int hc_mult, int tp,
                      int top_k, float rms_eps, float hc_eps, float norm_eps, hipStream_t stream) {
  const char *fn = "mhcb_finalize_glm";
  if (!hc_fn || !scale || !base || !norm_weight || !mixes_out || !layer_input)
    return fail(MHCB_EINVAL, "%s: hc_fn, scale, base, norm_weight, mixes_out and layer_input are required", fn);
  int rc = check_common(fn, residual, post, comb, scale, norm_weight, residual_out, layer_input,
                        nullptr, nullptr, M, hidden_size, hc_mult, tp, false);
  if (rc) return rc;
  if (hidden_size > kMaxHiddenGlm)
    return fail(MHCB_EUNSUPPORTED, "%s: hidden_size=%d exceeds %d", fn, hidden_size, kMaxHiddenGlm);
  if (!aligned(hc_fn, 16) || !aligned(base, 4) || !aligned(mixes_out, 4))
    return fail(MHCB_EALIGN, "%s: hc_fn must be 16-byte aligned, base and mixes_out 4-byte", fn);
  FinalizeView f;
  if ((rc = check_routes(fn, gemm2_permuted, gemm2_rank_stride, rows, expert_weights,
                         weights_rank_stride, weights_bf16, routed_scaling_factor, permuted_idx,
                         idx_rank_stride, shared_output, shared_rank_stride, tp, top_k, &f)))
    return rc;
  const int64_t need = mhcb_finalize_glm_workspace_bytes(M, hidden_size, tp);
  if (!workspace)
    return fail(MHCB_EINVAL, "%s: a workspace of %lld bytes is required", fn, (long long)need);
  if ((rc = check_workspace(fn, workspace, workspace_bytes, need))) return rc;
  // Up to kGlmTileRoutes routes a token: the stream pass computes the
  // ranks' contributions itself.  Beyond: publish every rank's
  // contribution, rank-major after the two-pass partials, and run the GLM
  // boundary on them as its rank partials.
  if ((int64_t)tp * top_k <= kGlmTileRoutes)
    return glm_two_pass(fn, nullptr, 0, residual, post, comb, hc_fn, scale, base, norm_weight,
                        residual_out, mixes_out, layer_input, workspace_parts(workspace), M,
                        hidden_size, tp, rms_eps, hc_eps, norm_eps, &f, stream);
  uint16_t *contrib = reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) + kSyncBytes +
                                                   kGlmPartBytes);
  if ((rc = launched(launch_finalize_to_owners(f, tp, 1, M, hidden_size, contrib, stream), fn)))
    return rc;
  return glm_two_pass(fn, contrib, (int64_t)M * hidden_size, residual, post, comb, hc_fn, scale,
                      base, norm_weight, residual_out, mixes_out, layer_input,
                      workspace_parts(workspace), M, hidden_size, tp, rms_eps, hc_eps, norm_eps,
                      nullptr, stream);
}

int mhcb_mixes(const float *mixes, const float *scale, const float *base, float *post_out,
               float *comb_out, int M, int hc_mult, float hc_eps, float post_mult,
               int sinkhorn_repeat, hipStream_t stream) {
  const char *fn = "mhcb_mixes";
  if (M < 1) return fail(MHCB_EINVAL, "%s: M=%d < 1", fn, M);
  if (hc_mult != kStreams) return fail(MHCB_EUNSUPPORTED, "%s: hc_mult=%d (only 4)", fn, hc_mult);
  if (sinkhorn_repeat < 0) return fail(MHCB_EINVAL, "%s: sinkhorn_repeat=%d < 0", fn, sinkhorn_repeat);
  if (!mixes || !scale || !base || !post_out || !comb_out)
    return fail(MHCB_EINVAL, "%s: every pointer is required", fn);
  if (!aligned(mixes, 4) || !aligned(scale, 4) || !aligned(base, 4) || !aligned(post_out, 4) ||
      !aligned(comb_out, 4))
    return fail(MHCB_EALIGN, "%s: FP32 tensors must be 4-byte aligned", fn);
  return launched(launch_mixes(mixes, scale, base, post_out, comb_out, M, hc_eps, post_mult,
                               sinkhorn_repeat, stream), fn);
}

static int finalize_impl(const char *fn, const uint16_t *gemm2_permuted, int64_t gemm2_rank_stride,
                         int64_t rows, const void *expert_weights, int64_t weights_rank_stride,
                         int weights_bf16, float routed_scaling_factor,
                         const int32_t *permuted_idx, int64_t idx_rank_stride,
                         const uint16_t *shared_output, int64_t shared_rank_stride,
                         const uint16_t *residual, const float *post, const float *comb,
                         const float *pre, const uint16_t *norm_weight, uint16_t *residual_out,
                         uint16_t *layer_input, uint8_t *mxfp8_values, uint8_t *mxfp8_scales,
                         int two_shot, void *workspace, int64_t workspace_bytes, int M,
                         int hidden_size, int hc_mult, int tp, int top_k, float norm_eps,
                         hipStream_t stream) {
  int rc = check_common(fn, residual, post, comb, pre, norm_weight, residual_out, layer_input,
                        mxfp8_values, mxfp8_scales, M, hidden_size, hc_mult, tp, true);
  if (rc) return rc;
  FinalizeView f;
  if ((rc = check_routes(fn, gemm2_permuted, gemm2_rank_stride, rows, expert_weights,
                         weights_rank_stride, weights_bf16, routed_scaling_factor, permuted_idx,
                         idx_rank_stride, shared_output, shared_rank_stride, tp, top_k, &f)))
    return rc;
  BoundaryArgs a = {};
  a.tp = tp;
  a.hc = hc_mult;
  a.residual = residual;
  a.post = post;
  a.comb = comb;
  a.pre = pre;
  a.gamma = norm_weight;
  a.residual_out = residual_out;
  a.layer_input = layer_input;
  a.mx_values = mxfp8_values;
  a.mx_scales = mxfp8_scales;
  a.M = M;
  a.H = hidden_size;
  a.norm_eps = norm_eps;
  if (!two_shot) {
    if ((rc = check_workspace(fn, workspace, workspace_bytes, kSyncBytes))) return rc;
    a.source = Source::kFinalize;
    a.fin = f;
    // About one workgroup per compute unit, at most five a token, up to
    // half as many tokens as compute units.  Measured on MI355X (H=5120,
    // tp=4, top_k=8; us per call): M=64 4 slices 11.6, 2 12.6, 8 13.7;
    // M=32 5 slices 10.85, 4 11.0, 8 11.8; M=8 5 slices 10.4, 10 slices
    // 10.5, 8 11.5; M=128 2 slices 15.6, none 17.4; M=160 3 slices 18.1,
    // none 18.0, 2 26.4.
    const int cus = device_cus();
    choose_slices(a, workspace, cus, 5, cus / 2 + 1);
    return launched(launch_boundary(a, stream), fn);
  }
  const int64_t need = mhcb_workspace_bytes(M, hidden_size, tp, 1);
  if (!workspace)
    return fail(MHCB_EINVAL, "%s: the two-shot emulation needs a %lld-byte workspace", fn, (long long)need);
  if ((rc = check_workspace(fn, workspace, workspace_bytes, need))) return rc;
  uint16_t *own = reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) + kSyncBytes);
  const int64_t slots = ((int64_t)M + tp - 1) / tp;
  uint16_t *reduced = own + (int64_t)tp * tp * slots * hidden_size;
  hipError_t e = launch_finalize_to_owners(f, tp, tp, M, hidden_size, own, stream);
  if (e == hipSuccess) e = launch_owner_reduce(own, tp, M, hidden_size, reduced, stream);
  if (e != hipSuccess) return launched(e, fn);
  a.source = Source::kPartials;
  a.partials = reduced;
  a.rank_stride = 0;
  a.tp = 1;
  choose_slices(a, workspace, device_cus(), 4);
  return launched(launch_boundary(a, stream), fn);
}

int mhcb_finalize(const uint16_t *gemm2_permuted, int64_t gemm2_rank_stride, int64_t rows,
                  const float *expert_weights, int64_t weights_rank_stride,
                  const int32_t *permuted_idx, int64_t idx_rank_stride,
                  const uint16_t *shared_output, int64_t shared_rank_stride,
                  const uint16_t *residual, const float *post, const float *comb, const float *pre,
                  const uint16_t *norm_weight, uint16_t *residual_out, uint16_t *layer_input,
                  uint8_t *mxfp8_values, uint8_t *mxfp8_scales, int two_shot, void *workspace,
                  int64_t workspace_bytes, int M, int hidden_size, int hc_mult, int tp, int top_k,
                  float norm_eps, hipStream_t stream) {
  return finalize_impl("mhcb_finalize", gemm2_permuted, gemm2_rank_stride, rows, expert_weights,
                       weights_rank_stride, 0, 1.0f, permuted_idx, idx_rank_stride, shared_output,
                       shared_rank_stride, residual, post, comb, pre, norm_weight, residual_out,
                       layer_input, mxfp8_values, mxfp8_scales, two_shot, workspace,
                       workspace_bytes, M, hidden_size, hc_mult, tp, top_k, norm_eps, stream);
}

int mhcb_finalize_ex(const uint16_t *gemm2_permuted, int64_t gemm2_rank_stride, int64_t rows,
                     const void *expert_weights, int64_t weights_rank_stride, int weights_bf16,
                     float routed_scaling_factor, const int32_t *permuted_idx,
                     int64_t idx_rank_stride, const uint16_t *shared_output,
                     int64_t shared_rank_stride, const uint16_t *residual, const float *post,
                     const float *comb, const float *pre, const uint16_t *norm_weight,
                     uint16_t *residual_out, uint16_t *layer_input, uint8_t *mxfp8_values,
                     uint8_t *mxfp8_scales, int two_shot, void *workspace, int64_t workspace_bytes,
                     int M, int hidden_size, int hc_mult, int tp, int top_k, float norm_eps,
                     hipStream_t stream) {
  return finalize_impl("mhcb_finalize_ex", gemm2_permuted, gemm2_rank_stride, rows,
                       expert_weights, weights_rank_stride, weights_bf16, routed_scaling_factor,
                       permuted_idx, idx_rank_stride, shared_output, shared_rank_stride, residual,
                       post, comb, pre, norm_weight, residual_out, layer_input, mxfp8_values,
                       mxfp8_scales, two_shot, workspace, workspace_bytes, M, hidden_size,
                       hc_mult, tp, top_k, norm_eps, stream);
}

// Validates the indexer's sizes; fills `rows`.
int check_indexer(const char *fn, int M, int K, int key_rows, int heads, int gate_rows, int &rows) {
  if (M < 1) return fail(MHCB_EINVAL, "%s: M=%d < 1", fn, M);
  if (key_rows < 0 || heads < 0 || gate_rows < 0 || key_rows + heads + gate_rows < 1)
    return fail(MHCB_EINVAL, "%s: rows (%d, %d, %d) must be >= 0 with at least one", fn, key_rows,
                heads, gate_rows);
  rows = key_rows + heads + gate_rows;
  if (rows > kIndexerMaxRows) return fail(MHCB_EUNSUPPORTED, "%s: %d rows exceed %d", fn, rows, kIndexerMaxRows);
  if (K <= 0 || K % 128 || K > kIndexerMaxK)
    return fail(MHCB_EUNSUPPORTED, "%s: K=%d must be a positive multiple of 128 up to %d", fn, K, kIndexerMaxK);
  return MHCB_OK;
}

int64_t mhcb_indexer_workspace_bytes(int M, int K, int key_rows, int heads, int gate_rows) {
  int rows = 0;
  if (check_indexer("mhcb_indexer_workspace_bytes", M, K, key_rows, heads, gate_rows, rows))
    return -1;
  return plan_indexer(M, K, rows, device_cus(), true).workspace_bytes;
}

int mhcb_indexer_workspace_init(void *workspace, int64_t workspace_bytes, hipStream_t stream) {
  const char *fn = "mhcb_indexer_workspace_init";
  if (!workspace || workspace_bytes < 0) return fail(MHCB_EINVAL, "%s: a workspace is required", fn);
  if (!aligned(workspace, 256)) return fail(MHCB_EALIGN, "%s: workspace must be 256-byte aligned", fn);
  return launched(launch_zero(workspace, workspace_bytes, stream), fn);
}

int mhcb_indexer_projection(const uint16_t *x, const uint16_t *weight, uint16_t *key_out,
                            float *heads_out, uint16_t *gate_out, void *workspace,
                            int64_t workspace_bytes, int M, int K, int key_rows, int heads,
                            int gate_rows, hipStream_t stream) {
  const char *fn = "mhcb_indexer_projection";
  int rows = 0;
  if (const int rc = check_indexer(fn, M, K, key_rows, heads, gate_rows, rows)) return rc;
  if (!x || !weight || (key_rows && !key_out) || (heads && !heads_out) || (gate_rows && !gate_out))
    return fail(MHCB_EINVAL, "%s: x, weight and every non-empty part's output are required", fn);
  if (!aligned(x, 16) || !aligned(weight, 16) || (key_out && !aligned(key_out, 2)) ||
      (heads_out && !aligned(heads_out, 4)) || (gate_out && !aligned(gate_out, 2)))
    return fail(MHCB_EALIGN, "%s: x and weight must be 16-byte aligned, the outputs element-aligned", fn);
  const IndexerPlan p = plan_indexer(M, K, rows, device_cus(), workspace != nullptr);
  if (workspace) {
    if (workspace_bytes < p.workspace_bytes)
      return fail(MHCB_EINVAL, "%s: workspace_bytes=%lld < %lld (mhcb_indexer_workspace_bytes)", fn,
                  (long long)workspace_bytes, (long long)p.workspace_bytes);
    if (!aligned(workspace, 256)) return fail(MHCB_EALIGN, "%s: workspace must be 256-byte aligned", fn);
  }
  char *ws = static_cast<char *>(workspace);
  IndexerArgs a = {x, weight, key_out, heads_out, gate_out,
                   p.splits > 1 ? reinterpret_cast<float *>(ws + p.counter_bytes) : nullptr,
                   p.splits > 1 ? reinterpret_cast<uint32_t *>(ws) : nullptr,
                   M, K, key_rows, heads, gate_rows, rows};
  return launched(launch_indexer(a, p, stream), fn);
}

int mhcb_quant_mxfp8(const uint16_t *x, uint8_t *values, uint8_t *scales, int M, int hidden_size,
                     hipStream_t stream) {
  const char *fn = "mhcb_quant_mxfp8";
  if (M < 1) return fail(MHCB_EINVAL, "%s: M=%d < 1", fn, M);
  if (hidden_size <= 0 || hidden_size % 128 || hidden_size > kMaxHidden)
    return fail(MHCB_EUNSUPPORTED, "%s: hidden_size=%d must be a positive multiple of 128 up to %d", fn, hidden_size, kMaxHidden);
  if (!x || !values || !scales) return fail(MHCB_EINVAL, "%s: every pointer is required", fn);
  if (!aligned(x, 16) || !aligned(values, 8) || !aligned(scales, 4))
    return fail(MHCB_EALIGN, "%s: x must be 16-byte aligned", fn);
  return launched(launch_quant_mxfp8(x, values, scales, M, hidden_size, stream), fn);
}

int mhcb_mailbox_init(const mhcb_mailbox *mailbox, hipStream_t stream) {
  const char *fn = "mhcb_mailbox_init";
  if (!mailbox) return fail(MHCB_EINVAL, "%s: mailbox is required", fn);
  if (mailbox->tp < 1 || mailbox->tp > kMaxTp) return fail(MHCB_EINVAL, "%s: tp=%d", fn, mailbox->tp);
  const int H = mailbox->hidden_size;
  if (H <= 0 || H % kFrag) return fail(MHCB_EUNSUPPORTED, "%s: hidden_size=%d", fn, H);
  int rc = check_mailbox(fn, mailbox, H, mailbox->tp, 1);
  if (rc) return rc;
  return launched(launch_mailbox_init(view_of(mailbox), mailbox->tp, H, stream), fn);
}

int mhcb_publish(const mhcb_mailbox *mailbox, const uint16_t *partials, int64_t rank_stride,
                 int rank_begin, int rank_count, int M, hipStream_t stream) {
  const char *fn = "mhcb_publish";
  if (!mailbox || !partials) return fail(MHCB_EINVAL, "%s: mailbox and partials are required", fn);
  const int H = mailbox->hidden_size;
  if (H <= 0 || H % kFrag) return fail(MHCB_EUNSUPPORTED, "%s: hidden_size=%d", fn, H);
  if (M < 1) return fail(MHCB_EINVAL, "%s: M=%d < 1", fn, M);
  int rc = check_mailbox(fn, mailbox, H, mailbox->tp, M);
  if (rc) return rc;
  if (rank_begin < 0 || rank_count < 1 || rank_begin + rank_count > mailbox->tp)
    return fail(MHCB_EINVAL, "%s: ranks [%d, %d) outside [0, %d)", fn, rank_begin, rank_begin + rank_count, mailbox->tp);
  if (rank_count > 1 && rank_stride < (int64_t)M * H)
    return fail(MHCB_EINVAL, "%s: rank_stride=%lld overlaps a rank's [M, hidden] block", fn, (long long)rank_stride);
  if (!aligned(partials, 16) || rank_stride % kFrag)
    return fail(MHCB_EALIGN, "%s: partials must be 16-byte aligned with rank_stride %% 8 == 0", fn);
  return launched(launch_publish(view_of(mailbox), mailbox->tp, H, partials, rank_stride, rank_begin,
                                 rank_count, M, stream), fn);
}

int mhcb_mailbox_status(const mhcb_mailbox *mailbox, int32_t *status_out, hipStream_t stream) {
  const char *fn = "mhcb_mailbox_status";
  if (!mailbox || !mailbox->status || !status_out)
    return fail(MHCB_EINVAL, "%s: the mailbox status words and status_out are required", fn);
  if (!aligned(mailbox->status, 4) || !aligned(status_out, 4))
    return fail(MHCB_EALIGN, "%s: status words must be 4-byte aligned", fn);
  return launched(launch_copy_words(reinterpret_cast<const uint32_t *>(mailbox->status),
                                    reinterpret_cast<uint32_t *>(status_out), 2, stream),
                  fn);
}

}  // extern "C"
