/*
 * mhcb.h -- C ABI of libmhcb: the fused TP-reduce + mHC + RMSNorm sublayer
 * boundary on AMD Instinct MI355X (gfx950).
 *
 * The operations are those of two web pages, cited by title and section:
 *   [DSV41] vllm.models.deepseek_v41.nvidia.ops.cute_dsl.all_reduce_mhc
 *           (AllReduceMHC.__call__ / .finalize / ._check / ._consumer,
 *            _LamportMHCDeviceKernel, _QuadFinalizePublishDeviceKernel,
 *            _OwnerReduceMulticastDeviceKernel, _SharedOnlyPublishDeviceKernel)
 *   [GLM]   vllm.models.glm5next.nvidia.specialized_decode.all_reduce_mhc
 *           (AllReduceMhcBoundary.__call__ / .join, _BoundaryDeviceKernel,
 *            _GroupBoundaryDeviceKernel, _MixesDeviceKernel, _PublishDeviceKernel)
 *   [IDX]   vllm.models.glm5next.nvidia.specialized_decode.indexer
 *           (IndexerProjection, _ProjectionKernel)
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE pointers owned by the caller unless stated; the
 *    library never allocates, frees or retains them.
 *  - BF16 tensors are uint16_t bit patterns, 16-byte aligned; FP32 tensors
 *    4-byte aligned; rank strides (in elements) keep 16-byte alignment.
 *  - Every call validates all arguments before any launch or any write to a
 *    mailbox or stage word ([DSV41] AllReduceMHC._consumer: a bad argument
 *    leaves the state untouched), then enqueues its kernels on `stream`
 *    (0 = the null stream) and returns without synchronizing.
 *  - Outputs must not alias inputs.
 *  - Return value: MHCB_OK or an error code; mhcb_last_error() gives the
 *    calling thread's message for the last failure.
 *  - hc_mult (residual streams): 1, 2, 4 or 8 for mhcb_boundary and the
 *    finalize calls ([DSV41] compiles _LamportMHCDeviceKernel for the
 *    module's hc_mult); exactly 4 for mhcb_boundary_glm and mhcb_mixes
 *    ([GLM] ties those kernels to four streams and 24 mixes).  hidden_size
 *    a multiple of 8 (16-byte fragments of 8 BF16 values) and at most 16384.
 */
#ifndef MHCB_H
#define MHCB_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum mhcb_status {
  MHCB_OK = 0,
  MHCB_EINVAL = 1,       /* bad size, shape, null pointer or combination     */
  MHCB_EALIGN = 2,       /* pointer or stride breaks the alignment rules     */
  MHCB_EUNSUPPORTED = 3, /* valid per the pages but not handled by libmhcb   */
  MHCB_ELAUNCH = 4,      /* the HIP runtime rejected a launch                */
  MHCB_ETIMEOUT = 5      /* a bounded wait gave up: the value a caller reports */
                         /* once a status word (mhcb_workspace_status,       */
                         /* mhcb_mailbox_status) reads non-zero              */
};

/* Message of the calling thread's last failed call ("" if none). */
const char *mhcb_last_error(void);

/* Library version as "major.minor.patch". */
const char *mhcb_version(void);

/* Bytes of the swizzled 128x4 UE8M0 scale array for an [M, hidden_size]
 * MXFP8 output: rows padded to a multiple of 128, hidden_size / 32 columns
 * ([DSV41] AllReduceMHC.__call__, mxfp8_scale_bytes).  Host-only. */
int64_t mhcb_mxfp8_scale_bytes(int64_t M, int64_t hidden_size);

/* Workspace.  The boundary entry points take an optional caller-owned
 * device workspace (256-byte aligned).  Its first part holds the state of
 * the cross-workgroup reduction that lets small-M calls spread each token
 * over several workgroups (with NULL every token takes one workgroup); it
 * must be initialized once (mhcb_workspace_init) before its first use.  Each
 * token slot has two copies of its exchange area, used by alternate calls;
 * a call clears the copy the previous call used while it works, so the
 * state is ready for the next call, with any slice count, with no reset at
 * the end.  Calls that may run concurrently (on different streams) must not
 * share a workspace.
 * Co-residency: the workgroups of one token wait for one another (bounded
 * by the workspace's spin limit).  They are dispatched consecutively, so on
 * an otherwise idle device the wait ends as soon as the slowest one stores
 * its value.  A kernel running concurrently that leaves fewer free
 * workgroup slots than a token's slice count (at most 16) can keep a slice
 * from starting until the others give up: those slices' results are then
 * NaN and the time-out is counted (mhcb_workspace_status).
 * mhcb_workspace_bytes gives the size for a call: the sync state, then a
 * scratch area of at least 8 MiB that holds the per-slice partials of the
 * two-pass GLM tiles (mhcb_boundary_glm, tokens_per_wg = -16) or, when
 * larger, the two-shot emulation's (mhcb_finalize, two_shot = 1) owner
 * mailboxes [tp][tp][ceil(M/tp)][hidden] and reduced sums [M][hidden]
 * (BF16).  mhcb_finalize_workspace_bytes is the same function under the
 * name the finalize call's documentation uses.  Host-only; -1 on bad
 * sizes. */
int64_t mhcb_workspace_bytes(int M, int hidden_size, int tp, int two_shot);
int64_t mhcb_finalize_workspace_bytes(int M, int hidden_size, int tp, int two_shot);

/* Writes the workspace's sync state (a kernel on `stream`): status word and
 * epochs zero, the spin limit back to its default, every exchange word the
 * empty marker.  After a timed-out call the status stays set until the
 * workspace is initialized again. */
int mhcb_workspace_init(void *workspace, int64_t workspace_bytes, hipStream_t stream);

/* Sets the number of re-reads after which a cross-workgroup wait of a call
 * on this workspace gives up (a kernel on `stream`, ordered before later
 * calls on it).  <= 0 restores the default, about a second of polling. */
int mhcb_workspace_set_spin_limit(void *workspace, int64_t spin_limit, hipStream_t stream);

/* Enqueues on `stream` a copy of the workspace's time-out count (cross-
 * workgroup waits of calls on this workspace that gave up since
 * mhcb_workspace_init) into *status_out: device memory, or pinned host
 * memory the device can write.  Never synchronizes; read *status_out after
 * the stream has reached that point. */
int mhcb_workspace_status(const void *workspace, uint32_t *status_out, hipStream_t stream);

/* Tuning: workgroups per token (or per GLM tile) for calls with a
 * workspace (1..64, of which the exchanging splits use at most 16 and the
 * two-pass GLM tiles at most 64; 0 = automatic, chosen by M from
 * measurements).  Applies to the later calls of the calling thread only
 * (thread-local; other threads keep their own setting); returns the
 * calling thread's previous value.  The BF16 sums, streams and the delayed
 * / finalize layer inputs do not depend on it; the GLM GEMV is summed over
 * the slices in FP32, so its raw mixes may change in the last bits. */
int mhcb_set_token_slices(int slices);

/* Three-generation Lamport mailbox ([GLM] AllReduceMhcBoundary.__init__,
 * [DSV41] module text): slots[generation][rank][token][hidden] BF16, every
 * empty slot holding the sentinel 0x8000 (BF16 -0); stage_state = {ACTIVE,
 * NEXT} of the rank that owns this view (on the pages every rank keeps its
 * own; two descriptors may share `slots` with separate stage_state, as a
 * peer publishing into this mailbox does); status[0] counts consumer polls
 * that gave up, status[1] the fragments the consumer found still empty
 * and re-read until they landed.  All three pointers are caller-owned
 * device memory; the struct itself is read on the host only. */
typedef struct mhcb_mailbox {
  uint16_t *slots;       /* [generations][tp][capacity][hidden_size]       */
  int32_t *stage_state;  /* [2]: ACTIVE, NEXT                              */
  int32_t *status;       /* [2]: poll time-outs, late fragments            */
  int generations;       /* must be 3                                      */
  int tp;                /* ranks                                          */
  int capacity;          /* max tokens per call                            */
  int hidden_size;
  int64_t spin_limit;    /* re-reads per fragment before giving up; <= 0:  */
                         /* the default (about a second of polling)        */
} mhcb_mailbox;

/* Delayed-mHC boundary ([DSV41] AllReduceMHC.__call__ with
 * _LamportMHCDeviceKernel), per token t and column c:
 *   xr      = bf16( ((0 + x_0) + x_1) + ... + x_{tp-1} )       (FP32 adds)
 *   y_j     = bf16( xr*post_j (+) sum_s residual_s * comb[s][j] )   (FMAs)
 *   p       = bf16( 0 (+) y_0*pre_0 (+) ... (+) y_{hc-1}*pre_{hc-1} )  (FMAs)
 *   out     = bf16( (p * inv) * norm_weight ),
 *             inv = 1/sqrt(sum_c p^2 / hidden + norm_eps)
 * Inputs: partials = tp BF16 [M, hidden] arrays rank_stride elements apart
 * (NULL iff mailbox is given: then the ACTIVE generation is polled until no
 * element is the sentinel, NEXT is advanced and the slots are reset; a
 * fragment still empty after spin_limit re-reads is read as NaN, so that
 * token's layer input and those columns of its residual_out come out NaN,
 * and the time-out is counted in status[0]);
 * residual [M, hc, hidden] BF16; post, pre [M, hc] FP32; comb [M, hc, hc]
 * FP32 indexed [source][target]; norm_weight [hidden] BF16 (hc = hc_mult).
 * Outputs: residual_out [M, hc, hidden] = y; layer_input [M, hidden] = out;
 * optionally mxfp8_values [M, hidden] E4M3 codes and mxfp8_scales
 * (mhcb_mxfp8_scale_bytes) UE8M0 scales of out, per 32 columns, in the
 * swizzled 128x4 layout, padding rows zeroed (hidden % 128 == 0 required).
 * pre == norm_weight == layer_input == NULL selects the residual-only
 * variant.  workspace: optional (see mhcb_workspace_bytes).
 * Errors: M < 1 or M > mailbox capacity, tp < 1 or tp > 64,
 * pre/norm_weight given alone, MXFP8 on a residual-only call -> EINVAL;
 * hidden % 8, hc_mult not 1, 2, 4 or 8, MXFP8 with hidden % 128
 * -> EUNSUPPORTED. */
int mhcb_boundary(const uint16_t *partials, int64_t rank_stride, const mhcb_mailbox *mailbox,
                  const uint16_t *residual, const float *post, const float *comb,
                  const float *pre, const uint16_t *norm_weight, uint16_t *residual_out,
                  uint16_t *layer_input, uint8_t *mxfp8_values, uint8_t *mxfp8_scales,
                  void *workspace, int64_t workspace_bytes, int M, int hidden_size, int hc_mult,
                  int tp, float norm_eps, hipStream_t stream);

/* GLM boundary ([GLM] AllReduceMhcBoundary.__call__ with
 * _BoundaryDeviceKernel / _GroupBoundaryDeviceKernel): xr and y as in
 * mhcb_boundary, then from the new streams
 *   g_k   = sum_{j,c} hc_fn[k][j*hidden + c] * y_j[c]   (k < 24)
 *   rstd  = 1/sqrt(sum_{j,c} y_j[c]^2 / (4*hidden) + rms_eps)
 *   mixes_out[t][k] = g_k * rstd                  (raw, for mhcb_mixes)
 *   pre_j = sigmoid(mixes_j * scale[0] + base[j]) + hc_eps
 *   p     = bf16((y_0*pre_0 + y_1*pre_1) + (y_2*pre_2 + y_3*pre_3))
 *   out   = bf16((p * inv) * norm_weight) as above.
 * hc_fn [24, 4*hidden] BF16; scale [3], base [24] FP32; mixes_out [M, 24]
 * FP32.  tokens_per_wg = 1, 2 or 4: that many tokens share one workgroup
 * and one read of hc_fn, and the outputs do not depend on the choice.
 * tokens_per_wg = 16: tiles of 16 tokens whose GEMV runs on the matrix
 * cores (needs a workspace); its FP32 sums are taken in another order, so
 * mixes_out may differ from the 1/2/4 results in the last bits (both agree
 * with the exact GEMV to about 1e-6 relative).  tokens_per_wg = -16: the
 * same 16-token tiles in two passes, with no cross-workgroup exchange: a
 * streaming pass writes residual_out and each column slice's partial GEMV
 * rows and sum of squares to the workspace's scratch area, then a pass with
 * one workgroup per token adds them in slice order and takes the collapse
 * and RMSNorm from residual_out (needs a workspace of
 * mhcb_workspace_bytes(...) bytes; results agree with the other forms to
 * the same tolerance).  0 = automatic: -16 when the workspace has
 * mhcb_workspace_bytes(...) bytes, else 16 from M = 256 when a smaller
 * workspace is given, else 1 or 2.  hidden <= 8192.
 * workspace: optional for 1, 2, 4 (see mhcb_workspace_bytes); calls that
 * share one must be ordered on one stream. */
int mhcb_boundary_glm(const uint16_t *partials, int64_t rank_stride, const uint16_t *residual,
                      const float *post, const float *comb, const uint16_t *hc_fn,
                      const float *scale, const float *base, const uint16_t *norm_weight,
                      uint16_t *residual_out, float *mixes_out, uint16_t *layer_input,
                      void *workspace, int64_t workspace_bytes, int M, int hidden_size,
                      int hc_mult, int tp, float rms_eps, float hc_eps, float norm_eps,
                      int tokens_per_wg, hipStream_t stream);

/* mhcb_boundary_glm for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without a workspace, always the two-pass 16-token tiles
 * (tokens_per_wg = -16; the same kernels, so the results are bit-identical
 * to mhcb_boundary_glm with a workspace of mhcb_workspace_bytes bytes).
 * Their per-slice partials go to a static device array of 8 MiB that the
 * library holds on each GPU it runs on until the process ends; the call
 * itself allocates and frees nothing.  Every call on a GPU shares that
 * GPU's array: calls that may overlap on one GPU (concurrent streams, or
 * with this library's other users of the array) race and must be ordered
 * by the caller.  A launch takes at most 1024 tokens (larger M is issued as
 * several launches on `stream`) and hidden <= 8192 (EUNSUPPORTED beyond), so
 * its partials (at most 1024 x 64 x 128 bytes) always fit the array.  The
 * first call on a device looks up the array's address there. */
int mhcb_boundary_glm_noalloc(const uint16_t *partials, int64_t rank_stride,
                              const uint16_t *residual, const float *post, const float *comb,
                              const uint16_t *hc_fn, const float *scale, const float *base,
                              const uint16_t *norm_weight, uint16_t *residual_out,
                              float *mixes_out, uint16_t *layer_input, int M, int hidden_size,
                              int hc_mult, int tp, float rms_eps, float hc_eps, float norm_eps,
                              hipStream_t stream);

/* Side-stream mixes for the next boundary ([GLM] _MixesDeviceKernel):
 *   post_out[t][j] = sigmoid(mixes[t][4+j] * scale[1] + base[4+j]) * post_mult
 *   comb_out[t]    = Sinkhorn(mixes[t][8+i] * scale[2] + base[8+i]), 4x4
 *                    row-major, eps = hc_eps, sinkhorn_repeat rounds.
 * mixes [M, 24]; post_out [M, 4]; comb_out [M, 4, 4] (FP32).  Meant for a
 * second stream that the caller joins before the next boundary reads it. */
int mhcb_mixes(const float *mixes, const float *scale, const float *base, float *post_out,
               float *comb_out, int M, int hc_mult, float hc_eps, float post_mult,
               int sinkhorn_repeat, hipStream_t stream);

/* MoE finalize boundary ([DSV41] AllReduceMHC.finalize with
 * _QuadFinalizePublishDeviceKernel): rank r's contribution to token t is
 *   c_r = bf16( (sum_k fma over k ascending of gemm2_r[idx_r[t][k]] * w_r[t][k])
 *               + shared_r[t] ), negative zero -> +0,
 * a route whose row index is -1 (expert not held by rank r) or outside
 * [0, rows) being skipped; then the boundary of mhcb_boundary on the c_r.
 * gemm2_permuted: per rank [rows, hidden] BF16, gemm2_rank_stride apart;
 * expert_weights [M, top_k] FP32 and permuted_idx [M, top_k] int32 per rank
 * (rank strides 0 = replicated); shared_output per rank [M, hidden] BF16.
 * two_shot = 1 runs the two-shot emulation instead: contributions stored
 * to owner t % tp, slot t / tp of owner mailboxes in `workspace`
 * (required then; mhcb_workspace_bytes with two_shot = 1), the owners'
 * FP32 rank-ordered sums, then the boundary reads one reduced value per
 * token; the results are bit-identical to two_shot = 0.
 * Errors as mhcb_boundary, plus top_k < 1, tp * top_k > 1024, a workspace
 * that is missing or too small -> EINVAL. */
int mhcb_finalize(const uint16_t *gemm2_permuted, int64_t gemm2_rank_stride, int64_t rows,
                  const float *expert_weights, int64_t weights_rank_stride,
                  const int32_t *permuted_idx, int64_t idx_rank_stride,
                  const uint16_t *shared_output, int64_t shared_rank_stride,
                  const uint16_t *residual, const float *post, const float *comb,
                  const float *pre, const uint16_t *norm_weight, uint16_t *residual_out,
                  uint16_t *layer_input, uint8_t *mxfp8_values, uint8_t *mxfp8_scales,
                  int two_shot, void *workspace, int64_t workspace_bytes, int M, int hidden_size,
                  int hc_mult, int tp, int top_k, float norm_eps, hipStream_t stream);

/* mhcb_finalize with the routing-weight options of the page
 * ([DSV41] _QuadFinalizePublishDeviceKernel, whose module compiles one
 * kernel per routing-weight dtype in AllReduceMHC.__init__): expert_weights
 * holds FP32 values (weights_bf16 = 0, 4-byte aligned) or BF16 bit patterns
 * (weights_bf16 = 1, 2-byte aligned), [M, top_k] per rank with
 * weights_rank_stride in elements; each weight is widened to FP32 and, when
 * routed_scaling_factor is not 1, multiplied by it in FP32 before its fused
 * multiply-add.  mhcb_finalize is this call with FP32 weights and factor 1.
 * Errors as mhcb_finalize, plus weights_bf16 not 0 or 1, or a factor that
 * is not finite -> EINVAL. */
int mhcb_finalize_ex(const uint16_t *gemm2_permuted, int64_t gemm2_rank_stride, int64_t rows,
                     const void *expert_weights, int64_t weights_rank_stride, int weights_bf16,
                     float routed_scaling_factor, const int32_t *permuted_idx,
                     int64_t idx_rank_stride, const uint16_t *shared_output,
                     int64_t shared_rank_stride, const uint16_t *residual, const float *post,
                     const float *comb, const float *pre, const uint16_t *norm_weight,
                     uint16_t *residual_out, uint16_t *layer_input, uint8_t *mxfp8_values,
                     uint8_t *mxfp8_scales, int two_shot, void *workspace, int64_t workspace_bytes,
                     int M, int hidden_size, int hc_mult, int tp, int top_k, float norm_eps,
                     hipStream_t stream);

/* GLM boundary of an MoE sublayer ([GLM] AllReduceMhcBoundary.__call__ with
 * an MoE output: the finalize publish of _QuadFinalizePublishDeviceKernel,
 * then the GLM boundary on the published contributions).  Every rank's
 * contribution
 *   c_r[t] = sanitize(bf16(sum_{k asc, row valid} w[t][k] * gemm2_r[row] + shared_r[t]))
 * (routing as in mhcb_finalize_ex: FP32 or BF16 weights times the routed
 * scaling factor, rows outside [0, rows) skipped) takes the place of rank
 * r's partial in mhcb_boundary_glm's arithmetic (two-pass tiles):
 * residual_out, mixes_out [M, 24] and layer_input as there.  Up to 128
 * routes a token (tp * top_k) the stream pass computes the contributions
 * itself; beyond, they are first written rank-major into the workspace.
 * The workspace is required, of at least
 * mhcb_finalize_glm_workspace_bytes(M, hidden_size, tp) bytes (the sync
 * state, the two-pass scratch, then room for tp * M * hidden BF16
 * contributions).  hc_mult = 4, hidden <= 8192. */
int64_t mhcb_finalize_glm_workspace_bytes(int M, int hidden_size, int tp);
int mhcb_finalize_glm(const uint16_t *gemm2_permuted, int64_t gemm2_rank_stride, int64_t rows,
                      const void *expert_weights, int64_t weights_rank_stride, int weights_bf16,
                      float routed_scaling_factor, const int32_t *permuted_idx,
                      int64_t idx_rank_stride, const uint16_t *shared_output,
                      int64_t shared_rank_stride, const uint16_t *residual, const float *post,
                      const float *comb, const uint16_t *hc_fn, const float *scale,
                      const float *base, const uint16_t *norm_weight, uint16_t *residual_out,
                      float *mixes_out, uint16_t *layer_input, void *workspace,
                      int64_t workspace_bytes, int M, int hidden_size, int hc_mult, int tp,
                      int top_k, float rms_eps, float hc_eps, float norm_eps, hipStream_t stream);

/* DSA indexer input projection ([IDX] vllm.models.glm5next.nvidia
 * .specialized_decode.indexer, IndexerProjection.__call__ /
 * _ProjectionKernel): the layer input x [M, K] BF16 times the concatenated
 * weight rows weight [key_rows + heads + gate_rows, K] BF16 (the indexer
 * key rows, the head-weight rows, the kpool gate rows, in that order),
 *   out[t][r] = sum_k x[t][k] * weight[r][k]   (FP32; products exact)
 * each part written in its own type: key_out [M, key_rows] BF16 (nearest
 * even), heads_out [M, heads] FP32, gate_out [M, gate_rows] BF16.
 *
 * Up to six tokens, each weight row is summed by one workgroup and no
 * workspace is used.  From seven tokens on, a workspace lets K be cut into
 * ranges summed by different workgroups, which spreads the weight read over
 * the device: partial sums and per-block counters (a fixed 4 KiB area at its
 * start) live in the workspace, and every call leaves the counters at zero
 * again.  Without a workspace, each output is summed by a single workgroup.
 *
 * workspace: NULL, or at least mhcb_indexer_workspace_bytes(...) bytes
 * (which depends on M, K and the row counts; 0 where K is not cut),
 * 256-byte aligned, set to zero by mhcb_indexer_workspace_init (or any zero
 * fill) before its first use; EINVAL if smaller.  Calls that share a
 * workspace must not overlap (same stream, or ordered).  Each output is
 * summed in a fixed order for a given M and workspace choice, so results
 * repeat bit for bit.  K a multiple of 128 up to 65536 and at most 4096 rows
 * (EUNSUPPORTED beyond); M >= 1; a part with no rows may pass NULL for its
 * output. */
int64_t mhcb_indexer_workspace_bytes(int M, int K, int key_rows, int heads, int gate_rows);
int mhcb_indexer_workspace_init(void *workspace, int64_t workspace_bytes, hipStream_t stream);
int mhcb_indexer_projection(const uint16_t *x, const uint16_t *weight, uint16_t *key_out,
                            float *heads_out, uint16_t *gate_out, void *workspace,
                            int64_t workspace_bytes, int M, int K, int key_rows, int heads,
                            int gate_rows, hipStream_t stream);

/* Standalone MXFP8 of a BF16 [M, hidden] array: the encoding of the
 * boundary's epilogue ([DSV41] _LamportMHCDeviceKernel, quantize): per 32
 * columns e = the smallest UE8M0 exponent with 2^(e-127) >= amax * fl(1/448),
 * codes = E4M3 round-to-nearest-even (saturating) of x * 2^(127-e); values
 * [M, hidden] bytes, scales mhcb_mxfp8_scale_bytes bytes. */
int mhcb_quant_mxfp8(const uint16_t *x, uint8_t *values, uint8_t *scales, int M, int hidden_size,
                     hipStream_t stream);

/* Fills every slot with the sentinel, zeroes stage_state and status. */
int mhcb_mailbox_init(const mhcb_mailbox *mailbox, hipStream_t stream);

/* Producer ([GLM] _PublishDeviceKernel, [DSV41]
 * _SharedOnlyPublishDeviceKernel): reads NEXT, stores ranks
 * [rank_begin, rank_begin + rank_count) of tokens [0, M) -- their partials
 * rank_stride elements apart -- with negative zero replaced by +0 into
 * generation NEXT, then sets ACTIVE = NEXT. */
int mhcb_publish(const mhcb_mailbox *mailbox, const uint16_t *partials, int64_t rank_stride,
                 int rank_begin, int rank_count, int M, hipStream_t stream);

/* Enqueues on `stream` a copy of the mailbox's two status words (poll
 * time-outs and late fragments since mhcb_mailbox_init) into status_out[2]:
 * device memory, or pinned host memory the device can write.  Never
 * synchronizes. */
int mhcb_mailbox_status(const mhcb_mailbox *mailbox, int32_t *status_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MHCB_H */
