/*
 * moe_a2a.h -- C ABI of the MI355X MoE token dispatch / combine library.
 *
 * One GPU holds the whole exchange: the ep_size destination regions of the
 * all-to-all are partitions of one workspace in local HBM.  Dispatch routes
 * every routed copy of a token into its region; combine gathers each token's
 * k expert outputs back and reduces them exactly once; the fused variant adds
 * the residual and applies RMSNorm in the same pass.
 *
 * Sources, cited by page title and section:
 *  [A2A]  InferenceX PR #2450, "CollectiveX: add FlashInfer one-sided NVLink
 *         EP for the GB SKUs": "The adapter" table (dispatch / combine phase
 *         contract, padded receive [ep_size, runtime_max_tokens_per_rank,
 *         hidden] read at valid slots only, workspace sized once from the
 *         ladder maximum with each call passing its rung); the on-metal probe
 *         comment (init / dispatch / combine signatures, the caller-provided
 *         output buffer of newer versions); "Update -- the correctness
 *         failures are resolved" (fp32 accumulation, one nearest-even
 *         narrowing store, expert outputs written in place in the workspace).
 *  [DR]   vLLM PR #41382, "[Bugfix] Fix double reduce in
 *         flashinfer_nvlink_two_sided and flashinfer_nvlink_one_sided
 *         backends": the all-to-all combine already sums over the experts
 *         dimension, so callers must not reduce its output again.
 *  [FUSE] magik.net, "Fusing the Allreduce: A Precision Investigation into
 *         FlashInfer's Verify-Path Optimization", section "The Message Itself:
 *         Explanation and Probe": residual add + RMSNorm fused onto the
 *         reduction that produces the hidden state.
 *
 * Conventions (all calls):
 *  - bf16 tensors are passed as uint16_t bit patterns; fp32 as float.
 *  - "device" pointers are HIP device memory of the GPU current when the call
 *    is made; "host" pointers are ordinary process memory.
 *  - Every buffer is allocated and freed by the caller.  The library never
 *    allocates, frees or synchronises, except moe_sync_status.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    dispatch and the combines only enqueue kernels on it and return.
 *  - Arguments are checked on the host before anything is enqueued; a
 *    failed check returns a negative MOE_ERR_* code and changes nothing.
 *  - Layout, symbols: T tokens, H hidden, k top-k, E experts, ep regions,
 *    epr = E / ep experts per region, cap = max_tokens_per_rank rows per
 *    region, f = t*k + j the flat index of token t's j-th routed copy.
 *  - Region of expert e is e / epr.  Expert id -1 means "no expert".
 *  - Row order inside a region is stable: region r holds its copies in
 *    increasing f.  ([A2A] "Verified: per-rank permutation" shows the order
 *    is the implementation's choice; this library fixes the stable one.)
 */
#ifndef MOE_A2A_H
#define MOE_A2A_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes -------------------------------------------------------- */
#define MOE_OK             0
#define MOE_ERR_ARG       (-1)  /* bad size, null or misaligned pointer      */
#define MOE_ERR_PHASE     (-2)  /* dispatch twice, or combine without dispatch */
#define MOE_ERR_OVERFLOW  (-3)  /* a region received more than cap copies    */
#define MOE_ERR_EXPERT_ID (-4)  /* an expert id outside [-1, E)              */
#define MOE_ERR_HIP       (-5)  /* a HIP runtime call failed (see hip_error, */
                                /* moe_last_hip_error)                     */
#define MOE_ERR_NOALLOC_SIZE (-6) /* a batch beyond the static scratch of  */
                                /* moe_dispatch_noalloc                    */
#define MOE_ERR_GAVE_UP   (-7)  /* a single-pass dispatch block gave up     */
                                /* waiting (its tokens were not dispatched) */

/* workspace layouts (moe_init) */
#define MOE_LAYOUT_PER_COPY   0     /* one row per routed copy (t, j)          */
#define MOE_LAYOUT_PER_REGION 1     /* one row per (token, destination region) */

/* bits of the device status word (moe_sync_status) */
#define MOE_STATUS_OVERFLOW  1
#define MOE_STATUS_EXPERT_ID 2
#define MOE_STATUS_GAVE_UP   4

/* ---- limits ---------------------------------------------------------------- */
#define MOE_MAX_EP          256     /* destination regions                     */
#define MOE_MAX_TOP_K        64     /* routed copies per token                 */
#define MOE_MAX_FUSED_HIDDEN 16384  /* hidden size of the fused epilogue       */
#define MOE_MAX_HIDDEN     1048576  /* hidden size (a row stays under 2^31 B)  */
#define MOE_MAX_PARTIALS     64     /* partials summed by moe_partials_reduce* */
#define MOE_NOALLOC_MAX_ITEMS 1048576 /* routed copies (T * k) per moe_dispatch_noalloc */
#define MOE_MAX_TOKENS     8388608  /* tokens per handle: the combine runs one */
                                    /* 256-lane block per token, and a launch */
                                    /* holds fewer than 2^32 lanes            */

/*
 * moe_handle -- host memory, owned by the caller.  Filled by moe_init; the
 * phase fields are updated by dispatch and the combines.  One handle serves
 * one stream at a time: calls on one handle must not overlap.
 */
typedef struct moe_handle {
    /* configuration (moe_init) */
    int32_t max_tokens;          /* ladder maximum: largest T of any call      */
    int32_t hidden;              /* H, multiple of 8                           */
    int32_t top_k;               /* k                                          */
    int32_t num_experts;         /* E                                          */
    int32_t ep_size;             /* ep                                         */
    int32_t experts_per_rank;    /* epr = E / ep                               */
    int32_t max_tokens_per_rank; /* cap: allocated rows per region             */
    int32_t layout;              /* MOE_LAYOUT_PER_COPY or MOE_LAYOUT_PER_REGION */
    /* device buffers owned by the caller (moe_init) */
    int32_t *counts;             /* [ep]          copies sent to each region   */
    int32_t *src_index;          /* [ep * cap]    f held by row (r, s)         */
    int32_t *slot_index;         /* [max_tokens * k] row r*cap+s of copy f, or -1 */
    int32_t *status;             /* [1]           MOE_STATUS_* bits, sticky    */
    void    *scratch;            /* moe_scratch_bytes(max_tokens, k, ep) bytes */
    size_t   scratch_bytes;
    /* per-call state */
    int32_t phase;               /* 0 idle, 1 dispatched                       */
    int32_t num_tokens;          /* T of the last dispatch                     */
    int32_t runtime_max_tokens_per_rank; /* R of the last dispatch             */
    int32_t hip_error;           /* hipError_t behind the last MOE_ERR_HIP     */
    /* single-pass dispatch (moe_init zeroes both)                         */
    uint32_t onepass_epoch;      /* epoch of the last one (library use only)   */
    int32_t  onepass_spin_limit; /* polls per word before a block gives up:   */
                                 /* 0 the default, < 0 give up at once (tests) */
} moe_handle;

/* Bytes of the padded workspace [ep, cap, H] bf16: the receive buffer
 * [A2A] "The adapter" sizes once from the ladder maximum ([ep_size,
 * max_tokens_per_rank, hidden]).  Returns 0 for a non-positive argument. */
size_t moe_workspace_bytes(int32_t ep_size, int32_t max_tokens_per_rank, int32_t hidden);

/* Bytes of routing scratch a handle needs (per-copy ranks and per-chunk
 * region histograms of the routing kernel, and the single-pass dispatch's
 * epoch-tagged words: 8 bytes per routed copy up to 65536 copies and per
 * chunk and region); returns 0 for arguments outside the limits.  Any
 * contents are accepted: the routing kernel writes what the copy kernel
 * reads, and a handle clears the words before its first single-pass
 * dispatch. */
size_t moe_scratch_bytes(int32_t max_tokens, int32_t top_k, int32_t ep_size);

/*
 * moe_init -- validate the configuration and bind the caller's buffers.
 * [A2A] on-metal probe: init(mapping, max_num_tokens, top_k, num_experts,
 * workspace_size_per_rank, hidden_size); the workspace is sized once from
 * the ladder maximum.
 *   h                    host, caller-owned; overwritten
 *   max_tokens           1 .. MOE_MAX_TOKENS, largest T any dispatch may pass
 *   hidden               8 .. MOE_MAX_HIDDEN, a multiple of 8
 *   top_k                1 .. MOE_MAX_TOP_K
 *   num_experts          multiple of ep_size
 *   ep_size              1 .. MOE_MAX_EP
 *   max_tokens_per_rank  >= 1; ep * cap and max_tokens * k must fit int32
 *   layout               MOE_LAYOUT_PER_COPY: one workspace row per routed
 *                        copy; MOE_LAYOUT_PER_REGION: one row per (token,
 *                        destination region), the form [A2A] measures ("Update
 *                        -- the correctness failures are resolved": a token is
 *                        sent once per destination rank and its duplicate-rank
 *                        top-k slots are blanked; "Bring-up progress": about
 *                        5.3 distinct ranks per token at top-8 over 8 ranks).
 *                        A token then contributes at most one row per region,
 *                        so cap = max_tokens always suffices.
 *   counts, src_index, slot_index, status, scratch: device, 4-byte aligned,
 *                        sized as in moe_handle; *status must be 0 before
 *                        the first dispatch (zero-filled memory); the scratch
 *                        belongs to this handle (two handles in flight at
 *                        once must not share it)
 *   scratch, scratch_bytes  may instead be NULL and 0: the handle then serves
 *                        moe_dispatch_noalloc only (moe_dispatch,
 *                        moe_dispatch_fp8 and moe_route_counts return
 *                        MOE_ERR_ARG)
 *   scratch_bytes        >= moe_scratch_bytes(max_tokens, top_k, ep_size)
 * Returns MOE_OK or MOE_ERR_ARG.  No HIP call is made.
 */
int moe_init(moe_handle *h, int32_t max_tokens, int32_t hidden, int32_t top_k,
             int32_t num_experts, int32_t ep_size, int32_t max_tokens_per_rank,
             int32_t layout, int32_t *counts, int32_t *src_index, int32_t *slot_index,
             int32_t *status, void *scratch, size_t scratch_bytes);

/*
 * moe_dispatch -- route every copy into its region.  [A2A] "The adapter":
 * dispatch(token_selected_experts, input_payloads, runtime_max_tokens_per_rank,
 * invalid_token_expert_id) into a padded receive; one-sided, each copy is
 * written straight into its destination region.
 *   x          device [T, H] bf16, 16-byte aligned
 *   topk_ids   device [T, k] int32 expert ids; -1 = no expert
 *   num_tokens T, 0 <= T <= runtime_max_tokens_per_rank
 *   runtime_max_tokens_per_rank  R, the rung of this call, R <= max_tokens
 *   workspace  device [ep, cap, H] bf16, 16-byte aligned
 * Writes: workspace rows (r, s) for s < min(counts[r], cap) with the source
 * token's row (bit copies); counts[r] = rows region r was sent (not clamped
 * to cap); slot_index[f]; src_index[r*cap + s] for valid rows.
 * Per-region layout: the token's first copy to region r takes the row
 * (src_index holds that copy's f); its later copies to r get the same
 * slot_index and write nothing.
 * Padding rows and src_index entries past the valid prefix are not touched.
 * Copies past cap are dropped (slot_index -1) and set MOE_STATUS_OVERFLOW;
 * ids outside [-1, E) are dropped and set MOE_STATUS_EXPERT_ID; both are
 * reported by moe_sync_status.
 * Batches of at most 4096 routed copies (T * k) run as one kernel launch.
 * In the per-copy layout, batches of 4097 to 65536 copies also run as one
 * launch (bf16 and fp8 payloads alike) whose first blocks rank the routing chunks into words tagged with
 * the dispatch's epoch (the handle's onepass_epoch; the handle's first such
 * dispatch, and the one after the epoch wraps, first clear the words with
 * hipMemsetAsync), while the other blocks wait for the words they need.
 * A block that waits too long (onepass_spin_limit polls of one word) gives
 * up: it writes nothing for its token, whose slot_index entries read -1, and
 * sets MOE_STATUS_GAVE_UP (moe_sync_status: MOE_ERR_GAVE_UP).  Under stream
 * capture, and for larger batches and the other layout, the routing kernel
 * runs first, then the copy kernel.
 * The workspace must not overlap x or topk_ids, and none of the three may
 * overlap the handle's device buffers (MOE_ERR_ARG).
 * Returns MOE_OK, MOE_ERR_ARG, MOE_ERR_PHASE (already dispatched) or
 * MOE_ERR_HIP (launch failed).  On success the handle is "dispatched".
 */
int moe_dispatch(moe_handle *h, const uint16_t *x, const int32_t *topk_ids,
                 int32_t num_tokens, int32_t runtime_max_tokens_per_rank,
                 uint16_t *workspace, void *stream);

/*
 * moe_dispatch_noalloc -- moe_dispatch for callers that cannot allocate
 * device memory at all (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the routing scratch (per-copy ranks
 * and per-chunk region histograms) comes from a static array in the
 * library's device code, 4 MiB + 64 KiB on each GPU the library runs on,
 * held until the process ends, instead of the handle's scratch (which may
 * be NULL).  The caller still passes x, topk_ids and the workspace, and the
 * handle still binds the output buffers.  Arguments, outputs, errors and the
 * phase as moe_dispatch, plus:
 *   num_tokens * top_k <= MOE_NOALLOC_MAX_ITEMS, else MOE_ERR_NOALLOC_SIZE
 * (checked before anything is enqueued).  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (on different streams,
 * or from different threads without ordering) race and give wrong results.
 * Nothing in the array needs clearing: each call's routing kernel writes
 * what its copy kernel reads.  Makes no allocating call; the first call on
 * a GPU looks up the array's device address (hipGetSymbolAddress).
 */
int moe_dispatch_noalloc(moe_handle *h, const uint16_t *x, const int32_t *topk_ids,
                         int32_t num_tokens, int32_t runtime_max_tokens_per_rank,
                         uint16_t *workspace, void *stream);

/*
 * moe_dispatch_fp8 -- moe_dispatch with an FP8 payload: each token row is
 * quantised once to OCP FP8 E4M3 with one fp32 scale, and the codes and the
 * scale travel to every destination row ([A2A] "The adapter" notes: an FP8
 * dispatch carries its scale as a second payload, checked against the
 * oracle's cast round-trip).  Per token row:
 *   amax  = max_h |x[t, h]|,   scale = amax / 448,
 *   q[h]  = e4m3_nearest_even( x[t, h] * (448 / amax) )      (fp32 ops)
 * so x ~ e4m3_value(q) * scale; an all-zero row gets scale 0 and zero codes.
 * x must be finite: a row holding an infinity or a NaN gets codes and a
 * scale that mean nothing (the copies and index maps are still exact).
 *   workspace  device [ep, cap, H] uint8 codes, 16-byte aligned
 *   scales     device [ep, cap] fp32, 4-byte aligned; scales[r*cap + s] is
 *              the scale of row (r, s), written for valid rows only
 * Other arguments, outputs (counts, slot_index, src_index), errors and the
 * phase as moe_dispatch, with the same launch choices (one launch up to
 * 4096 copies; the single pass, with its epoch words and give-up, for 4097
 * to 65536 per-copy copies outside capture; routing then copy kernels
 * otherwise); requires H <= MOE_MAX_FUSED_HIDDEN; workspace,
 * scales, x and topk_ids must not overlap each other (x and topk_ids
 * excepted) or the handle's device buffers (MOE_ERR_ARG).  The combine
 * that follows reads bf16 expert outputs from a buffer of the same
 * [ep, cap, H] layout (the experts dequantise and write it).
 */
int moe_dispatch_fp8(moe_handle *h, const uint16_t *x, const int32_t *topk_ids,
                     int32_t num_tokens, int32_t runtime_max_tokens_per_rank,
                     uint8_t *workspace, float *scales, void *stream);

/*
 * moe_combine -- reduce each token's k expert outputs exactly once.
 * [A2A] "Update -- the correctness failures are resolved": fp32
 * accumulation, one nearest-even narrowing store; [DR]: the result is final.
 *   expert_out   device [ep, cap, H] bf16, 16-byte aligned; the expert
 *                outputs in the dispatch layout (may be the workspace itself)
 *   topk_weights device [T, k] fp32 gates; read only when weighted != 0
 *   weighted     0: out = bf16(sum_j y_j); else out = bf16(sum_j w_j * y_j)
 *   out          device [T, H] bf16, 16-byte aligned; overwritten; overlapping
 *                expert_out, topk_weights (when weighted) or the handle's
 *                device buffers is MOE_ERR_ARG
 * Sum over j = 0..k-1 in order in fp32 (weighted terms as fused
 * multiply-adds), skipping copies with slot_index -1; padding rows are never
 * read.  A token with no valid copy gets +0.
 * Per-region layout: each row holds its region's message for the token (the
 * gated sum of the token's experts there, [A2A] "Bring-up progress": the
 * combine is an unweighted rank-sum), and each distinct row is added once,
 * in the order of its first copy; weighted must be 0 (else MOE_ERR_ARG).
 * Returns MOE_OK, MOE_ERR_ARG, MOE_ERR_PHASE (not dispatched) or MOE_ERR_HIP.
 * On success the handle returns to idle.
 */
int moe_combine(moe_handle *h, const uint16_t *expert_out, const float *topk_weights,
                int32_t weighted, uint16_t *out, void *stream);

/*
 * moe_combine_residual_rmsnorm -- combine, residual add and RMSNorm in one
 * pass ([FUSE]).  With s = (fp32 combine sum) + residual:
 *   residual_out = bf16(s)
 *   normed       = bf16( s / sqrt(mean_h(s^2) + eps) * gamma )
 * where the mean of squares, the root and the product are taken in fp64 (so
 * rows anywhere in bf16's range normalise) and the result is rounded to fp32,
 * then to bf16.  With eps = 0 a row of zeros gives NaN (0/0).
 *   residual     device [T, H] bf16, 16-byte aligned
 *   residual_out device [T, H] bf16; may be the same buffer as residual
 *   gamma        device [H] bf16, 16-byte aligned
 *   eps          finite, >= 0
 *   normed       device [T, H] bf16, 16-byte aligned
 * The outputs may not overlap expert_out, gamma, topk_weights (when
 * weighted), the handle's device buffers or each other, nor (normed) the
 * residual, and residual_out overlaps the residual only by being the same
 * buffer; otherwise MOE_ERR_ARG.
 * Other arguments as moe_combine.  Requires H <= MOE_MAX_FUSED_HIDDEN.
 */
int moe_combine_residual_rmsnorm(moe_handle *h, const uint16_t *expert_out,
                                 const float *topk_weights, int32_t weighted,
                                 const uint16_t *residual, uint16_t *residual_out,
                                 const uint16_t *gamma, float eps, uint16_t *normed,
                                 void *stream);

/*
 * moe_partials_reduce -- the reduction stage of a one-shot all-reduce under
 * tensor parallelism, on one GPU.  [FUSE] section "The Message Itself:
 * Explanation and Probe": each rank ends a layer with a partial hidden state
 * and an all-reduce sums them before the residual add and RMSNorm.  Once the
 * P partials sit in local memory (here they are simply a buffer the caller
 * fills), the sum is one reduction, taken like the combine's:
 *   out[t, h] = bf16( sum over p = 0..P-1 of f32(partials[p, t, h]) )
 * in fp32 in rank order, one nearest-even narrowing.  No handle, no phase.
 *   partials     device [P, T, H] bf16, 16-byte aligned
 *   num_partials P, 1 .. MOE_MAX_PARTIALS
 *   num_tokens   T, 0 .. MOE_MAX_TOKENS, with P * T < 2^31
 *   hidden       H, 8 .. MOE_MAX_HIDDEN, a multiple of 8
 *   out          device [T, H] bf16, 16-byte aligned; overwritten; overlapping
 *                partials is MOE_ERR_ARG
 * Asynchronous on `stream`.  Returns MOE_OK, MOE_ERR_ARG (checked before
 * anything is enqueued) or MOE_ERR_HIP (the launch failed; the hipError_t is
 * kept for moe_last_hip_error, as no handle holds it).
 */
int moe_partials_reduce(const uint16_t *partials, int32_t num_partials, int32_t num_tokens,
                        int32_t hidden, uint16_t *out, void *stream);

/*
 * moe_partials_reduce_residual_rmsnorm -- moe_partials_reduce fused with the
 * residual add and RMSNorm, the single kernel [FUSE] describes in place of
 * an all-reduce followed by the norm.  With s = (fp32 sum of the partials)
 * + residual, the outputs are those of moe_combine_residual_rmsnorm:
 *   residual_out = bf16(s),  normed = bf16( s / sqrt(mean_h(s^2) + eps) * gamma )
 *   residual     device [T, H] bf16, 16-byte aligned
 *   residual_out device [T, H] bf16; may be the same buffer as residual
 *   gamma        device [H] bf16, 16-byte aligned
 *   eps          finite, >= 0
 *   normed       device [T, H] bf16, 16-byte aligned
 * The outputs may not overlap partials, gamma or each other, nor (normed)
 * the residual, and residual_out overlaps the residual only by being the
 * same buffer; otherwise MOE_ERR_ARG.  Other arguments, limits and errors as
 * moe_partials_reduce; requires H <= MOE_MAX_FUSED_HIDDEN.
 */
int moe_partials_reduce_residual_rmsnorm(const uint16_t *partials, int32_t num_partials,
                                         int32_t num_tokens, int32_t hidden,
                                         const uint16_t *residual, uint16_t *residual_out,
                                         const uint16_t *gamma, float eps, uint16_t *normed,
                                         void *stream);

/*
 * moe_route_counts -- only the per-region copy counts of a routing, so a
 * caller can size max_tokens_per_rank before allocating the workspace
 * ([A2A] "The adapter": the receive is sized once, from the largest batch;
 * the counts are the dispatch's own, computed by its routing kernel).
 * Writes counts (and routing scratch); leaves the phase idle.
 *   topk_ids   device [T, k] int32;  0 <= num_tokens <= max_tokens
 * Returns MOE_OK, MOE_ERR_ARG, MOE_ERR_PHASE (a dispatch is pending) or
 * MOE_ERR_HIP.  Bad ids set MOE_STATUS_EXPERT_ID.
 */
int moe_route_counts(moe_handle *h, const int32_t *topk_ids, int32_t num_tokens,
                     void *stream);

/*
 * moe_sync_status -- wait for `stream`, read and clear the device status.
 * The device-side checks stand in for the host asserts of [A2A] "The
 * adapter" (ids outside the experts, a receive region past its capacity),
 * which a one-sided kernel cannot raise itself.
 *   bits  host, optional: receives the MOE_STATUS_* bits that were set
 * Returns MOE_ERR_EXPERT_ID, MOE_ERR_OVERFLOW or MOE_ERR_GAVE_UP if a kernel
 * flagged one since the last call (in that order when several were; `bits`
 * has them all), MOE_OK otherwise, MOE_ERR_HIP on a runtime failure.  The
 * only call that synchronises.
 */
int moe_sync_status(moe_handle *h, void *stream, int32_t *bits);

/* moe_reset -- return a dispatched handle to idle without combining: the
 * way out of the dispatch -> combine phase contract of [A2A] "The adapter"
 * when a dispatch is abandoned (e.g. after a device-detected error).
 * Returns MOE_OK, or MOE_ERR_ARG for a null handle. */
int moe_reset(moe_handle *h);

/* moe_output_is_reduced -- always 1: the combine output is final and must not
 * be summed over experts again ([DR]). */
int moe_output_is_reduced(void);

/* moe_strerror -- static text for a return code. */
const char *moe_strerror(int code);

/* moe_last_hip_error -- the hipError_t behind the most recent MOE_ERR_HIP
 * returned to the calling thread by any call of this library (0 if none);
 * the handle-free calls (moe_partials_reduce*) have no other place to keep
 * it.  Per thread; not cleared by later successful calls. */
int moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_A2A_H */
