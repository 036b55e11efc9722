// C ABI of the MoE dispatch / combine library: argument and phase checks on
// the host, then kernel launches on the caller's stream.  The phase contract
// (dispatch twice -> error, combine without dispatch -> error, combine
// returns the handle to idle) follows the "The adapter" table of InferenceX
// PR #2450, "CollectiveX: add FlashInfer one-sided NVLink EP for the GB SKUs".

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "launch.h"
#include "moe_a2a.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool dev_ok(const void *p, uintptr_t a) { return p != nullptr && aligned(p, a); }

// True if the byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && pa < pb + nb && pb < pa + na;
}

// The outputs of a fused epilogue against its inputs: `src` (the gathered
// rows), the residual, gamma, and each other.  residual_out may be the
// residual itself (updated in place), but not overlap it otherwise.
bool fused_outputs_overlap(const void *src, size_t src_bytes, const uint16_t *residual,
                           const uint16_t *residual_out, const uint16_t *gamma,
                           const uint16_t *normed, size_t row_bytes, size_t gamma_bytes) {
    return overlaps(residual_out, row_bytes, src, src_bytes) ||
           overlaps(normed, row_bytes, src, src_bytes) ||
           overlaps(normed, row_bytes, residual, row_bytes) ||
           overlaps(normed, row_bytes, residual_out, row_bytes) ||
           overlaps(residual_out, row_bytes, gamma, gamma_bytes) ||
           overlaps(normed, row_bytes, gamma, gamma_bytes) ||
           (residual_out != residual && overlaps(residual_out, row_bytes, residual, row_bytes));
}

// The hipError_t behind the calling thread's last MOE_ERR_HIP.
thread_local int32_t g_last_hip_error = 0;

int hip_fail(moe_handle *h, hipError_t e) {
    g_last_hip_error = static_cast<int32_t>(e);
    if (h != nullptr) h->hip_error = static_cast<int32_t>(e);
    return MOE_ERR_HIP;
}

// True if [p, p + bytes) shares a byte with any device buffer the handle
// binds (counts, src_index, slot_index, status, scratch), which dispatch
// writes and combine reads.
bool overlaps_handle(const moe_handle *h, const void *p, size_t bytes) {
    return overlaps(p, bytes, h->counts, (size_t)h->ep_size * 4) ||
           overlaps(p, bytes, h->src_index, (size_t)h->ep_size * h->max_tokens_per_rank * 4) ||
           overlaps(p, bytes, h->slot_index, (size_t)h->max_tokens * h->top_k * 4) ||
           overlaps(p, bytes, h->status, 4) ||
           overlaps(p, bytes, h->scratch, h->scratch_bytes);
}

// Routing scratch of moe_dispatch_noalloc: one array per GPU, in the
// library's device code (no allocation).  Holds the per-copy ranks of up to
// MOE_NOALLOC_MAX_ITEMS routed copies, then the per-chunk region histograms
// (kMaxChunks x MOE_MAX_EP int32).
constexpr size_t kStaticRankBytes = (size_t)MOE_NOALLOC_MAX_ITEMS * sizeof(int32_t);
constexpr size_t kStaticScratchBytes =
    kStaticRankBytes + (size_t)moe::kMaxChunks * MOE_MAX_EP * sizeof(int32_t);
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Device addresses of `scratch`, one per GPU, looked up on the first
// moe_dispatch_noalloc call with that GPU current.  In host code `scratch`
// names a host-side stand-in, so kernels get these addresses instead.
constexpr int kMaxDevices = 64;
void *g_scratch_dev[kMaxDevices];
std::mutex g_scratch_mu;

hipError_t static_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(int32_t ep_size, int32_t max_tokens_per_rank, int32_t hidden) {
    if (ep_size <= 0 || max_tokens_per_rank <= 0 || hidden <= 0) return 0;
    return (size_t)ep_size * (size_t)max_tokens_per_rank * (size_t)hidden * sizeof(uint16_t);
}

size_t moe_scratch_bytes(int32_t max_tokens, int32_t top_k, int32_t ep_size) {
    if (max_tokens < 1 || max_tokens > MOE_MAX_TOKENS || top_k < 1 || top_k > MOE_MAX_TOP_K ||
        ep_size < 1 || ep_size > MOE_MAX_EP)
        return 0;
    const int64_t items = (int64_t)max_tokens * top_k;
    if (items > INT32_MAX) return 0;
    const size_t bytes = (size_t)moe::scratch_words_offset(items, ep_size) +
                         (size_t)moe::scratch_words_count(items, ep_size) * sizeof(uint64_t);
    return (bytes + 255) & ~(size_t)255;
}

int moe_init(moe_handle *h, int32_t max_tokens, int32_t hidden, int32_t top_k,
             int32_t num_experts, int32_t ep_size, int32_t max_tokens_per_rank,
             int32_t layout, int32_t *counts, int32_t *src_index, int32_t *slot_index,
             int32_t *status, void *scratch, size_t scratch_bytes) {
    if (h == nullptr) return MOE_ERR_ARG;
    if (layout != MOE_LAYOUT_PER_COPY && layout != MOE_LAYOUT_PER_REGION) return MOE_ERR_ARG;
    if (max_tokens < 1 || max_tokens > MOE_MAX_TOKENS)
        return MOE_ERR_ARG;
    if (hidden < 8 || hidden > MOE_MAX_HIDDEN || hidden % 8 != 0)
        return MOE_ERR_ARG;
    if (top_k < 1 || top_k > MOE_MAX_TOP_K) return MOE_ERR_ARG;
    if (ep_size < 1 || ep_size > MOE_MAX_EP) return MOE_ERR_ARG;
    if (num_experts < ep_size || num_experts % ep_size != 0) return MOE_ERR_ARG;
    if (max_tokens_per_rank < 1) return MOE_ERR_ARG;
    if ((int64_t)ep_size * max_tokens_per_rank > INT32_MAX) return MOE_ERR_ARG;
    if ((int64_t)max_tokens * top_k > INT32_MAX) return MOE_ERR_ARG;
    if (!dev_ok(counts, 4) || !dev_ok(src_index, 4) || !dev_ok(slot_index, 4) ||
        !dev_ok(status, 4))
        return MOE_ERR_ARG;
    const size_t need = moe_scratch_bytes(max_tokens, top_k, ep_size);
    if (need == 0) return MOE_ERR_ARG;
    // no scratch (NULL, 0): a handle for moe_dispatch_noalloc only
    if (!(scratch == nullptr && scratch_bytes == 0) && (!dev_ok(scratch, 4) || scratch_bytes < need))
        return MOE_ERR_ARG;

    memset(h, 0, sizeof *h);
    h->max_tokens = max_tokens;
    h->hidden = hidden;
    h->top_k = top_k;
    h->num_experts = num_experts;
    h->ep_size = ep_size;
    h->experts_per_rank = num_experts / ep_size;
    h->max_tokens_per_rank = max_tokens_per_rank;
    h->layout = layout;
    h->counts = counts;
    h->src_index = src_index;
    h->slot_index = slot_index;
    h->status = status;
    h->scratch = scratch;
    h->scratch_bytes = scratch_bytes;
    return MOE_OK;
}

// The routing scratch of a call: the handle's, laid out for its largest
// batch, or the library's static array (moe_dispatch_noalloc), laid out for
// MOE_NOALLOC_MAX_ITEMS copies.
struct Scratch {
    void *base;
    int64_t max_items;
};

// log2 of experts_per_rank when it is a power of two (the kernels then map
// an expert to its region with a shift), else -1.
static int32_t epr_shift(const moe_handle *h) {
    for (int32_t s = 0; s < 31; ++s)
        if ((int32_t(1) << s) == h->experts_per_rank) return s;
    return -1;
}

static Scratch handle_scratch(const moe_handle *h) {
    return Scratch{h->scratch, (int64_t)h->max_tokens * h->top_k};
}

static moe::RouteArgs route_args(moe_handle *h, const Scratch &sc, const int32_t *topk_ids,
                                 int32_t num_tokens, const moe::RoutePlan &plan) {
    moe::RouteArgs ra;
    ra.ids = topk_ids;
    ra.rank = moe::scratch_rank(sc.base);
    ra.hist = moe::scratch_hist(sc.base, sc.max_items);
    ra.status = h->status;
    ra.n_items = (int64_t)num_tokens * h->top_k;
    ra.items_per_chunk = plan.tokens_per_chunk * h->top_k;
    ra.ep = h->ep_size;
    ra.epr = h->experts_per_rank;
    ra.n_experts = h->num_experts;
    ra.epr_shift = epr_shift(h);
    ra.k = h->top_k;
    ra.per_region = h->layout == MOE_LAYOUT_PER_REGION;
    return ra;
}

static int route(moe_handle *h, const Scratch &sc, const int32_t *topk_ids, int32_t num_tokens,
                 hipStream_t s, moe::RoutePlan *plan_out) {
    const moe::RoutePlan plan = moe::plan_route(num_tokens);
    const moe::RouteArgs ra = route_args(h, sc, topk_ids, num_tokens, plan);
    hipError_t e = moe::launch_route(ra, plan.n_chunks, s);
    if (e != hipSuccess) return hip_fail(h, e);
    *plan_out = plan;
    return MOE_OK;
}

static moe::DispatchArgs dispatch_args(moe_handle *h, const Scratch &sc, const uint16_t *x,
                                       const int32_t *ids, int32_t T, uint16_t *ws,
                                       const moe::RoutePlan &plan, int32_t count_only) {
    moe::DispatchArgs da;
    da.x = x;
    da.ids = ids;
    da.rank = moe::scratch_rank(sc.base);
    da.hist = moe::scratch_hist(sc.base, sc.max_items);
    da.ws = ws;
    da.counts = h->counts;
    da.slot_index = h->slot_index;
    da.src_index = h->src_index;
    da.status = h->status;
    da.T = T;
    da.H = h->hidden;
    da.k = h->top_k;
    da.ep = h->ep_size;
    da.epr = h->experts_per_rank;
    da.n_experts = h->num_experts;
    da.epr_shift = epr_shift(h);
    da.cap = h->max_tokens_per_rank;
    da.tokens_per_chunk = plan.tokens_per_chunk;
    da.n_chunks = plan.n_chunks;
    da.count_only = count_only;
    da.per_region = h->layout == MOE_LAYOUT_PER_REGION;
    da.fp8 = 0;
    da.ws8 = nullptr;
    da.scales = nullptr;
    da.t_base = 0;
    da.onepass = 0;
    da.route_blocks = 0;
    da.epoch = 0;
    da.spin_limit = 0;
    da.rank_w = nullptr;
    da.hist_w = nullptr;
    return da;
}


// True if `s` is being captured into a graph, and (conservatively) when the
// query fails; a failed query's error is cleared so that the launch check
// after the kernels does not report it as theirs.
static bool capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    return st != hipStreamCaptureStatusNone;
}

static int dispatch_checks(moe_handle *h, const uint16_t *x, const int32_t *topk_ids,
                           int32_t num_tokens, int32_t R, const void *workspace) {
    if (h == nullptr || h->max_tokens < 1) return MOE_ERR_ARG;
    if (h->phase != 0) return MOE_ERR_PHASE;
    if (R < 1 || R > h->max_tokens || num_tokens < 0 || num_tokens > R) return MOE_ERR_ARG;
    if (!dev_ok(workspace, 16)) return MOE_ERR_ARG;
    if (num_tokens > 0 && (!dev_ok(x, 16) || !dev_ok(topk_ids, 4))) return MOE_ERR_ARG;
    return MOE_OK;
}

// Bytes of the token rows a dispatch reads, and of its workspace (bf16 rows,
// or fp8 codes when elem == 1).
static size_t token_bytes(const moe_handle *h, int32_t num_tokens) {
    return (size_t)num_tokens * h->hidden * sizeof(uint16_t);
}
static size_t ws_bytes(const moe_handle *h, size_t elem) {
    return (size_t)h->ep_size * h->max_tokens_per_rank * h->hidden * elem;
}
// Bytes of the gates [T, k] fp32 of the last dispatch.
static size_t weight_bytes(const moe_handle *h) {
    return (size_t)h->num_tokens * h->top_k * sizeof(float);
}

// The inputs and outputs of a dispatch against each other and the handle's
// buffers: the workspace (and fp8 scales) may not overlap x, the ids or
// each other, and the handle's buffers, which the dispatch writes, may not
// overlap any of them.  (x and the ids are only read: they may overlap.)
static bool dispatch_overlaps(const moe_handle *h, const void *x, const void *ids,
                              int32_t num_tokens, const void *ws, size_t ws_bytes,
                              const void *scales, size_t scale_bytes) {
    const size_t xb = (size_t)num_tokens * h->hidden * sizeof(uint16_t);
    const size_t ib = (size_t)num_tokens * h->top_k * sizeof(int32_t);
    return overlaps(ws, ws_bytes, x, xb) || overlaps(ws, ws_bytes, ids, ib) ||
           overlaps(scales, scale_bytes, x, xb) || overlaps(scales, scale_bytes, ids, ib) ||
           overlaps(scales, scale_bytes, ws, ws_bytes) || overlaps_handle(h, x, xb) ||
           overlaps_handle(h, ids, ib) || overlaps_handle(h, ws, ws_bytes) ||
           overlaps_handle(h, scales, scale_bytes);
}

static int dispatch_launch(moe_handle *h, const Scratch &sc, moe::DispatchArgs da,
                           const int32_t *topk_ids, int32_t num_tokens, int32_t R, hipStream_t s,
                           bool words = false) {
    moe::RoutePlan plan = moe::plan_route(num_tokens);
    if (words && moe::dispatch_is_onepass(num_tokens, h->top_k, da.per_region) &&
        !capturing(s)) {
        uint64_t *rw = moe::scratch_rank_words(sc.base, sc.max_items, h->ep_size);
        // The handle's words are cleared on its first single-pass dispatch
        // (moe_init zeroes onepass_epoch; epoch 0 is never used) and whenever
        // the epoch would wrap; each dispatch then takes the next epoch.
        if (h->onepass_epoch == 0 || h->onepass_epoch >= 0x7FFFFFFFu) {
            const hipError_t me = hipMemsetAsync(
                rw, 0, moe::scratch_words_count(sc.max_items, h->ep_size) * sizeof(uint64_t), s);
            if (me != hipSuccess) return hip_fail(h, me);
            h->onepass_epoch = 0;
        }
        const uint32_t epoch = ++h->onepass_epoch;
        da.tokens_per_chunk = plan.tokens_per_chunk;
        da.n_chunks = plan.n_chunks;
        da.onepass = 1;
        da.epoch = epoch;
        da.spin_limit = h->onepass_spin_limit != 0 ? h->onepass_spin_limit : moe::kOnePassSpinLimit;
        da.rank_w = rw;
        da.hist_w = moe::scratch_hist_words(sc.base, sc.max_items, h->ep_size);
        const moe::RouteArgs ra = route_args(h, sc, topk_ids, num_tokens, plan);
        hipError_t e = moe::launch_dispatch_onepass(da, ra, s);
        if (e != hipSuccess) return hip_fail(h, e);
        h->phase = 1;
        h->num_tokens = num_tokens;
        h->runtime_max_tokens_per_rank = R;
        return MOE_OK;
    }
    if (!moe::dispatch_is_small(num_tokens, h->top_k)) {   // small batches need no routing kernel
        int rc = route(h, sc, topk_ids, num_tokens, s, &plan);
        if (rc != MOE_OK) return rc;
    }
    da.tokens_per_chunk = plan.tokens_per_chunk;
    da.n_chunks = plan.n_chunks;
    hipError_t e = moe::launch_dispatch_copy(da, s);
    if (e != hipSuccess) return hip_fail(h, e);
    h->phase = 1;
    h->num_tokens = num_tokens;
    h->runtime_max_tokens_per_rank = R;
    return MOE_OK;
}

int moe_dispatch(moe_handle *h, const uint16_t *x, const int32_t *topk_ids,
                 int32_t num_tokens, int32_t runtime_max_tokens_per_rank,
                 uint16_t *workspace, void *stream) {
    const int32_t R = runtime_max_tokens_per_rank;
    int rc = dispatch_checks(h, x, topk_ids, num_tokens, R, workspace);
    if (rc != MOE_OK) return rc;
    if (h->scratch == nullptr) return MOE_ERR_ARG;         // a handle for moe_dispatch_noalloc
    if (dispatch_overlaps(h, x, topk_ids, num_tokens, workspace, ws_bytes(h, sizeof(uint16_t)),
                          nullptr, 0))
        return MOE_ERR_ARG;
    const Scratch sc = handle_scratch(h);
    const moe::DispatchArgs da = dispatch_args(h, sc, x, topk_ids, num_tokens, workspace,
                                               moe::plan_route(num_tokens), 0);
    return dispatch_launch(h, sc, da, topk_ids, num_tokens, R, static_cast<hipStream_t>(stream), true);
}

int moe_dispatch_noalloc(moe_handle *h, const uint16_t *x, const int32_t *topk_ids,
                         int32_t num_tokens, int32_t runtime_max_tokens_per_rank,
                         uint16_t *workspace, void *stream) {
    const int32_t R = runtime_max_tokens_per_rank;
    int rc = dispatch_checks(h, x, topk_ids, num_tokens, R, workspace);
    if (rc != MOE_OK) return rc;
    if ((int64_t)num_tokens * h->top_k > MOE_NOALLOC_MAX_ITEMS) return MOE_ERR_NOALLOC_SIZE;
    if (dispatch_overlaps(h, x, topk_ids, num_tokens, workspace, ws_bytes(h, sizeof(uint16_t)),
                          nullptr, 0))
        return MOE_ERR_ARG;
    Scratch sc{nullptr, MOE_NOALLOC_MAX_ITEMS};
    const hipError_t e = static_scratch(&sc.base);
    if (e != hipSuccess) return hip_fail(h, e);
    const moe::DispatchArgs da = dispatch_args(h, sc, x, topk_ids, num_tokens, workspace,
                                               moe::plan_route(num_tokens), 0);
    return dispatch_launch(h, sc, da, topk_ids, num_tokens, R, static_cast<hipStream_t>(stream));
}

int moe_dispatch_fp8(moe_handle *h, const uint16_t *x, const int32_t *topk_ids,
                     int32_t num_tokens, int32_t runtime_max_tokens_per_rank,
                     uint8_t *workspace, float *scales, void *stream) {
    const int32_t R = runtime_max_tokens_per_rank;
    int rc = dispatch_checks(h, x, topk_ids, num_tokens, R, workspace);
    if (rc != MOE_OK) return rc;
    if (!dev_ok(scales, 4) || h->hidden > MOE_MAX_FUSED_HIDDEN) return MOE_ERR_ARG;
    if (h->scratch == nullptr) return MOE_ERR_ARG;         // a handle for moe_dispatch_noalloc
    const size_t scale_bytes = (size_t)h->ep_size * h->max_tokens_per_rank * sizeof(float);
    if (dispatch_overlaps(h, x, topk_ids, num_tokens, workspace, ws_bytes(h, 1), scales,
                          scale_bytes))
        return MOE_ERR_ARG;
    const Scratch sc = handle_scratch(h);
    moe::DispatchArgs da = dispatch_args(h, sc, x, topk_ids, num_tokens, nullptr,
                                         moe::plan_route(num_tokens), 0);
    da.fp8 = 1;
    da.ws8 = workspace;
    da.scales = scales;
    return dispatch_launch(h, sc, da, topk_ids, num_tokens, R, static_cast<hipStream_t>(stream), true);
}

int moe_route_counts(moe_handle *h, const int32_t *topk_ids, int32_t num_tokens, void *stream) {
    if (h == nullptr || h->max_tokens < 1) return MOE_ERR_ARG;
    if (h->phase != 0) return MOE_ERR_PHASE;
    if (num_tokens < 0 || num_tokens > h->max_tokens) return MOE_ERR_ARG;
    if (num_tokens > 0 && !dev_ok(topk_ids, 4)) return MOE_ERR_ARG;
    if (h->scratch == nullptr) return MOE_ERR_ARG;         // a handle for moe_dispatch_noalloc
    if (overlaps_handle(h, topk_ids, (size_t)num_tokens * h->top_k * sizeof(int32_t)))
        return MOE_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    moe::RoutePlan plan;
    const Scratch sc = handle_scratch(h);
    int rc = route(h, sc, topk_ids, num_tokens, s, &plan);
    if (rc != MOE_OK) return rc;
    const moe::DispatchArgs da = dispatch_args(h, sc, nullptr, topk_ids, num_tokens, nullptr, plan, 1);
    hipError_t e = moe::launch_dispatch_copy(da, s);
    if (e != hipSuccess) return hip_fail(h, e);
    return MOE_OK;
}

static int combine_common(moe_handle *h, const uint16_t *expert_out, const float *topk_weights,
                          int32_t weighted) {
    if (h == nullptr || h->max_tokens < 1) return MOE_ERR_ARG;
    if (h->phase != 1) return MOE_ERR_PHASE;
    if (weighted && h->layout == MOE_LAYOUT_PER_REGION) return MOE_ERR_ARG;
    if (h->num_tokens > 0) {
        if (!dev_ok(expert_out, 16)) return MOE_ERR_ARG;
        if (weighted && !dev_ok(topk_weights, 4)) return MOE_ERR_ARG;
    }
    return MOE_OK;
}

static moe::CombineArgs combine_args(moe_handle *h, const uint16_t *expert_out,
                                     const float *topk_weights, int32_t weighted) {
    moe::CombineArgs ca;
    memset(&ca, 0, sizeof ca);
    ca.y = expert_out;
    ca.slot_index = h->slot_index;
    ca.w = topk_weights;
    ca.T = h->num_tokens;
    ca.H = h->hidden;
    ca.k = h->top_k;
    ca.weighted = weighted ? 1 : 0;
    ca.per_region = h->layout == MOE_LAYOUT_PER_REGION;
    return ca;
}

int moe_combine(moe_handle *h, const uint16_t *expert_out, const float *topk_weights,
                int32_t weighted, uint16_t *out, void *stream) {
    int rc = combine_common(h, expert_out, topk_weights, weighted);
    if (rc != MOE_OK) return rc;
    if (h->num_tokens > 0 && !dev_ok(out, 16)) return MOE_ERR_ARG;
    const size_t ob = token_bytes(h, h->num_tokens);
    if (overlaps(out, ob, expert_out, ws_bytes(h, sizeof(uint16_t))) ||
        (weighted && overlaps(out, ob, topk_weights, weight_bytes(h))) || overlaps_handle(h, out, ob))
        return MOE_ERR_ARG;
    moe::CombineArgs ca = combine_args(h, expert_out, topk_weights, weighted);
    ca.out = out;
    hipError_t e = moe::launch_combine(ca, false, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(h, e);
    h->phase = 0;
    return MOE_OK;
}

int moe_combine_residual_rmsnorm(moe_handle *h, const uint16_t *expert_out,
                                 const float *topk_weights, int32_t weighted,
                                 const uint16_t *residual, uint16_t *residual_out,
                                 const uint16_t *gamma, float eps, uint16_t *normed,
                                 void *stream) {
    int rc = combine_common(h, expert_out, topk_weights, weighted);
    if (rc != MOE_OK) return rc;
    if (h->hidden > MOE_MAX_FUSED_HIDDEN) return MOE_ERR_ARG;
    if (!(eps >= 0.0f) || !isfinite(eps)) return MOE_ERR_ARG;
    if (h->num_tokens > 0 && (!dev_ok(residual, 16) || !dev_ok(residual_out, 16) ||
                              !dev_ok(gamma, 16) || !dev_ok(normed, 16)))
        return MOE_ERR_ARG;
    const size_t ob = token_bytes(h, h->num_tokens);
    if (fused_outputs_overlap(expert_out, ws_bytes(h, sizeof(uint16_t)), residual, residual_out,
                              gamma, normed, ob, (size_t)h->hidden * sizeof(uint16_t)) ||
        (weighted && (overlaps(residual_out, ob, topk_weights, weight_bytes(h)) ||
                      overlaps(normed, ob, topk_weights, weight_bytes(h)))) ||
        overlaps_handle(h, residual_out, ob) || overlaps_handle(h, normed, ob))
        return MOE_ERR_ARG;
    moe::CombineArgs ca = combine_args(h, expert_out, topk_weights, weighted);
    ca.residual = residual;
    ca.residual_out = residual_out;
    ca.gamma = gamma;
    ca.normed = normed;
    ca.eps = eps;
    hipError_t e = moe::launch_combine(ca, true, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(h, e);
    h->phase = 0;
    return MOE_OK;
}

static int partials_checks(const uint16_t *partials, int32_t num_partials, int32_t num_tokens,
                           int32_t hidden, int32_t max_hidden) {
    if (num_partials < 1 || num_partials > MOE_MAX_PARTIALS) return MOE_ERR_ARG;
    if (num_tokens < 0 || num_tokens > MOE_MAX_TOKENS) return MOE_ERR_ARG;
    if (hidden < 8 || hidden > max_hidden || hidden % 8 != 0) return MOE_ERR_ARG;
    if ((int64_t)num_partials * num_tokens > INT32_MAX) return MOE_ERR_ARG;
    if (num_tokens > 0 && !dev_ok(partials, 16)) return MOE_ERR_ARG;
    return MOE_OK;
}

static moe::CombineArgs partials_args(const uint16_t *partials, int32_t num_partials,
                                      int32_t num_tokens, int32_t hidden) {
    moe::CombineArgs ca;
    memset(&ca, 0, sizeof ca);
    ca.y = partials;
    ca.T = num_tokens;
    ca.H = hidden;
    ca.k = num_partials;
    ca.partials = 1;
    return ca;
}

int moe_partials_reduce(const uint16_t *partials, int32_t num_partials, int32_t num_tokens,
                        int32_t hidden, uint16_t *out, void *stream) {
    int rc = partials_checks(partials, num_partials, num_tokens, hidden, MOE_MAX_HIDDEN);
    if (rc != MOE_OK) return rc;
    if (num_tokens > 0 && !dev_ok(out, 16)) return MOE_ERR_ARG;
    const size_t row_bytes = (size_t)num_tokens * hidden * sizeof(uint16_t);
    if (overlaps(out, row_bytes, partials, row_bytes * num_partials)) return MOE_ERR_ARG;
    moe::CombineArgs ca = partials_args(partials, num_partials, num_tokens, hidden);
    ca.out = out;
    const hipError_t e = moe::launch_combine(ca, false, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(nullptr, e);
}

int moe_partials_reduce_residual_rmsnorm(const uint16_t *partials, int32_t num_partials,
                                         int32_t num_tokens, int32_t hidden,
                                         const uint16_t *residual, uint16_t *residual_out,
                                         const uint16_t *gamma, float eps, uint16_t *normed,
                                         void *stream) {
    int rc = partials_checks(partials, num_partials, num_tokens, hidden, MOE_MAX_FUSED_HIDDEN);
    if (rc != MOE_OK) return rc;
    if (!(eps >= 0.0f) || !isfinite(eps)) return MOE_ERR_ARG;
    if (num_tokens > 0 && (!dev_ok(residual, 16) || !dev_ok(residual_out, 16) ||
                           !dev_ok(gamma, 16) || !dev_ok(normed, 16)))
        return MOE_ERR_ARG;
    const size_t row_bytes = (size_t)num_tokens * hidden * sizeof(uint16_t);
    if (fused_outputs_overlap(partials, row_bytes * num_partials, residual, residual_out, gamma,
                              normed, row_bytes, (size_t)hidden * sizeof(uint16_t)))
        return MOE_ERR_ARG;
    moe::CombineArgs ca = partials_args(partials, num_partials, num_tokens, hidden);
    ca.residual = residual;
    ca.residual_out = residual_out;
    ca.gamma = gamma;
    ca.normed = normed;
    ca.eps = eps;
    const hipError_t e = moe::launch_combine(ca, true, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(nullptr, e);
}

int moe_sync_status(moe_handle *h, void *stream, int32_t *bits) {
    if (h == nullptr || h->status == nullptr) return MOE_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t host = 0;
    hipError_t e = hipMemcpyAsync(&host, h->status, sizeof host, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(h, e);
    if (host != 0) {
        e = hipMemsetAsync(h->status, 0, sizeof host, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(h, e);
    }
    if (bits) *bits = host;
    if (host & MOE_STATUS_EXPERT_ID) return MOE_ERR_EXPERT_ID;
    if (host & MOE_STATUS_OVERFLOW) return MOE_ERR_OVERFLOW;
    if (host & MOE_STATUS_GAVE_UP) return MOE_ERR_GAVE_UP;
    return MOE_OK;
}

int moe_reset(moe_handle *h) {
    if (h == nullptr) return MOE_ERR_ARG;
    h->phase = 0;
    return MOE_OK;
}

int moe_output_is_reduced(void) { return 1; }

int moe_last_hip_error(void) { return g_last_hip_error; }

const char *moe_strerror(int code) {
    switch (code) {
        case MOE_OK: return "success";
        case MOE_ERR_ARG: return "invalid argument (size, null or misaligned pointer)";
        case MOE_ERR_PHASE: return "phase error (dispatch twice, or combine without dispatch)";
        case MOE_ERR_OVERFLOW: return "a destination region received more copies than max_tokens_per_rank";
        case MOE_ERR_EXPERT_ID: return "expert id outside [-1, num_experts)";
        case MOE_ERR_HIP: return "HIP runtime error";
        case MOE_ERR_GAVE_UP:
            return "a single-pass dispatch block gave up waiting for the routing words "
                   "(its tokens were not dispatched)";
        case MOE_ERR_NOALLOC_SIZE:
            return "batch too large for the library's static routing scratch "
                   "(moe_dispatch_noalloc: num_tokens * top_k <= MOE_NOALLOC_MAX_ITEMS)";
        default: return "unknown error code";
    }
}

}  // extern "C"
