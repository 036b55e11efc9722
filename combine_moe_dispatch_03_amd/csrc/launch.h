// Internal interface between the C ABI (api.hip) and the gfx950 kernels
// (kernels.hip).  Not installed; the public surface is include/moe_a2a.h.
// The planning functions are inline so that every user of this header (the
// library, and the host-only sanitizer driver that stands in for the
// kernels) computes the same plan.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Routing is split into at most this many chunks of whole tokens.  Each
// dispatch block adds up the region histograms of the chunks before its own,
// so the bound keeps that prefix small (<= kMaxChunks * ep integers).
constexpr int kMaxChunks = 64;

// Batches of at most this many routed copies dispatch in one launch: each
// block counts the regions of all earlier copies itself (see
// dispatch_small_kernel), so no separate routing kernel runs.  Up to
// kSmallItemsShort copies each lane holds 8 of the ids, above that 16.
constexpr int kSmallItems = 4096;
constexpr int kSmallItemsShort = 2048;

// True when dispatch uses the single-launch path.
inline bool dispatch_is_small(int32_t num_tokens, int32_t top_k) {
    return (int64_t)num_tokens * top_k <= kSmallItems;
}

struct RoutePlan {
    int32_t tokens_per_chunk;
    int32_t n_chunks;
};

// Chunks of whole tokens for the routing kernel: at most kMaxChunks.
inline RoutePlan plan_route(int32_t num_tokens) {
    RoutePlan p;
    p.tokens_per_chunk = num_tokens > 0 ? (num_tokens + kMaxChunks - 1) / kMaxChunks : 1;
    p.n_chunks = num_tokens > 0 ? (num_tokens + p.tokens_per_chunk - 1) / p.tokens_per_chunk : 0;
    return p;
}

// Scratch layout: rank[max_tokens * k] then hist[kMaxChunks * ep] (int32),
// then, for a handle's own scratch, the single-pass dispatch's words:
// rank words [min(max_items, kOnePassItems)] and hist words
// [kMaxChunks * ep] (uint64, 8-byte aligned).
inline int32_t *scratch_rank(void *scratch) { return static_cast<int32_t *>(scratch); }
inline int32_t *scratch_hist(void *scratch, int64_t max_items) {
    return static_cast<int32_t *>(scratch) + max_items;
}
constexpr int64_t kOnePassWordItems = 65536;     // rank words: the single pass's largest batch
inline int64_t scratch_words_offset(int64_t max_items, int ep) {
    return ((max_items + (int64_t)kMaxChunks * ep) * 4 + 7) / 8 * 8;
}
inline int64_t scratch_words_count(int64_t max_items, int ep) {
    return (max_items < kOnePassWordItems ? max_items : kOnePassWordItems) + (int64_t)kMaxChunks * ep;
}
inline uint64_t *scratch_rank_words(void *scratch, int64_t max_items, int ep) {
    return reinterpret_cast<uint64_t *>(static_cast<char *>(scratch) + scratch_words_offset(max_items, ep));
}
inline uint64_t *scratch_hist_words(void *scratch, int64_t max_items, int ep) {
    return scratch_rank_words(scratch, max_items, ep) +
           (max_items < kOnePassWordItems ? max_items : kOnePassWordItems);
}


struct RouteArgs {
    const int32_t *ids;      // [T*k]
    int32_t *rank;           // [T*k] rank of the copy among its chunk's copies to the same region
    int32_t *hist;           // [n_chunks * ep] copies per (chunk, region)
    int32_t *status;         // MOE_STATUS_* bits
    int64_t n_items;         // T*k
    int32_t items_per_chunk;
    int32_t ep, epr, n_experts;
    int32_t epr_shift;       // log2(epr) when epr is a power of two, else -1
    int32_t k;
    int32_t per_region;      // 1: only a token's first copy to a region takes a row
};

struct DispatchArgs {
    const uint16_t *x;       // [T, H]
    const int32_t *ids;      // [T, k]
    const int32_t *rank;
    const int32_t *hist;
    uint16_t *ws;            // [ep, cap, H]
    int32_t *counts;         // [ep]
    int32_t *slot_index;     // [T*k]
    int32_t *src_index;      // [ep*cap]
    int32_t *status;
    int32_t T, H, k, ep, epr, n_experts, cap;
    int32_t epr_shift;       // log2(epr) when epr is a power of two, else -1
    int32_t tokens_per_chunk, n_chunks;
    int32_t count_only;      // 1: only write counts
    int32_t per_region;      // 1: one row per (token, region), duplicates share it
    int32_t fp8;             // 1: payload is e4m3 rows in ws8 plus one scale per row
    uint8_t *ws8;            // [ep, cap, H] e4m3 (fp8 payload)
    float *scales;           // [ep, cap]    row scales (fp8 payload)
    int32_t t_base;          // first token of this launch (set by launch_dispatch_copy)
    // single-pass dispatch (onepass != 0): the first route_blocks blocks rank
    // the chunks into rank_w / hist_w words of `epoch`; the others wait for
    // the words they need, giving up after spin_limit polls
    int32_t onepass;
    int32_t route_blocks;
    uint32_t epoch;
    int32_t spin_limit;      // < 0: every wait gives up at once (tests of the give-up path)
    uint64_t *rank_w;        // [T*k]
    uint64_t *hist_w;        // [n_chunks * ep]
};

struct CombineArgs {
    const uint16_t *y;       // [ep, cap, H] expert outputs in the dispatch layout
    const int32_t *slot_index;
    const float *w;          // [T, k] gates (weighted only)
    uint16_t *out;           // [T, H] (plain combine)
    const uint16_t *residual;     // [T, H] (fused)
    uint16_t *residual_out;       // [T, H] (fused; may alias residual)
    const uint16_t *gamma;        // [H]    (fused)
    uint16_t *normed;             // [T, H] (fused)
    float eps;
    int32_t T, H, k, weighted;
    int32_t per_region;      // 1: add each distinct row of a token once
    int32_t partials;        // 1: y holds [k, T, H] partials; row j of token t is j*T + t
                             //    (slot_index unused, every row valid)
    int32_t out_cached;      // set by launch_combine: output store cache policy (see kernels.hip)
};

// Batches of more than kSmallItems and at most kOnePassItems copies in the
// per-copy layout dispatch in one launch that ranks the chunks in its first
// blocks (dispatch_onepass_kernel).
constexpr int64_t kOnePassItems = kOnePassWordItems;
// The single pass loads each source row before its routing words for
// batches of more than kOnePassRowFirstFrom and at most kOnePassRowFirstItems
// copies, after them otherwise.
constexpr int64_t kOnePassRowFirstFrom = 28672;
constexpr int64_t kOnePassRowFirstItems = 32768;
inline bool dispatch_is_onepass(int32_t num_tokens, int32_t top_k, bool per_region) {
    const int64_t items = (int64_t)num_tokens * top_k;
    return !per_region && items > kSmallItems && items <= kOnePassItems;
}
// Polls of one word before a single-pass block gives up (each poll is a
// device-scope load after a short sleep).
constexpr int32_t kOnePassSpinLimit = 1 << 16;

hipError_t launch_route(const RouteArgs &a, int32_t n_chunks, hipStream_t s);
// The single-pass dispatch (see dispatch_onepass_kernel).
hipError_t launch_dispatch_onepass(const DispatchArgs &a, const RouteArgs &ra, hipStream_t s);
// Launches dispatch_small_kernel when dispatch_is_small(T, k) (no routing
// kernel needed), dispatch_copy_kernel otherwise (after launch_route).
hipError_t launch_dispatch_copy(const DispatchArgs &a, hipStream_t s);
hipError_t launch_combine(const CombineArgs &a, bool fused, hipStream_t s);

}  // namespace moe
