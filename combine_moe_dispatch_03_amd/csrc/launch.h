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

// Scratch layout: rank[max_tokens * k] then hist[kMaxChunks * ep].
inline int32_t *scratch_rank(void *scratch) { return static_cast<int32_t *>(scratch); }
inline int32_t *scratch_hist(void *scratch, int64_t max_items) {
    return static_cast<int32_t *>(scratch) + max_items;
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

hipError_t launch_route(const RouteArgs &a, int32_t n_chunks, hipStream_t s);
// Launches dispatch_small_kernel when dispatch_is_small(T, k) (no routing
// kernel needed), dispatch_copy_kernel otherwise (after launch_route).
hipError_t launch_dispatch_copy(const DispatchArgs &a, hipStream_t s);
hipError_t launch_combine(const CombineArgs &a, bool fused, hipStream_t s);

}  // namespace moe
