// Drives the host side of the C ABI (argument checks, phase machine, scratch
// carving, HIP error path) built with host-only AddressSanitizer and
// UndefinedBehaviorSanitizer by test_sanitizers.py.  The kernel launchers are
// replaced by stubs that check the argument blocks against the caller's
// buffers and count launches, so no GPU is needed; moe_sync_status runs into
// the HIP runtime and must either succeed or report MOE_ERR_HIP.  The stream
// capture query and the memset are stand-ins defined here (the executable's
// own definitions come before the runtime's), so that the single-pass branch
// (its epochs and the clearing of its words) runs on the host as well.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "launch.h"
#include "moe_a2a.h"

static const int32_t *g_scratch = nullptr;   // the scratch buffer handed to moe_init
static int64_t g_scratch_ints = 0;

static bool in_scratch(const int32_t *p, int64_t n) {
    return p >= g_scratch && n >= 0 && (p - g_scratch) + n <= g_scratch_ints;
}

// -1: the capture query fails (as it does with no device: the library then
// takes the capture-safe path), 0: the stream is not capturing, 1: it is.
static int g_capture = -1;
static int g_memsets = 0;                     // memsets that landed in the scratch buffer
extern "C" hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus *st) {
    if (g_capture < 0) return hipErrorNoDevice;
    *st = g_capture ? hipStreamCaptureStatusActive : hipStreamCaptureStatusNone;
    return hipSuccess;
}
extern "C" hipError_t hipMemsetAsync(void *dst, int value, size_t bytes, hipStream_t) {
    // the only device memory the dispatch clears is the single pass's words,
    // inside the scratch buffer (host memory here)
    const int32_t *p = static_cast<const int32_t *>(dst);
    if (bytes % 4 != 0 || !in_scratch(p, (int64_t)(bytes / 4))) std::abort();
    std::memset(dst, value, bytes);
    ++g_memsets;
    return hipSuccess;
}

namespace moe {
static int launches = 0;
static int fail_partials = 0;     // a partials launch of this many rows reports a HIP error
// plan_route and dispatch_is_small are the library's own (inline in launch.h)
hipError_t launch_route(const RouteArgs &a, int32_t n_chunks, hipStream_t) {
    if (n_chunks < 1 || n_chunks > kMaxChunks || a.n_items < 1) std::abort();
    if (!in_scratch(a.rank, a.n_items) || !in_scratch(a.hist, (int64_t)n_chunks * a.ep)) std::abort();
    if ((int64_t)a.items_per_chunk * n_chunks < a.n_items) std::abort();
    ++launches;
    return hipSuccess;
}
hipError_t launch_dispatch_copy(const DispatchArgs &a, hipStream_t) {
    if (a.T < 0 || a.n_chunks > kMaxChunks || (a.fp8 && (!a.ws8 || !a.scales))) std::abort();
    if (!dispatch_is_small(a.T, a.k) &&
        (!in_scratch(a.rank, (int64_t)a.T * a.k) || !in_scratch(a.hist, (int64_t)a.n_chunks * a.ep)))
        std::abort();
    ++launches;
    return hipSuccess;
}
static int onepass_launches = 0;
hipError_t launch_dispatch_onepass(const DispatchArgs &a, const RouteArgs &ra, hipStream_t) {
    // a mid-size per-copy batch whose words lie inside the scratch buffer
    if (!a.onepass || a.per_region || !dispatch_is_onepass(a.T, a.k, false)) std::abort();
    if (a.fp8 && (!a.ws8 || !a.scales)) std::abort();
    if (a.epoch == 0 || a.spin_limit == 0 || ra.n_items != (int64_t)a.T * a.k) std::abort();
    const char *lo = reinterpret_cast<const char *>(g_scratch);
    const char *hi = lo + g_scratch_ints * 4;
    const char *rw = reinterpret_cast<const char *>(a.rank_w), *hw = reinterpret_cast<const char *>(a.hist_w);
    if (rw < lo || rw + (int64_t)a.T * a.k * 8 > hi || hw < lo || hw + (int64_t)a.n_chunks * a.ep * 8 > hi)
        std::abort();
    if (reinterpret_cast<uintptr_t>(rw) % 8 != 0 || hw < rw + (int64_t)a.T * a.k * 8) std::abort();
    ++launches;
    ++onepass_launches;
    return hipSuccess;
}
hipError_t launch_combine(const CombineArgs &a, bool fused, hipStream_t) {
    if (a.T < 0 || a.k < 1 || (fused && (!a.residual || !a.gamma || !a.normed))) std::abort();
    // a partials reduction binds no handle: no slot_index, unweighted, every row p*T + t
    if (a.partials && (a.slot_index || a.weighted || a.per_region || a.w ||
                       (int64_t)a.k * a.T > INT32_MAX || (a.T > 0 && (!a.y || (!fused && !a.out)))))
        std::abort();
    if (!a.partials && !a.slot_index) std::abort();
    if (a.partials && a.k == fail_partials) return hipErrorInvalidValue;
    ++launches;
    return hipSuccess;
}
}  // namespace moe

#define CHECK(cond) do { if (!(cond)) { std::printf("FAILED: %s (line %d)\n", #cond, __LINE__); return 1; } } while (0)
// launches made by one call
#define LAUNCHES(call, n) do { int before_ = moe::launches; CHECK((call) == MOE_OK); CHECK(moe::launches - before_ == (n)); } while (0)

int main() {
    const int32_t T = 640, H = 128, k = 8, E = 64, ep = 8;
    // aligned host buffers stand in for device memory: the stubs never dereference them
    std::vector<int32_t> counts(ep), src(ep * T), slot(T * k), status(4);
    // stand-ins sized as the handle declares them (cap = T), so the overlap
    // checks see the real extents
    alignas(16) static uint16_t x[T * H], ws[ep * T * H], out[1 << 12];
    alignas(16) static uint16_t rows[3 * T * H];     // residual | normed | gamma, disjoint
    uint16_t *res = rows, *nrm = rows + T * H, *gam = rows + 2 * T * H;
    alignas(16) static uint8_t ws8[ep * T * H];
    static float w[T * k], scales[ep * T];
    static int32_t ids[T * k];
    const size_t sb = moe_scratch_bytes(T, k, ep);
    CHECK(sb >= (size_t)T * k * 4);
    std::vector<int32_t> scratch(sb / 4);
    g_scratch = scratch.data();
    g_scratch_ints = (int64_t)scratch.size();
    CHECK(moe_scratch_bytes(T, k, ep) == sb);

    moe_handle h;
    CHECK(moe_init(&h, T, H, k, E, ep, T, MOE_LAYOUT_PER_COPY, counts.data(), src.data(),
                   slot.data(), status.data(), scratch.data(), sb - 4) == MOE_ERR_ARG);
    CHECK(moe_init(&h, T, H, k, E, ep, T, MOE_LAYOUT_PER_COPY, counts.data(), src.data(),
                   slot.data(), status.data(), scratch.data(), sb) == MOE_OK);
    CHECK(moe_combine(&h, ws, w, 1, out, nullptr) == MOE_ERR_PHASE);
    LAUNCHES(moe_dispatch(&h, x, ids, T, T, ws, nullptr), 2);           // routed: route + copy
    CHECK(h.phase == 1 && h.num_tokens == T);
    CHECK(moe_dispatch(&h, x, ids, T, T, ws, nullptr) == MOE_ERR_PHASE);
    CHECK(moe_combine(&h, ws, nullptr, 1, out, nullptr) == MOE_ERR_ARG && h.phase == 1);
    LAUNCHES(moe_combine(&h, ws, w, 1, out, nullptr), 1);
    CHECK(h.phase == 0);
    LAUNCHES(moe_dispatch(&h, x, ids, 256, 256, ws, nullptr), 1);      // 2048 copies: single launch
    LAUNCHES(moe_combine_residual_rmsnorm(&h, ws, w, 1, res, res, gam, 1e-6f, nrm, nullptr), 1);
    LAUNCHES(moe_dispatch(&h, x, ids, 257, 300, ws, nullptr), 1);      // 2056 copies: single launch
    CHECK(moe_reset(&h) == MOE_OK && h.phase == 0);
    LAUNCHES(moe_dispatch(&h, x, ids, 512, 512, ws, nullptr), 1);      // 4096 copies: the last single launch
    CHECK(moe_reset(&h) == MOE_OK && h.phase == 0);
    LAUNCHES(moe_dispatch(&h, x, ids, 513, 600, ws, nullptr), 2);      // first routed size
    CHECK(moe_reset(&h) == MOE_OK && h.phase == 0);
    LAUNCHES(moe_dispatch_fp8(&h, x, ids, T, T, ws8, scales, nullptr), 2);
    CHECK(moe_reset(&h) == MOE_OK);
    LAUNCHES(moe_route_counts(&h, ids, T, nullptr), 2);
    CHECK(h.phase == 0);
    CHECK(moe_dispatch(&h, x, ids, T + 1, T, ws, nullptr) == MOE_ERR_ARG);
    CHECK(moe_dispatch(&h, x, ids, 10, T + 1, ws, nullptr) == MOE_ERR_ARG);
    CHECK(moe_dispatch(&h, x + 1, ids, 10, 10, ws, nullptr) == MOE_ERR_ARG);   // misaligned rows
    LAUNCHES(moe_dispatch(&h, x, ids, 0, 1, ws, nullptr), 1);          // empty batch
    LAUNCHES(moe_combine(&h, ws, nullptr, 0, nullptr, nullptr), 1);

    // the status read needs the HIP runtime; with no GPU it must fail cleanly
    int32_t bits = -1;
    const int rc = moe_sync_status(&h, nullptr, &bits);
    CHECK(rc == MOE_ERR_HIP || rc == MOE_OK);
    CHECK(rc != MOE_ERR_HIP || h.hip_error != 0);

    // the single pass: a mid-size per-copy batch on a stream that is not
    // capturing; the handle's first single-pass dispatch clears the words,
    // later ones only take the next epoch, the one after the last epoch
    // clears them again; under capture, and for the per-region layout, the
    // routing kernel and the copy kernel instead
    {
        g_capture = 0;
        moe_handle p;
        CHECK(moe_init(&p, T, H, k, E, ep, T, MOE_LAYOUT_PER_COPY, counts.data(), src.data(),
                       slot.data(), status.data(), scratch.data(), sb) == MOE_OK);
        const int m0 = g_memsets, o0 = moe::onepass_launches;
        LAUNCHES(moe_dispatch(&p, x, ids, T, T, ws, nullptr), 1);
        CHECK(p.onepass_epoch == 1 && g_memsets == m0 + 1 && moe::onepass_launches == o0 + 1);
        CHECK(moe_dispatch(&p, x, ids, T, T, ws, nullptr) == MOE_ERR_PHASE && p.onepass_epoch == 1);
        LAUNCHES(moe_combine(&p, ws, nullptr, 0, out, nullptr), 1);
        LAUNCHES(moe_dispatch_fp8(&p, x, ids, T, T, ws8, scales, nullptr), 1);
        CHECK(p.onepass_epoch == 2 && g_memsets == m0 + 1 && moe::onepass_launches == o0 + 2);
        CHECK(moe_reset(&p) == MOE_OK);
        LAUNCHES(moe_dispatch(&p, x, ids, 512, 512, ws, nullptr), 1);   // 4096 copies: single launch
        CHECK(p.onepass_epoch == 2 && moe::onepass_launches == o0 + 2);
        CHECK(moe_reset(&p) == MOE_OK);
        p.onepass_epoch = 0x7FFFFFFF;
        LAUNCHES(moe_dispatch(&p, x, ids, 513, 600, ws, nullptr), 1);   // after the last epoch
        CHECK(p.onepass_epoch == 1 && g_memsets == m0 + 2);
        CHECK(moe_reset(&p) == MOE_OK);
        g_capture = 1;
        LAUNCHES(moe_dispatch(&p, x, ids, T, T, ws, nullptr), 2);
        CHECK(moe_reset(&p) == MOE_OK);
        LAUNCHES(moe_dispatch_fp8(&p, x, ids, T, T, ws8, scales, nullptr), 2);
        CHECK(moe_reset(&p) == MOE_OK);
        CHECK(p.onepass_epoch == 1 && g_memsets == m0 + 2 && moe::onepass_launches == o0 + 3);
        g_capture = 0;
        moe_handle q;
        CHECK(moe_init(&q, T, H, k, E, ep, T, MOE_LAYOUT_PER_REGION, counts.data(), src.data(),
                       slot.data(), status.data(), scratch.data(), sb) == MOE_OK);
        LAUNCHES(moe_dispatch(&q, x, ids, T, T, ws, nullptr), 2);
        CHECK(q.onepass_epoch == 0 && moe::onepass_launches == o0 + 3);
        g_capture = -1;
    }

    // per-region layout rejects a weighted combine
    moe_handle g;
    CHECK(moe_init(&g, T, H, k, E, ep, T, MOE_LAYOUT_PER_REGION, counts.data(), src.data(),
                   slot.data(), status.data(), scratch.data(), sb) == MOE_OK);
    LAUNCHES(moe_dispatch(&g, x, ids, T, T, ws, nullptr), 2);
    CHECK(moe_combine(&g, ws, w, 1, out, nullptr) == MOE_ERR_ARG);
    LAUNCHES(moe_combine(&g, ws, nullptr, 0, out, nullptr), 1);
    for (int code = -6; code <= 1; ++code) CHECK(moe_strerror(code) != nullptr);

    // buffers overlapping what a call reads are rejected before any launch
    {
        moe_handle o;
        CHECK(moe_init(&o, T, H, k, E, ep, T, MOE_LAYOUT_PER_COPY, counts.data(), src.data(),
                       slot.data(), status.data(), scratch.data(), sb) == MOE_OK);
        CHECK(moe_dispatch(&o, ws + 8 * H, ids, 16, 16, ws, nullptr) == MOE_ERR_ARG);  // x inside ws
        CHECK(moe_dispatch_fp8(&o, x, ids, 16, 16, ws8, reinterpret_cast<float *>(ws8 + 64),
                               nullptr) == MOE_ERR_ARG);                            // scales inside ws8
        CHECK(moe_dispatch(&o, x, reinterpret_cast<const int32_t *>(ws), 16, 16, ws, nullptr) ==
              MOE_ERR_ARG);                                                         // ids inside ws
        CHECK(moe_dispatch(&o, reinterpret_cast<const uint16_t *>(scratch.data()), ids, 16, 16, ws,
                           nullptr) == MOE_ERR_ARG);                                // x over scratch
        CHECK(moe_dispatch(&o, x, slot.data(), 16, 16, ws, nullptr) == MOE_ERR_ARG);  // ids = slot_index
        CHECK(moe_dispatch(&o, x, ids, 16, 16, reinterpret_cast<uint16_t *>(src.data()), nullptr) ==
              MOE_ERR_ARG);                                                         // ws over src_index
        CHECK(moe_dispatch_fp8(&o, x, ids, 16, 16, ws8, reinterpret_cast<float *>(counts.data()),
                               nullptr) == MOE_ERR_ARG);                            // scales = counts
        CHECK(moe_route_counts(&o, counts.data(), 1, nullptr) == MOE_ERR_ARG);     // ids = counts
        CHECK(o.phase == 0);
        LAUNCHES(moe_dispatch(&o, x, ids, 16, 16, ws, nullptr), 1);
        CHECK(moe_combine(&o, ws, nullptr, 0, ws + 16 * H, nullptr) == MOE_ERR_ARG);  // out inside ws
        CHECK(moe_combine(&o, ws, reinterpret_cast<const float *>(out), 1, out, nullptr) ==
              MOE_ERR_ARG);                                                         // out over weights
        CHECK(moe_combine(&o, ws, nullptr, 0, reinterpret_cast<uint16_t *>(slot.data()), nullptr) ==
              MOE_ERR_ARG);                                                         // out over slot_index
        CHECK(moe_combine(&o, ws, nullptr, 0, reinterpret_cast<uint16_t *>(status.data()), nullptr) ==
              MOE_ERR_ARG);                                                         // out over status
        CHECK(moe_combine_residual_rmsnorm(&o, ws, reinterpret_cast<const float *>(nrm), 1, res, res,
                                           gam, 1e-6f, nrm, nullptr) == MOE_ERR_ARG);  // normed over weights
        CHECK(moe_combine_residual_rmsnorm(&o, ws, nullptr, 0, res,
                                           reinterpret_cast<uint16_t *>(scratch.data()), gam, 1e-6f,
                                           nrm, nullptr) == MOE_ERR_ARG);         // residual_out over scratch
        CHECK(moe_combine_residual_rmsnorm(&o, ws, nullptr, 0, res, res, gam, 1e-6f, res + 8 * H,
                                           nullptr) == MOE_ERR_ARG);              // normed over residual
        CHECK(moe_combine_residual_rmsnorm(&o, ws, nullptr, 0, res, res, gam, 1e-6f, ws + H,
                                           nullptr) == MOE_ERR_ARG);              // normed inside ws
        CHECK(moe_combine_residual_rmsnorm(&o, ws, nullptr, 0, res, res + 8, gam, 1e-6f, nrm,
                                           nullptr) == MOE_ERR_ARG);              // residual_out shifted
        CHECK(o.phase == 1);
        LAUNCHES(moe_combine_residual_rmsnorm(&o, ws, nullptr, 0, res, res, gam, 1e-6f, nrm,
                                              nullptr), 1);                       // in-place residual
        CHECK(o.phase == 0);
    }

    // partials reduction: no handle, one launch per call, nothing for an empty batch
    // beyond the (skipped-inside) launch call, checks before anything is enqueued
    LAUNCHES(moe_partials_reduce(ws, 8, 4, H, out, nullptr), 1);
    LAUNCHES(moe_partials_reduce_residual_rmsnorm(ws, 8, 4, H, out, out, out + 1024, 1e-6f,
                                                  out + 2048, nullptr), 1);
    LAUNCHES(moe_partials_reduce(nullptr, 8, 0, H, nullptr, nullptr), 1);
    CHECK(moe_partials_reduce(ws, 0, 4, H, out, nullptr) == MOE_ERR_ARG);
    CHECK(moe_partials_reduce(ws, MOE_MAX_PARTIALS + 1, 4, H, out, nullptr) == MOE_ERR_ARG);
    CHECK(moe_partials_reduce(ws + 1, 8, 4, H, out, nullptr) == MOE_ERR_ARG);
    CHECK(moe_partials_reduce_residual_rmsnorm(ws, 8, 4, MOE_MAX_FUSED_HIDDEN + 8, out, out, out,
                                               1e-6f, out, nullptr) == MOE_ERR_ARG);
    // outputs overlapping their inputs or each other are rejected; the
    // in-place residual (residual_out == residual) is allowed
    {
        alignas(16) static uint16_t pool[8 * 4 * 16 + 6 * 4 * 16];
        const int32_t P = 8, Tn = 4, Hn = 16, n = Tn * Hn;
        uint16_t *parts = pool, *res = pool + P * n, *nrm = res + n, *gam = nrm + n;
        CHECK(moe_partials_reduce(parts, P, Tn, Hn, parts + (P - 1) * n + 8, nullptr) == MOE_ERR_ARG);
        LAUNCHES(moe_partials_reduce(parts, P, Tn, Hn, res, nullptr), 1);
        LAUNCHES(moe_partials_reduce_residual_rmsnorm(parts, P, Tn, Hn, res, res, gam, 1e-6f, nrm,
                                                      nullptr), 1);
        CHECK(moe_partials_reduce_residual_rmsnorm(parts, P, Tn, Hn, res, res, gam, 1e-6f, res,
                                                   nullptr) == MOE_ERR_ARG);
        CHECK(moe_partials_reduce_residual_rmsnorm(parts, P, Tn, Hn, res, res + 8, gam, 1e-6f, nrm,
                                                   nullptr) == MOE_ERR_ARG);
        CHECK(moe_partials_reduce_residual_rmsnorm(parts, P, Tn, Hn, res, res, nrm, 1e-6f, nrm,
                                                   nullptr) == MOE_ERR_ARG);
    }
    // a handle without scratch serves moe_dispatch_noalloc only; that call
    // rejects batches beyond its static scratch before anything else
    {
        moe_handle n;
        CHECK(moe_init(&n, T, H, k, E, ep, T, MOE_LAYOUT_PER_COPY, counts.data(), src.data(),
                       slot.data(), status.data(), nullptr, 0) == MOE_OK);
        CHECK(moe_init(&n, T, H, k, E, ep, T, MOE_LAYOUT_PER_COPY, counts.data(), src.data(),
                       slot.data(), status.data(), nullptr, 4) == MOE_ERR_ARG);
        CHECK(moe_init(&n, T, H, k, E, ep, T, MOE_LAYOUT_PER_COPY, counts.data(), src.data(),
                       slot.data(), status.data(), nullptr, 0) == MOE_OK);
        const int before = moe::launches;
        CHECK(moe_dispatch(&n, x, ids, T, T, ws, nullptr) == MOE_ERR_ARG);
        CHECK(moe_dispatch_fp8(&n, x, ids, T, T, ws8, scales, nullptr) == MOE_ERR_ARG);
        CHECK(moe_route_counts(&n, ids, T, nullptr) == MOE_ERR_ARG);
        CHECK(moe::launches == before && n.phase == 0);
        moe_handle big;
        const int32_t Tb = MOE_NOALLOC_MAX_ITEMS / k + 1;
        CHECK(moe_init(&big, Tb, H, k, E, ep, 1, MOE_LAYOUT_PER_COPY, counts.data(), src.data(),
                       slot.data(), status.data(), nullptr, 0) == MOE_OK);
        CHECK(moe_dispatch_noalloc(&big, x, ids, Tb, Tb, ws, nullptr) == MOE_ERR_NOALLOC_SIZE);
        CHECK(moe::launches == before && big.phase == 0);
    }

    // a failed partials launch keeps its hipError_t for moe_last_hip_error
    moe::fail_partials = 5;
    CHECK(moe_partials_reduce(ws, 5, 4, H, out, nullptr) == MOE_ERR_HIP);
    CHECK(moe_last_hip_error() == (int)hipErrorInvalidValue);
    CHECK(moe_partials_reduce_residual_rmsnorm(ws, 5, 4, H, out, out, out + 1024, 1e-6f, out + 2048,
                                               nullptr) == MOE_ERR_HIP);
    CHECK(moe_last_hip_error() == (int)hipErrorInvalidValue);
    moe::fail_partials = 0;
    // outside the block above the capture query fails, which the library
    // reads as capture: those routed dispatches take the two-kernel path
    std::printf("sanitized ABI driver: ok (%d launches, %d single-pass, sync_status rc %d)\n",
                moe::launches, moe::onepass_launches, rc);
    return 0;
}
