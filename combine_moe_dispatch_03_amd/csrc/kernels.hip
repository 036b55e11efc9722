// gfx950 kernels of the MoE dispatch / combine path.
//
// Nothing here is a dense contraction, so nothing uses MFMA: the path is
// bound by HBM bandwidth.  Five kernels:
//
//  route_rank_kernel     per chunk of tokens: each routed copy's rank among
//                        the chunk's copies to the same region (a stable
//                        wave-ballot scan), and the chunk's region histogram.
//  dispatch_copy_kernel  per pair of routed copies (four for the fp8
//                        payload, a whole token for rows under 8 KB; x column
//                        block): the slots of its token's copies (chunk
//                        prefix + rank), the index maps, and the 16-byte row
//                        copies x[t] -> workspace rows.  A token's blocks run
//                        on one XCD, so its source row comes from that XCD's
//                        L2 after the first read.
//  dispatch_small_kernel the whole dispatch in one launch for small batches
//                        (decode): each block counts the earlier copies
//                        itself instead of reading route_rank_kernel's output.
//  dispatch_onepass_kernel routing and copy in one launch for mid-size
//                        batches (per-copy layout, bf16 or fp8): its first blocks do
//                        route_rank_kernel's work and publish it as
//                        epoch-tagged words, which the copy blocks wait for.
//  combine_kernel        per token (x column block): gathers the k rows
//                        (routed copies, or the partials of an all-reduce),
//                        accumulates in fp32 in j order, narrows once to
//                        bf16 (nearest-even); optionally adds the residual
//                        and applies RMSNorm with a block-reduced sum of
//                        squares (the whole row stays in registers).
//
// Sources: InferenceX PR #2450 "CollectiveX: add FlashInfer one-sided NVLink
// EP for the GB SKUs" ("The adapter" table; "Kernel arithmetic read from
// source": 16-byte stores, nearest-even narrowing; "Update -- the correctness
// failures are resolved": fp32 accumulator, single narrowing); vLLM PR #41382
// "[Bugfix] Fix double reduce ..." (one reduction over the experts); magik.net
// "Fusing the Allreduce: ..." section "The Message Itself: Explanation and
// Probe" (residual + RMSNorm fused onto the producing reduction).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "launch.h"
#include "moe_a2a.h"

namespace moe {
namespace {

static_assert(MOE_MAX_PARTIALS <= MOE_MAX_TOP_K, "partials use the combine's per-token row arrays");
static_assert(MOE_MAX_TOP_K <= 64, "one wave compacts a token's rows");

constexpr int kThreads = 256;            // 4 wave64 per workgroup
constexpr int kWaves = kThreads / 64;
// Cache policy of the combine's output stores (out, residual_out, normed):
// each row is written once here and read by the next layer, not by this
// kernel.  The policy bits of a gfx950 vector memory instruction are sc0 = 1,
// nt = 2, sc1 = 16.  Measured at the prefill shape (combine after a dispatch):
// plain stores 91.8 us, non-temporal 90.1 us, sc1 86.0-86.6 us.  With sc1 the
// rows stay in the 256 MB Infinity Cache, which only pays while a launch's
// outputs fit there beside the rest of the step: at H = 7168, top-8, a step
// (dispatch + combine) gains 4-8 us up to T = 8192 (117 MB of output) but
// loses 35-85 us from T = 10240 (147 MB) on, because the next kernel pays for
// writing the rows back (dispatch 230 -> 268 us at T = 10240).  So outputs up
// to kOutCachedBytes per launch are stored with sc1 and larger ones
// non-temporally.  The gathered loads stay non-temporal (every policy with nt
// measured the same, the others 5 us slower), and so do the dispatch's
// workspace stores (sc1 there is 10 % slower).
constexpr int kPolicyNT = 2;
constexpr int kPolicySC1 = 16;
constexpr int64_t kOutCachedBytes = int64_t(120) << 20;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16 is the high half of a binary32 pattern: widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16 pair, nearest-even (gfx950 v_cvt_pk_bf16_f32).
// The element at the lower address goes to the low half.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// fp64 -> fp32 rounded to odd: the truncation toward zero, with its last bit
// set when the conversion is inexact.  fp32 carries 16 more bits than bf16
// (also among subnormals), so a nearest-even narrowing of this value to bf16
// equals the direct nearest-even rounding of the fp64 value: Boldo and
// Melquiond, "When double rounding is odd" (2005).  NaN and infinities pass
// through; a finite value beyond fp32's range becomes the largest finite
// fp32 (odd), which still narrows to the bf16 infinity.
__device__ __forceinline__ float f64_to_f32_odd(double d) {
    float f = (float)d;                          // nearest-even
    const double back = (double)f;
    if (back != d && d == d) {                   // inexact (and not NaN)
        uint32_t b = __float_as_uint(f);
        if (__builtin_fabs(back) > __builtin_fabs(d)) b -= 1;   // back to the truncation
        f = __uint_as_float(b | 1u);
    }
    return f;
}

__device__ __forceinline__ void unpack8(const u32x4 &r, float (&f)[8]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f[2 * q] = bf16_lo(r[q]);
        f[2 * q + 1] = bf16_hi(r[q]);
    }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = pack_bf16(f[2 * q], f[2 * q + 1]);
    return r;
}

__device__ __forceinline__ u32x4 load16(const uint16_t *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// A buffer resource over one output row of H bf16 values (raw addressing,
// the gfx9 default data format word); `row` is uniform across the wave.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(uint16_t *row, int H) {
    return __builtin_amdgcn_make_buffer_rsrc(row, 0, H * (int)sizeof(uint16_t), 0x00020000);
}

// 16-byte store of element offset `off` of an output row; `cached` (uniform
// across the launch) selects sc1 over non-temporal.
__device__ __forceinline__ void store_out16(__amdgpu_buffer_rsrc_t row, int64_t off, const u32x4 &v,
                                            bool cached) {
    const int byte_off = (int)(off * sizeof(uint16_t));
    if (cached)
        __builtin_amdgcn_raw_buffer_store_b128(v, row, byte_off, 0, kPolicySC1);
    else
        __builtin_amdgcn_raw_buffer_store_b128(v, row, byte_off, 0, kPolicyNT);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Orders this wave's LDS accesses before the call against those after it
// (between lanes of one wave; other waves are not waited for).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// base[r] += sum of hist[i] over i < n with i % ep == r (LDS, all threads).
// When ep divides the block size every entry a thread visits belongs to the
// same region, so the thread adds its entries in a register (loads in flight
// together) and issues one LDS atomic.
__device__ __forceinline__ void add_region_sums(int32_t *base, const int32_t *hist, int n, int ep,
                                                int tid) {
    if (kThreads % ep == 0) {
        int sum = 0;
        for (int i = tid; i < n; i += kThreads) sum += hist[i];
        if (sum != 0) atomicAdd(&base[tid % ep], sum);
    } else {
        for (int i = tid; i < n; i += kThreads) atomicAdd(&base[i % ep], hist[i]);
    }
}

// cbase[j] += sum of hist[c*ep + dests[j]] over chunks c < n_chunks, for the
// token's copies j < k with dests[j] >= 0 (LDS, all threads): the copies of
// earlier chunks in each copy's own region.  kThreads / kp lanes share a copy
// (kp = k rounded up to a power of two), each summing a stride of chunks in a
// register and adding it with one LDS atomic; k x n_chunks loads in all,
// against ep x n_chunks for add_region_sums.
__device__ __forceinline__ void add_copy_sums(int32_t *cbase, const int32_t *dests,
                                              const int32_t *hist, int n_chunks, int ep, int k,
                                              int tid) {
    int kp = 1;
    while (kp < k) kp <<= 1;
    const int lanes = kThreads / kp;
    const int j = tid / lanes, sub = tid % lanes;
    if (j >= k) return;
    const int d = dests[j];
    if (d < 0) return;
    int sum = 0;
    for (int c = sub; c < n_chunks; c += lanes) sum += hist[(int64_t)c * ep + d];
    if (sum != 0) atomicAdd(&cbase[j], sum);
}

// Region of expert e (0 <= e < E): a shift when experts_per_rank is a power
// of two (epr_shift >= 0), else a division.
template <typename Args>
__device__ __forceinline__ int region_of(const Args &a, int e) {
    return a.epr_shift >= 0 ? e >> a.epr_shift : e / a.epr;
}

// Lanes of this wave bound for the same region as this lane (d >= 0), found
// by intersecting one ballot per bit of the region number.  Every lane must
// call this (ballots).
__device__ __forceinline__ uint64_t region_group(int d, int region_bits) {
    uint64_t same = __ballot(d >= 0);
    for (int b = 0; b < region_bits; ++b) {
        const bool bit = d >= 0 && ((d >> b) & 1);
        const uint64_t m = __ballot(bit);
        same &= bit ? m : ~m;
    }
    return same;
}

// Lanes 0 .. n-1 of a wave.
__device__ __forceinline__ uint64_t low_lanes(int n) { return n == 0 ? 0ull : ~0ull >> (64 - n); }

// Per-region layout: true if no earlier copy of the same token (flat indices
// token_base .. i-1) is bound for region d.  Reads the token's ids from L1/L2.
__device__ __forceinline__ bool first_to_region(const int32_t *ids, int64_t token_base, int64_t i,
                                                int d, int epr, int n_experts) {
    for (int64_t q = token_base; q < i; ++q) {
        const int e = ids[q];
        if (e >= 0 && e < n_experts && e / epr == d) return false;
    }
    return true;
}

// The lanes a copy is ranked with: region_group of its region d.  Under the
// per-region layout only a token's first copy to each region is ranked, so
// later copies get d = -1 and leave every group.  A wave's items are
// consecutive flat indices starting at a multiple of k (tiles of 256 from a
// chunk start); when k divides 64 a token's copies are therefore the lanes
// lane - lane % k .. lane, and a copy is first iff none of the earlier ones is
// in its group (one more ballot then drops the later copies).  Otherwise the
// token's earlier ids are re-read before grouping.  Called by every lane with
// uniform k; `active` lanes hold a copy.
template <typename Args>
__device__ __forceinline__ uint64_t rank_group(const Args &a, int &d, int64_t i, bool active,
                                               int region_bits) {
    const bool wave_form = a.per_region && 64 % a.k == 0;
    if (a.per_region && !wave_form && active && d >= 0 &&
        !first_to_region(a.ids, i - i % a.k, i, d, a.epr, a.n_experts))
        d = -1;
    uint64_t same = region_group(d, region_bits);
    if (wave_form) {
        const int lane = threadIdx.x & 63;
        const uint64_t earlier = low_lanes(lane) & ~low_lanes(lane - lane % a.k);
        const bool first = d >= 0 && (same & earlier) == 0;
        same &= __ballot(first);
        if (!first) d = -1;
    }
    return same;
}

// ---------------------------------------------------------------------------
// route_rank_kernel: grid = n_chunks, one workgroup per chunk of whole tokens.
// Items of the chunk are taken 256 at a time (one per thread, flat order).
// Under the per-region layout only a token's first copy to each region is
// ranked (later copies share its row).
// Within a wave, lanes with the same region are found with ballots
// (rank_group); a lane's rank is the number of such lanes below it.  Per-wave
// counts go through LDS to give wave offsets, and a per-region carry runs
// across tiles, so ranks follow the flat order f.
// The ids of kTileGroup tiles are loaded before the first of them is ranked
// (clamped to the chunk, so the loads are unconditional and all in flight),
// instead of one dependent load per tile after the previous tile's barriers.
constexpr int kTileGroup = 4;

// Words of the single-pass dispatch: a 32-bit value under the 32-bit epoch of
// the dispatch that wrote it, stored and loaded whole at device scope (vector
// memory instructions with sc1), so a reader that sees its own epoch in a
// word has that word's value; no other memory is ordered by it.
__device__ __forceinline__ uint64_t load_word(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_word(uint64_t *p, uint32_t epoch, int32_t v) {
    __hip_atomic_store(p, ((uint64_t)epoch << 32) | (uint32_t)v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
// The value of word p once it carries `epoch`; false after `limit` further
// polls (each after a short sleep) without it, or at once when limit < 0.
__device__ __forceinline__ bool wait_word(const uint64_t *p, uint32_t epoch, int limit, int &v) {
    if (limit < 0) return false;                // a forced give-up
    uint64_t w = load_word(p);
    for (int n = 0; (uint32_t)(w >> 32) != epoch; ++n) {
        if (n >= limit) return false;
        __builtin_amdgcn_s_sleep(2);
        w = load_word(p);
    }
    v = (int)(uint32_t)w;
    return true;
}

// The body of route_rank_kernel for one chunk.  WORDS: ranks and the chunk
// histogram go to rank_w / hist_w as words of `epoch` (the single-pass
// dispatch) instead of a.rank / a.hist.
template <bool WORDS>
__device__ __forceinline__ void rank_chunk(const RouteArgs &a, int chunk, int32_t *wave_cnt,
                                           int32_t *carry, uint64_t *rank_w, uint64_t *hist_w,
                                           uint32_t epoch) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ep = a.ep;
    const int64_t begin = (int64_t)chunk * a.items_per_chunk;
    const int64_t end = min(begin + (int64_t)a.items_per_chunk, a.n_items);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    int region_bits = 0;
    while ((1 << region_bits) < ep) ++region_bits;

    for (int r = tid; r < ep; r += kThreads) carry[r] = 0;
    bool bad = false;

    for (int64_t group = begin; group < end; group += kTileGroup * kThreads) {
        int ids[kTileGroup];
#pragma unroll
        for (int g = 0; g < kTileGroup; ++g)       // end > begin: the chunk is never empty
            ids[g] = a.ids[min(group + g * kThreads + tid, end - 1)];
#pragma unroll
        for (int g = 0; g < kTileGroup; ++g) {
            const int64_t tile = group + g * kThreads;
            if (tile >= end) break;                  // uniform
            for (int r = tid; r < kWaves * ep; r += kThreads) wave_cnt[r] = 0;
            __syncthreads();

            const int64_t i = tile + tid;
            int d = -1;
            if (i < end) {
                const int e = ids[g];
                if (e >= 0 && e < a.n_experts)
                    d = region_of(a, e);
                else if (e != -1)
                    bad = true;
            }
            const uint64_t same = a.per_region ? rank_group(a, d, i, i < end, region_bits)
                                               : region_group(d, region_bits);
            const int lane_rank = __popcll(same & below);
            if (d >= 0 && (same >> lane) == 1ull)          // highest lane of its group
                wave_cnt[wave * ep + d] = __popcll(same);
            __syncthreads();

            if (d >= 0) {
                int off = carry[d];
                for (int w = 0; w < wave; ++w) off += wave_cnt[w * ep + d];
                if constexpr (WORDS)
                    store_word(&rank_w[i], epoch, off + lane_rank);
                else
                    a.rank[i] = off + lane_rank;
            }
            __syncthreads();
            for (int r = tid; r < ep; r += kThreads) {
                int add = 0;
                for (int w = 0; w < kWaves; ++w) add += wave_cnt[w * ep + r];
                carry[r] += add;
            }
            __syncthreads();
        }
    }

    if (bad) atomicOr(a.status, MOE_STATUS_EXPERT_ID);
    for (int r = tid; r < ep; r += kThreads) {
        if constexpr (WORDS)
            store_word(&hist_w[(int64_t)chunk * ep + r], epoch, carry[r]);
        else
            a.hist[(int64_t)chunk * ep + r] = carry[r];
    }
}

__global__ __launch_bounds__(kThreads) void route_rank_kernel(RouteArgs a) {
    __shared__ int32_t wave_cnt[kWaves * MOE_MAX_EP];
    __shared__ int32_t carry[MOE_MAX_EP];
    rank_chunk<false>(a, blockIdx.x, wave_cnt, carry, nullptr, nullptr, 0);
}

// ---------------------------------------------------------------------------
// Dispatch helpers.
// Rows of token t's copies: thread tid < k holds copy tid's region d,
// `before` (copies of earlier tokens in region d) and its rank after them;
// writes slot_index / src_index (when cb == 0) and, in copy_rows, the rows
// this block must fill.  Under the per-region layout a copy whose region
// already has a row for this token takes that row and fills nothing.  One
// block barrier: copy_rows is complete after it, and a later copy reads its
// first copy's row from `rows` only after it.
__device__ __forceinline__ void assign_rows(const DispatchArgs &a, int d, int tid, int cb,
                                            int64_t f, int before, int rank,
                                            const int32_t *dests, int32_t *rows,
                                            int32_t *copy_rows) {
    int first = tid;
    if (tid < a.k && d >= 0 && a.per_region)
        for (int j = 0; j < tid; ++j)
            if (dests[j] == d) { first = j; break; }
    int row = -1;
    if (tid < a.k && first == tid) {
        if (d >= 0) {
            const int s = before + rank;
            if (s < a.cap)
                row = d * a.cap + s;
            else if (cb == 0)
                atomicOr(a.status, MOE_STATUS_OVERFLOW);
        }
        rows[tid] = row;
        if (cb == 0 && row >= 0) a.src_index[row] = (int32_t)f;
    }
    if (tid < a.k) copy_rows[tid] = first == tid ? row : -1;
    __syncthreads();
    if (tid < a.k && cb == 0) a.slot_index[f] = first == tid ? row : rows[first];
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Payload writers: the token's row (VPT vectors of 8 bf16 per thread, lanes
// with col >= vpr hold a duplicate vector and store nothing) goes to the rows
// copy_rows[j0 .. j1-1] (-1 = nothing to write), with buffer stores of cache
// policy POLICY (a uniform row base; offsets stay inside the row).
template <int VPT, int POLICY>
__device__ __forceinline__ void store_rows_bf16(const DispatchArgs &a, const u32x4 (&v)[VPT],
                                                const int (&col)[VPT], const int64_t (&off)[VPT],
                                                int vpr, const int32_t *copy_rows, int j0, int j1) {
    for (int j = j0; j < j1; ++j) {
        const int row = uniform(copy_rows[j]);
        if (row < 0) continue;
        const __amdgpu_buffer_rsrc_t dst = row_rsrc(a.ws + (int64_t)row * a.H, a.H);
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            if (col[q] >= vpr) continue;
            __builtin_amdgcn_raw_buffer_store_b128(v[q], dst, (int)(off[q] * sizeof(uint16_t)), 0, POLICY);
        }
    }
}

// FP8 payload: one scale per row.  amax = max |x| over the row (block
// reduction: wave shuffles, then the 4 wave maxima in LDS); scale = amax/448,
// q = e4m3(x * (448/amax)) with gfx950's nearest-even conversion
// (v_cvt_pk_fp8_f32), 8 codes per 8-byte store; an all-zero row gets scale 0
// and zero codes.  The whole row must be in the block (one column block).
template <int VPT, int POLICY>
__device__ __forceinline__ void store_rows_fp8(const DispatchArgs &a, const u32x4 (&v)[VPT],
                                               const int (&col)[VPT], const int64_t (&off)[VPT],
                                               int vpr, const int32_t *copy_rows, float *red,
                                               int tid, int j0, int j1) {
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
        if (col[q] >= vpr) continue;
        float f[8];
        unpack8(v[q], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(f[e]));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    float amax = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) amax = fmaxf(amax, red[w]);
    const float scale = amax / 448.0f;
    const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
    u32x2 qv[VPT];
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
        float f[8];
        unpack8(v[q], f);
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0] * inv, f[1] * inv, 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2] * inv, f[3] * inv, lo, true);
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4] * inv, f[5] * inv, 0, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6] * inv, f[7] * inv, hi, true);
        qv[q] = u32x2{(uint32_t)lo, (uint32_t)hi};
    }
    for (int j = j0; j < j1; ++j) {
        const int row = uniform(copy_rows[j]);
        if (row < 0) continue;
        const __amdgpu_buffer_rsrc_t dst =
            __builtin_amdgcn_make_buffer_rsrc(a.ws8 + (int64_t)row * a.H, 0, a.H, 0x00020000);
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            if (col[q] >= vpr) continue;
            __builtin_amdgcn_raw_buffer_store_b64(qv[q], dst, (int)off[q], 0, POLICY);
        }
        if (tid == 0) a.scales[row] = scale;
    }
}

// dispatch_copy_kernel<VPT, POLICY, FP8, C, ROW_FIRST>: grid = (blocks of C copies, column
// blocks), a launch covering tokens t_base ... ; each thread moves VPT 16-byte
// vectors of the token's row, vector v of block cb at (cb*VPT + v)*256 + tid,
// so every vector step is one coalesced 4 KB stripe.
// Block order: block b holds copy group (b/8) % n of token
// t_base + ((b/8) / n)*8 + b%8, n = ceil(k/C).  Workgroups go round-robin
// over the 8 XCDs, so the n blocks of a token (8 apart) share an XCD: its L2
// serves the source row after the first read.  Measured at T = 4096,
// H = 7168, top-8 (copy alone): one token per block (C = k) 90.4-91.0 us; one
// copy per block 84.2-85.8 us in this order but 131 us in token-major order
// (then each copy's block fetches the row into another XCD's L2); two copies
// per block 85.7-86.6 us; four 88.0 us.  In the dispatch -> combine loop
// (dispatch us, warm / after a 1 GiB cache-evicting read, T = 4096):
//            one block per token   C = 1        C = 2        C = 4
//   bf16     98.4 / 109            89 / 131     95 / 98.5    95 / 110
//   region   68.2 / 79             69 / 108     65 / 75      67 / 81
//   fp8      55.1 / 64             80 / 103     53 / 70      54 / 60
// With C = 1 a token's 8 blocks miss on the same source lines at once, which
// costs more than the split gains once the row is not in the Infinity Cache;
// so bf16 payloads use C = 2 and the fp8 payload (each block also finds the
// row's scale and converts the whole row) C = 4.
// Every block computes the slots of all its token's copies (a few hundred
// bytes from L2); only group 0, column block 0 writes the index maps.
// Load order: vector memory loads complete in the order they are issued, so a
// wait for one load also waits for every load issued before it.  With
// ROW_FIRST the source row's loads go first, then the token's ids and
// in-chunk ranks; the earlier chunks' histogram entries are read after the
// first barrier.  Without it the slot computation's loads (ids, ranks and the
// histogram entries, at most kPreLoads per thread) are issued first and the
// row's last, so the slots are computed while the row is still in flight and
// only the stores wait for it.  When the prefix is summed per copy its
// histogram entries depend on the copies' regions, so there the ids' round
// trip comes before them.  Dispatch us, warm / after a 1 GiB cache-evicting
// read, row first -> row last: prefill 92.5 / 96.1 -> 93.1 / 99.9, fused
// 50.2 / 52.7 -> 49.8 / 53.7, skewed 180.3 / 187.4 -> 180.6 / 186.5,
// per-region prefill 61.6 / 72.9 -> 63.2 / 69.3, per-region skewed
// 90.8 / 118.1 -> 86.4 / 106.2, fp8 prefill 51.2 / 59.5 -> 50.6 / 57.4,
// per-region fp8 prefill 42.2 / 47.0 -> 40.3 / 45.6.  A block that writes
// few rows per row it reads (the per-region layout, ~5.3 rows per token at
// top-8 of 8 regions; the fp8 payload, a quarter of the bytes per row) gains
// from overlapping the row's latency with its slot computation; the
// per-copy bf16 copy writes 8 rows per row read and is faster cold with the
// row requested first.  Issuing its histogram loads together with the ids
// (one round trip fewer) made the skewed dispatch faster warm (180 -> 172)
// but slower cold (188 -> 202) and prefill 6 us slower cold, so that case
// keeps the order above.  Loads of the row are unconditional (lanes past the
// row end re-read the row's last vector and store nothing).
// POLICY is the cache policy of the workspace stores; FP8 writes e4m3 codes
// and a row scale instead of the bf16 row (each block finds the row's scale).
constexpr int kPreLoads = 4;                   // prefix loads per thread issued with the slots' own
template <int VPT, int POLICY, bool FP8, int C, bool ROW_FIRST>
__global__ __launch_bounds__(kThreads) void dispatch_copy_kernel(DispatchArgs a) {
    __shared__ int32_t base[MOE_MAX_EP];
    __shared__ int32_t cbase[MOE_MAX_TOP_K];
    __shared__ int32_t dests[MOE_MAX_TOP_K];
    __shared__ int32_t rows[MOE_MAX_TOP_K];
    __shared__ int32_t copy_rows[MOE_MAX_TOP_K];
    __shared__ float red[kWaves];

    const int tid = threadIdx.x;
    const int cb = blockIdx.y;
    const int ep = a.ep;
    const int n = (a.k + C - 1) / C;            // copy groups per token
    const int b = blockIdx.x;
    const int grp = (b >> 3) % n;
    const int t = a.t_base + ((b >> 3) / n) * 8 + (b & 7);

    if (a.t_base == 0 && b == 0 && cb == 0) {   // region totals over all chunks
        for (int r = tid; r < ep; r += kThreads) base[r] = 0;
        __syncthreads();
        add_region_sums(base, a.hist, a.n_chunks * ep, ep, tid);
        __syncthreads();
        for (int r = tid; r < ep; r += kThreads) a.counts[r] = base[r];
        __syncthreads();
    }
    if (a.count_only || t >= a.T) return;

    const int vpr = a.H >> 3;                   // 16-byte vectors per row
    const uint16_t *src = a.x + (int64_t)t * a.H;
    u32x4 v[VPT];
    int col[VPT];
    int64_t off[VPT];
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
        col[q] = (cb * VPT + q) * kThreads + tid;
        off[q] = (int64_t)min(col[q], vpr - 1) * 8;
    }
    if constexpr (ROW_FIRST) {
#pragma unroll
        for (int q = 0; q < VPT; ++q) v[q] = load16(src + off[q]);
    }

    // This token's ids and in-chunk ranks.
    const int64_t f0 = (int64_t)t * a.k;
    const int64_t f = f0 + tid;
    int e = -1, rank = 0;
    if (tid < a.k) {
        e = a.ids[f];
        rank = a.rank[f];                       // meaningful only for a ranked copy
    }

    // Slots of this token's copies: copies of earlier chunks come first,
    // summed per region, or per copy when there are more regions than copies
    // (for the per-region layout, more than twice as many).  Measured with
    // 16 regions, top-8: per-copy sums took the skewed dispatch from 197 to
    // 188 us after a cache-evicting read (warm equal) but slowed the skewed
    // per-region dispatch from 86 to 88 us warm and 119 to 127 us cold; with
    // 256 regions they lifted T = 4096 from 56.5 to 64.7 % of the HBM peak
    // cold.
    int kp = 1;
    while (kp < a.k) kp <<= 1;
    const bool by_copy = a.per_region ? 2 * kp < ep : kp < ep;
    const int chunk = t / a.tokens_per_chunk;
    // Per region: entries i = tid + q*256 of the chunk * ep entries before
    // this chunk.  Per copy: copy j = tid / lanes sums chunks sub, sub +
    // lanes, ... of its own region (lanes = 256 / kp threads per copy).
    const int lanes = kThreads / kp;
    const int pj = tid / lanes, sub = tid % lanes;
    int pd = -1;                                // per copy: region of copy pj
    int pre[kPreLoads];
    if constexpr (ROW_FIRST) {
        // the histogram entries are read after the first barrier
    } else if (by_copy) {
        if (pj < a.k) {
            const int ej = a.ids[f0 + pj];
            if (ej >= 0 && ej < a.n_experts) pd = region_of(a, ej);
        }
#pragma unroll
        for (int q = 0; q < kPreLoads; ++q) {
            const int c = sub + q * lanes;
            pre[q] = (pd >= 0 && c < chunk) ? a.hist[(int64_t)c * ep + pd] : 0;
        }
    } else {
        const int n_pre = chunk * ep;
#pragma unroll
        for (int q = 0; q < kPreLoads; ++q) {
            const int i = tid + q * kThreads;
            pre[q] = i < n_pre ? a.hist[i] : 0;
        }
    }

    if constexpr (!ROW_FIRST) {                 // the source row, after every load the slots need
#pragma unroll
        for (int q = 0; q < VPT; ++q) v[q] = load16(src + off[q]);
    }

    int d = -1;
    if (tid < a.k) {
        if (e >= 0 && e < a.n_experts) d = region_of(a, e);
        dests[tid] = d;
    }
    if (by_copy) {
        if (tid < a.k) cbase[tid] = 0;
    } else {
        for (int r = tid; r < ep; r += kThreads) base[r] = 0;
    }
    __syncthreads();
    if constexpr (ROW_FIRST) {
        if (by_copy)
            add_copy_sums(cbase, dests, a.hist, chunk, ep, a.k, tid);
        else
            add_region_sums(base, a.hist, chunk * ep, ep, tid);
    } else if (by_copy) {
        if (pj < a.k && pd >= 0) {
            int sum = 0;
#pragma unroll
            for (int q = 0; q < kPreLoads; ++q) sum += pre[q];
            for (int c = sub + kPreLoads * lanes; c < chunk; c += lanes)   // k > 16 only
                sum += a.hist[(int64_t)c * ep + pd];
            if (sum != 0) atomicAdd(&cbase[pj], sum);
        }
    } else {
        const int n_pre = chunk * ep;
        if (kThreads % ep == 0) {               // every entry of this thread is region tid % ep
            int sum = 0;
#pragma unroll
            for (int q = 0; q < kPreLoads; ++q) sum += pre[q];
            for (int i = tid + kPreLoads * kThreads; i < n_pre; i += kThreads) sum += a.hist[i];
            if (sum != 0) atomicAdd(&base[tid % ep], sum);
        } else {
#pragma unroll
            for (int q = 0; q < kPreLoads; ++q) {
                const int i = tid + q * kThreads;
                if (i < n_pre) atomicAdd(&base[i % ep], pre[q]);
            }
            for (int i = tid + kPreLoads * kThreads; i < n_pre; i += kThreads)
                atomicAdd(&base[i % ep], a.hist[i]);
        }
    }
    __syncthreads();
    const int before = d < 0 ? 0 : by_copy ? cbase[tid] : base[d];
    assign_rows(a, d, tid, cb | grp, f, before, rank, dests, rows, copy_rows);
    const int j0 = grp * C, j1 = min(a.k, j0 + C);
    if constexpr (FP8)
        store_rows_fp8<VPT, POLICY>(a, v, col, off, vpr, copy_rows, red, tid, j0, j1);
    else
        store_rows_bf16<VPT, POLICY>(a, v, col, off, vpr, copy_rows, j0, j1);
}

// dispatch_onepass_kernel<VPT, POLICY, C, ROW_FIRST, FP8>: routing and copy
// in one launch for mid-size batches (per-copy layout; the bf16 payload, or
// with FP8 the e4m3 codes and a row scale, whole rows in one block).  Blocks
// 0 .. route_blocks-1 (a multiple of 8, so the copy blocks keep the copy
// kernel's XCD grouping) rank one chunk each, exactly as route_rank_kernel,
// into words of this dispatch's epoch (ranks, and the chunk's per-region
// histogram).  They have the lowest block indices, so they are placed on the
// GPU before any copy block.  Every other block is a copy kernel block: its
// lanes read their rank and histogram words, each polled until it carries
// the epoch (a block of an early chunk needs only the chunks before its
// own), and it loads its source row before those reads (ROW_FIRST) or after
// them.  Measured: for 28673 to 32768 copies the row first is faster (4096
// tokens, hidden 7168, top-8: dispatch 86.4 us against 89.2, step 167.5
// against 169.4); elsewhere the row after the words, which leaves HBM to the
// routing blocks' id reads while the first copy blocks wait (8192 tokens,
// 65536 copies: step 333 us against 341; 1536 to 3584 tokens: steps 0.5 to
// 1.5 us faster, the dispatch after a cache-evicting read 2 to 4 us faster).
// A block that has polled a word spin_limit times without the epoch gives
// up: it sets MOE_STATUS_GAVE_UP, its token's index maps read -1 and it
// writes no row, so every block ends.  Copy block 0, column block 0 also
// sums every chunk's histogram into counts.
template <int VPT, int POLICY, int C, bool ROW_FIRST, bool FP8>
__global__ __launch_bounds__(kThreads) void dispatch_onepass_kernel(DispatchArgs a, RouteArgs ra) {
    __shared__ float red[kWaves];
    __shared__ int32_t wave_cnt[kWaves * MOE_MAX_EP];
    __shared__ int32_t carry[MOE_MAX_EP];
    __shared__ int32_t base[MOE_MAX_EP];
    __shared__ int32_t cbase[MOE_MAX_TOP_K];
    __shared__ int32_t dests[MOE_MAX_TOP_K];
    __shared__ int32_t rows[MOE_MAX_TOP_K];
    __shared__ int32_t copy_rows[MOE_MAX_TOP_K];
    __shared__ int32_t gave_up;

    const int tid = threadIdx.x;
    if ((int)blockIdx.x < a.route_blocks) {
        if (blockIdx.y == 0 && (int)blockIdx.x < a.n_chunks) {
            rank_chunk<true>(ra, blockIdx.x, wave_cnt, carry, a.rank_w, a.hist_w, a.epoch);
        }
        return;
    }
    const int cb = blockIdx.y;
    const int ep = a.ep;
    const int n = (a.k + C - 1) / C;
    const int b = blockIdx.x - a.route_blocks;
    const int grp = (b >> 3) % n;
    const int t = ((b >> 3) / n) * 8 + (b & 7);
    const bool totals = b == 0 && cb == 0;
    if (!totals && t >= a.T) return;

    const int vpr = a.H >> 3;
    const uint16_t *src = a.x + (int64_t)min(t, a.T - 1) * a.H;
    u32x4 v[VPT];
    int col[VPT];
    int64_t off[VPT];
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
        col[q] = (cb * VPT + q) * kThreads + tid;
        off[q] = (int64_t)min(col[q], vpr - 1) * 8;
    }
    if constexpr (ROW_FIRST) {
#pragma unroll
        for (int q = 0; q < VPT; ++q) v[q] = load16(src + off[q]);
    }
    const int64_t f0 = (int64_t)t * a.k;
    const int64_t f = f0 + tid;
    int e = -1;
    if (tid < a.k && t < a.T) e = a.ids[f];
    int d = -1;
    if (tid < a.k) {
        if (e >= 0 && e < a.n_experts) d = region_of(a, e);
        dests[tid] = d;
    }
    int kp = 1;
    while (kp < a.k) kp <<= 1;
    const bool by_copy = a.per_region ? 2 * kp < ep : kp < ep;
    const int chunk = t / a.tokens_per_chunk;
    if (by_copy) {
        if (tid < a.k) cbase[tid] = 0;
    } else {
        for (int r = tid; r < ep; r += kThreads) base[r] = 0;
    }
    if (tid == 0) gave_up = 0;
    __syncthreads();
    bool ok = true;
    if (totals && ok) {                         // region totals over all chunks (in carry)
        for (int r = tid; r < ep; r += kThreads) carry[r] = 0;
        __syncthreads();
        for (int i = tid; i < a.n_chunks * ep; i += kThreads) {
            int w = 0;
            if (!wait_word(a.hist_w + i, a.epoch, a.spin_limit, w)) ok = false;
            if (w != 0) atomicAdd(&carry[i % ep], w);
        }
        __syncthreads();
        for (int r = tid; r < ep; r += kThreads) a.counts[r] = carry[r];
    }
    if (t >= a.T) {                             // the totals block past the batch
        if (!ok) atomicOr(a.status, MOE_STATUS_GAVE_UP);
        return;
    }
    // this token's ranks (a rank word exists only for a ranked copy: one with
    // a region, and under the per-region layout its token's first to it)
    int rank = 0;
    if (ok && tid < a.k && d >= 0) {
        bool ranked = true;
        if (a.per_region)
            for (int j = 0; j < tid; ++j)
                if (dests[j] == d) { ranked = false; break; }
        if (ranked && !wait_word(a.rank_w + f, a.epoch, a.spin_limit, rank)) ok = false;
    }
    if (ok) {
        if (by_copy) {
            const int lanes = kThreads / kp;
            const int j = tid / lanes, sub = tid % lanes;
            if (j < a.k && dests[j] >= 0) {
                int sum = 0;
                for (int c = sub; c < chunk; c += lanes) {
                    int w = 0;
                    if (!wait_word(a.hist_w + (int64_t)c * ep + dests[j], a.epoch, a.spin_limit, w)) ok = false;
                    sum += w;
                }
                if (sum != 0) atomicAdd(&cbase[j], sum);
            }
        } else {
            int sum = 0;
            const bool same_region = kThreads % ep == 0;
            for (int i = tid; i < chunk * ep; i += kThreads) {
                int w = 0;
                if (!wait_word(a.hist_w + i, a.epoch, a.spin_limit, w)) ok = false;
                if (same_region)
                    sum += w;
                else if (w != 0)
                    atomicAdd(&base[i % ep], w);
            }
            if (same_region && sum != 0) atomicAdd(&base[tid % ep], sum);
        }
    }
    if (!ok) gave_up = 1;
    __syncthreads();
    if (gave_up) {                              // uniform: nothing written for this token
        if ((cb | grp) == 0) {
            if (tid < a.k) a.slot_index[f] = -1;
            if (tid == 0) atomicOr(a.status, MOE_STATUS_GAVE_UP);
        }
        return;
    }
    if constexpr (!ROW_FIRST) {
#pragma unroll
        for (int q = 0; q < VPT; ++q) v[q] = load16(src + off[q]);
    }
    const int before = d < 0 ? 0 : by_copy ? cbase[tid] : base[d];
    assign_rows(a, d, tid, cb | grp, f, before, rank, dests, rows, copy_rows);
    const int j0 = grp * C, j1 = min(a.k, j0 + C);
    if constexpr (FP8)
        store_rows_fp8<VPT, POLICY>(a, v, col, off, vpr, copy_rows, red, tid, j0, j1);
    else
        store_rows_bf16<VPT, POLICY>(a, v, col, off, vpr, copy_rows, j0, j1);
}

template <bool NT>
__device__ __forceinline__ u32x4 load_row16(const uint16_t *p) {
    const u32x4 *v = reinterpret_cast<const u32x4 *>(p);
    return NT ? __builtin_nontemporal_load(v) : *v;
}

// acc += g * row (weighted, fused multiply-add) or acc += row, element order fixed.
template <int VPT, bool WEIGHTED>
__device__ __forceinline__ void accumulate(float (&acc)[VPT][8], const u32x4 (&raw)[VPT], float g) {
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
        float f[8];
        unpack8(raw[q], f);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[q][e] = WEIGHTED ? __builtin_fmaf(g, f[e], acc[q][e]) : acc[q][e] + f[e];
    }
}

// ---------------------------------------------------------------------------
// dispatch_small_kernel<VPT, POLICY, FP8, C, PER>: the whole dispatch in one launch,
// for batches of at most kSmallItems routed copies (decode).  Grid and block
// order as dispatch_copy_kernel: blocks of C copies of one token, a token's
// blocks 8 indices apart so they share an XCD, x column blocks.  In place of
// the routing kernel's chunk histograms each block counts, per region, the
// copies of all earlier tokens itself: at most kSmallItems ids from L2,
// loaded together with the source row, one LDS add per copy (under the
// per-region layout one per ballot group of first copies, as in
// route_rank_kernel) into its wave's own row of counts, which the wave clears
// itself, so one block barrier publishes the counts and the token's regions.
// After it every wave sums the four rows for its copies' regions and adds
// each copy's rank among its own token's earlier copies to the same region,
// so the slots follow the stable order of the routed path.  Each token's
// first block flags the token's bad ids and writes its index maps; the last
// token's first block writes counts (the earlier tokens' copies plus its
// own).
// PER: earlier ids per lane, kSmallItemsShort / 256 or kSmallItems / 256 (the
// smaller form keeps decode's register and load count down: 16 per lane made
// the decode dispatch 6.3 -> 6.9 us).
static_assert(kSmallItems % kThreads == 0 && kSmallItemsShort % kThreads == 0,
              "small-batch ids are split evenly over a block");

template <int VPT, int POLICY, bool FP8, int C, int PER>
__global__ __launch_bounds__(kThreads) void dispatch_small_kernel(DispatchArgs a) {
    __shared__ int32_t cnt[kWaves * MOE_MAX_EP];        // per wave: earlier copies per region
    __shared__ int32_t dests[MOE_MAX_TOP_K];
    __shared__ int32_t wave_rows[kWaves * MOE_MAX_TOP_K]; // per wave: the rows this block fills
    __shared__ float red[kWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cb = blockIdx.y;
    const int ep = a.ep;
    const int n = (a.k + C - 1) / C;            // copy groups per token
    const int b = blockIdx.x;
    const int grp = (b >> 3) % n;
    const int t = ((b >> 3) / n) * 8 + (b & 7);
    if (t >= a.T) return;                       // past the batch in the last group of 8 tokens
    const bool first_block = (grp | cb) == 0;   // writes the token's index maps

    // loads: this token's ids and the ids of every earlier token, then the
    // source row (loads complete in issue order: the count below waits only
    // for the ids, the stores for the row)
    const int64_t mine = (int64_t)t * a.k;      // this token's first copy
    const int own_id = tid < a.k ? a.ids[mine + tid] : -1;
    int eid[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int64_t i = (int64_t)p * kThreads + tid;
        eid[p] = i < mine ? a.ids[i] : -1;
    }
    const int vpr = a.H >> 3;
    const uint16_t *src = a.x + (int64_t)t * a.H;
    u32x4 v[VPT];
    int col[VPT];
    int64_t off[VPT];
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
        col[q] = (cb * VPT + q) * kThreads + tid;
        off[q] = (int64_t)min(col[q], vpr - 1) * 8;
        v[q] = load16(src + off[q]);
    }
    int32_t *wave_cnt = cnt + wave * ep;        // this wave's counts: no other wave uses them
    for (int r = lane; r < ep; r += 64) wave_cnt[r] = 0;
    wave_sync();
    int d = -1;
    if (tid < a.k) {
        if (own_id >= 0 && own_id < a.n_experts)
            d = region_of(a, own_id);
        else if (own_id != -1 && first_block)
            atomicOr(a.status, MOE_STATUS_EXPERT_ID);
        dests[tid] = d;
    }

    // copies of the earlier tokens, per region
    if (a.per_region) {
        int region_bits = 0;
        while ((1 << region_bits) < ep) ++region_bits;
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            if ((int64_t)p * kThreads >= mine) break;     // uniform
            const int64_t i = (int64_t)p * kThreads + tid;
            int de = -1;
            if (i < mine && eid[p] >= 0 && eid[p] < a.n_experts) de = region_of(a, eid[p]);
            const uint64_t same = rank_group(a, de, i, i < mine, region_bits);
            if (de >= 0 && (same >> lane) == 1ull) atomicAdd(&wave_cnt[de], __popcll(same));
        }
    } else {
#pragma unroll
        for (int p = 0; p < PER; ++p)
            if (eid[p] >= 0 && eid[p] < a.n_experts) atomicAdd(&wave_cnt[region_of(a, eid[p])], 1);
    }
    __syncthreads();                            // the only block barrier before the stores

    // Row of copy j: its region's copies of earlier tokens (the four waves'
    // counts) plus its rank among the token's earlier copies to that region.
    // Under the per-region layout a token's copies to one region share the
    // row of the first of them (rank 0), and only that one fills it.
    auto row_of = [&](int j, bool &fills) -> int {
        const int dj = dests[j];
        fills = false;
        if (dj < 0) return -1;
        int rank = 0;
        for (int i = 0; i < j; ++i) rank += (dests[i] == dj);
        fills = !a.per_region || rank == 0;
        if (a.per_region) rank = 0;
        int s = rank;
        for (int w = 0; w < kWaves; ++w) s += cnt[w * ep + dj];
        return s < a.cap ? dj * a.cap + s : -1;
    };
    if (first_block && tid < a.k) {             // the token's index maps
        bool fills;
        const int row = row_of(tid, fills);
        if (fills && d >= 0 && row < 0) atomicOr(a.status, MOE_STATUS_OVERFLOW);
        a.slot_index[mine + tid] = row;
        if (fills && row >= 0) a.src_index[row] = (int32_t)(mine + tid);
    }
    if (first_block && t == a.T - 1) {          // totals: the earlier tokens' copies plus this one's
        for (int r = tid; r < ep; r += kThreads) {
            int own = 0;
            for (int j = 0; j < a.k; ++j) own += (dests[j] == r);
            int earlier = 0;
            for (int w = 0; w < kWaves; ++w) earlier += cnt[w * ep + r];
            a.counts[r] = earlier + (a.per_region ? (own > 0) : own);
        }
    }
    // every wave finds the rows of this block's copies itself (no second
    // block barrier)
    const int j0 = grp * C, j1 = min(a.k, j0 + C);
    int32_t *rows_w = wave_rows + wave * MOE_MAX_TOP_K;
    for (int j = j0 + lane; j < j1; j += 64) {
        bool fills;
        const int row = row_of(j, fills);
        rows_w[j] = fills ? row : -1;
    }
    wave_sync();
    if constexpr (FP8)
        store_rows_fp8<VPT, POLICY>(a, v, col, off, vpr, rows_w, red, tid, j0, j1);
    else
        store_rows_bf16<VPT, POLICY>(a, v, col, off, vpr, rows_w, j0, j1);
}

// G rows starting at compacted copy j0: all G x VPT loads, then the adds in
// copy order.
template <int G, int VPT, bool WEIGHTED, bool NT>
__device__ __forceinline__ void gather_group(float (&acc)[VPT][8], const uint16_t *y, int H,
                                             const int32_t *rows, const float *gates, int j0,
                                             const int64_t (&off)[VPT]) {
    u32x4 raw[G][VPT];
#pragma unroll
    for (int u = 0; u < G; ++u) {
        const uint16_t *src = y + (int64_t)uniform(rows[j0 + u]) * H;
#pragma unroll
        for (int q = 0; q < VPT; ++q) raw[u][q] = load_row16<NT>(src + off[q]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < G; ++u) accumulate<VPT, WEIGHTED>(acc, raw[u], gates[j0 + u]);
}

// ---------------------------------------------------------------------------
// combine_kernel<VPT, JU, WEIGHTED, FUSED, NT>: grid = (T, column blocks);
// FUSED runs with one column block so the whole row is in the workgroup.
//
// With `partials` set the k rows of token t are the partial sums j*T + t of
// a [k, T, H] buffer (the local reduction of an all-reduce), all valid.
// Otherwise wave 0 first compacts the token's valid copies (slot_index >= 0) into LDS,
// keeping j order, so only rows holding valid copies are ever read (padding
// rows never are).  Under the per-region layout a row named by an earlier
// copy of the token is dropped: each region's message is added once.  Lane j
// of wave 0 loads copy j's slot and gate together and compares rows with the
// earlier lanes through shuffles, so the prologue is one round trip and one
// block barrier (with a first barrier before the gates' loads, the decode
// combine took 7.0 instead of 6.6 us after a cache-evicting read, the skewed
// per-region one 86.9 instead of 86.4 us; others equal).  Rows
// are then fetched JU at a time with every load of a group issued before the
// first add, and no load under a branch (a branch around a load makes the
// compiler wait for all outstanding loads).  Lanes
// past the end of the row load the row's last vector instead and store
// nothing.  Adds run in j order, so the fp32 sum is the same sequence of
// roundings for every layout.  NT marks the gathered rows non-temporal (each
// is read once).
template <int VPT, int JU, bool WEIGHTED, bool FUSED, bool NT>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
    __shared__ int32_t rows[MOE_MAX_TOP_K];
    __shared__ float gates[MOE_MAX_TOP_K];
    __shared__ int32_t n_valid;
    __shared__ double partial[kWaves];

    const int tid = threadIdx.x;
    const int t = blockIdx.x;
    const int cb = blockIdx.y;
    const int k = a.k;

    if (tid < 64) {                             // wave 0 (k <= 64): compact valid copies
        int row = -1;
        float g = 0.0f;
        if (tid < k) {                          // the copy's row and gate, in one round trip
            row = a.partials ? tid * a.T + t : a.slot_index[(int64_t)t * k + tid];
            g = WEIGHTED ? a.w[(int64_t)t * k + tid] : 1.0f;
        }
        if (a.per_region) {                     // a row already added for this token
            const int mine = row;
            for (int j = 0; j + 1 < k; ++j) {
                const int rj = __shfl(mine, j);
                if (j < tid && mine >= 0 && rj == mine) row = -1;
            }
        }
        const uint64_t valid = __ballot(row >= 0);
        if (row >= 0) {
            const int pos = __popcll(valid & ((tid == 0) ? 0ull : (~0ull >> (64 - tid))));
            rows[pos] = row;
            gates[pos] = g;
        }
        if (tid == 0) n_valid = __popcll(valid);
    }
    __syncthreads();
    const int nv = uniform(n_valid);

    const int vpr = a.H >> 3;
    int col[VPT];
    int64_t off[VPT];                           // element offset of the vector, clamped into the row
    float acc[VPT][8];
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
        col[q] = (cb * VPT + q) * kThreads + tid;
        off[q] = (int64_t)min(col[q], vpr - 1) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[q][e] = 0.0f;
    }

    // Rows in groups of JU, then one group each of 4, 2 and 1 for the rest:
    // every load of a group is issued before its first add (the scheduling
    // barrier keeps the compiler from sinking loads to their uses).
    int j0 = 0;
    for (; j0 + JU <= nv; j0 += JU)
        gather_group<JU, VPT, WEIGHTED, NT>(acc, a.y, a.H, rows, gates, j0, off);
    if (JU > 4 && j0 + 4 <= nv) {
        gather_group<4, VPT, WEIGHTED, NT>(acc, a.y, a.H, rows, gates, j0, off);
        j0 += 4;
    }
    if (JU > 2 && j0 + 2 <= nv) {
        gather_group<2, VPT, WEIGHTED, NT>(acc, a.y, a.H, rows, gates, j0, off);
        j0 += 2;
    }
    if (j0 < nv) gather_group<1, VPT, WEIGHTED, NT>(acc, a.y, a.H, rows, gates, j0, off);

    const int64_t row_off = (int64_t)t * a.H;
    const bool cached = a.out_cached != 0;
    if constexpr (!FUSED) {
#pragma unroll
        for (int q = 0; q < VPT; ++q)
            if (col[q] < vpr) store_out16(row_rsrc(a.out + row_off, a.H), off[q], pack8(acc[q]), cached);
        return;
    } else {
        // s = sum + residual (fp32); residual_out = bf16(s).  The sum of
        // squares, its root and the normalising product are taken in fp64:
        // in fp32, s^2 summed over a row overflows once the elements pass
        // ~2e17 (bf16 reaches 3e38) and, with eps = 0, underflows for tiny
        // rows, where fp64 covers the whole bf16 range.  The fp64 product
        // is rounded to fp32 with round-to-odd, then to bf16 nearest-even,
        // which together round it to bf16 nearest-even exactly once.  The
        // fp64 work is a few dozen operations per thread in a memory-bound
        // kernel.
        double ss = 0.0;
        // the residual and gamma in one round trip (gamma overlaps neither
        // output, so its loads may come before the residual_out stores)
        u32x4 rv[VPT], gv[VPT];
#pragma unroll
        for (int q = 0; q < VPT; ++q) rv[q] = load16(a.residual + row_off + off[q]);
#pragma unroll
        for (int q = 0; q < VPT; ++q) gv[q] = load16(a.gamma + off[q]);
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            float r[8];
            unpack8(rv[q], r);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q][e] = acc[q][e] + r[e];
            if (col[q] < vpr) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    ss = __builtin_fma((double)acc[q][e], (double)acc[q][e], ss);
                store_out16(row_rsrc(a.residual_out + row_off, a.H), off[q], pack8(acc[q]), cached);
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        if ((tid & 63) == 0) partial[tid >> 6] = ss;
        __syncthreads();
        double total = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) total += partial[w];
        const double inv = 1.0 / __builtin_sqrt(total / (double)a.H + (double)a.eps);
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            if (col[q] >= vpr) continue;
            float g[8];
            unpack8(gv[q], g);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[q][e] = f64_to_f32_odd(((double)acc[q][e] * inv) * (double)g[e]);
            store_out16(row_rsrc(a.normed + row_off, a.H), off[q], pack8(acc[q]), cached);
        }
    }
}

// Smallest power-of-two vectors-per-thread (<= 8) covering a row in one block.
int full_row_vpt(int32_t H) {
    const int vpr = H / 8;
    int vpt = 1;
    while (vpt < 8 && vpt * kThreads < vpr) vpt *= 2;
    return vpt;
}

// Vectors per thread for the streaming kernels: a whole row per block when
// there are enough rows (T of them, one per block) to fill the chip, smaller
// blocks otherwise.
int streaming_vpt(int64_t T, int32_t H) {
    constexpr int64_t kWantBlocks = 1024;      // 256 CUs x 4
    const int vpr = H / 8;
    int vpt = full_row_vpt(H);
    while (vpt > 1) {
        const int64_t blocks = (int64_t)T * ((vpr + vpt * kThreads - 1) / (vpt * kThreads));
        if (blocks >= kWantBlocks) break;
        vpt /= 2;
    }
    return vpt;
}

int column_blocks(int32_t H, int vpt) {
    const int vpr = H / 8;
    return (vpr + vpt * kThreads - 1) / (vpt * kThreads);
}

// Launch choices, measured on MI355X at the prefill shape (T = 4096,
// H = 7168, top-8): non-temporal workspace stores and gathers move the copy
// from 4.98 to 5.68 TB/s and the combine from 3.77 to 5.70 TB/s; a group of
// 8 rows x 4 vectors (32 loads in flight per thread) is the best plain
// combine shape.  Wider rows (8 vectors per thread) use groups of 4 rows to
// keep the register count near 200.
// Workspace store policy.  The routed copy stores non-temporal with sc1 set.
// Step us, back-to-back dispatch -> combine, nt -> nt + sc1 (two runs each):
// prefill 175.0, 174.5 -> 174.0, 173.0; fused 99.8, 99.6 -> 98.6, 98.9;
// skewed 344.6, 345.3 -> 339.3, 342.4; per-region prefill 122.8, 122.9 ->
// 119.9, 119.3; per-region skewed 172.4, 172.5 -> 173.1, 172.3 (its
// dispatch 87.0 -> 83.7).  nt + sc0 + sc1 measured the same as nt + sc1, and
// nt + sc0 the same as nt.  Plain stores made the prefill dispatch 84 us but
// its combine 84 -> 90 us and the skewed step 345 -> 366 us: the dirty rows'
// write-back moves into the next kernel.  The single-launch decode dispatch
// stays plain non-temporal: with sc1 its combine, which then reads the rows
// from HBM rather than the caches, took 5.8 instead of 4.4 us (decode step
// 8.9 -> 11.1 us).  The same holds while a routed copy's rows fit the caches
// (T = 512, 59 MB: step 26.4 -> 28.9 us with sc1), so sc1 is set only above
// kCopyWriteThroughBytes of rows (T = 1024, 117 MB: 49.0 either way;
// T = 1536: 69.8 -> 69.0; T = 2048: 91.0 -> 89.3), and only for the per-copy
// bf16 layout (the per-region skewed step lost 5 us with it, the fp8 payload
// measured the same).
constexpr int kCopyPolicy = kPolicyNT | kPolicySC1;
constexpr int kSmallPolicy = kPolicyNT;
constexpr int64_t kCopyWriteThroughBytes = int64_t(128) << 20;
// Copies per dispatch_copy_kernel block (bf16 and fp8 payloads), and the
// most blocks along x in one launch (a launch must hold fewer than 2^32
// lanes).
constexpr int kCopiesPerBlock = 2;
constexpr int kCopiesPerBlockFp8 = 4;
constexpr int64_t kOnePassFp8WholeTokenItems = 8192;
constexpr int64_t kRegionWholeTokenItems = 8192;
constexpr int64_t kRegionWholeTokenItemsFp8 = 24576;
// Smaller rows (under 8 KB of bf16) keep one block per token: after a cache-
// evicting read, T = 4096, H = 2048, top-8 copies ran at 48.8 % of the HBM
// peak split in pairs against 60.8 % whole (T = 32768: 54.9 % against 68.7 %;
// warm steps gain 1-2 points from the split).  At H = 4096 the split is even
// cold (64.5 against 64.6 %) and 4 points ahead warm.
constexpr int kSplitMinHidden = 4096;
constexpr int64_t kMaxBlocksX = int64_t(1) << 22;
constexpr bool kCombineNT = true;
// Rows per gather group.  Eight is best only for the plain per-copy combine
// with more than four rows per token; everywhere else groups of 4 measured
// better: the fused epilogue keeps the residual and gamma in registers too
// (6.23 vs 6.07 TB/s with 8), and with few rows per token (top-k <= 4, or
// the per-region layout's ~5.3 distinct rows at top-8) the smaller register
// footprint lets more waves run (T = 4096, H = 7168: top-2 33.4 -> 31.3 us,
// top-4 49.9 -> 48.4 us, per-region top-8 65.2 -> 62.8 us).
int combine_group(int vpt, bool fused, const CombineArgs &a) {
    return (fused || vpt >= 8 || a.k <= 4 || a.per_region) ? 4 : 8;
}

template <int VPT, bool FP8, int C>
void launch_copy_c(const DispatchArgs &a, dim3 grid, hipStream_t s, bool small) {
    if (small) {
        if ((int64_t)a.T * a.k <= kSmallItemsShort)
            hipLaunchKernelGGL((dispatch_small_kernel<VPT, kSmallPolicy, FP8, C, kSmallItemsShort / kThreads>),
                               grid, dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL((dispatch_small_kernel<VPT, kSmallPolicy, FP8, C, kSmallItems / kThreads>),
                               grid, dim3(kThreads), 0, s, a);
        return;
    }
    // the source row first only for the per-copy bf16 copy (see dispatch_copy_kernel),
    // which also stores with sc1 once its rows outgrow kCopyWriteThroughBytes
    if constexpr (!FP8) {
        if (!a.per_region) {
            const int64_t written = (int64_t)a.T * a.k * a.H * (int64_t)sizeof(uint16_t);
            if (written > kCopyWriteThroughBytes)
                hipLaunchKernelGGL((dispatch_copy_kernel<VPT, kCopyPolicy, FP8, C, true>), grid,
                                   dim3(kThreads), 0, s, a);
            else
                hipLaunchKernelGGL((dispatch_copy_kernel<VPT, kPolicyNT, FP8, C, true>), grid,
                                   dim3(kThreads), 0, s, a);
            return;
        }
    }
    hipLaunchKernelGGL((dispatch_copy_kernel<VPT, kPolicyNT, FP8, C, false>), grid, dim3(kThreads), 0, s,
                       a);
}

template <int VPT, bool FP8>
void launch_copy_vpt(const DispatchArgs &a, dim3 grid, hipStream_t s, bool small, int c) {
    constexpr int kSplit = FP8 ? kCopiesPerBlockFp8 : kCopiesPerBlock;
    if (c == kSplit)
        launch_copy_c<VPT, FP8, kSplit>(a, grid, s, small);
    else
        launch_copy_c<VPT, FP8, MOE_MAX_TOP_K>(a, grid, s, small);
}

// c: copies per dispatch_copy_kernel block (kCopiesPerBlock[Fp8], or
// MOE_MAX_TOP_K for a whole token).
template <bool FP8>
void launch_copy(const DispatchArgs &a, int vpt, dim3 grid, hipStream_t s, bool small, int c) {
    switch (vpt) {
        case 1: launch_copy_vpt<1, FP8>(a, grid, s, small, c); break;
        case 2: launch_copy_vpt<2, FP8>(a, grid, s, small, c); break;
        case 4: launch_copy_vpt<4, FP8>(a, grid, s, small, c); break;
        default: launch_copy_vpt<8, FP8>(a, grid, s, small, c); break;
    }
}

template <int VPT, int JU, bool FUSED>
void launch_combine_group(const CombineArgs &a, dim3 grid, hipStream_t s) {
    if (a.weighted)
        hipLaunchKernelGGL((combine_kernel<VPT, JU, true, FUSED, kCombineNT>), grid,
                           dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((combine_kernel<VPT, JU, false, FUSED, kCombineNT>), grid,
                           dim3(kThreads), 0, s, a);
}

template <int VPT, bool FUSED>
void launch_combine_vpt(const CombineArgs &a, dim3 grid, hipStream_t s) {
    if constexpr (!FUSED && VPT < 8) {
        if (combine_group(VPT, FUSED, a) == 8) {
            launch_combine_group<VPT, 8, FUSED>(a, grid, s);
            return;
        }
    }
    launch_combine_group<VPT, 4, FUSED>(a, grid, s);
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, int32_t n_chunks, hipStream_t s) {
    if (n_chunks > 0)
        hipLaunchKernelGGL(route_rank_kernel, dim3(n_chunks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

namespace {
template <int VPT, int C>
void launch_onepass_c(const DispatchArgs &a, const RouteArgs &ra, dim3 grid, hipStream_t s) {
    if (!a.per_region) {
        const int64_t items = (int64_t)a.T * a.k;
        const int64_t written = items * a.H * (int64_t)sizeof(uint16_t);
        const bool row_first = items > kOnePassRowFirstFrom && items <= kOnePassRowFirstItems;
        if (items > kOnePassRowFirstItems || (written > kCopyWriteThroughBytes && !row_first))
            hipLaunchKernelGGL((dispatch_onepass_kernel<VPT, kCopyPolicy, C, false, false>), grid, dim3(kThreads), 0,
                               s, a, ra);
        else if (written > kCopyWriteThroughBytes)
            hipLaunchKernelGGL((dispatch_onepass_kernel<VPT, kCopyPolicy, C, true, false>), grid, dim3(kThreads), 0,
                               s, a, ra);
        else if (row_first)
            hipLaunchKernelGGL((dispatch_onepass_kernel<VPT, kPolicyNT, C, true, false>), grid, dim3(kThreads), 0, s,
                               a, ra);
        else
            hipLaunchKernelGGL((dispatch_onepass_kernel<VPT, kPolicyNT, C, false, false>), grid, dim3(kThreads), 0, s,
                               a, ra);
        return;
    }
    hipLaunchKernelGGL((dispatch_onepass_kernel<VPT, kPolicyNT, C, false, false>), grid, dim3(kThreads), 0, s, a,
                       ra);
}

template <int VPT>
void launch_onepass_vpt(const DispatchArgs &a, const RouteArgs &ra, dim3 grid, hipStream_t s, int c) {
    if (c == kCopiesPerBlock)
        launch_onepass_c<VPT, kCopiesPerBlock>(a, ra, grid, s);
    else
        launch_onepass_c<VPT, MOE_MAX_TOP_K>(a, ra, grid, s);
}
}  // namespace

// The fp8 payload: whole rows in a block (one column block), copies per
// block as in the copy kernel (every copy of a token under kSplitMinHidden,
// four above) except that batches of at most kOnePassFp8WholeTokenItems
// copies keep a whole token per block (H = 7168, top-8, step / dispatch
// after a cache-evicting read, us, three runs each: 640 tokens 25.7 / 14.8
// -> 25.3 / 13.7; 1024 tokens 39.0 / 21.4 -> 38.5 / 18.4; at 2048 tokens
// four per block stay ahead, 78.5 / 32.9 against 79.8 / 34.1; the bf16
// payload lost at 640-1024 tokens), the row loaded after the routing words,
// and non-temporal stores.  Measured against the routing kernel + copy kernel (dispatch us
// warm / cold, two runs each): 4096 tokens, H = 7168, top-8
// 49.5 / 57.75 -> 48.5 / 57.7; 2048 tokens 30.05 / 33.45 -> 28.8 / 33.2;
// skewed 8192 tokens 92.1 / 109.4 -> 90.25 / 110.05; 1024 tokens
// 18.95 / 20.75 -> 17.65 / 21.0.
template <int VPT>
void launch_onepass_fp8(const DispatchArgs &a, const RouteArgs &ra, dim3 grid, hipStream_t s, int c) {
    if (c == kCopiesPerBlockFp8)
        hipLaunchKernelGGL((dispatch_onepass_kernel<VPT, kPolicyNT, kCopiesPerBlockFp8, false, true>), grid,
                           dim3(kThreads), 0, s, a, ra);
    else
        hipLaunchKernelGGL((dispatch_onepass_kernel<VPT, kPolicyNT, MOE_MAX_TOP_K, false, true>), grid,
                           dim3(kThreads), 0, s, a, ra);
}

hipError_t launch_dispatch_onepass(const DispatchArgs &args, const RouteArgs &ra, hipStream_t s) {
    DispatchArgs a = args;
    a.t_base = 0;
    if (a.fp8) {
        const bool whole = a.H < kSplitMinHidden || (int64_t)a.T * a.k <= kOnePassFp8WholeTokenItems;
        const int c = whole ? MOE_MAX_TOP_K : kCopiesPerBlockFp8;
        const int n = (a.k + c - 1) / c;
        const int64_t t_pad = ((int64_t)a.T + 7) / 8 * 8;
        a.route_blocks = (a.n_chunks + 7) / 8 * 8;   // keeps the copy blocks' XCD grouping
        const dim3 grid((uint32_t)(a.route_blocks + t_pad * n), 1);
        switch (full_row_vpt(a.H)) {
            case 1: launch_onepass_fp8<1>(a, ra, grid, s, c); break;
            case 2: launch_onepass_fp8<2>(a, ra, grid, s, c); break;
            case 4: launch_onepass_fp8<4>(a, ra, grid, s, c); break;
            default: launch_onepass_fp8<8>(a, ra, grid, s, c); break;
        }
        return hipGetLastError();
    }
    const int c = a.H < kSplitMinHidden ? MOE_MAX_TOP_K : kCopiesPerBlock;
    const int n = (a.k + c - 1) / c;
    const int64_t t_pad = ((int64_t)a.T + 7) / 8 * 8;
    const int vpt = streaming_vpt(t_pad * n, a.H);
    a.route_blocks = (a.n_chunks + 7) / 8 * 8;   // keeps the copy blocks' XCD grouping
    const dim3 grid((uint32_t)(a.route_blocks + t_pad * n), column_blocks(a.H, vpt));
    switch (vpt) {
        case 1: launch_onepass_vpt<1>(a, ra, grid, s, c); break;
        case 2: launch_onepass_vpt<2>(a, ra, grid, s, c); break;
        case 4: launch_onepass_vpt<4>(a, ra, grid, s, c); break;
        default: launch_onepass_vpt<8>(a, ra, grid, s, c); break;
    }
    return hipGetLastError();
}

hipError_t launch_dispatch_copy(const DispatchArgs &args, hipStream_t s) {
    DispatchArgs a = args;
    a.t_base = 0;
    if (a.count_only || a.T == 0) {             // the totals only (an empty batch: zeros)
        const dim3 grid(1, 1);
        if (a.fp8)
            launch_copy<true>(a, full_row_vpt(a.H), grid, s, false, MOE_MAX_TOP_K);
        else
            launch_copy<false>(a, 1, grid, s, false, MOE_MAX_TOP_K);
        return hipGetLastError();
    }
    // Blocks of c copies in XCD order (both copy kernels), over tokens
    // padded to a multiple of 8.  Rows under kSplitMinHidden stay one block
    // per token.  The fp8 payload needs the whole row in a block for its
    // scale.
    // The single-launch kernel above kSmallItemsShort copies counts up to
    // 4096 earlier ids in every block, so it takes a whole token per block
    // there (one count per token instead of one per pair of copies): ladder
    // T = 512 roundtrip 25.9 -> 25.0 us, T = 384 step 20.6 -> 19.7 us, other
    // sizes unchanged; 4 copies per block measured the same at T = 512 but
    // 0.8 us slower at T = 448.
    // The routed copy of the per-region layout takes a whole token per block
    // up to kRegionWholeTokenItems copies, the fp8 payload up to
    // kRegionWholeTokenItemsFp8 (H = 7168, top-8, step / dispatch after a
    // cache-evicting read, us, three runs each: 640 tokens 25.4 / 19.1 ->
    // 25.2 / 17.1; 1024 tokens 37.5 / 24.6 -> 37.1 / 22.8; 1536 tokens
    // 51.9 / 31.7 -> 52.9 / 32.9 and 2048 tokens 75.5 / 39.4 -> 76.8 / 41.4
    // stay in pairs; fp8 1024 tokens 31.2 / 17.8 -> 30.9 / 17.4, 1536
    // tokens 43.3 / 23.8 -> 43.6 / 21.1, 2048 tokens 64.4 / 27.8 ->
    // 64.2 / 25.1, 3072 tokens 77.5 / 36.7 -> 76.7 / 36.5; at 4096 tokens
    // four per block stay, 98.9 / 45.8 against 98.2 / 47.1).
    const int64_t items = (int64_t)a.T * a.k;
    const bool small_long = dispatch_is_small(a.T, a.k) && items > kSmallItemsShort;
    const bool region_whole = a.per_region && !dispatch_is_small(a.T, a.k) &&
                              items <= (a.fp8 ? kRegionWholeTokenItemsFp8 : kRegionWholeTokenItems);
    const int c = (a.H < kSplitMinHidden || small_long || region_whole) ? MOE_MAX_TOP_K
                  : a.fp8 ? kCopiesPerBlockFp8 : kCopiesPerBlock;
    const int n = (a.k + c - 1) / c;
    const int64_t t_pad = ((int64_t)a.T + 7) / 8 * 8;
    const int vpt = a.fp8 ? full_row_vpt(a.H) : streaming_vpt(t_pad * n, a.H);
    if (dispatch_is_small(a.T, a.k)) {          // one launch, no routing kernel before it
        const dim3 grid((uint32_t)(t_pad * n), column_blocks(a.H, vpt));
        if (a.fp8)
            launch_copy<true>(a, vpt, grid, s, true, c);
        else
            launch_copy<false>(a, vpt, grid, s, true, c);
        return hipGetLastError();
    }
    // Routed: launches of at most kMaxBlocksX blocks along x.
    const int64_t slab = std::max<int64_t>(8, kMaxBlocksX / n / 8 * 8);    // tokens per launch
    for (int64_t t0 = 0; t0 < a.T; t0 += slab) {
        a.t_base = (int32_t)t0;
        const int64_t tokens = std::min<int64_t>(slab, t_pad - t0);
        const dim3 grid((uint32_t)(tokens * n), column_blocks(a.H, vpt));
        if (a.fp8)
            launch_copy<true>(a, vpt, grid, s, false, c);
        else
            launch_copy<false>(a, vpt, grid, s, false, c);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_combine(const CombineArgs &args, bool fused, hipStream_t s) {
    if (args.T == 0) return hipSuccess;
    CombineArgs a = args;
    const int64_t out_bytes = (int64_t)a.T * a.H * (int64_t)sizeof(uint16_t) * (fused ? 2 : 1);
    a.out_cached = out_bytes <= kOutCachedBytes;
    const int vpt = fused ? full_row_vpt(a.H) : streaming_vpt(a.T, a.H);
    const dim3 grid(a.T, fused ? 1 : column_blocks(a.H, vpt));
    if (fused) {
        switch (vpt) {
            case 1: launch_combine_vpt<1, true>(a, grid, s); break;
            case 2: launch_combine_vpt<2, true>(a, grid, s); break;
            case 4: launch_combine_vpt<4, true>(a, grid, s); break;
            default: launch_combine_vpt<8, true>(a, grid, s); break;
        }
    } else {
        switch (vpt) {
            case 1: launch_combine_vpt<1, false>(a, grid, s); break;
            case 2: launch_combine_vpt<2, false>(a, grid, s); break;
            case 4: launch_combine_vpt<4, false>(a, grid, s); break;
            default: launch_combine_vpt<8, false>(a, grid, s); break;
        }
    }
    return hipGetLastError();
}

}  // namespace moe
