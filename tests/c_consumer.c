/* A plain C caller of the library, with no Python and no torch: device
 * buffers come from the HIP runtime API, the calls go through
 * include/moe_a2a.h, and every result is checked on the host against values
 * this program derives itself.
 *
 * Batch: T = 50 tokens of H = 64, top-4 of 16 experts over 4 regions; every
 * fifth token leaves its last copy unrouted (-1).  Token rows hold small
 * multiples of 1/4, so all sums below are exact in bf16.  The expert stage
 * is the identity (the combine reads the dispatched rows in place), hence:
 *   counts[r] = number of copies whose expert / 4 == r;
 *   src_index and slot_index are inverse maps, regions in flat-index order;
 *   every dispatched row equals its token's row;
 *   unweighted combine = (routed copies of t) * x[t];
 *   weighted combine with every gate 1/4 = (routed copies of t) / 4 * x[t].
 * Then the handle-free partials reduction: 8 partials, partial p holding 2^p
 * everywhere, sum exactly 255; fused with a zero residual, gamma 1 and eps 0,
 * residual_out 255 and normed exactly 1.
 * Exit status 0 and "c consumer: ok" on success. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_a2a.h"

#define T 50
#define H 64
#define K 4
#define E 16
#define EP 4
#define EPR (E / EP)
#define CAP (T * K)

#define HIP_CHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
    printf("HIP error %d at line %d\n", (int)e_, __LINE__); return 1; } } while (0)
#define MOE_CHECK(x) do { int c_ = (x); if (c_ != MOE_OK) { \
    printf("library error %s at line %d\n", moe_strerror(c_), __LINE__); return 1; } } while (0)
#define EXPECT(cond) do { if (!(cond)) { printf("check failed: %s (line %d)\n", #cond, __LINE__); \
    return 1; } } while (0)

static uint16_t bf16_of(float f) {            /* exact for the values used here */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static float f32_of(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint16_t x[T * H], ws_host[EP * CAP * H], out[T * H];
static int32_t ids[T * K], counts[EP], slot[T * K], src[EP * CAP];
static float w[T * K];

static int check_combine(const char *what, float scale) {
    for (int t = 0; t < T; ++t) {
        int routed = 0;
        for (int j = 0; j < K; ++j) routed += ids[t * K + j] >= 0;
        for (int h = 0; h < H; ++h)
            if (f32_of(out[t * H + h]) != scale * (float)routed * f32_of(x[t * H + h])) {
                printf("%s: token %d element %d is %g\n", what, t, h, f32_of(out[t * H + h]));
                return 1;
            }
    }
    return 0;
}

int main(void) {
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) x[t * H + h] = bf16_of((float)((t * H + h) % 17 - 8) / 4.0f);
        for (int j = 0; j < K; ++j) ids[t * K + j] = (t * 7 + j * 5) % E;   /* distinct within a token */
        if (t % 5 == 0) ids[t * K + K - 1] = -1;
    }
    for (int f = 0; f < T * K; ++f) w[f] = 0.25f;

    uint16_t *dx, *dws, *dout;
    int32_t *dids, *dcounts, *dsrc, *dslot, *dstatus;
    float *dw;
    void *dscratch;
    const size_t scratch_bytes = moe_scratch_bytes(T, K, EP);
    EXPECT(scratch_bytes > 0 && moe_workspace_bytes(EP, CAP, H) == sizeof ws_host);
    HIP_CHECK(hipMalloc((void **)&dx, sizeof x));
    HIP_CHECK(hipMalloc((void **)&dws, sizeof ws_host));
    HIP_CHECK(hipMalloc((void **)&dout, sizeof out));
    HIP_CHECK(hipMalloc((void **)&dids, sizeof ids));
    HIP_CHECK(hipMalloc((void **)&dw, sizeof w));
    HIP_CHECK(hipMalloc((void **)&dcounts, sizeof counts));
    HIP_CHECK(hipMalloc((void **)&dsrc, sizeof src));
    HIP_CHECK(hipMalloc((void **)&dslot, sizeof slot));
    HIP_CHECK(hipMalloc((void **)&dstatus, sizeof(int32_t)));
    HIP_CHECK(hipMalloc(&dscratch, scratch_bytes));
    HIP_CHECK(hipMemcpy(dx, x, sizeof x, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dids, ids, sizeof ids, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dw, w, sizeof w, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemset(dsrc, 0xff, sizeof src));                /* -1: no copy */
    HIP_CHECK(hipMemset(dstatus, 0, sizeof(int32_t)));

    moe_handle h;
    MOE_CHECK(moe_init(&h, T, H, K, E, EP, CAP, MOE_LAYOUT_PER_COPY, dcounts, dsrc, dslot,
                       dstatus, dscratch, scratch_bytes));
    EXPECT(moe_combine(&h, dws, NULL, 0, dout, NULL) == MOE_ERR_PHASE);

    /* dispatch, then the maps and rows */
    int32_t bits = -1;
    MOE_CHECK(moe_dispatch(&h, dx, dids, T, T, dws, NULL));
    MOE_CHECK(moe_sync_status(&h, NULL, &bits));
    EXPECT(bits == 0);
    HIP_CHECK(hipMemcpy(counts, dcounts, sizeof counts, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(slot, dslot, sizeof slot, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(src, dsrc, sizeof src, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(ws_host, dws, sizeof ws_host, hipMemcpyDeviceToHost));
    int want[EP] = {0};
    for (int f = 0; f < T * K; ++f)
        if (ids[f] >= 0) want[ids[f] / EPR]++;
    for (int r = 0; r < EP; ++r) {
        EXPECT(counts[r] == want[r]);
        for (int s = 0; s < counts[r]; ++s) {
            const int f = src[r * CAP + s];
            EXPECT(f >= 0 && f < T * K && ids[f] / EPR == r && slot[f] == r * CAP + s);
            EXPECT(s == 0 || f > src[r * CAP + s - 1]);
            EXPECT(memcmp(&ws_host[(size_t)(r * CAP + s) * H], &x[(f / K) * H], H * sizeof(uint16_t)) == 0);
        }
        for (int s = counts[r]; s < CAP; ++s) EXPECT(src[r * CAP + s] == -1);
    }
    for (int f = 0; f < T * K; ++f) EXPECT((ids[f] < 0) == (slot[f] < 0));

    /* identity experts: the combine reads the dispatched rows in place */
    MOE_CHECK(moe_combine(&h, dws, NULL, 0, dout, NULL));
    HIP_CHECK(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
    if (check_combine("unweighted", 1.0f)) return 1;
    EXPECT(moe_combine(&h, dws, NULL, 0, dout, NULL) == MOE_ERR_PHASE);

    MOE_CHECK(moe_dispatch(&h, dx, dids, T, T, dws, NULL));
    MOE_CHECK(moe_combine(&h, dws, dw, 1, dout, NULL));
    HIP_CHECK(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
    if (check_combine("weighted", 0.25f)) return 1;
    EXPECT(moe_output_is_reduced() == 1);

    /* the partials reduction: no handle, no phase */
    {
        enum { P = 8 };
        static uint16_t parts[P * T * H], res[T * H], gam[H], nrm[T * H];
        for (int p = 0; p < P; ++p)
            for (int i = 0; i < T * H; ++i) parts[p * T * H + i] = bf16_of((float)(1 << p));
        for (int i = 0; i < H; ++i) gam[i] = bf16_of(1.0f);
        uint16_t *dparts, *dres, *dgam, *dnrm;
        HIP_CHECK(hipMalloc((void **)&dparts, sizeof parts));
        HIP_CHECK(hipMalloc((void **)&dres, sizeof res));
        HIP_CHECK(hipMalloc((void **)&dgam, sizeof gam));
        HIP_CHECK(hipMalloc((void **)&dnrm, sizeof nrm));
        HIP_CHECK(hipMemcpy(dparts, parts, sizeof parts, hipMemcpyHostToDevice));
        HIP_CHECK(hipMemcpy(dgam, gam, sizeof gam, hipMemcpyHostToDevice));
        HIP_CHECK(hipMemset(dres, 0, sizeof res));
        EXPECT(moe_partials_reduce(dparts, P, T, H, dparts + 8, NULL) == MOE_ERR_ARG);
        MOE_CHECK(moe_partials_reduce(dparts, P, T, H, dout, NULL));
        HIP_CHECK(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
        for (int i = 0; i < T * H; ++i) EXPECT(f32_of(out[i]) == 255.0f);
        MOE_CHECK(moe_partials_reduce_residual_rmsnorm(dparts, P, T, H, dres, dres, dgam, 0.0f,
                                                       dnrm, NULL));
        HIP_CHECK(hipMemcpy(res, dres, sizeof res, hipMemcpyDeviceToHost));
        HIP_CHECK(hipMemcpy(nrm, dnrm, sizeof nrm, hipMemcpyDeviceToHost));
        for (int i = 0; i < T * H; ++i) EXPECT(f32_of(res[i]) == 255.0f && f32_of(nrm[i]) == 1.0f);
        HIP_CHECK(hipFree(dparts));
        HIP_CHECK(hipFree(dres));
        HIP_CHECK(hipFree(dgam));
        HIP_CHECK(hipFree(dnrm));
    }

    HIP_CHECK(hipFree(dx));
    HIP_CHECK(hipFree(dws));
    HIP_CHECK(hipFree(dout));
    HIP_CHECK(hipFree(dids));
    HIP_CHECK(hipFree(dw));
    HIP_CHECK(hipFree(dcounts));
    HIP_CHECK(hipFree(dsrc));
    HIP_CHECK(hipFree(dslot));
    HIP_CHECK(hipFree(dstatus));
    HIP_CHECK(hipFree(dscratch));
    printf("c consumer: ok\n");
    return 0;
}
