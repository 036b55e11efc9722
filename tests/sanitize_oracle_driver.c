/* Drives every oracle function through ordinary and edge inputs; built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by test_sanitizers.py.
 * Exits 0 when every call returned; the sanitizers abort on a memory or
 * undefined-behaviour error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_dispatch(const uint16_t *, const int32_t *, int64_t, int64_t, int64_t, int64_t,
                    int64_t, int64_t, uint16_t *, int32_t *, int32_t *, int32_t *);
int oracle_dispatch_region(const uint16_t *, const int32_t *, int64_t, int64_t, int64_t, int64_t,
                           int64_t, int64_t, uint16_t *, int32_t *, int32_t *, int32_t *);
int oracle_combine(const uint16_t *, const int32_t *, const float *, int, int64_t, int64_t,
                   int64_t, uint16_t *);
int oracle_combine_region(const uint16_t *, const int32_t *, int64_t, int64_t, int64_t, uint16_t *);
int oracle_combine_residual_rmsnorm(const uint16_t *, const int32_t *, const float *, int, int64_t,
                                    int64_t, int64_t, const uint16_t *, const uint16_t *, float,
                                    uint16_t *, uint16_t *, double *, float *);
int oracle_combine_residual_rmsnorm_region(const uint16_t *, const int32_t *, int64_t, int64_t,
                                           int64_t, const uint16_t *, const uint16_t *, float,
                                           uint16_t *, uint16_t *, double *, float *);
int oracle_partials_reduce(const uint16_t *, int64_t, int64_t, int64_t, uint16_t *);
int oracle_partials_reduce_residual_rmsnorm(const uint16_t *, int64_t, int64_t, int64_t,
                                            const uint16_t *, const uint16_t *, float, uint16_t *,
                                            uint16_t *, double *, float *);
uint16_t oracle_f64_to_bf16(double);
float oracle_e4m3_to_f32(uint8_t);
uint8_t oracle_f32_to_e4m3(float);
void oracle_quantize_e4m3_rows(const uint16_t *, int64_t, int64_t, uint8_t *, float *);

static uint32_t state = 12345u;
static uint32_t next(void) { state = state * 1664525u + 1013904223u; return state >> 8; }

static void run(int64_t T, int64_t H, int64_t k, int64_t ep, int64_t epr, int64_t cap, int bad)
{
    int64_t E = ep * epr;
    uint16_t *x = malloc(sizeof(uint16_t) * (size_t)(T * H));
    int32_t *ids = malloc(sizeof(int32_t) * (size_t)(T * k));
    for (int64_t i = 0; i < T * H; ++i) x[i] = (uint16_t)(0x3F80 + (next() % 512) - 256);
    for (int64_t i = 0; i < T * k; ++i) {
        uint32_t r = next() % 10;
        ids[i] = r == 0 ? -1 : (int32_t)(next() % (uint32_t)E);
        if (bad && r == 1) ids[i] = (int32_t)(E + (int64_t)(next() % 5));
        if (bad && r == 2) ids[i] = -2 - (int32_t)(next() % 5);
    }
    uint16_t *ws = malloc(sizeof(uint16_t) * (size_t)(ep * cap * H));
    int32_t *counts = malloc(sizeof(int32_t) * (size_t)ep);
    int32_t *slot = malloc(sizeof(int32_t) * (size_t)(T * k));
    int32_t *src = malloc(sizeof(int32_t) * (size_t)(ep * cap));
    float *w = malloc(sizeof(float) * (size_t)(T * k));
    uint16_t *out = malloc(sizeof(uint16_t) * (size_t)(T * H));
    uint16_t *res = malloc(sizeof(uint16_t) * (size_t)(T * H));
    uint16_t *normed = malloc(sizeof(uint16_t) * (size_t)(T * H));
    uint16_t *gamma = malloc(sizeof(uint16_t) * (size_t)H);
    double *n64 = malloc(sizeof(double) * (size_t)(T * H));
    float *scratch = malloc(sizeof(float) * (size_t)H);
    uint8_t *q = malloc((size_t)(T * H));
    float *scale = malloc(sizeof(float) * (size_t)(T));
    for (int64_t i = 0; i < ep * cap * H; ++i) ws[i] = 0x3F80;
    for (int64_t i = 0; i < T * k; ++i) w[i] = (float)(next() % 1000) / 1000.0f;
    for (int64_t i = 0; i < T * H; ++i) res[i] = x[(i * 7) % (T * H)];
    for (int64_t i = 0; i < H; ++i) gamma[i] = 0x3F80;
    for (int layout = 0; layout < 2; ++layout) {
        if (layout == 0)
            oracle_dispatch(x, ids, T, H, k, ep, epr, cap, ws, counts, slot, src);
        else
            oracle_dispatch_region(x, ids, T, H, k, ep, epr, cap, ws, counts, slot, src);
        if (layout == 0) {
            oracle_combine(ws, slot, w, 1, T, H, k, out);
            oracle_combine(ws, slot, w, 0, T, H, k, out);
            oracle_combine_residual_rmsnorm(ws, slot, w, 1, T, H, k, res, gamma, 1e-6f, res, normed,
                                            n64, scratch);
        } else {
            oracle_combine_region(ws, slot, T, H, k, out);
            oracle_combine_residual_rmsnorm_region(ws, slot, T, H, k, res, gamma, 1e-6f, res,
                                                   normed, NULL, scratch);
        }
    }
    oracle_quantize_e4m3_rows(x, T, H, q, scale);
    /* partials reduction: k partials of [T, H], buffers sized exactly */
    uint16_t *parts = malloc(sizeof(uint16_t) * (size_t)(k * T * H) + 1);
    for (int64_t i = 0; i < k * T * H; ++i) parts[i] = x[i % (T * H > 0 ? T * H : 1)];
    oracle_partials_reduce(parts, k, T, H, out);
    oracle_partials_reduce_residual_rmsnorm(parts, k, T, H, res, gamma, 1e-6f, res, normed, n64,
                                            scratch);
    free(parts);
    free(x); free(ids); free(ws); free(counts); free(slot); free(src); free(w); free(out);
    free(res); free(normed); free(gamma); free(n64); free(scratch); free(q); free(scale);
}

int main(void)
{
    run(0, 8, 2, 2, 2, 1, 0);          /* empty batch */
    run(1, 8, 1, 1, 1, 1, 0);          /* one token, one region */
    run(37, 24, 3, 4, 3, 200, 1);      /* ragged, bad ids */
    run(64, 16, 8, 8, 4, 20, 1);       /* overflow: cap below the per-region counts */
    run(20, 8, 64, 256, 2, 40, 0);     /* the limits: k = 64, ep = 256 */
    for (int i = 0; i < 256; ++i)      /* every e4m3 code, and back */
        (void)oracle_f32_to_e4m3(oracle_e4m3_to_f32((uint8_t)i));
    double special[] = {0.0, -0.0, INFINITY, -INFINITY, NAN, 1e-45, 1e-40, 3.4e38, 1e300, -1e-300};
    for (size_t i = 0; i < sizeof special / sizeof *special; ++i) {
        (void)oracle_f64_to_bf16(special[i]);
        (void)oracle_f32_to_e4m3((float)special[i]);
    }
    puts("sanitized oracle driver: ok");
    return 0;
}
