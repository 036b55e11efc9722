/*
 * CPU oracle for MoE token dispatch, reduce-once combine, and the fused
 * residual-add + RMSNorm epilogue.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library; it is plain scalar C, slow on purpose, written so that each
 * loop can be checked against the pages by eye.
 *
 * Sources (web pages; the build cites them by title and section):
 *  [A2A]  InferenceX PR #2450, "CollectiveX: add FlashInfer one-sided NVLink
 *         EP for the GB SKUs".  Sections used: "The adapter" table (padded
 *         [ep_size, runtime_max_tokens_per_rank, hidden] receive, valid slots
 *         only, workspace sized once), "Verified: per-rank permutation"
 *         (slot order inside a region is the implementation's choice),
 *         "Kernel arithmetic read from source" (nearest-even narrowing, one
 *         narrowing store), "Update -- the correctness failures are resolved"
 *         (the combine accumulates in fp32 and narrows once; a bf16
 *         accumulator was the defect).
 *  [DR]   vLLM PR #41382, "[Bugfix] Fix double reduce in
 *         flashinfer_nvlink_two_sided and flashinfer_nvlink_one_sided
 *         backends", description and review thread: the all-to-all combine
 *         already sums over the experts dimension, so its output is final and
 *         must not be reduced a second time.
 *  [FUSE] magik.net, "Fusing the Allreduce: A Precision Investigation into
 *         FlashInfer's Verify-Path Optimization", section "The Message
 *         Itself: Explanation and Probe": residual add and RMSNorm fused onto
 *         the reduction that produces the hidden state.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - one workspace row per routed copy (t, j); region of expert e = e / epr;
 *  - rows fill a region in increasing flat index f = t*k + j (stable order);
 *  - expert id -1 means "no expert" (no row, contributes nothing); any other
 *    id outside [0, E) is an error and is likewise skipped;
 *  - a copy whose region is already full is an overflow error, not written;
 *    counts[r] still reports how many copies region r was sent;
 *  - weighted combine term: fmaf(w, y, acc); unweighted: acc + y; terms taken
 *    in j = 0..k-1 order, fp32 accumulator, single nearest-even narrowing;
 *  - fused epilogue: s = acc + residual in fp32 (the accumulator is not
 *    narrowed first); residual_out = bf16(s); the mean of squares, the
 *    reciprocal square root and the scaling by gamma in fp64 (the oracle is
 *    the more precise side), eps inside the square root, mean over H;
 *  - reduction of tensor-parallel partials ([FUSE]'s all-reduce, local
 *    half): the P partials [P, T, H] are summed in fp32 in rank order and
 *    narrowed once, and the fused form applies the combine's epilogue to that
 *    sum;
 *  - per-region layout (the FlashInfer form): one row per (token, region),
 *    taken by the token's first copy to that region; the row's message (the
 *    region's gated, fp32-summed, once-narrowed expert outputs) is added once,
 *    in the order of first copies, unweighted.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_STATUS_OVERFLOW 1
#define ORACLE_STATUS_BAD_ID 2

/* ---- bf16 codec, from the IEEE 754 definition -------------------------------
 * bfloat16 is binary32 with the low 16 fraction bits dropped: 1 sign bit,
 * 8 exponent bits (bias 127), 7 stored fraction bits.  Decoding is exact: the
 * 16 stored bits are the high half of the binary32 pattern.  Encoding rounds
 * a real value to the nearest bfloat16, ties to the even significand:
 * normal numbers in [2^(e-1), 2^e) are spaced 2^(e-8); subnormals (below
 * 2^-126) are spaced 2^-133; magnitudes that round beyond the largest finite
 * value (2 - 2^-7) * 2^127 become infinity. */

float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

uint16_t oracle_f64_to_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);                      /* a in [2^(e-1), 2^e) */
    int qexp = e - 8;                  /* spacing of 8-significant-bit values */
    if (qexp < -133)
        qexp = -133;                   /* subnormal spacing */
    double q = nearbyint(ldexp(a, -qexp));   /* default mode: ties to even */
    double r = ldexp(q, qexp);
    if (r >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);
    float rf = (float)r;               /* exact: r has <= 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &rf, sizeof bits);
    return (uint16_t)(sign | (bits >> 16));
}

uint16_t oracle_f32_to_bf16(float v)
{
    return oracle_f64_to_bf16((double)v);    /* float -> double is exact */
}

/* ---- dispatch ([A2A] "The adapter" table) -----------------------------------
 * x         [T, H] bf16, ids [T, k] int32 (flat index f = t*k + j)
 * ws        [ep, cap, H] bf16; row (r, s) receives copy number s of region r
 * counts    [ep]   copies sent to each region (not clamped to cap)
 * slot_index[T*k]  r*cap + s of the row holding copy f, or -1
 * src_index [ep*cap] f of the copy held by row (r, s), for s < min(counts, cap);
 *           entries past the valid prefix are left untouched, as are the
 *           padding rows of ws.
 * Returns a bit set of ORACLE_STATUS_* flags. */
int oracle_dispatch(const uint16_t *x, const int32_t *ids,
                    int64_t T, int64_t H, int64_t k, int64_t ep, int64_t epr,
                    int64_t cap, uint16_t *ws, int32_t *counts,
                    int32_t *slot_index, int32_t *src_index)
{
    int status = 0;
    int64_t E = ep * epr;
    for (int64_t r = 0; r < ep; ++r)
        counts[r] = 0;
    for (int64_t f = 0; f < T * k; ++f) {
        int32_t e = ids[f];
        slot_index[f] = -1;
        if (e == -1)
            continue;
        if (e < 0 || e >= E) {
            status |= ORACLE_STATUS_BAD_ID;
            continue;
        }
        int64_t r = e / epr;
        int64_t s = counts[r];
        counts[r] += 1;
        if (s >= cap) {
            status |= ORACLE_STATUS_OVERFLOW;
            continue;
        }
        int64_t row = r * cap + s;
        slot_index[f] = (int32_t)row;
        src_index[row] = (int32_t)f;
        memcpy(ws + row * H, x + (f / k) * H, (size_t)H * sizeof(uint16_t));
    }
    return status;
}

/* ---- per-region layout ([A2A] "Update -- the correctness failures are
 * resolved": the FlashInfer dispatch sends a token once per destination
 * rank and blanks the duplicate-rank top-k slots; "Bring-up progress":
 * about 5.3 distinct ranks per token for top-8 over 8 ranks; "Synthesis":
 * duplicate experts on one rank are read once; the combine is an unweighted
 * sum of one message per rank).
 * One row per (token, region): the first copy f = t*k + j of token t bound
 * for region r takes the next row of r; later copies of t bound for r share
 * that row (slot_index equal, src_index holds the first copy).  Rows fill a
 * region in increasing f of their first copy.  Overflow, bad ids and -1 as in
 * oracle_dispatch. */
static int first_copy_to_region(const int32_t *ids, int64_t t, int64_t j, int64_t k,
                                int64_t epr, int64_t E, int64_t *first_j)
{
    int64_t r = ids[t * k + j] / epr;
    for (int64_t i = 0; i < j; ++i) {
        int32_t e = ids[t * k + i];
        if (e >= 0 && e < E && e / epr == r) {
            *first_j = i;
            return 0;
        }
    }
    *first_j = j;
    return 1;
}

int oracle_dispatch_region(const uint16_t *x, const int32_t *ids,
                           int64_t T, int64_t H, int64_t k, int64_t ep, int64_t epr,
                           int64_t cap, uint16_t *ws, int32_t *counts,
                           int32_t *slot_index, int32_t *src_index)
{
    int status = 0;
    int64_t E = ep * epr;
    for (int64_t r = 0; r < ep; ++r)
        counts[r] = 0;
    for (int64_t f = 0; f < T * k; ++f) {
        int32_t e = ids[f];
        slot_index[f] = -1;
        if (e == -1)
            continue;
        if (e < 0 || e >= E) {
            status |= ORACLE_STATUS_BAD_ID;
            continue;
        }
        int64_t t = f / k, j = f % k, first_j;
        if (!first_copy_to_region(ids, t, j, k, epr, E, &first_j)) {
            slot_index[f] = slot_index[t * k + first_j];
            continue;
        }
        int64_t r = e / epr;
        int64_t s = counts[r];
        counts[r] += 1;
        if (s >= cap) {
            status |= ORACLE_STATUS_OVERFLOW;
            continue;
        }
        int64_t row = r * cap + s;
        slot_index[f] = (int32_t)row;
        src_index[row] = (int32_t)f;
        memcpy(ws + row * H, x + t * H, (size_t)H * sizeof(uint16_t));
    }
    return status;
}

/* True if an earlier copy of token t already names the same row: under the
 * per-region layout that row's message has been added, so it is skipped. */
static int row_seen_before(const int32_t *slot_index, int64_t t, int64_t j, int64_t k)
{
    for (int64_t i = 0; i < j; ++i)
        if (slot_index[t * k + i] == slot_index[t * k + j])
            return 1;
    return 0;
}

/* ---- combine: reduce exactly once ([A2A] "Update -- ... resolved", [DR]) ----
 * out[t, h] = bf16( sum over j = 0..k-1 with slot_index[t,j] >= 0 of
 *                   c_j * f32(y[slot_index[t,j], h]) )
 * accumulated in fp32 in j order; c_j = w[t, j] (weighted) or 1 (unweighted).
 * out is overwritten, never accumulated into. */
static float combine_accumulate(const uint16_t *y, const int32_t *slot_index,
                                const float *w, int weighted, int64_t t,
                                int64_t h, int64_t H, int64_t k, int once_per_row)
{
    float acc = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
        int32_t row = slot_index[t * k + j];
        if (row < 0)
            continue;
        if (once_per_row && row_seen_before(slot_index, t, j, k))
            continue;
        float v = oracle_bf16_to_f32(y[(int64_t)row * H + h]);
        if (weighted)
            acc = fmaf(w[t * k + j], v, acc);
        else
            acc = acc + v;
    }
    return acc;
}

static void combine_rows(const uint16_t *y, const int32_t *slot_index, const float *w,
                         int weighted, int64_t T, int64_t H, int64_t k, int once_per_row,
                         uint16_t *out)
{
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h)
            out[t * H + h] = oracle_f32_to_bf16(
                combine_accumulate(y, slot_index, w, weighted, t, h, H, k, once_per_row));
}

int oracle_combine(const uint16_t *y, const int32_t *slot_index, const float *w,
                   int weighted, int64_t T, int64_t H, int64_t k, uint16_t *out)
{
    combine_rows(y, slot_index, w, weighted, T, H, k, 0, out);
    return 0;
}

/* Per-region layout: each distinct row of a token is added once, in the order
 * of its first copy; the messages already carry the gates (unweighted). */
int oracle_combine_region(const uint16_t *y, const int32_t *slot_index,
                          int64_t T, int64_t H, int64_t k, uint16_t *out)
{
    combine_rows(y, slot_index, NULL, 0, T, H, k, 1, out);
    return 0;
}

/* ---- combine + residual add + RMSNorm ([FUSE]) ------------------------------
 * s[h]            = acc[h] + f32(residual[t, h])          (fp32)
 * residual_out    = bf16(s)
 * normed[t, h]    = bf16( s[h] / sqrt(mean_h(s^2) + eps) * f32(gamma[h]) )
 * residual_out may alias residual (each element is read before it is written).
 * normed_f64, if not NULL, receives the unrounded fp64 normed values.
 * s_scratch is caller memory of H floats. */
static void fused_rows(const uint16_t *y, const int32_t *slot_index, const float *w,
                       int weighted, int once_per_row, int64_t T, int64_t H, int64_t k,
                       const uint16_t *residual, const uint16_t *gamma, float eps,
                       uint16_t *residual_out, uint16_t *normed, double *normed_f64,
                       float *s_scratch)
{
    for (int64_t t = 0; t < T; ++t) {
        double sumsq = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            float acc = combine_accumulate(y, slot_index, w, weighted, t, h, H, k, once_per_row);
            float s = acc + oracle_bf16_to_f32(residual[t * H + h]);
            s_scratch[h] = s;
            sumsq += (double)s * (double)s;
        }
        double inv = 1.0 / sqrt(sumsq / (double)H + (double)eps);
        for (int64_t h = 0; h < H; ++h) {
            double n = (double)s_scratch[h] * inv * (double)oracle_bf16_to_f32(gamma[h]);
            residual_out[t * H + h] = oracle_f32_to_bf16(s_scratch[h]);
            normed[t * H + h] = oracle_f64_to_bf16(n);
            if (normed_f64)
                normed_f64[t * H + h] = n;
        }
    }
}

int oracle_combine_residual_rmsnorm(const uint16_t *y, const int32_t *slot_index,
                                    const float *w, int weighted, int64_t T,
                                    int64_t H, int64_t k, const uint16_t *residual,
                                    const uint16_t *gamma, float eps,
                                    uint16_t *residual_out, uint16_t *normed,
                                    double *normed_f64, float *s_scratch)
{
    fused_rows(y, slot_index, w, weighted, 0, T, H, k, residual, gamma, eps, residual_out,
               normed, normed_f64, s_scratch);
    return 0;
}

int oracle_combine_residual_rmsnorm_region(const uint16_t *y, const int32_t *slot_index,
                                           int64_t T, int64_t H, int64_t k,
                                           const uint16_t *residual, const uint16_t *gamma,
                                           float eps, uint16_t *residual_out,
                                           uint16_t *normed, double *normed_f64,
                                           float *s_scratch)
{
    fused_rows(y, slot_index, NULL, 0, 1, T, H, k, residual, gamma, eps, residual_out, normed,
               normed_f64, s_scratch);
    return 0;
}

/* ---- reduction stage of a one-shot all-reduce + residual + RMSNorm ([FUSE]) --
 * Under tensor parallelism every rank ends a layer with a partial hidden state
 * and an all-reduce sums them; [FUSE] replaces that all-reduce followed by
 * the residual add and RMSNorm with one kernel.  On one GPU the exchange is
 * done once all P partials sit in local memory, partials[p, t, h], and what
 * remains is their sum.  The same "reduce once, narrow once" reading as the
 * combine:
 *   acc[t, h] = sum over p = 0..P-1 of f32(partials[p, t, h])   (fp32, p order)
 *   out       = bf16(acc)                                      (plain reduce)
 * and, fused, the epilogue of the combine above with acc in place of the
 * combine's sum. */
static float partials_accumulate(const uint16_t *partials, int64_t P, int64_t T,
                                 int64_t H, int64_t t, int64_t h)
{
    float acc = 0.0f;
    for (int64_t p = 0; p < P; ++p)
        acc = acc + oracle_bf16_to_f32(partials[(p * T + t) * H + h]);
    return acc;
}

int oracle_partials_reduce(const uint16_t *partials, int64_t P, int64_t T, int64_t H,
                           uint16_t *out)
{
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h)
            out[t * H + h] = oracle_f32_to_bf16(partials_accumulate(partials, P, T, H, t, h));
    return 0;
}

int oracle_partials_reduce_residual_rmsnorm(const uint16_t *partials, int64_t P, int64_t T,
                                            int64_t H, const uint16_t *residual,
                                            const uint16_t *gamma, float eps,
                                            uint16_t *residual_out, uint16_t *normed,
                                            double *normed_f64, float *s_scratch)
{
    for (int64_t t = 0; t < T; ++t) {
        double sumsq = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            float sum = partials_accumulate(partials, P, T, H, t, h);
            float s = sum + oracle_bf16_to_f32(residual[t * H + h]);
            s_scratch[h] = s;
            sumsq += (double)s * (double)s;
        }
        double rinv = 1.0 / sqrt(sumsq / (double)H + (double)eps);
        for (int64_t h = 0; h < H; ++h) {
            double n = (double)s_scratch[h] * rinv * (double)oracle_bf16_to_f32(gamma[h]);
            residual_out[t * H + h] = oracle_f32_to_bf16(s_scratch[h]);
            normed[t * H + h] = oracle_f64_to_bf16(n);
            if (normed_f64)
                normed_f64[t * H + h] = n;
        }
    }
    return 0;
}

/* ---- FP8 payload (InferenceX PR #2450, "The adapter" notes: an FP8 dispatch
 * carries its scale as a second payload, checked against the oracle's cast
 * round-trip) -------------------------------------------------------------------
 * OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 stored
 * fraction bits; normal numbers in [2^(e-1), 2^e) are spaced 2^(e-4), the
 * smallest normal is 2^-6 and subnormals are spaced 2^-9; the largest finite
 * value is 448 (exponent field 15, fraction 110); exponent 15 with fraction
 * 111 is NaN and there is no infinity, so a magnitude that rounds past 448
 * (at or beyond the tie point 464) becomes NaN.  Encoding rounds to nearest,
 * ties to the even significand. */

float oracle_e4m3_to_f32(uint8_t c)
{
    int sign = c >> 7, exp = (c >> 3) & 15, frac = c & 7;
    double v;
    if (exp == 15 && frac == 7)
        v = NAN;
    else if (exp == 0)
        v = ldexp((double)frac, -9);
    else
        v = ldexp(1.0 + frac / 8.0, exp - 7);
    return (float)(sign ? -v : v);
}

uint8_t oracle_f32_to_e4m3(float f)
{
    double v = (double)f;
    uint8_t sign = signbit(v) ? 0x80u : 0u;
    if (isnan(v))
        return (uint8_t)(sign | 0x7Fu);
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    int e = 0;
    if (!isinf(a))
        frexp(a, &e);                  /* a in [2^(e-1), 2^e) */
    int qexp = e - 4;                  /* spacing of 4-significant-bit values */
    if (qexp < -9)
        qexp = -9;                     /* subnormal spacing */
    double r = isinf(a) ? INFINITY : ldexp(nearbyint(ldexp(a, -qexp)), qexp);
    if (r > 448.0)
        return (uint8_t)(sign | 0x7Fu);          /* no infinity: NaN */
    if (r < ldexp(1.0, -6))                       /* subnormal: fraction = r / 2^-9 */
        return (uint8_t)(sign | (uint8_t)ldexp(r, 9));
    int re;
    double m = frexp(r, &re);                     /* r = m * 2^re, m in [0.5, 1) */
    int frac = (int)ldexp(m * 2.0 - 1.0, 3);      /* 1.fff */
    return (uint8_t)(sign | ((re - 1 + 7) << 3) | frac);
}

/* Row quantisation for the FP8 payload: one fp32 scale per token row,
 *   amax     = max_h |x[t, h]|
 *   scale[t] = amax / 448          (fp32 division; 0 for an all-zero row)
 *   inv      = 448 / amax          (fp32 division; 0 for an all-zero row)
 *   q[t, h]  = e4m3( fp32(x[t, h]) * inv )   (fp32 product, then nearest-even)
 * so the row's largest magnitude maps to 448 and x ~ e4m3_value(q) * scale.
 * Inputs are finite. */
void oracle_quantize_e4m3_rows(const uint16_t *x, int64_t T, int64_t H, uint8_t *q,
                               float *scale)
{
    for (int64_t t = 0; t < T; ++t) {
        float amax = 0.0f;
        for (int64_t h = 0; h < H; ++h) {
            float a = fabsf(oracle_bf16_to_f32(x[t * H + h]));
            if (a > amax)
                amax = a;
        }
        float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
        scale[t] = amax / 448.0f;
        for (int64_t h = 0; h < H; ++h)
            q[t * H + h] = oracle_f32_to_e4m3(oracle_bf16_to_f32(x[t * H + h]) * inv);
    }
}

/* ---- array forms of the codec, for the test suite ---------------------------- */
void oracle_e4m3_to_f32_array(const uint8_t *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_to_f32(in[i]);
}

void oracle_f32_to_e4m3_array(const float *in, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_e4m3(in[i]);
}

void oracle_bf16_to_f32_array(const uint16_t *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_to_f32(in[i]);
}

void oracle_f32_to_bf16_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_bf16(in[i]);
}

void oracle_f64_to_bf16_array(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f64_to_bf16(in[i]);
}
