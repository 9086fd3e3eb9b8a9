/*
 * tests/c/fullcheck.c -- the parity checks of tests/parity.py, element by
 * element in C, for the tests that compare every element of a rank shard of
 * hundreds of millions of parameters with the oracle (test-side only; the
 * expected values come from the oracle, oracle/rank_step.c).
 *
 * For one block of n elements it takes the state before the step (the
 * oracle's inputs: p0, m0, v0 and the slices), the oracle's results in double
 * (g, p, m, v) and the GPU's results (fp32 p, m, v, optionally the stored
 * gradient and the bf16 copy), and counts:
 *
 *   - elements beyond the mixed tolerance |x_gpu - x_ref| <= tol*max(|x_ref|, s_x)
 *     with the floors of tests/parity.py (s_G = mean_q |x_q|,
 *     s_m = b1|m0| + (1-b1)s_G, s_v = b2 v0 + (1-b2)s_G^2,
 *     s_p = |p0|(1 - lr wd) + lr (s_m/bc1) / (sqrt(vhat) + eps)),
 *     NaN where the other side is not, and infinities that differ;
 *   - the largest share of the allowance used, err / (tol*max(|x_ref|, s_x));
 *   - elements beyond the literal bound |err| <= tol*|x_ref|;
 *   - bf16: words that are not the RNE of the GPU's own fp32 value, words
 *     more than 1 ulp from RNE(oracle) where the fp32 allowance is below half
 *     a bf16 ulp, and all words that differ from RNE(oracle).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { OUT_G = 0, OUT_P = 1, OUT_M = 2, OUT_V = 3, N_OUT = 4 };

typedef struct {
    int64_t n_bad[N_OUT];      /* beyond the mixed tolerance (or NaN / infinity mismatch) */
    int64_t first_bad[N_OUT];  /* index of the first such element, -1 if none */
    int64_t n_literal[N_OUT];  /* beyond the literal relative bound */
    double worst[N_OUT];       /* largest err / allowance over the finite results */
    int64_t bf16_not_own;      /* bf16 word != RNE of the GPU's own fp32 p' */
    int64_t bf16_far;          /* judged words more than 1 ulp from RNE(oracle p') */
    int64_t bf16_diff;         /* words != RNE(oracle p') */
    int64_t first_bf16_bad;    /* first word failing one of the first two rules, -1 if none */
} check_stats;

static double widen_bf16(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double slice_elem(const void* slices, int32_t slice_is_bf16, int64_t stride, int32_t q,
                         int64_t k) {
    if (slice_is_bf16) return widen_bf16(((const uint16_t*)slices)[q * stride + k]);
    return (double)((const float*)slices)[q * stride + k];
}

/* RNE of a double to bf16 (see oracle/rank_step.c for the rule), from the
 * definition: the general path. */
static uint16_t rne_general(double x) {
    const uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
    if (isinf(x)) return (uint16_t)(sign | 0x7F80u);
    const double a = fabs(x);
    if (a == 0.0) return sign;
    int e2;
    (void)frexp(a, &e2);
    int lead = e2 - 1;
    if (lead < -126) lead = -126;
    const int ulp_exp = lead - 7;
    const double val = ldexp(rint(ldexp(a, -ulp_exp)), ulp_exp);
    if (val >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    const float f = (float)val;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

/* The same rounding on the bits of the double where the result is a normal
 * bf16 or overflows (binary exponent -126..127): round the 52 fraction bits
 * to 7, ties to even, the carry rising into the exponent; the exponent is
 * rebiased from 1023 to 127.  Zeros, subnormal results, NaN and infinities
 * take the general path. */
uint16_t fullcheck_rne(double x) {
    uint64_t u;
    memcpy(&u, &x, sizeof u);
    const int e = (int)((u >> 52) & 0x7FFu) - 1023;
    if (e < -126 || e > 127) return rne_general(x);
    const uint64_t sign = u >> 63;
    const uint64_t r = u + ((UINT64_C(1) << 44) - 1) + ((u >> 45) & 1u);
    const int er = (int)((r >> 52) & 0x7FFu) - 1023;
    if (er > 127) return (uint16_t)((sign << 15) | 0x7F80u);
    return (uint16_t)((sign << 15) | ((uint64_t)(er + 127) << 7) | ((r >> 45) & 0x7Fu));
}

static uint16_t rne(double x) { return fullcheck_rne(x); }

/* signed-magnitude bf16 bits -> integers in value order */
static int32_t monotone(uint16_t b) { return (b & 0x8000u) ? -(int32_t)(b & 0x7FFFu) : (int32_t)b; }

static void judge(check_stats* s, int o, int64_t k, double got, double ref, double floor, double tol) {
    if (isnan(got) != isnan(ref)) {
        if (s->n_bad[o]++ == 0) s->first_bad[o] = k;
        return;
    }
    if (isinf(ref)) {
        if (got != ref && s->n_bad[o]++ == 0) s->first_bad[o] = k;
        return;
    }
    if (isnan(ref)) return;
    const double err = fabs(got - ref);
    const double lim = tol * fmax(fabs(ref), floor);
    if (err > lim && s->n_bad[o]++ == 0) s->first_bad[o] = k;
    if (err > tol * fabs(ref)) s->n_literal[o]++;
    if (isfinite(got)) {
        const double r = lim > 0 ? err / lim : (err > 0 ? INFINITY : 0.0);
        if (r > s->worst[o]) s->worst[o] = r;
    }
}

void fullcheck_init(check_stats* s) {
    memset(s, 0, sizeof *s);
    for (int o = 0; o < N_OUT; ++o) s->first_bad[o] = -1;
    s->first_bf16_bad = -1;
}

/*
 * Check elements [0, n) of one block.  gpu_g and gpu_bf16 may be NULL.
 * `base` is added to the indices recorded in the stats.
 */
void fullcheck_block(int64_t n, int64_t base, const float* p0, const float* m0, const float* v0,
                     const void* slices, int32_t slice_is_bf16, int64_t stride, int32_t n_slices,
                     int64_t t, double lr, double beta1, double beta2, double eps,
                     double weight_decay, double tol, const double* ref_g, const double* ref_p,
                     const double* ref_m, const double* ref_v, const float* gpu_p,
                     const float* gpu_m, const float* gpu_v, const float* gpu_g,
                     const uint16_t* gpu_bf16, check_stats* s) {
    const double bc1 = 1.0 - pow(beta1, (double)t);
    const double bc2 = 1.0 - pow(beta2, (double)t);
    const double half_ulp_scale = ldexp(1.0, -9);
    for (int64_t k = 0; k < n; ++k) {
        double sg = 0.0;
        for (int32_t q = 0; q < n_slices; ++q) sg += fabs(slice_elem(slices, slice_is_bf16, stride, q, k));
        sg /= (double)n_slices;
        const double s_m = beta1 * fabs((double)m0[k]) + (1.0 - beta1) * sg;
        const double s_v = beta2 * (double)v0[k] + (1.0 - beta2) * sg * sg;
        const double vhat = ref_v[k] / bc2;
        const double s_p = fabs((double)p0[k]) * (1.0 - lr * weight_decay) +
                           lr * (s_m / bc1) / (sqrt(vhat) + eps);
        const int64_t at = base + k;
        if (gpu_g) judge(s, OUT_G, at, (double)gpu_g[k], ref_g[k], sg, tol);
        judge(s, OUT_P, at, (double)gpu_p[k], ref_p[k], s_p, tol);
        judge(s, OUT_M, at, (double)gpu_m[k], ref_m[k], s_m, tol);
        judge(s, OUT_V, at, (double)gpu_v[k], ref_v[k], s_v, tol);
        if (gpu_bf16) {
            const uint16_t got = gpu_bf16[k];
            const uint16_t own = rne((double)gpu_p[k]);
            const uint16_t want = rne(ref_p[k]);
            int bad = got != own;
            if (bad) s->bf16_not_own++;
            if (got != want) s->bf16_diff++;
            const double rp = ref_p[k];
            if (!isnan(rp) && tol * fmax(fabs(rp), s_p) < fabs(rp) * half_ulp_scale) {
                const int32_t d = monotone(got) - monotone(want);
                if (d > 1 || d < -1) {
                    s->bf16_far++;
                    bad = 1;
                }
            }
            if (bad && s->first_bf16_bad < 0) s->first_bf16_bad = at;
        }
    }
}

/* Adds the counts of b into a (the first indices and maxima combine too). */
void fullcheck_merge(check_stats* a, const check_stats* b) {
    for (int o = 0; o < N_OUT; ++o) {
        if (b->first_bad[o] >= 0 && (a->first_bad[o] < 0 || b->first_bad[o] < a->first_bad[o]))
            a->first_bad[o] = b->first_bad[o];
        a->n_bad[o] += b->n_bad[o];
        a->n_literal[o] += b->n_literal[o];
        if (b->worst[o] > a->worst[o]) a->worst[o] = b->worst[o];
    }
    if (b->first_bf16_bad >= 0 && (a->first_bf16_bad < 0 || b->first_bf16_bad < a->first_bf16_bad))
        a->first_bf16_bad = b->first_bf16_bad;
    a->bf16_not_own += b->bf16_not_own;
    a->bf16_far += b->bf16_far;
    a->bf16_diff += b->bf16_diff;
}
