/*
 * oracle/rank_step.c -- the oracle's rank step in plain C, float64 throughout.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load it.  It shares no code, constants or
 * helpers with the HIP library in rank_step_amd/ and includes nothing from
 * there.
 *
 * The same arithmetic as oracle/step.py (which cites the pages step by step),
 * written element by element so that the parity tests can run the oracle over
 * every element of a rank shard of hundreds of millions of parameters.  For
 * each element k < n of one shard:
 *
 *   1. G = (x_0 + x_1 + ... + x_{N-1}) / N: the mean of the N incoming
 *      gradient slices, each widened exactly to double, summed in rank order
 *      and divided once ("PyTorch 训练框架内核深度解析, 第18章 FSDP" §18.3 and
 *      §18.6, reduce-scatter with reduce_dtype=float32; NCCL ZeRO/FSDP state
 *      sharding post, "Optimizer Step 的所有权": replicas step with averaged
 *      gradients).
 *   2. decoupled-weight-decay AdamW on the shard only (FSDP chapter §18.21 and
 *      §18.43, torch.optim.AdamW; the post's "FSDP Sharded Optimizer"):
 *         p1 = p * (1 - lr*wd)
 *         m' = beta1*m + (1 - beta1)*G
 *         v' = beta2*v + (1 - beta2)*G*G
 *         mhat = m' / (1 - beta1^t),  vhat = v' / (1 - beta2^t)
 *         p' = p1 - lr*mhat / (sqrt(vhat) + eps)
 *   3. the bf16 copy: round to nearest, ties to even, from the format's
 *      definition (FSDP chapter §18.6 and §18.10: bf16 on the wire, fp32
 *      master).
 *
 * Every operation is one IEEE double operation, in the order oracle/step.py
 * takes them (built with -ffp-contract=off, so no fused multiply-add), so the
 * two agree bit for bit; the CPU tests check that on seeded inputs and on the
 * special values.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* bf16 bit pattern -> double, exactly (bf16 is the top half of an fp32). */
static double widen_bf16(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Slice q's element k, widened exactly to double. */
static double slice_elem(const void* slices, int32_t slice_is_bf16, int64_t stride, int32_t q,
                         int64_t k) {
    if (slice_is_bf16) return widen_bf16(((const uint16_t*)slices)[q * stride + k]);
    return (double)((const float*)slices)[q * stride + k];
}

/* The mean of element k's slices, then its AdamW update, from the state
 * p, m, v (already in double). */
static void step_elem(double p, double m, double v, const void* slices, int32_t slice_is_bf16,
                      int64_t stride, int32_t n_slices, int64_t k, double lr, double beta1,
                      double beta2, double eps, double decay, double bc1, double bc2, double* g_out,
                      double* p_out, double* m_out, double* v_out) {
    /* 1. the mean of the slices */
    double acc = 0.0;
    for (int32_t q = 0; q < n_slices; ++q) acc = acc + slice_elem(slices, slice_is_bf16, stride, q, k);
    const double g = acc / (double)n_slices;
    /* 2. AdamW */
    const double p1 = p * decay;
    const double m_new = beta1 * m + (1.0 - beta1) * g;
    const double v_new = beta2 * v + ((1.0 - beta2) * g) * g;
    const double mhat = m_new / bc1;
    const double vhat = v_new / bc2;
    *g_out = g;
    *p_out = p1 - (lr * mhat) / (sqrt(vhat) + eps);
    *m_out = m_new;
    *v_out = v_new;
}

/*
 * One rank step over elements [0, n) of a shard whose fp32 state before the
 * step is p, m, v, and whose N gradient slices start `stride` elements apart
 * (bf16 bit patterns when slice_is_bf16, else fp32).  Writes the reduced
 * gradient and the updated state, in double.  Returns 0, or -1 for bad
 * arguments (n < 0, N < 1, t < 1).
 */
int oracle_rank_step(const float* p, const float* m, const float* v, const void* slices,
                     int32_t slice_is_bf16, int64_t stride, int32_t n_slices, int64_t n,
                     int64_t t, double lr, double beta1, double beta2, double eps,
                     double weight_decay, double* g_out, double* p_out, double* m_out,
                     double* v_out) {
    if (n < 0 || n_slices < 1 || t < 1) return -1;
    const double decay = 1.0 - lr * weight_decay;
    const double bc1 = 1.0 - pow(beta1, (double)t);
    const double bc2 = 1.0 - pow(beta2, (double)t);
    for (int64_t k = 0; k < n; ++k)
        step_elem((double)p[k], (double)m[k], (double)v[k], slices, slice_is_bf16, stride, n_slices, k,
                  lr, beta1, beta2, eps, decay, bc1, bc2, g_out + k, p_out + k, m_out + k, v_out + k);
    return 0;
}

/* The same step from a state held in double (the oracle's own trajectory
 * carried from step to step). */
int oracle_rank_step_f64(const double* p, const double* m, const double* v, const void* slices,
                         int32_t slice_is_bf16, int64_t stride, int32_t n_slices, int64_t n,
                         int64_t t, double lr, double beta1, double beta2, double eps,
                         double weight_decay, double* g_out, double* p_out, double* m_out,
                         double* v_out) {
    if (n < 0 || n_slices < 1 || t < 1) return -1;
    const double decay = 1.0 - lr * weight_decay;
    const double bc1 = 1.0 - pow(beta1, (double)t);
    const double bc2 = 1.0 - pow(beta2, (double)t);
    for (int64_t k = 0; k < n; ++k)
        step_elem(p[k], m[k], v[k], slices, slice_is_bf16, stride, n_slices, k, lr, beta1, beta2, eps,
                  decay, bc1, bc2, g_out + k, p_out + k, m_out + k, v_out + k);
    return 0;
}

/*
 * 3. bf16 round to nearest even of double values: the representable bf16
 * value nearest to x (1 sign, 8 exponent and 7 fraction bits), ties to the
 * one with an even last fraction bit; magnitudes that round past the largest
 * finite value give infinity; NaN gives the quiet NaN 0x7FC0 with x's sign;
 * signed zeros keep their sign.
 */
static uint16_t bf16_rne(double x) {
    const uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
    if (isinf(x)) return (uint16_t)(sign | 0x7F80u);
    const double a = fabs(x);
    if (a == 0.0) return sign;
    int e2;
    (void)frexp(a, &e2);                  /* a = f * 2^e2, 0.5 <= f < 1 */
    int lead = e2 - 1;                    /* a in [2^lead, 2^(lead+1)) */
    if (lead < -126) lead = -126;         /* below the normal range the spacing is fixed */
    const int ulp_exp = lead - 7;
    const double val = ldexp(rint(ldexp(a, -ulp_exp)), ulp_exp);   /* rint: ties to even */
    if (val >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    const float f = (float)val;           /* exact: every finite bf16 value is an fp32 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

/* bf16 bits of n double values. */
void oracle_bf16_rne(const double* x, int64_t n, uint16_t* out) {
    for (int64_t k = 0; k < n; ++k) out[k] = bf16_rne(x[k]);
}
