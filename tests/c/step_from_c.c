/* A plain C11 consumer of the whole path: HIP runtime calls for memory, the
 * library's C ABI for the step, no PyTorch.  Three shards (one with padding)
 * of 8 bf16 gradient slices each get seeded inputs, one fused multi-tensor
 * step at t = 1, and the inputs and outputs are written to the file named by
 * argv[1] for the test to check against the oracle:
 *   per shard: int64 S, int64 valid, uint16 slices[8][S], float p0[S], m0[S],
 *   v0[S], float p1[S], m1[S], v1[S], uint16 bf16[S]. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fsdp_step.h"

#define NS 8
#define NSHARDS 3

static uint32_t lcg = 12345u;
static float uniform(void) { /* [-1, 1) */
    lcg = lcg * 1664525u + 1013904223u;
    return (float)(lcg >> 8) * (1.0f / 8388608.0f) - 1.0f;
}
static uint16_t to_bf16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

#define HIP_OK(x)                                                                  \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                \
            return 1;                                                              \
        }                                                                          \
    } while (0)

int main(int argc, char** argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s OUTPUT\n", argv[0]);
        return 2;
    }
    const int64_t S[NSHARDS] = {5000, 2048, 777};
    const int64_t V[NSHARDS] = {4990, 2048, 777};
    uint16_t* h_sl[NSHARDS];
    float *h_p[NSHARDS], *h_m[NSHARDS], *h_v[NSHARDS];
    void *d_sl[NSHARDS], *d_p[NSHARDS], *d_m[NSHARDS], *d_v[NSHARDS], *d_out[NSHARDS];
    fsdp_mt_tensor t[NSHARDS];
    memset(t, 0, sizeof t);
    for (int i = 0; i < NSHARDS; ++i) {
        const int64_t n = S[i];
        h_sl[i] = malloc(NS * n * 2);
        h_p[i] = malloc(n * 4);
        h_m[i] = malloc(n * 4);
        h_v[i] = malloc(n * 4);
        if (!h_sl[i] || !h_p[i] || !h_m[i] || !h_v[i]) return 1;
        for (int64_t k = 0; k < n; ++k) {
            const int pad = k >= V[i];
            h_p[i][k] = pad ? 12345.0f : 0.02f * uniform();
            h_m[i][k] = pad ? -7.0f : 1e-3f * uniform();
            const float u = uniform();
            h_v[i][k] = pad ? 3.0f : 1e-6f * u * u;
            for (int q = 0; q < NS; ++q) h_sl[i][q * n + k] = pad ? 0x7fc0u : to_bf16_bits(1e-2f * uniform());
        }
        HIP_OK(hipMalloc(&d_sl[i], NS * n * 2));
        HIP_OK(hipMalloc(&d_p[i], n * 4));
        HIP_OK(hipMalloc(&d_m[i], n * 4));
        HIP_OK(hipMalloc(&d_v[i], n * 4));
        HIP_OK(hipMalloc(&d_out[i], n * 2));
        HIP_OK(hipMemcpy(d_sl[i], h_sl[i], NS * n * 2, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(d_p[i], h_p[i], n * 4, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(d_m[i], h_m[i], n * 4, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(d_v[i], h_v[i], n * 4, hipMemcpyHostToDevice));
        t[i].param_fp32 = d_p[i];
        t[i].exp_avg = d_m[i];
        t[i].exp_avg_sq = d_v[i];
        t[i].grad_slices = d_sl[i];
        t[i].slice_stride = n;
        t[i].unshard_bf16_out = d_out[i];
        t[i].shard_numel = n;
        t[i].valid = V[i];
    }
    fsdp_mt_plan* plan = NULL;
    int32_t st = fsdp_mt_plan_create(&plan, t, NSHARDS, NS, FSDP_DT_BF16, NULL);
    if (st != FSDP_OK) {
        fprintf(stderr, "plan: %d %s\n", st, fsdp_last_error());
        return 1;
    }
    const fsdp_adamw_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.01, 1};
    st = fsdp_mt_step(plan, &hp, NULL);
    if (st != FSDP_OK) {
        fprintf(stderr, "step: %d %s\n", st, fsdp_last_error());
        return 1;
    }
    HIP_OK(hipDeviceSynchronize());
    FILE* f = fopen(argv[1], "wb");
    if (!f) return 1;
    for (int i = 0; i < NSHARDS; ++i) {
        const int64_t n = S[i];
        float* o = malloc(n * 4);
        uint16_t* b = malloc(n * 2);
        if (!o || !b) return 1;
        fwrite(&S[i], 8, 1, f);
        fwrite(&V[i], 8, 1, f);
        fwrite(h_sl[i], 2, NS * n, f);
        fwrite(h_p[i], 4, n, f);
        fwrite(h_m[i], 4, n, f);
        fwrite(h_v[i], 4, n, f);
        void* const outs[3] = {d_p[i], d_m[i], d_v[i]};
        for (int j = 0; j < 3; ++j) {
            HIP_OK(hipMemcpy(o, outs[j], n * 4, hipMemcpyDeviceToHost));
            fwrite(o, 4, n, f);
        }
        HIP_OK(hipMemcpy(b, d_out[i], n * 2, hipMemcpyDeviceToHost));
        fwrite(b, 2, n, f);
        free(o);
        free(b);
    }
    fclose(f);
    st = fsdp_mt_plan_destroy(plan);
    for (int i = 0; i < NSHARDS; ++i) {
        hipFree(d_sl[i]);
        hipFree(d_p[i]);
        hipFree(d_m[i]);
        hipFree(d_v[i]);
        hipFree(d_out[i]);
        free(h_sl[i]);
        free(h_p[i]);
        free(h_m[i]);
        free(h_v[i]);
    }
    return st == FSDP_OK ? 0 : 1;
}
