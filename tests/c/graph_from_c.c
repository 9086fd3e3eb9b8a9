/* A plain C11 consumer of the capturable step: HIP runtime calls for memory,
 * streams and graphs, the library's C ABI for the steps, no PyTorch.  Two
 * copies of the same three shards (one with padding, 8 bf16 gradient slices
 * each, shared read-only) are stepped side by side: copy A by fsdp_mt_step
 * at t = 1, 2, 3, 4, copy B by replays of one HIP graph that captured
 * fsdp_mt_step_capturable once.  The learning rate follows a schedule
 * (linear warmup, then decay): A passes each step's rate in its hparams, B
 * reads it from a device double that the host writes before each replay.
 * After every replay the two copies' state and bf16 outputs must be equal
 * bit for bit and the device count must equal the replays made.  Prints
 * "graph_from_c: ok" and exits 0, else prints what differs and exits 1. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fsdp_step.h"

#define NS 8
#define NSHARDS 3
#define REPLAYS 4

static uint32_t lcg = 777u;
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

#define FSDP_OK_OR_FAIL(x)                                                         \
    do {                                                                           \
        int32_t s_ = (x);                                                          \
        if (s_ != FSDP_OK) {                                                       \
            fprintf(stderr, "%s: %d %s\n", #x, s_, fsdp_last_error());             \
            return 1;                                                              \
        }                                                                          \
    } while (0)

/* Device buffers of one copy of the shards. */
typedef struct {
    void *p[NSHARDS], *m[NSHARDS], *v[NSHARDS], *out[NSHARDS];
} copy_bufs;

/* Equal bytes of n-byte device buffers a and b (host scratch h1, h2). */
static int same_bytes(const void* a, const void* b, size_t n, unsigned char* h1, unsigned char* h2) {
    if (hipMemcpy(h1, a, n, hipMemcpyDeviceToHost) != hipSuccess) return 0;
    if (hipMemcpy(h2, b, n, hipMemcpyDeviceToHost) != hipSuccess) return 0;
    return memcmp(h1, h2, n) == 0;
}

int main(void) {
    const int64_t S[NSHARDS] = {6000, 2048, 515};
    const int64_t V[NSHARDS] = {5990, 2048, 515};
    void* d_sl[NSHARDS];
    copy_bufs c[2];
    fsdp_mt_tensor t[2][NSHARDS];
    memset(t, 0, sizeof t);
    unsigned char *h1 = malloc(6000 * 4), *h2 = malloc(6000 * 4);
    if (!h1 || !h2) return 1;
    for (int i = 0; i < NSHARDS; ++i) {
        const int64_t n = S[i];
        uint16_t* hs = malloc(NS * n * 2);
        float *hp = malloc(n * 4), *hm = malloc(n * 4), *hv = malloc(n * 4);
        if (!hs || !hp || !hm || !hv) return 1;
        for (int64_t k = 0; k < n; ++k) {
            const int pad = k >= V[i];
            hp[k] = pad ? 0.0f : 0.02f * uniform();
            hm[k] = pad ? 0.0f : 1e-3f * uniform();
            const float u = uniform();
            hv[k] = pad ? 0.0f : 1e-6f * u * u;
            for (int q = 0; q < NS; ++q) hs[q * n + k] = to_bf16_bits(1e-2f * uniform());
        }
        HIP_OK(hipMalloc(&d_sl[i], NS * n * 2));
        HIP_OK(hipMemcpy(d_sl[i], hs, NS * n * 2, hipMemcpyHostToDevice));
        for (int a = 0; a < 2; ++a) {
            HIP_OK(hipMalloc(&c[a].p[i], n * 4));
            HIP_OK(hipMalloc(&c[a].m[i], n * 4));
            HIP_OK(hipMalloc(&c[a].v[i], n * 4));
            HIP_OK(hipMalloc(&c[a].out[i], n * 2));
            HIP_OK(hipMemcpy(c[a].p[i], hp, n * 4, hipMemcpyHostToDevice));
            HIP_OK(hipMemcpy(c[a].m[i], hm, n * 4, hipMemcpyHostToDevice));
            HIP_OK(hipMemcpy(c[a].v[i], hv, n * 4, hipMemcpyHostToDevice));
            t[a][i].param_fp32 = c[a].p[i];
            t[a][i].exp_avg = c[a].m[i];
            t[a][i].exp_avg_sq = c[a].v[i];
            t[a][i].grad_slices = d_sl[i];
            t[a][i].slice_stride = n;
            t[a][i].unshard_bf16_out = c[a].out[i];
            t[a][i].shard_numel = n;
            t[a][i].valid = V[i];
        }
        free(hs);
        free(hp);
        free(hm);
        free(hv);
    }
    hipStream_t stream;
    HIP_OK(hipStreamCreateWithFlags(&stream, hipStreamNonBlocking));
    fsdp_mt_plan *plan_a = NULL, *plan_b = NULL;
    FSDP_OK_OR_FAIL(fsdp_mt_plan_create(&plan_a, t[0], NSHARDS, NS, FSDP_DT_BF16, stream));
    FSDP_OK_OR_FAIL(fsdp_mt_plan_create(&plan_b, t[1], NSHARDS, NS, FSDP_DT_BF16, stream));
    int64_t* d_count;
    double* d_lr;
    HIP_OK(hipMalloc((void**)&d_count, 8));
    HIP_OK(hipMemset(d_count, 0, 8));
    HIP_OK(hipMalloc((void**)&d_lr, 8));
    HIP_OK(hipDeviceSynchronize());

    /* capture one capturable step, its learning rate read from d_lr */
    fsdp_adamw_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.01, 1};
    const double schedule[REPLAYS] = {2.5e-4, 5e-4, 1e-3, 7.5e-4};
    hipGraph_t graph;
    hipGraphExec_t exec;
    HIP_OK(hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal));
    FSDP_OK_OR_FAIL(fsdp_mt_step_capturable(plan_b, &hp, d_count, d_lr, stream));
    HIP_OK(hipStreamEndCapture(stream, &graph));
    HIP_OK(hipGraphInstantiate(&exec, graph, NULL, NULL, 0));

    int bad = 0;
    for (int r = 1; r <= REPLAYS && !bad; ++r) {
        hp.step = r;
        hp.lr = schedule[r - 1];
        FSDP_OK_OR_FAIL(fsdp_mt_step(plan_a, &hp, stream));
        HIP_OK(hipMemcpyAsync(d_lr, &schedule[r - 1], 8, hipMemcpyHostToDevice, stream));
        HIP_OK(hipGraphLaunch(exec, stream));
        HIP_OK(hipStreamSynchronize(stream));
        int64_t count = -1;
        HIP_OK(hipMemcpy(&count, d_count, 8, hipMemcpyDeviceToHost));
        if (count != r) {
            fprintf(stderr, "replay %d: device count %lld\n", r, (long long)count);
            bad = 1;
        }
        for (int i = 0; i < NSHARDS; ++i) {
            const size_t n = (size_t)S[i];
            if (!same_bytes(c[0].p[i], c[1].p[i], n * 4, h1, h2) ||
                !same_bytes(c[0].m[i], c[1].m[i], n * 4, h1, h2) ||
                !same_bytes(c[0].v[i], c[1].v[i], n * 4, h1, h2) ||
                !same_bytes(c[0].out[i], c[1].out[i], n * 2, h1, h2)) {
                fprintf(stderr, "replay %d: shard %d differs from the eager step\n", r, i);
                bad = 1;
            }
        }
    }
    HIP_OK(hipGraphExecDestroy(exec));
    HIP_OK(hipGraphDestroy(graph));
    FSDP_OK_OR_FAIL(fsdp_mt_plan_destroy(plan_a));
    FSDP_OK_OR_FAIL(fsdp_mt_plan_destroy(plan_b));
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipStreamDestroy(stream));
    for (int i = 0; i < NSHARDS; ++i) {
        (void)hipFree(d_sl[i]);
        for (int a = 0; a < 2; ++a) {
            (void)hipFree(c[a].p[i]);
            (void)hipFree(c[a].m[i]);
            (void)hipFree(c[a].v[i]);
            (void)hipFree(c[a].out[i]);
        }
    }
    (void)hipFree(d_count);
    (void)hipFree(d_lr);
    free(h1);
    free(h2);
    if (bad) return 1;
    printf("graph_from_c: ok\n");
    return 0;
}
