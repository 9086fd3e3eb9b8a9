/* A plain C consumer of librank_step.so: includes the header as C, calls the
 * host-only layout entry point for the 4-tensor MLP at N=4 on every rank and
 * prints the views and summaries as JSON lines; then checks that a bad
 * argument comes back as FSDP_E_ARG with a message.  No device is needed. */
#include <stdio.h>
#include <string.h>

#include "fsdp_step.h"

int main(void) {
    const fsdp_tensor_shape shapes[4] = {
        {256 * 256, 256, FSDP_DT_F32, 0},
        {256, 256, FSDP_DT_F32, 0},
        {1024 * 256, 1024, FSDP_DT_F32, 0},
        {256 * 1024, 256, FSDP_DT_F32, 0},
    };
    for (int mode = FSDP_LAYOUT_FLAT; mode <= FSDP_LAYOUT_OWNER; ++mode) {
        for (int r = 0; r < 4; ++r) {
            fsdp_shard_view v[4];
            fsdp_layout_summary s;
            const int32_t st = fsdp_shard_layout(mode, 4, r, shapes, 4, 0, v, &s);
            if (st != FSDP_OK) {
                printf("{\"error\": %d}\n", st);
                return 1;
            }
            printf("{\"mode\": %d, \"rank\": %d, \"views\": [", mode, r);
            for (int i = 0; i < 4; ++i)
                printf("%s[%lld, %lld, %lld, %lld, %lld, %lld, %lld]", i ? ", " : "",
                       (long long)v[i].shard_numel, (long long)v[i].valid, (long long)v[i].global_offset,
                       (long long)v[i].view_offset, (long long)v[i].view_numel,
                       (long long)v[i].tensor_offset, (long long)v[i].owner);
            printf("], \"summary\": [%lld, %lld, %lld, %lld, %lld, %lld, %lld, %lld, %lld]}\n",
                   (long long)s.logical_numel, (long long)s.physical_numel, (long long)s.shard_numel,
                   (long long)s.pad_numel, (long long)s.bytes_param, (long long)s.bytes_grad,
                   (long long)s.bytes_optim, (long long)s.bytes_master, (long long)s.bytes_grad_unsharded);
        }
    }
    fsdp_shard_view v[4];
    fsdp_layout_summary s;
    const int32_t bad = fsdp_shard_layout(FSDP_LAYOUT_FLAT, 4, 4, shapes, 4, 0, v, &s);
    printf("{\"bad_rank\": %d, \"message\": %d}\n", bad, (int)(strlen(fsdp_last_error()) > 0));
    return 0;
}
