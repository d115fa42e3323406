/*
 * A plain C11 consumer of libzero's host-side ABI: no Python, no torch, no GPU.
 * Builds a layout, reads it back through every accessor (with the capacity
 * protocol), checks the memory accounting against the page formulas
 * ("ZeRO Optimizer", "Theoretical Reductions"), the commit rule, and that every
 * device entry point rejects bad arguments before it would launch anything.
 * Exit status 0 on success; prints the first failed check otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "zero.h"

static int fails = 0;
#define CHECK(c)                                                                   \
    do {                                                                           \
        if (!(c)) {                                                                \
            fprintf(stderr, "check failed at line %d: %s (%s)\n", __LINE__, #c,    \
                    zero_last_error());                                            \
            fails++;                                                               \
        }                                                                          \
    } while (0)

/* a 16-byte aligned address that is never dereferenced: every call below fails
   validation before any device access */
#define FAKE ((uintptr_t)1 << 40)

int main(void) {
    CHECK(strncmp(zero_version(), "libzero", 7) == 0);

    const int64_t numels[3] = {1000, 2048, 1000};
    zero_layout* L = NULL;
    CHECK(zero_layout_build(numels, 3, 2, 1, 8, &L) == ZERO_OK && L != NULL);
    zero_layout_info info;
    CHECK(zero_layout_info_get(L, &info) == ZERO_OK);
    CHECK(info.n_tensors == 3 && info.psi == 4048 && info.used_L == 4048);
    CHECK(info.shard_S == 2024 && info.padded_L == 4048 && info.world_N == 2);
    int64_t off[3];
    CHECK(zero_layout_offsets(L, off) == ZERO_OK && off[0] == 0 && off[1] == 1000 && off[2] == 3048);

    int64_t n = -1;
    CHECK(zero_layout_segments(L, 1, NULL, 0, &n) == ZERO_OK && n == 2);
    zero_segment seg[2];
    zero_segment one[1];
    CHECK(zero_layout_segments(L, 1, one, 1, &n) == ZERO_E_RANGE && n == 2);
    CHECK(zero_layout_segments(L, 1, seg, 2, &n) == ZERO_OK);
    CHECK(seg[0].tensor == 1 && seg[0].tensor_off == 1024 && seg[0].shard_off == 0 && seg[0].len == 1024);
    CHECK(seg[1].tensor == 2 && seg[1].tensor_off == 0 && seg[1].shard_off == 1024 && seg[1].len == 1000);
    CHECK(zero_layout_segments(L, 2, seg, 2, &n) == ZERO_E_RANGE);

    zero_bucket bk[8];
    CHECK(zero_layout_buckets(L, 1, 512, bk, 8, &n) == ZERO_OK && n == 4);
    CHECK(bk[0].shard_off == 0 && bk[0].len == 512 && bk[0].tensor == 1);
    CHECK(bk[2].shard_off == 1024 && bk[2].len == 512 && bk[2].tensor == 2);
    CHECK(bk[3].shard_off == 1536 && bk[3].len == 488);
    CHECK(sizeof(zero_bucket) == 16 && sizeof(zero_stats) == 16);

    int64_t v[4];
    const int64_t P = info.padded_L, S = info.shard_S;
    CHECK(zero_layout_mem_values(L, 0, v) == ZERO_OK && v[3] == 4 * P);
    CHECK(zero_layout_mem_values(L, 1, v) == ZERO_OK && v[3] == 2 * P + 2 * S);
    CHECK(zero_layout_mem_values(L, 2, v) == ZERO_OK && v[3] == P + 3 * S);
    CHECK(zero_layout_mem_values(L, 3, v) == ZERO_OK && v[3] == 4 * S);
    CHECK(zero_layout_mem_bytes(L, 2, v) == ZERO_OK && v[3] == 2 * P + 14 * S);
    CHECK(zero_layout_mem_values(L, 7, v) == ZERO_E_INVAL);
    zero_layout_free(L);

    CHECK(zero_layout_build(numels, 3, 0, 1, 8, &L) == ZERO_E_INVAL);
    const int64_t neg[2] = {4, -1};
    CHECK(zero_layout_build(neg, 2, 2, 1, 8, &L) == ZERO_E_INVAL);
    CHECK(zero_layout_build(numels, 3, 2, 1, 8, NULL) == ZERO_E_INVAL);

    /* the commit rule */
    zero_train_state ts = {0, 0, 65536.0, 1.0, 1, 0};
    zero_stats clean = {0u, 0u, 1.0}, bad = {1u, 0u, 0.0};
    CHECK(zero_commit_rule(&ts, &clean) == ZERO_COMMIT && ts.t == 1);
    CHECK(zero_commit_rule(&ts, &bad) == ZERO_SKIP && ts.t == 1 && ts.loss_scale == 32768.0);
    CHECK(ts.n_skipped == 1);
    CHECK(zero_commit_rule(NULL, &bad) == ZERO_E_INVAL);

    /* device entry points: argument checks only */
    const size_t ws = zero_workspace_bytes(64);
    CHECK(ws >= 24);
    const void* reps[2] = {(const void*)FAKE, (const void*)(FAKE + 4096)};
    CHECK(zero_reduce_shard(reps, 2, ZERO_BF16, 64, NULL, 0, 0.0, NULL, (zero_stats*)(FAKE + 8192),
                            (void*)(FAKE + 12288), ws, NULL) == ZERO_E_INVAL);       /* loss scale 0 */
    CHECK(zero_reduce_shard(reps, 0, ZERO_BF16, 64, NULL, 0, 1.0, NULL, (zero_stats*)(FAKE + 8192),
                            (void*)(FAKE + 12288), ws, NULL) == ZERO_E_RANGE);
    zero_adam_args a;
    memset(&a, 0, sizeof(a));
    a.replicas = reps;
    a.n_replicas = 2;
    a.grad_dtype = ZERO_BF16;
    a.p_in = a.p_out = (float*)(FAKE + 16384);                /* aliased: fused must be out of place */
    a.m_in = (const float*)(FAKE + 20480);
    a.m_out = (float*)(FAKE + 24576);
    a.v_in = (const float*)(FAKE + 28672);
    a.v_out = (float*)(FAKE + 32768);
    a.shard_S = 64;
    a.lr = 1e-3; a.beta1 = 0.9; a.beta2 = 0.999; a.eps = 1e-8; a.loss_scale = 1.0; a.step_t = 1;
    a.stats_dev = (zero_stats*)(FAKE + 8192);
    a.workspace_dev = (void*)(FAKE + 12288);
    a.ws_bytes = ws;
    CHECK(zero_adam_step(&a, NULL) == ZERO_E_INVAL);
    a.p_out = (float*)(FAKE + 16384 + 4);
    CHECK(zero_adam_step(&a, NULL) == ZERO_E_ALIGN);
    CHECK(zero_adam_step(NULL, NULL) == ZERO_E_INVAL);

    zero_train_args t;
    memset(&t, 0, sizeof(t));
    t.replicas = reps;
    t.n_replicas = 2;
    t.grad_dtype = ZERO_BF16;
    t.shard_S = 64;
    t.p[0] = t.p[1] = (float*)(FAKE + 16384);                 /* the two sets alias */
    t.m[0] = (float*)(FAKE + 20480); t.m[1] = (float*)(FAKE + 24576);
    t.v[0] = (float*)(FAKE + 28672); t.v[1] = (float*)(FAKE + 32768);
    t.lr = 1e-3; t.eps = 1e-8;
    t.state_dev = (zero_device_state*)(FAKE + 36864);
    t.stats_dev = (zero_stats*)(FAKE + 8192);
    t.workspace_dev = (void*)(FAKE + 12288);
    t.ws_bytes = ws;
    CHECK(zero_train_step(&t, NULL) == ZERO_E_INVAL);
    CHECK(zero_device_state_init(NULL, (void*)(FAKE + 12288), ws, 0.9, 0.999, 1.0, 1.0, 0, NULL) == ZERO_E_INVAL);
    CHECK(zero_gather_slot((const float*)FAKE, 64, (uint16_t*)(FAKE + 8), NULL) == ZERO_E_ALIGN);

    if (fails) return 1;
    printf("abi_host ok\n");
    return 0;
}
