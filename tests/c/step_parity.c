/*
 * A plain C11 program that drives the device-commit step through libzero's ABI
 * and the HIP runtime's C API only (no Python, no torch), and checks it against
 * the CPU oracle's C entry point (or_step, test infrastructure) bit for bit:
 * three steps of a ragged shard (S = 100003, N = 8 bf16 replicas, AdamW), the
 * second with an injected +inf that must be skipped.
 * Inputs come from a splitmix64 stream local to this test.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero.h"

/* the oracle's C entry point (oracle/oracle.c) */
int or_step(const void* const* reps, int32_t N, int32_t dtype, int64_t n, double loss_scale, float* p,
            float* m, float* v, uint16_t* slot, double lr, double beta1, double beta2, double eps,
            double wd, int64_t t, double* sumsq_out, int32_t nthreads);
uint16_t or_f32_to_bf16(float x);

#define HIPCK(x)                                                                     \
    do {                                                                             \
        hipError_t e_ = (x);                                                         \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 2;                                                                \
        }                                                                            \
    } while (0)
#define ZCK(x)                                                                       \
    do {                                                                             \
        int r_ = (x);                                                                \
        if (r_ != ZERO_OK) {                                                         \
            fprintf(stderr, "libzero error %d at line %d: %s\n", r_, __LINE__, zero_last_error()); \
            return 3;                                                                \
        }                                                                            \
    } while (0)

static uint64_t sm_state = 0x5eed5eed5eedULL;
static uint64_t splitmix64(void) {
    uint64_t z = (sm_state += 0x9E3779B97F4A7C15ULL);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}
/* a bf16 pattern with random sign, exponent in [2^-17, 2^-2), random mantissa */
static uint16_t rand_bf16(void) {
    uint64_t r = splitmix64();
    uint16_t sign = (uint16_t)((r & 1u) << 15);
    uint16_t exp = (uint16_t)(110u + (r >> 1) % 15u);
    uint16_t man = (uint16_t)((r >> 8) & 0x7Fu);
    return (uint16_t)(sign | (exp << 7) | man);
}
static float rand_param(void) {
    uint64_t r = splitmix64();
    uint32_t sign = (uint32_t)(r & 1u) << 31;
    uint32_t exp = 118u + (uint32_t)((r >> 1) % 6u);
    uint32_t man = (uint32_t)(r >> 16) & 0x7FFFFFu;
    uint32_t u = sign | (exp << 23) | man;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

enum { S = 100003, N = 8, STEPS = 3 };

int main(void) {
    const double lr = 1e-3, b1 = 0.9, b2 = 0.999, eps = 1e-8, wd = 0.01, ls = 1.0;
    static uint16_t reps_h[STEPS][N][S];
    static float p_h[S], m_h[S], v_h[S];
    static uint16_t slot_h[S];
    for (int s = 0; s < STEPS; ++s)
        for (int j = 0; j < N; ++j)
            for (int i = 0; i < S; ++i) reps_h[s][j][i] = rand_bf16();
    reps_h[1][5][777] = 0x7F80;                                 /* +inf on the second step */
    for (int i = 0; i < S; ++i) {
        p_h[i] = rand_param();
        m_h[i] = v_h[i] = 0.0f;
        slot_h[i] = or_f32_to_bf16(p_h[i]);
    }

    /* device buffers */
    void* reps_d[STEPS][N];
    for (int s = 0; s < STEPS; ++s)
        for (int j = 0; j < N; ++j) {
            HIPCK(hipMalloc(&reps_d[s][j], sizeof(uint16_t) * S));
            HIPCK(hipMemcpy(reps_d[s][j], reps_h[s][j], sizeof(uint16_t) * S, hipMemcpyHostToDevice));
        }
    float *p_d[2], *m_d[2], *v_d[2];
    uint16_t* slot_d[2];
    for (int k = 0; k < 2; ++k) {
        HIPCK(hipMalloc((void**)&p_d[k], sizeof(float) * S));
        HIPCK(hipMalloc((void**)&m_d[k], sizeof(float) * S));
        HIPCK(hipMalloc((void**)&v_d[k], sizeof(float) * S));
        HIPCK(hipMalloc((void**)&slot_d[k], sizeof(uint16_t) * S));
        HIPCK(hipMemset(m_d[k], 0, sizeof(float) * S));
        HIPCK(hipMemset(v_d[k], 0, sizeof(float) * S));
        HIPCK(hipMemset(p_d[k], 0, sizeof(float) * S));
    }
    HIPCK(hipMemcpy(p_d[0], p_h, sizeof(float) * S, hipMemcpyHostToDevice));
    zero_device_state* rec_d;
    zero_stats* stats_d;
    void* ws_d;
    const size_t ws = zero_workspace_bytes(S);
    HIPCK(hipMalloc((void**)&rec_d, 128));
    HIPCK(hipMalloc((void**)&stats_d, 16));
    HIPCK(hipMalloc(&ws_d, ws));
    ZCK(zero_gather_slot(p_d[0], S, slot_d[0], NULL));
    ZCK(zero_device_state_init(rec_d, ws_d, ws, b1, b2, ls, 1.0, 1, NULL));

    int64_t t_host = 0;
    int mismatch = 0;
    for (int s = 0; s < STEPS; ++s) {
        zero_train_args a;
        memset(&a, 0, sizeof(a));
        a.replicas = (const void* const*)reps_d[s];
        a.n_replicas = N;
        a.grad_dtype = ZERO_BF16;
        for (int k = 0; k < 2; ++k) {
            a.p[k] = p_d[k];
            a.m[k] = m_d[k];
            a.v[k] = v_d[k];
            a.slot[k] = slot_d[k];
        }
        a.shard_S = S;
        a.lr = lr; a.eps = eps; a.weight_decay = wd;
        a.state_dev = rec_d;
        a.stats_dev = stats_d;
        a.workspace_dev = ws_d;
        a.ws_bytes = ws;
        ZCK(zero_train_step(&a, NULL));
        ZCK(zero_device_state_flush(rec_d, stats_d, ws_d, ws, NULL));

        const void* hr[N];
        for (int j = 0; j < N; ++j) hr[j] = reps_h[s][j];
        double sumsq = 0.0;
        const int flag = or_step(hr, N, 1, S, ls, p_h, m_h, v_h, slot_h, lr, b1, b2, eps, wd, t_host + 1,
                                 &sumsq, 4);
        if (!flag) t_host++;

        HIPCK(hipDeviceSynchronize());
        zero_device_state rec;
        zero_stats st;
        HIPCK(hipMemcpy(&rec, rec_d, sizeof(rec), hipMemcpyDeviceToHost));
        HIPCK(hipMemcpy(&st, stats_d, sizeof(st), hipMemcpyDeviceToHost));
        if ((int)st.overflow != flag || rec.t != t_host || (int)rec.last_overflow != flag) {
            fprintf(stderr, "step %d: flag gpu %u oracle %d, t gpu %lld oracle %lld\n", s, st.overflow,
                    flag, (long long)rec.t, (long long)t_host);
            return 4;
        }
        if (!flag && fabs(st.sumsq - sumsq) > 1e-9 * sumsq) {
            fprintf(stderr, "step %d: sumsq gpu %.17g oracle %.17g\n", s, st.sumsq, sumsq);
            return 4;
        }
        static float p_g[S], m_g[S], v_g[S];
        static uint16_t slot_g[S];
        const int c = (int)(rec.cur & 1u);
        HIPCK(hipMemcpy(p_g, p_d[c], sizeof(float) * S, hipMemcpyDeviceToHost));
        HIPCK(hipMemcpy(m_g, m_d[c], sizeof(float) * S, hipMemcpyDeviceToHost));
        HIPCK(hipMemcpy(v_g, v_d[c], sizeof(float) * S, hipMemcpyDeviceToHost));
        HIPCK(hipMemcpy(slot_g, slot_d[c], sizeof(uint16_t) * S, hipMemcpyDeviceToHost));
        if (memcmp(p_g, p_h, sizeof(p_h)) || memcmp(m_g, m_h, sizeof(m_h)) ||
            memcmp(v_g, v_h, sizeof(v_h)) || memcmp(slot_g, slot_h, sizeof(slot_h))) {
            fprintf(stderr, "step %d: committed state differs from the oracle\n", s);
            mismatch = 1;
        }
        printf("step %d: flag %d, t %lld, sumsq %.6e, state bit-identical: %s\n", s, flag,
               (long long)rec.t, st.sumsq, mismatch ? "no" : "yes");
        fflush(stdout);
        if (mismatch) return 5;
    }
    for (int s = 0; s < STEPS; ++s)
        for (int j = 0; j < N; ++j) HIPCK(hipFree(reps_d[s][j]));
    for (int k = 0; k < 2; ++k) {
        HIPCK(hipFree(p_d[k])); HIPCK(hipFree(m_d[k])); HIPCK(hipFree(v_d[k])); HIPCK(hipFree(slot_d[k]));
    }
    HIPCK(hipFree(rec_d)); HIPCK(hipFree(stats_d)); HIPCK(hipFree(ws_d));
    printf("step_parity ok\n");
    return 0;
}
