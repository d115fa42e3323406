// offload.cpp -- the host side of a step whose optimizer state lives in host
// memory ("ZeRO Optimizer", "Advanced Optimizations", ZeRO-Offload: the
// optimizer states move to CPU memory, and GPU-CPU transfers are balanced
// against the work). The GPU folds the gradient replicas (zero_reduce_shard);
// the averaged fp32 gradient crosses to the host in chunks; host threads run
// Adam/AdamW on each chunk as it lands and send its bf16 values back while the
// next chunks are still crossing.
//
// The host update is the device's operation sequence, one IEEE fp32 operation
// per source operation (the library is built with -ffp-contract=off; x86 vector
// division and square root are correctly rounded), so it matches zero_adam_step
// bit for bit. The loop is compiled for AVX-512, AVX2 and baseline x86-64 and
// the loader picks the widest one the CPU has.
#include <hip/hip_runtime.h>
#include <sched.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <thread>
#include <vector>

#include "zero.h"
#include "zero_internal.h"

namespace {

using zl::set_error;

constexpr int kMaxThreads = 256;
constexpr int64_t kDefaultChunk = int64_t(1) << 20;

// Adam / AdamW over n elements, in place, optionally with the bf16 slot.
__attribute__((target_clones("avx512f", "avx2", "default"))) void adam_span(
    const float* __restrict g, float* __restrict p, float* __restrict m, float* __restrict v,
    uint16_t* __restrict slot, int64_t n, const zk::Scalars s) {
    const float b1 = s.b1, b2 = s.b2, omb1 = s.omb1, omb2 = s.omb2;
    const float bc1 = s.bc1, bc2 = s.bc2, lr = s.lr, eps = s.eps, decay = s.decay;
    for (int64_t i = 0; i < n; ++i) {
        const float gi = g[i];
        const float mt = b1 * m[i];
        const float mg = omb1 * gi;
        const float m1 = mt + mg;
        const float gg = gi * gi;
        const float vt = b2 * v[i];
        const float vg = omb2 * gg;
        const float v1 = vt + vg;
        const float mh = m1 / bc1;
        const float vh = v1 / bc2;
        const float den = __builtin_elementwise_sqrt(vh) + eps;
        const float u = mh / den;
        const float p1 = p[i] * decay;
        const float lu = lr * u;
        const float pn = p1 - lu;
        m[i] = m1;
        v[i] = v1;
        p[i] = pn;
        if (slot) {
            uint32_t w;
            memcpy(&w, &pn, 4);
            // round to nearest even; any NaN becomes the quiet NaN 0x7FC0
            slot[i] = (w & 0x7fffffffu) > 0x7f800000u
                          ? (uint16_t)0x7fc0u
                          : (uint16_t)((w + 0x7fffu + ((w >> 16) & 1u)) >> 16);
        }
    }
}

// Worker threads: as requested, else one per CPU this process may run on.
int thread_count(int32_t requested, int64_t work_items) {
    int t = requested;
    if (t <= 0) {
        cpu_set_t set;
        CPU_ZERO(&set);
        t = sched_getaffinity(0, sizeof(set), &set) == 0 ? CPU_COUNT(&set)
                                                          : (int)std::thread::hardware_concurrency();
    }
    if (t < 1) t = 1;
    if (t > kMaxThreads) t = kMaxThreads;
    if ((int64_t)t > work_items) t = (int)(work_items > 0 ? work_items : 1);
    return t;
}

bool finite_in(double x, double lo, double hi) { return x == x && x >= lo && x < hi; }
bool finite_nonneg(double x) { return x == x && x >= 0 && x < 1e308; }

int check_hyper(const char* fn, double lr, double beta1, double beta2, double eps, double wd,
                int64_t t) {
    if (!finite_in(beta1, 0.0, 1.0) || !finite_in(beta2, 0.0, 1.0) || !finite_nonneg(lr) ||
        !finite_nonneg(eps) || !finite_nonneg(wd) || t < 1) {
        set_error("%s: lr=%g beta1=%g beta2=%g eps=%g weight_decay=%g step_t=%lld out of domain",
                  fn, lr, beta1, beta2, eps, wd, (long long)t);
        return ZERO_E_INVAL;
    }
    return ZERO_OK;
}

}  // namespace

extern "C" {

int zero_host_adam(const zero_host_adam_args* args) {
    static const char* fn = "zero_host_adam";
    if (!args) {
        set_error("%s: args is NULL", fn);
        return ZERO_E_INVAL;
    }
    const zero_host_adam_args& a = *args;
    if (a.n < 0) {
        set_error("%s: n=%lld is negative", fn, (long long)a.n);
        return ZERO_E_RANGE;
    }
    if (a.n > 0 && (!a.g || !a.p || !a.m || !a.v)) {
        set_error("%s: g, p, m or v is NULL", fn);
        return ZERO_E_INVAL;
    }
    int rc = check_hyper(fn, a.lr, a.beta1, a.beta2, a.eps, a.weight_decay, a.step_t);
    if (rc) return rc;
    if (a.n == 0) return ZERO_OK;
    const zk::Scalars s = zl::update_scalars(a.lr, a.beta1, a.beta2, a.eps, a.weight_decay,
                                             a.step_t);
    // contiguous stripes of at least 64K elements, one per thread
    const int T = thread_count(a.nthreads, (a.n + 65535) / 65536);
    std::vector<std::thread> pool;
    for (int k = 0; k < T; ++k) {
        const int64_t lo = a.n * k / T, hi = a.n * (k + 1) / T;
        auto run = [&a, &s, lo, hi] {
            adam_span(a.g + lo, a.p + lo, a.m + lo, a.v + lo, a.slot_bf16 ? a.slot_bf16 + lo : nullptr,
                      hi - lo, s);
        };
        if (k == T - 1) run();
        else pool.emplace_back(run);
    }
    for (auto& th : pool) th.join();
    return ZERO_OK;
}

int zero_offload_step(const zero_offload_args* args, void* stream, zero_stats* stats_out) {
    static const char* fn = "zero_offload_step";
    if (!args) {
        set_error("%s: args is NULL", fn);
        return ZERO_E_INVAL;
    }
    const zero_offload_args& a = *args;
    const int64_t S = a.shard_S;
    if (!a.state || !a.stats_dev) {
        set_error("%s: state or stats_dev is NULL", fn);
        return ZERO_E_INVAL;
    }
    if (S > 0 && (!a.g_dev || !a.g_host || !a.p_host || !a.m_host || !a.v_host || !a.slot_host ||
                  !a.slot_dev)) {
        set_error("%s: a gradient, state or slot buffer is NULL", fn);
        return ZERO_E_INVAL;
    }
    if (a.chunk_elems < 0) {
        set_error("%s: chunk_elems=%lld is negative", fn, (long long)a.chunk_elems);
        return ZERO_E_RANGE;
    }
    int rc = check_hyper(fn, a.lr, a.beta1, a.beta2, a.eps, a.weight_decay, a.state->t + 1);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipStream_t up = a.stream_h2d ? static_cast<hipStream_t>(a.stream_h2d) : st;

    // 1. fold, average, flag and norm on the GPU; the stats come back first
    rc = zero_reduce_shard(a.replicas, a.n_replicas, a.grad_dtype, S, nullptr, 0,
                           a.state->loss_scale, a.g_dev, a.stats_dev, a.workspace_dev, a.ws_bytes,
                           stream);
    if (rc) return rc;
    zero_stats stats{};
    rc = zl::hip_error(hipMemcpyAsync(&stats, a.stats_dev, sizeof(stats), hipMemcpyDeviceToHost, st),
                       fn);
    if (rc) return rc;
    rc = zl::hip_error(hipStreamSynchronize(st), fn);
    if (rc) return rc;
    if (stats_out) *stats_out = stats;

    // 2. overflow: skip
    if (stats.overflow) return zero_commit_rule(a.state, &stats);

    // 3. chunks cross to the host in order; host threads update them as they land
    const int64_t C = a.chunk_elems > 0 ? a.chunk_elems : kDefaultChunk;
    const int64_t n_chunks = (S + C - 1) / C;
    std::vector<hipEvent_t> ev((size_t)n_chunks, nullptr);
    int err = ZERO_OK;
    for (int64_t c = 0; c < n_chunks && !err; ++c) {
        const int64_t lo = c * C, len = (S - lo) < C ? (S - lo) : C;
        err = zl::hip_error(hipEventCreateWithFlags(&ev[c], hipEventDisableTiming), fn);
        if (!err)
            err = zl::hip_error(hipMemcpyAsync(a.g_host + lo, a.g_dev + lo, (size_t)len * 4,
                                               hipMemcpyDeviceToHost, st),
                                fn);
        if (!err) err = zl::hip_error(hipEventRecord(ev[c], st), fn);
    }
    if (!err) {
        const zk::Scalars s = zl::update_scalars(a.lr, a.beta1, a.beta2, a.eps, a.weight_decay,
                                                 a.state->t + 1);
        // Every thread takes its stripe of every chunk, chunk after chunk; the
        // thread that finishes a chunk's last stripe sends that chunk's bf16 values
        // up. A chunk is thus updated by all threads as soon as it lands, and its
        // upload overlaps the next chunks' copies and updates.
        const int T = thread_count(a.nthreads, (C + 16383) / 16384);
        std::vector<std::atomic<int>> left((size_t)n_chunks);
        for (auto& x : left) x.store(T);
        std::atomic<int> first_err{(int)hipSuccess};   // a hipError_t; the text is set below
        auto worker = [&](int k) {
            for (int64_t c = 0; c < n_chunks; ++c) {
                if (first_err.load() != (int)hipSuccess) return;
                const int64_t lo = c * C, len = (S - lo) < C ? (S - lo) : C;
                // stripes of whole 16-element groups, so stripes never split a cache line
                const int64_t groups = (len + 15) / 16;
                const int64_t a0 = lo + 16 * (groups * k / T);
                const int64_t a1 = k == T - 1 ? lo + len : lo + 16 * (groups * (k + 1) / T);
                hipError_t e = hipEventSynchronize(ev[c]);
                if (e == hipSuccess && a1 > a0)
                    adam_span(a.g_host + a0, a.p_host + a0, a.m_host + a0, a.v_host + a0,
                              a.slot_host + a0, a1 - a0, s);
                if (e == hipSuccess && left[c].fetch_sub(1) == 1)
                    e = hipMemcpyAsync(a.slot_dev + lo, a.slot_host + lo, (size_t)len * 2,
                                       hipMemcpyHostToDevice, up);
                if (e != hipSuccess) {
                    int expected = (int)hipSuccess;
                    first_err.compare_exchange_strong(expected, (int)e);
                    return;
                }
            }
        };
        std::vector<std::thread> pool;
        for (int k = 0; k + 1 < T; ++k) pool.emplace_back(worker, k);
        worker(T - 1);
        for (auto& th : pool) th.join();
        err = zl::hip_error((hipError_t)first_err.load(), fn);
    }
    // drain both streams before the events go and before the caller reuses g_host / slot_host
    const int e1 = zl::hip_error(hipStreamSynchronize(st), fn);
    const int e2 = up != st ? zl::hip_error(hipStreamSynchronize(up), fn) : ZERO_OK;
    for (hipEvent_t e : ev)
        if (e) (void)hipEventDestroy(e);
    if (err) return err;
    if (e1) return e1;
    if (e2) return e2;
    return zero_commit_rule(a.state, &stats);
}

}  // extern "C"
