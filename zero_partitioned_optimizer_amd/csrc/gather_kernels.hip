// gather_kernels.hip -- the stage-3 fetch: copy whole tensors out of the rank
// shards of the flat parameter buffer into contiguous temporaries, before the
// layer that uses them ("ZeRO Optimizer", "ZeRO Stages" stage 3 and
// "Communication Patterns": parameters are all-gathered before each layer,
// only the required subset). Tensor t occupies [o_t, o_t + n_t) of the flat
// buffer and rank r holds [r*S, (r+1)*S) of it, so each tensor is at most a few
// contiguous pieces, one per rank it touches. On one GPU the N shards are
// resident buffers (in a multi-GPU build: the peers' shards mapped over xGMI).
//
// Pure copy, HBM-bound (2 x element bytes per element): workgroups take fixed
// tasks of kGatherChunk output elements, so a launch has about one task per
// 16 KB of bf16 output whatever the tensor sizes; pieces whose source and
// destination share their 16-byte alignment move as 16-byte vectors, others
// element by element (still coalesced). Up to kGatherTensors tensors go into one
// launch (as many as the kernel argument block holds), so a model's fetch takes
// few launches, each with its own tail.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_internal.h"

namespace zk {

constexpr int kGatherTensors = 48;                      // tensors per launch
constexpr int64_t kGatherChunk = 8192;                  // output elements per task
constexpr int64_t kGatherMaxTasks = int64_t(1) << 20;   // workgroups per gather launch

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct GatherParams {
    const void* shard[kGatherMaxShards];
    int64_t S;
    double inv_S;                             // 1 / S, rounded once
    int32_t n_tensors;
    int32_t reserved;
    int64_t offset[kGatherTensors];
    int64_t numel[kGatherTensors];
    void* out[kGatherTensors];
    int64_t first_task[kGatherTensors + 1];   // prefix sums of the tensors' task counts
    int64_t task_base;                        // task of workgroup 0 of this launch
};
static_assert(sizeof(GatherParams) <= 4096, "the gather arguments fit the kernel argument block");

// len elements from src to dst by the whole workgroup. Each lane issues up to
// four 16-byte loads before its stores, so a full task (16 KB of bf16) is one
// round of loads in flight per lane.
template <typename E>
__device__ __forceinline__ void copy_piece(const E* __restrict__ src, E* __restrict__ dst,
                                           int64_t len) {
    constexpr int64_t V = 16 / sizeof(E);
    const uintptr_t sa = reinterpret_cast<uintptr_t>(src), da = reinterpret_cast<uintptr_t>(dst);
    int64_t done = 0;
    if (((sa ^ da) & 15u) == 0) {
        int64_t h = (int64_t)(((16u - (sa & 15u)) & 15u) / sizeof(E));
        if (h > len) h = len;
        for (int64_t k = threadIdx.x; k < h; k += kBlock) dst[k] = src[k];
        const int64_t nv = (len - h) / V;
        const u32x4* __restrict__ s4 = reinterpret_cast<const u32x4*>(src + h);
        u32x4* __restrict__ d4 = reinterpret_cast<u32x4*>(dst + h);
        int64_t k = threadIdx.x;
        for (; k + 3 * kBlock < nv; k += 4 * kBlock) {
            const u32x4 a = __builtin_nontemporal_load(s4 + k);
            const u32x4 b = __builtin_nontemporal_load(s4 + k + kBlock);
            const u32x4 c = __builtin_nontemporal_load(s4 + k + 2 * kBlock);
            const u32x4 d = __builtin_nontemporal_load(s4 + k + 3 * kBlock);
            d4[k] = a;
            d4[k + kBlock] = b;
            d4[k + 2 * kBlock] = c;
            d4[k + 3 * kBlock] = d;
        }
        for (; k < nv; k += kBlock) d4[k] = __builtin_nontemporal_load(s4 + k);
        done = h + nv * V;
    }
    for (int64_t k = done + threadIdx.x; k < len; k += kBlock) dst[k] = src[k];
}

template <typename E>
__global__ void __launch_bounds__(kBlock) k_gather(const GatherParams g) {
    const int64_t task = g.task_base + blockIdx.x;
    // the task's tensor: the last t with first_task[t] <= task (first_task does
    // not decrease). Lane i of every wave reads entry i, and the number of entries
    // at or below the task, over the wave, is t + 1: one round of loads whatever
    // the tensor's position, where a scan of the entries takes up to 47 in a row.
    static_assert(kGatherTensors <= 64, "one entry per lane");
    const int lane = threadIdx.x & 63;
    const int64_t ft = lane < g.n_tensors ? g.first_task[lane] : INT64_MAX;
    const int t = __popcll(__ballot(ft <= task)) - 1;
    const int64_t n = g.numel[t];
    const int64_t e0 = (task - g.first_task[t]) * kGatherChunk;
    const int64_t e1 = e0 + kGatherChunk < n ? e0 + kGatherChunk : n;
    E* out = static_cast<E*>(g.out[t]);
    const int64_t f = g.offset[t] + e0;
    // rank r = floor(f / S) from the reciprocal (within one of it for any f below
    // 2^51), then corrected: no 64-bit division
    int64_t r = (int64_t)((double)f * g.inv_S);
    if (r * g.S > f) --r;
    else if ((r + 1) * g.S <= f) ++r;
    int64_t off = f - r * g.S;
    for (int64_t e = e0; e < e1; ++r, off = 0) {
        const int64_t rest = g.S - off;
        const int64_t len = e1 - e < rest ? e1 - e : rest;
        copy_piece<E>(static_cast<const E*>(g.shard[r]) + off, out + e, len);
        e += len;
    }
}

hipError_t launch_gather(const void* const* shards, int32_t n_shards, int64_t S, int32_t elem_bytes,
                         const int64_t* offsets, const int64_t* numels, void* const* outs,
                         int32_t n_tensors, hipStream_t st) {
    GatherParams g{};
    for (int r = 0; r < kGatherMaxShards; ++r) g.shard[r] = r < n_shards ? shards[r] : nullptr;
    g.S = S;
    g.inv_S = S > 0 ? 1.0 / (double)S : 0.0;
    for (int32_t base = 0; base < n_tensors; base += kGatherTensors) {
        const int32_t k = n_tensors - base < kGatherTensors ? n_tensors - base : kGatherTensors;
        g.n_tensors = k;
        g.first_task[0] = 0;
        for (int32_t i = 0; i < k; ++i) {
            g.offset[i] = offsets[base + i];
            g.numel[i] = numels[base + i];
            g.out[i] = outs[base + i];
            g.first_task[i + 1] = g.first_task[i] + (g.numel[i] + kGatherChunk - 1) / kGatherChunk;
        }
        const int64_t tasks = g.first_task[k];
        // at most kGatherMaxTasks workgroups (8G elements) per launch; a group
        // with more tasks takes several launches over consecutive task ranges
        for (int64_t t0 = 0; t0 < tasks; t0 += kGatherMaxTasks) {
            const int64_t n = tasks - t0 < kGatherMaxTasks ? tasks - t0 : kGatherMaxTasks;
            g.task_base = t0;
            if (elem_bytes == 2)
                hipLaunchKernelGGL(k_gather<uint16_t>, dim3((unsigned)n), dim3(kBlock), 0, st, g);
            else
                hipLaunchKernelGGL(k_gather<uint32_t>, dim3((unsigned)n), dim3(kBlock), 0, st, g);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace zk
