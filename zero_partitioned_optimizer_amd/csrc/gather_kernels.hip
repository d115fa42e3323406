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
// tasks of kGatherChunk output elements (kSmallChunk in calls too small to fill
// the chip), so a launch has about one task per 16 KB of bf16 output whatever
// the tensor sizes; pieces whose source and
// destination share their 16-byte alignment move as 16-byte vectors, others
// element by element (still coalesced); outputs go through the caches when the
// call's outputs fit in the Infinity Cache and past them otherwise. The tensor
// table travels in the kernel argument block, sized to the call's shard count
// (a table of 8, 64 or 256 shard pointers, then as many tensors as the rest of
// the 4 KB block holds: 143, 127 or 72), so a model's fetch takes few launches,
// each with its own fill and tail.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_internal.h"

namespace zk {

constexpr int64_t kGatherChunk = 8192;                  // output elements per task
constexpr int64_t kSmallChunk = 4096;                   // ... in calls too small to fill the chip
constexpr int64_t kSmallCallTasks = 2048;               // tasks of kGatherChunk below which a
                                                        // call takes tasks of kSmallChunk
constexpr int64_t kGatherMaxTasks = int64_t(1) << 20;   // workgroups per gather launch
constexpr int kArgBytes = 4096;                         // the kernel argument block

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One launch's arguments for calls over at most NSH shards: the header and the
// shard table, then per tensor its flat offset, length, output and first task
// (the prefix sum of the task counts, relative to the launch's group; the
// entries past the group's last tensor, up to kTensors, all hold its total).
template <int NSH>
struct GatherArgs {
    static constexpr int kHead = 8 * NSH + 24;
    static constexpr int kTensors = (kArgBytes - kHead - 4) / 28;
    const void* shard[NSH];
    int64_t S;
    double inv_S;                             // 1 / S, rounded once
    int64_t task_base;                        // task of workgroup 0 of this launch
    int64_t offset[kTensors];
    int64_t numel[kTensors];
    void* out[kTensors];
    int32_t first_task[kTensors + 1];
};
static_assert(sizeof(GatherArgs<8>) <= kArgBytes && sizeof(GatherArgs<64>) <= kArgBytes &&
                  sizeof(GatherArgs<kGatherMaxShards>) <= kArgBytes,
              "the gather arguments fit the kernel argument block");
static_assert(GatherArgs<kGatherMaxShards>::kTensors >= 64, "at least one lane's worth of tensors");

// 16-byte store: nontemporal (NTS, past the caches) or plain (allocating in them).
template <bool NTS>
__device__ __forceinline__ void st16(u32x4* p, u32x4 v) {
    if constexpr (NTS) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// len elements from src to dst by the whole workgroup. Each lane issues up to
// four 16-byte loads before its stores, so a full task (16 KB of bf16) is one
// round of loads in flight per lane.
template <typename E, bool NTS>
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
            st16<NTS>(d4 + k, a);
            st16<NTS>(d4 + k + kBlock, b);
            st16<NTS>(d4 + k + 2 * kBlock, c);
            st16<NTS>(d4 + k + 3 * kBlock, d);
        }
        for (; k < nv; k += kBlock) st16<NTS>(d4 + k, __builtin_nontemporal_load(s4 + k));
        done = h + nv * V;
    }
    for (int64_t k = done + threadIdx.x; k < len; k += kBlock) dst[k] = src[k];
}

template <typename E, int NSH, bool NTS, int64_t CHUNK>
__global__ void __launch_bounds__(kBlock) k_gather(const GatherArgs<NSH> g) {
    constexpr int KT = GatherArgs<NSH>::kTensors;
    const int64_t task = g.task_base + blockIdx.x;
    // the task's tensor: the last t with first_task[t] <= task (first_task does
    // not decrease). Lane i of every wave reads entries i, i + 64, ..., and the
    // number of entries at or below the task, over the wave, is t + 1: one round
    // of loads whatever the tensor's position. The entries past the group hold
    // its total, which exceeds every task of the launch; the loads depend on
    // nothing but the lane, so that they are all in flight together.
    const int lane = threadIdx.x & 63;
    int32_t ft[(KT + 63) / 64];
#pragma unroll
    for (int i = 0; i < (KT + 63) / 64; ++i) {
        const int j = 64 * i + lane;
        ft[i] = g.first_task[j < KT ? j : KT];
    }
    int t = -1;
#pragma unroll
    for (int i = 0; i < (KT + 63) / 64; ++i) t += __popcll(__ballot((int64_t)ft[i] <= task));
    const int64_t n = g.numel[t];
    const int64_t e0 = (task - g.first_task[t]) * CHUNK;
    const int64_t e1 = e0 + CHUNK < n ? e0 + CHUNK : n;
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
        copy_piece<E, NTS>(static_cast<const E*>(g.shard[r]) + off, out + e, len);
        e += len;
    }
}

template <int NSH, bool NTS, int64_t CHUNK>
static hipError_t gather_groups(const void* const* shards, int32_t n_shards, int64_t S,
                                int32_t elem_bytes, const int64_t* offsets, const int64_t* numels,
                                void* const* outs, int32_t n_tensors, hipStream_t st) {
    constexpr int KT = GatherArgs<NSH>::kTensors;
    GatherArgs<NSH> g{};
    for (int r = 0; r < NSH; ++r) g.shard[r] = r < n_shards ? shards[r] : nullptr;
    g.S = S;
    g.inv_S = 1.0 / (double)S;
    for (int32_t base = 0; base < n_tensors; base += KT) {
        const int32_t k = n_tensors - base < KT ? n_tensors - base : KT;
        int64_t tasks = 0;
        for (int32_t i = 0; i < k; ++i) {
            g.offset[i] = offsets[base + i];
            g.numel[i] = numels[base + i];
            g.out[i] = outs[base + i];
            g.first_task[i] = (int32_t)tasks;
            tasks += (g.numel[i] + CHUNK - 1) / CHUNK;
            // a group's tasks are counted in 32 bits (2^31 tasks: 16T elements)
            if (tasks > INT32_MAX) return hipErrorInvalidValue;
        }
        for (int32_t i = k; i <= KT; ++i) g.first_task[i] = (int32_t)tasks;
        // at most kGatherMaxTasks workgroups (8G elements) per launch; a group
        // with more tasks takes several launches over consecutive task ranges
        for (int64_t t0 = 0; t0 < tasks; t0 += kGatherMaxTasks) {
            const int64_t n = tasks - t0 < kGatherMaxTasks ? tasks - t0 : kGatherMaxTasks;
            g.task_base = t0;
            if (elem_bytes == 2)
                hipLaunchKernelGGL((k_gather<uint16_t, NSH, NTS, CHUNK>), dim3((unsigned)n), dim3(kBlock), 0,
                                   st, g);
            else
                hipLaunchKernelGGL((k_gather<uint32_t, NSH, NTS, CHUNK>), dim3((unsigned)n), dim3(kBlock), 0,
                                   st, g);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

template <bool NTS, int64_t CHUNK>
static hipError_t gather_by_shards(const void* const* shards, int32_t n_shards, int64_t S,
                                   int32_t elem_bytes, const int64_t* offsets, const int64_t* numels,
                                   void* const* outs, int32_t n_tensors, hipStream_t st) {
    if (n_shards <= 8)
        return gather_groups<8, NTS, CHUNK>(shards, n_shards, S, elem_bytes, offsets, numels, outs,
                                            n_tensors, st);
    if (n_shards <= 64)
        return gather_groups<64, NTS, CHUNK>(shards, n_shards, S, elem_bytes, offsets, numels, outs,
                                             n_tensors, st);
    return gather_groups<kGatherMaxShards, NTS, CHUNK>(shards, n_shards, S, elem_bytes, offsets, numels,
                                                       outs, n_tensors, st);
}

// A call whose outputs fit in the 256 MB Infinity Cache stores them through the
// caches, where the layer that reads them right after finds them; a larger one
// could not keep them there and streams them past the caches, which leaves the
// cache to the other traffic (Llama-7B layer 139 -> 127 us, model 4.72 -> 4.56
// ms; a GPT-2 layer or model keeps the cached stores).
constexpr int64_t kCachedOutBytes = int64_t(256) << 20;

// A call of fewer than kSmallCallTasks tasks (a layer of a small model: GPT-2
// small's 865) leaves most of the 256 compute units' slots empty; tasks of half
// the size double its workgroups (GPT-2 layers in turn 8.6 -> 8.1 us). Larger
// calls keep the full tasks, with which they run faster (GPT-2 model 78 against
// 82 us with half tasks, Llama-7B layer 127 against 129 us).
hipError_t launch_gather(const void* const* shards, int32_t n_shards, int64_t S, int32_t elem_bytes,
                         const int64_t* offsets, const int64_t* numels, void* const* outs,
                         int32_t n_tensors, hipStream_t st) {
    int64_t out_bytes = 0, tasks = 0;
    for (int32_t k = 0; k < n_tensors && out_bytes <= kCachedOutBytes; ++k) {
        out_bytes += numels[k] * elem_bytes;
        tasks += (numels[k] + kGatherChunk - 1) / kGatherChunk;
    }
    if (out_bytes > kCachedOutBytes)
        return gather_by_shards<true, kGatherChunk>(shards, n_shards, S, elem_bytes, offsets, numels, outs,
                                                    n_tensors, st);
    if (tasks < kSmallCallTasks)
        return gather_by_shards<false, kSmallChunk>(shards, n_shards, S, elem_bytes, offsets, numels, outs,
                                                    n_tensors, st);
    return gather_by_shards<false, kGatherChunk>(shards, n_shards, S, elem_bytes, offsets, numels, outs,
                                                 n_tensors, st);
}

}  // namespace zk
