// hbm_probe.hip -- achievable HBM bandwidth of plain streams on this GPU, for
// context beside the step kernel's roofline: read-only, write-only, copy, and
// k:1 read:write mixes (2:1 is the step's mix at N = 8 with bf16 replicas,
// 28 B read : 14 B written per element; 5:1 is near its mix at N = 32).
// Every kernel streams dwordx4 with nontemporal hints over 1 GiB buffers (or the
// size in MiB given as the argument) from a
// grid-stride loop with a bounds check on every access. Prints one JSON object.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kB = 256;

// K reads of independent buffers and (W = 1) one write, or (W = 0) none.
template <int K, int W>
__global__ void __launch_bounds__(kB) k_mix(const f4* const* __restrict__ src, f4* __restrict__ dst,
                                          int64_t n4, float* sink) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    const int64_t stride = (int64_t)gridDim.x * kB * 2;
    for (int64_t i = (int64_t)blockIdx.x * kB * 2 + threadIdx.x; i < n4; i += stride) {
        f4 v[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t j = i + u * kB;
            if (j < n4) {
#pragma unroll
                for (int k = 0; k < K; ++k) v[u] += __builtin_nontemporal_load(src[k] + j);
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t j = i + u * kB;
            if (W && j < n4) __builtin_nontemporal_store(v[u], dst + j);
            acc += v[u];
        }
    }
    if (!W && acc.x == 1234.5f) sink[blockIdx.x] = acc.y;
}

__global__ void __launch_bounds__(kB) k_write(f4* __restrict__ dst, int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * kB;
    for (int64_t i = (int64_t)blockIdx.x * kB + threadIdx.x; i < n4; i += stride)
        __builtin_nontemporal_store(f4{1.f, 2.f, 3.f, 4.f}, dst + i);
}

#define CK(x)                                                                              \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            fprintf(stderr, "hbm_probe: %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 1;                                                                      \
        }                                                                                  \
    } while (0)

int main(int argc, char** argv) {
    // optional argument: MiB per buffer (default 1024; six buffers are allocated)
    int64_t mib = argc > 1 ? atoll(argv[1]) : 1024;
    if (mib < 16) mib = 16;
    if (mib > 16384) mib = 16384;
    const int64_t bytes = mib << 20;
    const int64_t n4 = bytes / 16;
    const int kMaxK = 5;
    f4* buf[kMaxK + 1];
    for (auto& b : buf) {
        CK(hipMalloc(&b, bytes));
        CK(hipMemset(b, 0, bytes));
    }
    const f4** srcs;
    CK(hipMalloc(&srcs, sizeof(f4*) * kMaxK));
    CK(hipMemcpy(srcs, buf, sizeof(f4*) * kMaxK, hipMemcpyHostToDevice));
    float* sink;
    CK(hipMalloc(&sink, sizeof(float) * 65536));
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    const int grid = 16384;
    auto time_it = [&](auto launch) -> double {
        for (int w = 0; w < 2; ++w) launch();
        std::vector<float> ts;
        for (int r = 0; r < 9; ++r) {
            hipEventRecord(e0);
            launch();
            hipEventRecord(e1);
            hipEventSynchronize(e1);
            float ms = 0.f;
            hipEventElapsedTime(&ms, e0, e1);
            ts.push_back(ms);
        }
        std::sort(ts.begin(), ts.end());
        return ts[ts.size() / 2] * 1e-3;
    };
    f4* dst = buf[kMaxK];
    const double t_read = time_it([&] { hipLaunchKernelGGL((k_mix<1, 0>), grid, kB, 0, 0, srcs, dst, n4, sink); });
    const double t_write = time_it([&] { hipLaunchKernelGGL(k_write, grid, kB, 0, 0, dst, n4); });
    const double t_copy = time_it([&] { hipLaunchKernelGGL((k_mix<1, 1>), grid, kB, 0, 0, srcs, dst, n4, sink); });
    const double t_mix2 = time_it([&] { hipLaunchKernelGGL((k_mix<2, 1>), grid, kB, 0, 0, srcs, dst, n4, sink); });
    const double t_mix5 = time_it([&] { hipLaunchKernelGGL((k_mix<5, 1>), grid, kB, 0, 0, srcs, dst, n4, sink); });
    CK(hipGetLastError());
    CK(hipDeviceSynchronize());
    const double b = (double)bytes;
    printf("{\"unit\": \"GB/s\", \"buffer_bytes\": %lld, \"grid\": %d, \"read\": %.1f, \"write\": %.1f, "
           "\"copy\": %.1f, \"mix_2to1\": %.1f, \"mix_5to1\": %.1f}\n",
           (long long)bytes, grid, b / t_read / 1e9, b / t_write / 1e9, 2 * b / t_copy / 1e9,
           3 * b / t_mix2 / 1e9, 6 * b / t_mix5 / 1e9);
    for (auto& p : buf) CK(hipFree(p));
    CK(hipFree(srcs));
    CK(hipFree(sink));
    return 0;
}
