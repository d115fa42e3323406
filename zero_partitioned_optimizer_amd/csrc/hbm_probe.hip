// hbm_probe.hip -- achievable HBM bandwidth of plain streams on this GPU, for
// context beside the step kernel's roofline: read-only, write-only, copy, and
// k:1 read:write mixes (2:1 is the step's mix at N = 8 with bf16 replicas,
// 28 B read : 14 B written per element; 5:1 is near its mix at N = 32).
// Every kernel streams dwordx4 with nontemporal hints over 1 GiB buffers (or the
// size in MiB given as the first argument) from a grid-stride loop with a bounds
// check on every access.
//
// Given a shard size S and a replica count N as well, it also times a stream of
// the fused step's own shape at that size: N bf16 replica reads (dwordx2), three
// fp32 reads and three fp32 writes (dwordx4) and one bf16 write (dwordx2) per
// quad, one quad per lane and one trip per workgroup, with trivial arithmetic;
// once with p, m, v as three arrays per state set and once with each set one
// buffer of 8192-element tiles [p | m | v] (the step's two state layouts).
//
// All buffers hold pseudo-random small normal values, not zeros: streams of
// zeros run measurably faster on this part, and the step's data is not zero.
// Prints one JSON object.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u2 __attribute__((ext_vector_type(2)));

constexpr int kB = 256;

__device__ __forceinline__ uint32_t mix32(uint64_t i, uint32_t seed) {
    uint32_t x = (uint32_t)i * 2654435761u ^ (uint32_t)(i >> 32) ^ seed;
    x ^= x >> 15;
    x *= 2246822519u;
    x ^= x >> 13;
    return x;
}

// n 32-bit words of values in +-[0.5, 1): every 16-bit half is such a bf16, and
// every word such an fp32.
__global__ void __launch_bounds__(kB) k_fill(uint32_t* __restrict__ p, int64_t n, uint32_t seed) {
    const int64_t stride = (int64_t)gridDim.x * kB;
    for (int64_t i = (int64_t)blockIdx.x * kB + threadIdx.x; i < n; i += stride)
        p[i] = (mix32((uint64_t)i, seed) & 0x807f807fu) | 0x3f003f00u;
}

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
    for (int64_t i = (int64_t)blockIdx.x * kB + threadIdx.x; i < n4; i += stride) {
        const uint32_t h = (mix32((uint64_t)i, 7u) & 0x807f807fu) | 0x3f003f00u;
        const float x = __uint_as_float(h);
        __builtin_nontemporal_store(f4{x, x + 1.f, x + 2.f, x + 3.f}, dst + i);
    }
}

// The step's shape: quad q of this lane, one trip per workgroup. TILED: p, m, v
// point at one set buffer (m, v one and two 2048-quad sections after p) and the
// quad's state index is (q / 2048) * 6144 + q % 2048.
template <bool TILED>
__global__ void __launch_bounds__(kB) k_step_shape(const u2* const* __restrict__ rep, int n_rep,
                                                 const f4* __restrict__ p, const f4* __restrict__ m,
                                                 const f4* __restrict__ v, f4* __restrict__ po,
                                                 f4* __restrict__ mo, f4* __restrict__ vo,
                                                 u2* __restrict__ slot, int64_t nq) {
    const int64_t q = (int64_t)blockIdx.x * kB + threadIdx.x;
    if (q >= nq) return;
    const int64_t s = TILED ? (q >> 11) * 6144 + (q & 2047) : q;
    const f4 a = __builtin_nontemporal_load(p + s);
    const f4 b = __builtin_nontemporal_load(m + s);
    const f4 c = __builtin_nontemporal_load(v + s);
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < n_rep; j += 8) {
        u2 r[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) r[k] = __builtin_nontemporal_load(rep[j + k < n_rep ? j + k : j] + q);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (j + k < n_rep) {
                acc.x += __uint_as_float(r[k].x << 16);
                acc.y += __uint_as_float(r[k].x & 0xffff0000u);
                acc.z += __uint_as_float(r[k].y << 16);
                acc.w += __uint_as_float(r[k].y & 0xffff0000u);
            }
        }
    }
    __builtin_nontemporal_store(a + acc, po + s);
    __builtin_nontemporal_store(b * acc, mo + s);
    __builtin_nontemporal_store(c - acc, vo + s);
    const f4 n = a - acc;
    u2 w;
    w.x = (__float_as_uint(n.x) >> 16) | (__float_as_uint(n.y) & 0xffff0000u);
    w.y = (__float_as_uint(n.z) >> 16) | (__float_as_uint(n.w) & 0xffff0000u);
    __builtin_nontemporal_store(w, slot + q);
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
    // optional arguments: MiB per buffer (default 1024; six buffers are
    // allocated), then shard size S (a multiple of 4) and replica count N for the
    // step-shaped stream
    int64_t mib = argc > 1 ? atoll(argv[1]) : 1024;
    const int64_t shape_S = argc > 3 ? atoll(argv[2]) : 0;
    const int shape_N = argc > 3 ? atoi(argv[3]) : 0;
    if (argc > 3 && (shape_S < 4 || shape_S % 4 != 0 || shape_S > (int64_t(1) << 32) ||
                     shape_N < 1 || shape_N > 256)) {
        fprintf(stderr, "hbm_probe: S must be a positive multiple of 4 up to 2^32 and N in [1, 256]\n");
        return 1;
    }
    if (mib < 16) mib = 16;
    if (mib > 16384) mib = 16384;
    const int64_t bytes = mib << 20;
    const int64_t n4 = bytes / 16;
    const int kMaxK = 5;
    f4* buf[kMaxK + 1];
    uint32_t seed = 1;
    for (auto& b : buf) {
        CK(hipMalloc(&b, bytes));
        hipLaunchKernelGGL(k_fill, 4096, kB, 0, 0, reinterpret_cast<uint32_t*>(b), bytes / 4, seed++);
    }
    CK(hipGetLastError());
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
    for (auto& p : buf) CK(hipFree(p));
    const double b = (double)bytes;
    printf("{\"unit\": \"GB/s\", \"buffer_bytes\": %lld, \"grid\": %d, \"data\": \"random\", "
           "\"read\": %.1f, \"write\": %.1f, \"copy\": %.1f, \"mix_2to1\": %.1f, \"mix_5to1\": %.1f",
           (long long)bytes, grid, b / t_read / 1e9, b / t_write / 1e9, 2 * b / t_copy / 1e9,
           3 * b / t_mix2 / 1e9, 6 * b / t_mix5 / 1e9);
    if (shape_S > 0) {
        // N replicas of S bf16, p/m/v in and out (fp32), one bf16 slot
        const int64_t nq = shape_S / 4;
        std::vector<u2*> reps((size_t)shape_N, nullptr);
        for (auto& r : reps) {
            CK(hipMalloc(&r, shape_S * 2));
            hipLaunchKernelGGL(k_fill, 4096, kB, 0, 0, reinterpret_cast<uint32_t*>(r), shape_S / 2, seed++);
        }
        f4* st[6];
        for (auto& x : st) {
            CK(hipMalloc(&x, shape_S * 4));
            hipLaunchKernelGGL(k_fill, 4096, kB, 0, 0, reinterpret_cast<uint32_t*>(x), shape_S, seed++);
        }
        u2* slot;
        CK(hipMalloc(&slot, shape_S * 2));
        const u2** rtab;
        CK(hipMalloc(&rtab, sizeof(u2*) * shape_N));
        CK(hipMemcpy(rtab, reps.data(), sizeof(u2*) * shape_N, hipMemcpyHostToDevice));
        CK(hipGetLastError());
        // tiled state sets: 3 * S rounded up to whole 8192-element tiles, in floats
        const int64_t tiled_floats = 3 * ((shape_S + 8191) / 8192) * 8192;
        f4* ts[2];
        for (auto& x : ts) {
            CK(hipMalloc(&x, tiled_floats * 4));
            hipLaunchKernelGGL(k_fill, 4096, kB, 0, 0, reinterpret_cast<uint32_t*>(x), tiled_floats, seed++);
        }
        CK(hipGetLastError());
        const int64_t sgrid = (nq + kB - 1) / kB;
        const double t_shape = time_it([&] {
            hipLaunchKernelGGL(k_step_shape<false>, dim3((unsigned)sgrid), kB, 0, 0, rtab, shape_N, st[0],
                               st[1], st[2], st[3], st[4], st[5], slot, nq);
        });
        const double t_tiled = time_it([&] {
            hipLaunchKernelGGL(k_step_shape<true>, dim3((unsigned)sgrid), kB, 0, 0, rtab, shape_N, ts[0],
                               ts[0] + 2048, ts[0] + 4096, ts[1], ts[1] + 2048, ts[1] + 4096, slot, nq);
        });
        CK(hipGetLastError());
        CK(hipDeviceSynchronize());
        const double sb = (double)shape_S * (2.0 * shape_N + 26.0);
        printf(", \"step_shape\": {\"shard_elems\": %lld, \"n_replicas\": %d, \"bytes\": %.0f, "
               "\"us\": %.2f, \"gbps\": %.1f}",
               (long long)shape_S, shape_N, sb, t_shape * 1e6, sb / t_shape / 1e9);
        printf(", \"step_shape_tiled\": {\"us\": %.2f, \"gbps\": %.1f}", t_tiled * 1e6,
               sb / t_tiled / 1e9);
        for (auto& r : reps) CK(hipFree(r));
        for (auto& x : st) CK(hipFree(x));
        for (auto& x : ts) CK(hipFree(x));
        CK(hipFree(slot));
        CK(hipFree(rtab));
    }
    printf("}\n");
    CK(hipFree(srcs));
    CK(hipFree(sink));
    return 0;
}
