// step_kernels.hip -- gfx950 kernels of the per-rank ZeRO stage-1/2 shard step.
//
// One pass over this rank's shard: fold the N gradient replicas in slot order
// (the ring order of the reduce-scatter walk in "Why DeepSpeed ZeRO paper says
// reduce-scatter (or all-gather) has data movement of Psi elements?",
// GuanhuaWang's reply), average and unscale, flag overflow and accumulate the
// squared norm, update fp32 master / m / v with Adam, and write the bf16 result
// into this rank's slot of the gathered parameter buffer ("[REQUEST] Direct
// Correspondence between Gradient and Optimizer States to Reduce
// Communication", "Problem").
//
// The work is pure streaming: (N * gradient bytes + 26) bytes per element against
// about 25 fp32 operations (three divisions and a square root among them), far
// under the fp32 vector ridge, so HBM bandwidth bounds it. There is no dense
// contraction and no MFMA. Design points:
//  - wave64 lanes each own one quad (4 consecutive elements) per row: bf16
//    replicas come in as dwordx2, fp32 state as dwordx4, so a wave reads 512 B
//    (bf16) or 1 KiB (fp32) contiguous per instruction;
//  - every lane issues its p/m/v loads and the first batch of up to 8 replica
//    loads (slots 0 .. 7) before the first add, then the remaining replicas in
//    batches of 8, each batch all in flight before its adds;
//  - one short workgroup per 1,024 elements (one quad per lane, one trip),
//    far more workgroups than are resident, so faster CUs take more of them
//    and the tail is one short workgroup; beyond kGridMax workgroups the grid
//    strides over the shard with the same number of trips per workgroup; small
//    shards are instead split evenly over a multiple of 256 workgroups;
//  - fp32 state as three arrays or in tiles of p | m | v (state_q, state_e);
//  - a bucket table confines the step to its buckets: one workgroup per bucket,
//    or, for a short table of long buckets, chunks of 1,024 elements dealt over
//    the grid; a quad cut by a bucket edge is loaded whole like the others and
//    masked to the bucket's elements;
//  - the flag and the fp64 squared norm are reduced with wave shuffles, then
//    LDS, then one partial per workgroup, summed in workgroup order (by a
//    one-workgroup finalize kernel, or, with the device commit, by workgroup 0
//    of the next launch on the record), so the norm is bit-reproducible; there
//    are no float atomics and no memsets;
//  - loads of data read once use the nontemporal hint, and so do the stores.
// Arithmetic is one IEEE fp32 operation per source operation, built with
// -ffp-contract=off; division and sqrt are the correctly rounded forms.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "zero_internal.h"

#ifndef ZERO_NT
#define ZERO_NT 1
#endif
#ifndef ZERO_WAVES_PER_EU
#define ZERO_WAVES_PER_EU 0
#endif
#if ZERO_WAVES_PER_EU > 0
#define ZERO_STEP_BOUNDS __launch_bounds__(kBlock, ZERO_WAVES_PER_EU)
#else
#define ZERO_STEP_BOUNDS __launch_bounds__(kBlock)
#endif

namespace zk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct KParams {
    const void* rep[kArgReplicas];          // replica pointers, slot order (up to kArgReplicas)
    const void* const* rep_ext;             // device table of all n_rep pointers (n_rep > kArgReplicas)
    int32_t n_rep;
    int32_t part_base;                      // device commit: partial slot of workgroup 0
    int32_t collect_n;                      // device commit: > 0: workgroup 0 folds the pending step
                                            // in, and this step (collect_n partials) becomes
                                            // pending; 0: a part before the last
    int32_t even_blocks;                    // whole shard: > 0: split evenly over this many
                                            // blocks of kEvenBlockQuads quads; bucket table:
                                            // > 0: buckets cut into chunks of kChunk elements
    int64_t S;
    const zero_bucket* buckets;
    int64_t n_buckets;
    const float* p_in;
    const float* m_in;
    const float* v_in;
    float* p_out;
    float* m_out;
    float* v_out;
    float* set_p[2];                        // device-commit path: both state sets
    float* set_m[2];
    float* set_v[2];
    const zero_device_state* ctrl;          // device-commit path: committed t, scale, set
    zero_device_state* ctrl_rw;             // the same record, written by workgroup 0 (commit)
    zero_stats* stats;
    uint16_t* set_slot[2];                  // device-commit path with a double-buffered slot
    uint16_t* slot;
    float* g_out;
    Partial* partials;
    uint64_t* ws_half[2];                   // device commit: tagged partials, by step number parity
    uint64_t* ws_started;                   // device commit: start marks, one per workgroup slot
    uint64_t* ws_flags;                     // device commit: overflow flag words, by step number parity
    Scalars sc;
};

// What one workgroup works with: the update's scalars and the in/out state.
struct Res {
    Scalars sc;
    const float* p_in;
    const float* m_in;
    const float* v_in;
    float* p_out;
    float* m_out;
    float* v_out;
    uint16_t* slot;                         // where the bf16 result goes, or nullptr
    uint32_t tag;                           // device-commit: number of this step
    uint64_t mark;                          // device-commit: start mark (tag, and a checksum of the
                                            // record words read, so it waits for all of them)
    uint32_t err;                           // device-commit: the record's sticky error code
};

// ---------------------------------------------------------------------------
// memory access
// ---------------------------------------------------------------------------

// Where quad q / element e of the fp32 state lives in a set's buffer. Split
// layout: p, m and v are three arrays indexed by element. Tiled layout: one
// array of tiles of kStateTile elements, each holding that range of p, then of
// m, then of v; the m and v bases are the p base plus one and two sections, so
// the same index serves all three.
template <bool TILED>
__device__ __forceinline__ int64_t state_q(int64_t q) {
    if constexpr (TILED)
        return (q >> kStateTileQuadsLog2) * (3 * kStateTileQuads) + (q & (kStateTileQuads - 1));
    else
        return q;
}
template <bool TILED>
__device__ __forceinline__ int64_t state_e(int64_t e) {
    if constexpr (TILED)
        return (e >> kStateTileLog2) * (3 * kStateTile) + (e & (kStateTile - 1));
    else
        return e;
}

template <typename T>
__device__ __forceinline__ T ld(const T* p) {
#if ZERO_NT
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

template <typename T>
__device__ __forceinline__ void st(T* p, T v) {
#if ZERO_NT
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

__device__ __forceinline__ float bf2f(uint32_t h16) { return __uint_as_float(h16 << 16); }

// fp32 -> bf16, round to nearest even; any NaN becomes 0x7FC0.
__device__ __forceinline__ uint32_t f2bf(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ bool nonfinite(float x) {
    return (__float_as_uint(x) & 0x7f800000u) == 0x7f800000u;
}

// x as a bf16 buffer holds it: rounded to nearest even, any NaN the quiet NaN.
__device__ __forceinline__ float hold_bf16(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return __uint_as_float(0x7fc00000u);
    return __uint_as_float((u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u);
}

// Replica element type tags: uint16_t (bf16), float, and WireBf16 -- bf16
// replicas whose running sum is held in bf16 after every add, as in a ring whose
// buffers and messages are bf16.
struct WireBf16 {};

// A quad (4 consecutive elements) of one gradient replica, widened to fp32, and
// one hop of the fold (add is fp32 except on the bf16 wire).
template <typename RT>
struct Quad;

template <>
struct Quad<uint16_t> {
    using V = u32x2;
    static __device__ __forceinline__ f32x4 add(f32x4 acc, f32x4 x) { return acc + x; }
    static __device__ __forceinline__ float add1(float acc, float x) { return acc + x; }
    static __device__ __forceinline__ V load(const void* base, int64_t q) {
        return ld(reinterpret_cast<const u32x2*>(base) + q);
    }
    static __device__ __forceinline__ f32x4 widen(V w) {
        f32x4 r;
        r.x = __uint_as_float(w.x << 16);
        r.y = __uint_as_float(w.x & 0xffff0000u);
        r.z = __uint_as_float(w.y << 16);
        r.w = __uint_as_float(w.y & 0xffff0000u);
        return r;
    }
    static __device__ __forceinline__ float one(const void* base, int64_t e) {
        return bf2f(reinterpret_cast<const uint16_t*>(base)[e]);
    }
};

template <>
struct Quad<WireBf16> : Quad<uint16_t> {
    static __device__ __forceinline__ f32x4 add(f32x4 acc, f32x4 x) {
        const f32x4 s = acc + x;
        return f32x4{hold_bf16(s.x), hold_bf16(s.y), hold_bf16(s.z), hold_bf16(s.w)};
    }
    static __device__ __forceinline__ float add1(float acc, float x) { return hold_bf16(acc + x); }
};

template <>
struct Quad<float> {
    using V = f32x4;
    static __device__ __forceinline__ f32x4 add(f32x4 acc, f32x4 x) { return acc + x; }
    static __device__ __forceinline__ float add1(float acc, float x) { return acc + x; }
    static __device__ __forceinline__ V load(const void* base, int64_t q) {
        return ld(reinterpret_cast<const f32x4*>(base) + q);
    }
    static __device__ __forceinline__ f32x4 widen(V w) { return w; }
    static __device__ __forceinline__ float one(const void* base, int64_t e) {
        return reinterpret_cast<const float*>(base)[e];
    }
};

// Where a launch finds replica pointer j: in its kernel arguments (up to
// kArgReplicas replicas), or, for a replica type wrapped in Ext, in a device table
// (more replicas than the argument block holds). Ext<T> folds exactly as T.
template <typename T>
struct Ext {};

template <typename T>
struct Quad<Ext<T>> : Quad<T> {};

template <typename RT>
struct Reps {
    static __device__ __forceinline__ const void* at(const KParams& a, int j) { return a.rep[j]; }
};

template <typename T>
struct Reps<Ext<T>> {
    static __device__ __forceinline__ const void* at(const KParams& a, int j) { return a.rep_ext[j]; }
};

// ---------------------------------------------------------------------------
// arithmetic
// ---------------------------------------------------------------------------

// Adam / AdamW on one element, one fp32 operation per line (no contraction).
__device__ __forceinline__ void adam1(float g, float p, float m, float v, const Scalars& s,
                                      float& pn, float& m1, float& v1) {
    const float mt = s.b1 * m;
    const float mg = s.omb1 * g;
    m1 = mt + mg;
    const float gg = g * g;
    const float vt = s.b2 * v;
    const float vg = s.omb2 * gg;
    v1 = vt + vg;
    const float mh = m1 / s.bc1;
    const float vh = v1 / s.bc2;
    const float den = sqrtf(vh) + s.eps;
    const float u = mh / den;
    const float p1 = p * s.decay;
    const float lu = s.lr * u;
    pn = p1 - lu;
}

// Load K replicas (slots j .. j+K-1) for ROWS quads, then add them in slot order.
template <typename RT, int ROWS, int K>
__device__ __forceinline__ void fold_batch(const KParams& a, int j, int64_t q0, int64_t qs,
                                           f32x4 (&acc)[ROWS]) {
    typename Quad<RT>::V buf[K][ROWS];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const void* base = Reps<RT>::at(a, j + k);
#pragma unroll
        for (int r = 0; r < ROWS; ++r) buf[k][r] = Quad<RT>::load(base, q0 + r * qs);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) acc[r] = Quad<RT>::add(acc[r], Quad<RT>::widen(buf[k][r]));
    }
}

// Slots 0 .. K-1 as the first batch: all K loads in flight, then acc = R_0 and
// R_1 .. R_{K-1} added in slot order.
template <typename RT, int ROWS, int K>
__device__ __forceinline__ void fold_head(const KParams& a, int64_t q0, int64_t qs,
                                          f32x4 (&acc)[ROWS]) {
    typename Quad<RT>::V buf[K][ROWS];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const void* base = Reps<RT>::at(a, k);
#pragma unroll
        for (int r = 0; r < ROWS; ++r) buf[k][r] = Quad<RT>::load(base, q0 + r * qs);
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r) acc[r] = Quad<RT>::widen(buf[0][r]);
#pragma unroll
    for (int k = 1; k < K; ++k) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) acc[r] = Quad<RT>::add(acc[r], Quad<RT>::widen(buf[k][r]));
    }
}

// acc = R_0 + R_1 + ... + R_{N-1}, left to right, for ROWS quads: slots 0 .. 7
// in one batch (with the state loads already issued, a lane's first memory
// round trip carries up to eight replica loads), then batches of 8 and the rest.
template <typename RT, int ROWS>
__device__ __forceinline__ void fold(const KParams& a, int64_t q0, int64_t qs, f32x4 (&acc)[ROWS]) {
    const int n = a.n_rep;
    switch (n < 8 ? n : 8) {
        case 8: fold_head<RT, ROWS, 8>(a, q0, qs, acc); break;
        case 7: fold_head<RT, ROWS, 7>(a, q0, qs, acc); break;
        case 6: fold_head<RT, ROWS, 6>(a, q0, qs, acc); break;
        case 5: fold_head<RT, ROWS, 5>(a, q0, qs, acc); break;
        case 4: fold_head<RT, ROWS, 4>(a, q0, qs, acc); break;
        case 3: fold_head<RT, ROWS, 3>(a, q0, qs, acc); break;
        case 2: fold_head<RT, ROWS, 2>(a, q0, qs, acc); break;
        default: fold_head<RT, ROWS, 1>(a, q0, qs, acc); break;
    }
    int j = 8;
    for (; j + 8 <= n; j += 8) fold_batch<RT, ROWS, 8>(a, j, q0, qs, acc);
    switch (n - j) {
        case 7: fold_batch<RT, ROWS, 7>(a, j, q0, qs, acc); break;
        case 6: fold_batch<RT, ROWS, 6>(a, j, q0, qs, acc); break;
        case 5: fold_batch<RT, ROWS, 5>(a, j, q0, qs, acc); break;
        case 4: fold_batch<RT, ROWS, 4>(a, j, q0, qs, acc); break;
        case 3: fold_batch<RT, ROWS, 3>(a, j, q0, qs, acc); break;
        case 2: fold_batch<RT, ROWS, 2>(a, j, q0, qs, acc); break;
        case 1: fold_batch<RT, ROWS, 1>(a, j, q0, qs, acc); break;
        default: break;
    }
}

// The first trip of workgroup bx in a grid of G. Consecutive workgroup indices
// are dispatched to the 8 XCDs in turn, so workgroup bx runs on XCD bx % 8 as
// its (bx / 8)-th: XCD x's l-th workgroup takes trip (l / K) * 8K + x*K + l % K,
// a permutation of the first 8 * floor(G / 8) trips (the last partial run
// shrinks K; the rest of the grid keeps its index). Each XCD then walks runs of
// K consecutive trips (K = 64: 128 KB of each bf16 replica) instead of every
// eighth trip: Llama-7B 1.6-2.9% faster, Llama-70B 0.3-0.4%, GPT-2 0-2%. The
// evenly split small launches permute their shares, and bucket launches their
// chunks or buckets, the same way.
constexpr int64_t kXcdRun = 64;
__device__ __forceinline__ int64_t xcd_trip(int64_t bx, int64_t G) {
    const int64_t L = G >> 3;
    if (bx >= 8 * L) return bx;
    const int64_t x = bx & 7, l = bx >> 3, full = L / kXcdRun, rem = L % kXcdRun;
    return l < full * kXcdRun ? (l / kXcdRun) * 8 * kXcdRun + x * kXcdRun + l % kXcdRun
                              : full * 8 * kXcdRun + x * rem + (l - full * kXcdRun);
}

// The first batch of a lane's replica quads (slots 0 .. min(N, 8) - 1) for its
// first quad, loaded before the committed-state record is read: the replica
// addresses do not depend on it, so with a cold cache the record's round trip
// and these loads overlap.
template <typename RT>
struct Head {
    typename Quad<RT>::V v[8];
};

template <typename RT>
__device__ __forceinline__ void head_load(const KParams& a, int64_t q, Head<RT>& h) {
    // fewer than 8 replicas: the spare loads repeat the last slot and are dropped
    const int n = a.n_rep;
#pragma unroll
    for (int k = 0; k < 8; ++k) h.v[k] = Quad<RT>::load(Reps<RT>::at(a, k < n ? k : n - 1), q);
}

// fold() for one quad whose first batch is already loaded.
template <typename RT>
__device__ __forceinline__ void fold_pre(const KParams& a, int64_t q0, const Head<RT>& h,
                                         f32x4 (&acc)[1]) {
    const int n = a.n_rep;
    acc[0] = Quad<RT>::widen(h.v[0]);
#pragma unroll
    for (int k = 1; k < 8; ++k)
        if (k < n) acc[0] = Quad<RT>::add(acc[0], Quad<RT>::widen(h.v[k]));
    int j = 8;
    for (; j + 8 <= n; j += 8) fold_batch<RT, 1, 8>(a, j, q0, 0, acc);
    switch (n - j > 0 ? n - j : 0) {
        case 7: fold_batch<RT, 1, 7>(a, j, q0, 0, acc); break;
        case 6: fold_batch<RT, 1, 6>(a, j, q0, 0, acc); break;
        case 5: fold_batch<RT, 1, 5>(a, j, q0, 0, acc); break;
        case 4: fold_batch<RT, 1, 4>(a, j, q0, 0, acc); break;
        case 3: fold_batch<RT, 1, 3>(a, j, q0, 0, acc); break;
        case 2: fold_batch<RT, 1, 2>(a, j, q0, 0, acc); break;
        case 1: fold_batch<RT, 1, 1>(a, j, q0, 0, acc); break;
        default: break;
    }
}

// Host-commit launches carry everything in the kernel arguments. Device-commit
// launches read the committed state's record: which state set is current, the
// loss scale and beta^t; each workgroup derives the update's scalars from it
// with the same double operations, rounded once to fp32, that the host uses.
// Relaxed agent-scope loads: coherent across XCDs, for words that other
// workgroups of the same launch write (partials, start marks).
__device__ __forceinline__ uint32_t rd32(const uint32_t* p) {
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t rd64(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double rdf64(const double* p) {
    return __longlong_as_double((long long)rd64(reinterpret_cast<const uint64_t*>(p)));
}
__device__ __forceinline__ uint32_t fold32(uint64_t x) { return (uint32_t)x ^ (uint32_t)(x >> 32); }
// The record's words are the same in every lane: keep them in scalar registers.
__device__ __forceinline__ uint32_t uni32(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint64_t uni64(uint64_t x) {
    return ((uint64_t)uni32((uint32_t)(x >> 32)) << 32) | uni32((uint32_t)x);
}

// Workgroup barrier for LDS traffic: every wave's LDS operations before it are
// done and visible to every wave after it. Unlike __syncthreads, whose workgroup
// fence also waits for each wave's outstanding global loads and stores, it lets
// the state and slot stores of a finished tile drain while the workgroup
// reduces its partial and ends.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The committed state as a launch sees it: the record (state after its `seq`
// finalized steps) with the pending step -- the one that ran after them, if
// pending_n > 0 -- folded in by the skip rule: a clean pending step advances the
// current set and beta^t, an overflowed one halves a dynamic loss scale. Every
// workgroup derives it from the same words, so all agree; workgroup 0 writes it
// back into the record later in the launch.
struct RecView {
    uint32_t seq, pend, cur, dynamic, err;
    uint64_t flag;                          // flag word of the pending step's parity
    double b1, b2, pow1, pow2, ls, min_ls;  // pow: beta^t of the committed t
    uint32_t sum;                           // checksum of every word read
};

// The record and the flag words are read with plain loads: what earlier
// launches wrote is visible at a launch's start (caches are written back and
// invalidated between launches), and within a launch workgroup 0 rewrites the
// record only after every workgroup has posted its start mark, whose value
// depends on every word read here, so no workgroup can see the new record.
__device__ __forceinline__ RecView read_record(const zero_device_state* c, const uint64_t* flags) {
    RecView v;
    v.seq = uni32(c->seq);
    v.pend = uni32(c->pending_n);
    v.cur = uni32(c->cur);
    v.dynamic = uni32(c->dynamic);
    v.err = uni32(c->error);
    const uint64_t b1 = uni64((uint64_t)__double_as_longlong(c->beta1));
    const uint64_t b2 = uni64((uint64_t)__double_as_longlong(c->beta2));
    const uint64_t p1 = uni64((uint64_t)__double_as_longlong(c->beta1_pow));
    const uint64_t p2 = uni64((uint64_t)__double_as_longlong(c->beta2_pow));
    const uint64_t ls = uni64((uint64_t)__double_as_longlong(c->loss_scale));
    const uint64_t ml = uni64((uint64_t)__double_as_longlong(c->min_loss_scale));
    // both flag words, so that neither load waits for seq
    const uint64_t f0 = uni64(flags[0]), f1 = uni64(flags[1]);
    v.flag = ((v.seq + 1u) & 1u) ? f1 : f0;
    v.b1 = __longlong_as_double((long long)b1);
    v.b2 = __longlong_as_double((long long)b2);
    v.pow1 = __longlong_as_double((long long)p1);
    v.pow2 = __longlong_as_double((long long)p2);
    v.ls = __longlong_as_double((long long)ls);
    v.min_ls = __longlong_as_double((long long)ml);
    v.sum = v.seq ^ v.pend ^ v.cur ^ v.dynamic ^ v.err ^ fold32(b1) ^ fold32(b2) ^ fold32(p1) ^ fold32(p2) ^
            fold32(ls) ^ fold32(ml) ^ fold32(v.flag);
    v.cur &= 1u;
    return v;
}

// Did the pending step overflow? Its workgroups that saw a non-finite gradient
// stored its number into the flag word of its parity; an older number there is
// a step two or more back.
__device__ __forceinline__ bool pending_overflow(const RecView& v) {
    return v.flag == (uint64_t)(v.seq + 1u);
}

// The skip rule applied to the pending step (the same operations as the
// zero_commit_rule of the host).
__device__ __forceinline__ void apply_pending(RecView& v) {
    if (!v.pend) return;
    if (!pending_overflow(v)) {
        v.cur ^= 1u;
        v.pow1 = v.pow1 * v.b1;
        v.pow2 = v.pow2 * v.b2;
    } else if (v.dynamic) {
        const double half = v.ls / 2.0;
        v.ls = half > v.min_ls ? half : v.min_ls;
    }
}

template <bool CTRL, bool TILED>
__device__ __forceinline__ Res resolve(const KParams& a) {
    Res r;
    r.sc = a.sc;
    if constexpr (!CTRL) {
        r.p_in = a.p_in;
        r.m_in = a.m_in;
        r.v_in = a.v_in;
        r.p_out = a.p_out;
        r.m_out = a.m_out;
        r.v_out = a.v_out;
        r.slot = a.slot;
        r.tag = 0u;
        r.mark = 0u;
        r.err = 0u;
    } else {
        RecView v = read_record(a.ctrl, a.ws_flags);
        const uint32_t tag = v.seq + (v.pend ? 2u : 1u);
        r.err = v.err;
        r.tag = tag;
        r.mark = ((uint64_t)tag << 32) | v.sum;
        apply_pending(v);
        const uint32_t cur = v.cur, nxt = cur ^ 1u;
        const double b1 = v.b1, b2 = v.b2;
        const double pow1 = v.pow1 * b1;            // beta^(t+1), one more factor of the product
        const double pow2 = v.pow2 * b2;
        r.sc.inv = (float)(1.0 / ((double)a.n_rep * v.ls));
        r.sc.b1 = (float)b1;
        r.sc.b2 = (float)b2;
        r.sc.omb1 = (float)(1.0 - b1);
        r.sc.omb2 = (float)(1.0 - b2);
        r.sc.bc1 = (float)(1.0 - pow1);
        r.sc.bc2 = (float)(1.0 - pow2);
        r.p_in = a.set_p[cur];
        r.m_in = a.set_m[cur];
        r.v_in = a.set_v[cur];
        r.p_out = a.set_p[nxt];
        r.m_out = a.set_m[nxt];
        r.v_out = a.set_v[nxt];
        // a double-buffered slot takes the candidate in the out buffer, like the state
        r.slot = a.set_slot[1] ? a.set_slot[nxt] : a.slot;
    }
    if constexpr (TILED) {
        // one buffer per set: m and v sit one and two sections after p in each tile
        r.m_in = r.p_in + kStateTile;
        r.v_in = r.p_in + 2 * kStateTile;
        r.m_out = r.p_out + kStateTile;
        r.v_out = r.p_out + 2 * kStateTile;
    }
    return r;
}

// The update of ROWS quads, held in registers until it is stored.
template <int ROWS>
struct Outs {
    f32x4 pn[ROWS], m1[ROWS], v1[ROWS];
};

// ROWS quads at q0, q0 + qs, ...: fold, average, flag, g^2 and (with ADAM) the
// update of 4*ROWS elements of this lane. Reduce-only launches store g here;
// the update is returned in `o` for quads_store. MASKED (one row): only the
// elements whose bits are set in `mask` (bit c: element 4*q0 + c) count towards
// the flag and g^2 and are stored; the others are loaded and computed, since the
// quad lies inside the shard's buffers, and dropped.
template <typename RT, bool ADAM, bool WRITE_G, bool TILED, int ROWS, bool MASKED = false>
__device__ __forceinline__ void quads_compute(const KParams& a, const Res& rs, int64_t q0,
                                              int64_t qs, double& sq, uint32_t& bad,
                                              Outs<ROWS>& o, uint32_t mask = 0xFu) {
    static_assert(!MASKED || ROWS == 1, "masked quads come one at a time");
    f32x4 p[ROWS], m[ROWS], v[ROWS];
    if constexpr (ADAM) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const int64_t q = state_q<TILED>(q0 + r * qs);
            p[r] = ld(reinterpret_cast<const f32x4*>(rs.p_in) + q);
            m[r] = ld(reinterpret_cast<const f32x4*>(rs.m_in) + q);
            v[r] = ld(reinterpret_cast<const f32x4*>(rs.v_in) + q);
        }
    }
    f32x4 acc[ROWS];
    fold<RT, ROWS>(a, q0, qs, acc);
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const int64_t q = q0 + r * qs;
        f32x4 g = acc[r] * rs.sc.inv;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool in = !MASKED || ((mask >> c) & 1u);
            bad |= (in && nonfinite(g[c])) ? 1u : 0u;
            const double gd = (double)g[c];
            sq += in ? gd * gd : 0.0;
        }
        if constexpr (WRITE_G) {
            if (!MASKED || mask == 0xFu) {
                st(reinterpret_cast<f32x4*>(a.g_out) + q, g);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if ((mask >> c) & 1u) a.g_out[q * 4 + c] = g[c];
            }
        }
        if constexpr (ADAM) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float x, y, z;
                adam1(g[c], p[r][c], m[r][c], v[r][c], rs.sc, x, y, z);
                o.pn[r][c] = x;
                o.m1[r][c] = y;
                o.v1[r][c] = z;
            }
        }
    }
}

template <bool TILED, int ROWS, bool MASKED = false>
__device__ __forceinline__ void quads_store(const Res& rs, int64_t q0, int64_t qs,
                                            const Outs<ROWS>& o, uint32_t mask = 0xFu) {
    if constexpr (MASKED) {
        if (mask != 0xFu) {
            // a quad cut by a bucket edge: its own elements one by one
            const int64_t qt = state_q<TILED>(q0);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (!((mask >> c) & 1u)) continue;
                rs.p_out[qt * 4 + c] = o.pn[0][c];
                rs.m_out[qt * 4 + c] = o.m1[0][c];
                rs.v_out[qt * 4 + c] = o.v1[0][c];
                if (rs.slot) rs.slot[q0 * 4 + c] = (uint16_t)f2bf(o.pn[0][c]);
            }
            return;
        }
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const int64_t q = q0 + r * qs;
        const int64_t qt = state_q<TILED>(q);
        st(reinterpret_cast<f32x4*>(rs.p_out) + qt, o.pn[r]);
        st(reinterpret_cast<f32x4*>(rs.m_out) + qt, o.m1[r]);
        st(reinterpret_cast<f32x4*>(rs.v_out) + qt, o.v1[r]);
        if (rs.slot) {
            u32x2 w;
            w.x = f2bf(o.pn[r].x) | (f2bf(o.pn[r].y) << 16);
            w.y = f2bf(o.pn[r].z) | (f2bf(o.pn[r].w) << 16);
            st(reinterpret_cast<u32x2*>(rs.slot) + q, w);
        }
    }
}

// The whole step for ROWS quads of this lane.
// quads() for one quad whose first replica batch is already loaded (MASKED: as
// in quads_compute, only the elements whose bits are set in `mask` count and are
// stored).
template <typename RT, bool ADAM, bool WRITE_G, bool TILED, bool MASKED = false>
__device__ __forceinline__ void quad_pre(const KParams& a, const Res& rs, int64_t q0,
                                         const Head<RT>& h, double& sq, uint32_t& bad,
                                         uint32_t mask = 0xFu) {
    f32x4 p[1], m[1], v[1];
    if constexpr (ADAM) {
        const int64_t q = state_q<TILED>(q0);
        p[0] = ld(reinterpret_cast<const f32x4*>(rs.p_in) + q);
        m[0] = ld(reinterpret_cast<const f32x4*>(rs.m_in) + q);
        v[0] = ld(reinterpret_cast<const f32x4*>(rs.v_in) + q);
    }
    f32x4 acc[1];
    fold_pre<RT>(a, q0, h, acc);
    f32x4 g[1];
    Outs<1> o;
    g[0] = acc[0] * rs.sc.inv;
    if constexpr (ADAM) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float x, y, z;
            adam1(g[0][c], p[0][c], m[0][c], v[0][c], rs.sc, x, y, z);
            o.pn[0][c] = x;
            o.m1[0][c] = y;
            o.v1[0][c] = z;
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const bool in = !MASKED || ((mask >> c) & 1u);
        bad |= (in && nonfinite(g[0][c])) ? 1u : 0u;
        const double gd = (double)g[0][c];
        sq += in ? gd * gd : 0.0;
    }
    if constexpr (WRITE_G) {
        if (!MASKED || mask == 0xFu) {
            st(reinterpret_cast<f32x4*>(a.g_out) + q0, g[0]);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if ((mask >> c) & 1u) a.g_out[q0 * 4 + c] = g[0][c];
        }
    }
    if constexpr (ADAM) quads_store<TILED, 1, MASKED>(rs, q0, 0, o, mask);
}

template <typename RT, bool ADAM, bool WRITE_G, bool TILED, int ROWS, bool MASKED = false>
__device__ __forceinline__ void quads(const KParams& a, const Res& rs, int64_t q0, int64_t qs,
                                      double& sq, uint32_t& bad, uint32_t mask = 0xFu) {
    Outs<ROWS> o;
    quads_compute<RT, ADAM, WRITE_G, TILED, ROWS, MASKED>(a, rs, q0, qs, sq, bad, o, mask);
    if constexpr (ADAM) quads_store<TILED, ROWS, MASKED>(rs, q0, qs, o, mask);
}

// One element, for the shard's last S % 4 elements (the buffers do not hold them
// as a whole quad).
template <typename RT, bool ADAM, bool WRITE_G, bool TILED>
__device__ __forceinline__ void one_elem(const KParams& a, const Res& rs, int64_t e, double& sq,
                                         uint32_t& bad) {
    // replica loads in batches of 8, all in flight before their adds (a spare load
    // repeats the batch's first slot and is dropped): a lane on the tail makes
    // N / 8 memory round trips, not N
    const int n = a.n_rep;
    float acc = Quad<RT>::one(Reps<RT>::at(a, 0), e);
    for (int j = 1; j < n; j += 8) {
        const int cnt = n - j < 8 ? n - j : 8;
        float x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = Quad<RT>::one(Reps<RT>::at(a, k < cnt ? j + k : j), e);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float s = Quad<RT>::add1(acc, x[k]);
            acc = k < cnt ? s : acc;
        }
    }
    const float g = acc * rs.sc.inv;
    bad |= nonfinite(g) ? 1u : 0u;
    const double gd = (double)g;
    sq += gd * gd;
    if constexpr (WRITE_G) a.g_out[e] = g;
    if constexpr (ADAM) {
        float pn, m1, v1;
        const int64_t es = state_e<TILED>(e);
        adam1(g, rs.p_in[es], rs.m_in[es], rs.v_in[es], rs.sc, pn, m1, v1);
        rs.p_out[es] = pn;
        rs.m_out[es] = m1;
        rs.v_out[es] = v1;
        if (rs.slot) rs.slot[e] = (uint16_t)f2bf(pn);
    }
}

// All elements of [lo, hi) by the threads of one workgroup, one quad per lane
// per round. A quad cut by an edge of the range goes through the same loads as
// the others, masked to the range's elements, so the lanes on the edges make the
// same memory round trips as the rest; only the shard's last partial quad (when
// S % 4 != 0), which the buffers do not hold whole, goes element by element.
// HEAD: the lane's first quad of the range, (lo >> 2) + threadIdx.x, has its first
// replica batch in `h` already (range_first_quad, when it is below range_qend).
__device__ __forceinline__ int64_t range_qend(const KParams& a, int64_t hi) {
    const int64_t qw = a.S >> 2;            // the shard's whole quads
    const int64_t qhi = (hi + 3) >> 2;      // one past the quad holding element hi - 1
    return qhi < qw ? qhi : qw;
}

__device__ __forceinline__ uint32_t edge_mask(int64_t q, int64_t lo, int64_t hi) {
    const int64_t e = q << 2;
    uint32_t mask = 0xFu;
    if (e < lo) mask &= 0xFu << (uint32_t)(lo - e);
    if (e + 4 > hi) mask &= 0xFu >> (uint32_t)(e + 4 - hi);
    return mask;
}

template <typename RT, bool ADAM, bool WRITE_G, bool TILED, bool HEAD = false>
__device__ __forceinline__ void range(const KParams& a, const Res& rs, int64_t lo, int64_t hi,
                                      double& sq, uint32_t& bad, const Head<RT>* h = nullptr) {
    if (lo >= hi) return;
    const int tid = threadIdx.x;
    const int64_t qw = a.S >> 2;
    const int64_t qhi = range_qend(a, hi);
    int64_t q = (lo >> 2) + tid;
    if constexpr (HEAD) {
        if (q < qhi) quad_pre<RT, ADAM, WRITE_G, TILED, true>(a, rs, q, *h, sq, bad, edge_mask(q, lo, hi));
        q += kBlock;
    }
    for (; q < qhi; q += kBlock)
        quads<RT, ADAM, WRITE_G, TILED, 1, true>(a, rs, q, 0, sq, bad, edge_mask(q, lo, hi));
    const int64_t et = qw << 2;
    for (int64_t e = (lo > et ? lo : et) + tid; e < hi; e += kBlock)
        one_elem<RT, ADAM, WRITE_G, TILED>(a, rs, e, sq, bad);
}

// Wave64 shuffles, then LDS across the workgroup's waves, in a fixed order.
__device__ __forceinline__ void block_reduce(double& sq, uint32_t& bad, uint32_t& badb) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        sq += __shfl_xor(sq, off, 64);
        bad |= __shfl_xor(bad, off, 64);
        badb += __shfl_xor(badb, off, 64);
    }
    constexpr int kWaves = kBlock / 64;
    __shared__ double s_sq[kWaves];
    __shared__ uint32_t s_bad[kWaves];
    __shared__ uint32_t s_badb[kWaves];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) {
        s_sq[w] = sq;
        s_bad[w] = bad;
        s_badb[w] = badb;
    }
    lds_barrier();
    if (threadIdx.x == 0) {
        double t = s_sq[0];
        uint32_t b = s_bad[0], bb = s_badb[0];
#pragma unroll
        for (int i = 1; i < kWaves; ++i) {
            t += s_sq[i];
            b |= s_bad[i];
            bb += s_badb[i];
        }
        sq = t;
        bad = b;
        badb = bb;
    }
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------

// Device commit. A launch does not commit its own step: every workgroup leaves
// its partial (three 64-bit words tagged with the step's number) in the
// workspace half of that number's parity, and one that finds a non-finite
// gradient stores the number into the flag word of that parity. The next launch
// on the record -- or zero_device_state_flush -- folds the step in: its
// workgroups all derive the committed state from the record and the flag word
// (apply_pending), and its workgroup 0 sums the pending step's partials (long
// complete) and rewrites the record once every workgroup of its own launch has
// read it, which each signals with a start mark. Nobody waits for the last
// workgroup to finish, and nothing runs after it.
//
// Waits are bounded by kCollectTimeout ticks of the 100 MHz real-time counter.
// If one runs out (which a correct launch never does) workgroup 0 freezes the
// record instead of folding: it stores a ZERO_RECORD_E_* code in the record's
// error word and touches nothing else there, and the stats carry the marker
// bad_buckets = 0xFFFFFFFF. A workgroup that finds the code set returns at once,
// in this launch and every later one, so no update lands on state that a late
// workgroup may still be reading.
constexpr uint64_t kCollectTimeout = 200000000ull;   // 2 s

// OR of a per-thread flag over the workgroup, in every thread.
__device__ __forceinline__ uint32_t block_or(uint32_t x) {
    __shared__ uint32_t s_or[kBlock / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x |= __shfl_xor(x, off, 64);
    lds_barrier();
    if ((threadIdx.x & 63) == 0) s_or[threadIdx.x >> 6] = x;
    lds_barrier();
    uint32_t r = 0u;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) r |= s_or[w];
    return r;
}

// Sum n partials tagged `tag` at `base` in slot order (thread t takes partials t,
// t + kBlock, ..., kBatch at a time with their loads all in flight; then the
// fixed tree of block_reduce, which leaves the totals in thread 0). Partials are
// polled until they carry the tag; a thread whose wait runs out sets
// ZERO_RECORD_E_COLLECT in tmo.
__device__ __forceinline__ void collect(const uint64_t* base, int n, uint32_t tag, uint64_t t0,
                                       double& sq, uint32_t& bad, uint32_t& badb, uint32_t& tmo) {
    constexpr int kBatch = 4;
    bool timed_out = false;
    for (int b = threadIdx.x; b < n && !timed_out; b += kBatch * kBlock) {
        uint64_t w[kBatch][3];
        uint32_t want = 0u, have = 0u;
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
            if (b + k * kBlock < n) want |= 1u << k;
        for (;;) {
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                if (!((want & ~have) >> k & 1u)) continue;
                const uint64_t* q = base + 3 * (int64_t)(b + k * kBlock);
                w[k][0] = rd64(q);
                w[k][1] = rd64(q + 1);
                w[k][2] = rd64(q + 2);
            }
#pragma unroll
            for (int k = 0; k < kBatch; ++k)
                if ((uint32_t)(w[k][0] >> 32) == tag && (uint32_t)(w[k][1] >> 32) == tag &&
                    (uint32_t)(w[k][2] >> 32) == tag)
                    have |= (want >> k & 1u) << k;
            if (have == want) break;
            if (__builtin_amdgcn_s_memrealtime() - t0 > kCollectTimeout) {
                timed_out = true;
                break;
            }
            __builtin_amdgcn_s_sleep(8);
        }
        if (timed_out) break;
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (!(want >> k & 1u)) continue;
            const uint64_t bits = ((w[k][0] & 0xffffffffull) << 32) | (w[k][1] & 0xffffffffull);
            sq += __longlong_as_double((long long)bits);
            bad |= (uint32_t)(w[k][2] & 1u);
            badb += (uint32_t)(w[k][2] & 0xffffffffull) >> 1;
        }
    }
    if (timed_out) tmo |= (uint32_t)ZERO_RECORD_E_COLLECT;
    block_reduce(sq, bad, badb);
}

// Wait until the n start marks at `marks` carry `tag`: every workgroup of this
// launch has read the record. Thread t checks marks t, t + kBlock, ..., kBatch at
// a time with their loads all in flight, re-polling the ones not yet in; a thread
// whose wait runs out sets ZERO_RECORD_E_MARKS in tmo.
__device__ __forceinline__ void wait_marks(const uint64_t* marks, int n, uint32_t tag, uint64_t t0,
                                          uint32_t& tmo) {
    constexpr int kBatch = 4;
    for (int b = threadIdx.x; b < n; b += kBatch * kBlock) {
        uint32_t want = 0u, have = 0u;
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
            if (b + k * kBlock < n) want |= 1u << k;
        for (;;) {
            uint64_t w[kBatch];
#pragma unroll
            for (int k = 0; k < kBatch; ++k)
                w[k] = ((want & ~have) >> k & 1u) ? rd64(marks + b + k * kBlock) : 0ull;
#pragma unroll
            for (int k = 0; k < kBatch; ++k)
                if ((uint32_t)(w[k] >> 32) == tag) have |= (want >> k & 1u) << k;
            if (have == want) break;
            if (__builtin_amdgcn_s_memrealtime() - t0 > kCollectTimeout) {
                tmo |= (uint32_t)ZERO_RECORD_E_MARKS;
                return;
            }
            __builtin_amdgcn_s_sleep(8);
        }
    }
}

// The stats of a frozen record: overflow, every bucket counted bad, NaN norm.
__device__ __forceinline__ void error_stats(zero_stats* stats) {
    stats->overflow = 1u;
    stats->bad_buckets = 0xffffffffu;
    stats->sumsq = __longlong_as_double(0x7ff8000000000000ll);
}

// Thread 0: fold the pending step into the record (with the squared norm and
// bucket count summed from its partials) and write its stats; the step that
// just ran (new_pending partials; 0 for a flush) becomes the pending one. If a
// wait ran out (tmo holds ZERO_RECORD_E_* bits), freeze the record instead: only
// its error word changes, so every other field still describes the state before
// this launch, whichever words a late reader of the record sees.
__device__ __forceinline__ void fold_pending(zero_device_state* c, zero_stats* stats,
                                             const uint64_t* flags, double sq, uint32_t badb,
                                             uint32_t tmo, uint32_t new_pending) {
    if (tmo) {
        error_stats(stats);
        c->error = (tmo & (uint32_t)ZERO_RECORD_E_COLLECT) ? (uint32_t)ZERO_RECORD_E_COLLECT
                                                          : (uint32_t)ZERO_RECORD_E_MARKS;
        return;
    }
    RecView v = read_record(c, flags);
    if (v.pend) {
        const bool overflow = pending_overflow(v);
        stats->overflow = overflow ? 1u : 0u;
        stats->bad_buckets = badb;
        stats->sumsq = sq;
        c->last_overflow = overflow ? 1u : 0u;
        c->last_sumsq = sq;
        if (!overflow) c->t = c->t + 1;
        else c->n_skipped = c->n_skipped + 1;
        apply_pending(v);
        c->cur = v.cur;
        c->beta1_pow = v.pow1;
        c->beta2_pow = v.pow2;
        c->loss_scale = v.ls;
        c->seq = v.seq + 1u;
    }
    c->pending_n = new_pending;
}

// Workgroup 0 of the launch that ends a step (all its threads): fold the pending
// step into the record once every workgroup of this launch has read it.
__device__ __forceinline__ void finalize_launch(const KParams& a, uint32_t tag) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    const zero_device_state* c = a.ctrl;
    const uint32_t seq = rd32(&c->seq), pend = rd32(&c->pending_n);
    double sq = 0.0;
    uint32_t bad = 0u, badb = 0u, tmo = 0u;
    if (pend) collect(a.ws_half[(seq + 1u) & 1u], (int)pend, seq + 1u, t0, sq, bad, badb, tmo);
    wait_marks(a.ws_started + a.part_base, (int)gridDim.x, tag, t0, tmo);
    tmo = block_or(tmo);
    if (threadIdx.x == 0) fold_pending(a.ctrl_rw, a.stats, a.ws_flags, sq, badb, tmo,
                                       (uint32_t)a.collect_n);
}

// Device commit: post this workgroup's start mark once every one of its waves
// has read the record. Each wave's checksum of the words it read goes through
// LDS (its write waits for those reads), and thread 0 stores the step's number
// with the XOR of all of them, so the mark cannot become visible before any
// wave's reads are done; workgroup 0 rewrites the record only once every mark of
// the launch is in. (A mark posted by wave 0 alone would not cover a sibling wave
// whose record loads were still in flight.)
__device__ __forceinline__ void post_mark(const KParams& a, const Res& rs) {
    constexpr int kWaves = kBlock / 64;
    __shared__ uint32_t s_mark[kWaves];
    if ((threadIdx.x & 63) == 0) s_mark[threadIdx.x >> 6] = (uint32_t)rs.mark;
    lds_barrier();
    if (threadIdx.x == 0) {
        uint32_t x = 0u;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) x ^= s_mark[k];
        __hip_atomic_store(a.ws_started + ((int64_t)a.part_base + blockIdx.x),
                           ((uint64_t)rs.tag << 32) | x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// PRE (device commit, one row, launches of at most kPreGrid workgroups over the
// whole shard or over a table of short buckets): each lane's first quad and its
// first replica batch are taken before the committed-state record is read, so
// that with a cold cache the record's round trip overlaps those loads.
template <typename RT, bool BUCKETS, bool ADAM, bool WRITE_G, bool CTRL, bool TILED, int ROWS,
          bool PRE = false>
__global__ void ZERO_STEP_BOUNDS k_step(const KParams a) {
    static_assert(!PRE || (CTRL && ROWS == 1), "the prefetch serves one-row device-commit launches");
    Head<RT> head;
    if constexpr (PRE && BUCKETS) {
        // a table of short buckets, one per workgroup in turn (never the chunked
        // table): the first bucket's descriptor, then the lane's first quad in it
        const int64_t b = xcd_trip(blockIdx.x, gridDim.x);
        if (b < a.n_buckets) {
            const zero_bucket bk = a.buckets[b];
            const int64_t lo = bk.shard_off, len = bk.len;
            if (lo >= 0 && len > 0 && lo <= a.S && len <= a.S - lo) {
                const int64_t q = (lo >> 2) + threadIdx.x;
                if (q < range_qend(a, lo + len)) head_load<RT>(a, q, head);
            }
        }
    } else if constexpr (PRE) {
        const int64_t nq = a.S >> 2, g = gridDim.x;
        const int64_t b = xcd_trip(blockIdx.x, gridDim.x);
        int64_t q = -1;
        if (a.even_blocks > 0) {
            const int64_t nb = a.even_blocks;
            int64_t qhi = ((b + 1) * nb / g) * kEvenBlockQuads;
            if (qhi > nq) qhi = nq;
            q = (b * nb / g) * kEvenBlockQuads + threadIdx.x;
            if (q >= qhi) q = -1;
        } else if (b < nq / kBlock) {
            q = b * kBlock + threadIdx.x;
        }
        if (q >= 0) head_load<RT>(a, q, head);
    }
    const Res rs = resolve<CTRL, TILED>(a);
    if constexpr (CTRL) {
        // a frozen record (a wait of an earlier launch ran out): no work at all
        if (rs.err) return;
        post_mark(a, rs);
    }
    double sq = 0.0;
    uint32_t bad = 0u, badb = 0u;
    if constexpr (!BUCKETS) {
        if (a.even_blocks > 0) {
            // blocks [b*NB/G, (b+1)*NB/G) of the shard's quads, and the last S % 4
            // elements with the one that takes the last blocks (b: the workgroup's
            // share, permuted over the XCDs like the trips of a larger launch)
            const int64_t nq = a.S >> 2, nb = a.even_blocks, g = gridDim.x;
            const int64_t b = xcd_trip(blockIdx.x, gridDim.x);
            const int64_t qlo = (b * nb / g) * kEvenBlockQuads;
            int64_t qhi = ((b + 1) * nb / g) * kEvenBlockQuads;
            if (qhi > nq) qhi = nq;
            int64_t q = qlo + threadIdx.x;
            if constexpr (PRE) {
                if (q < qhi) quad_pre<RT, ADAM, WRITE_G, TILED>(a, rs, q, head, sq, bad);
                q += kBlock;
            }
            for (; q < qhi; q += kBlock)
                quads<RT, ADAM, WRITE_G, TILED, 1>(a, rs, q, 0, sq, bad);
            if (b == (int64_t)gridDim.x - 1) {
                const int64_t e = nq * 4 + threadIdx.x;
                if (e < a.S) one_elem<RT, ADAM, WRITE_G, TILED>(a, rs, e, sq, bad);
            }
        } else {
            const int64_t nq = a.S >> 2;
            const int64_t per_trip = (int64_t)ROWS * kBlock;
            const int64_t ntrips = nq / per_trip;
            int64_t trip = xcd_trip(blockIdx.x, gridDim.x);
            if constexpr (PRE) {
                if (trip < ntrips)
                    quad_pre<RT, ADAM, WRITE_G, TILED>(a, rs, trip * per_trip + threadIdx.x, head, sq, bad);
                trip += gridDim.x;
            }
            for (; trip < ntrips; trip += gridDim.x)
                quads<RT, ADAM, WRITE_G, TILED, ROWS>(a, rs, trip * per_trip + threadIdx.x, kBlock, sq, bad);
            // whole quads after the last full trip, and the last S % 4 elements
            if ((int64_t)blockIdx.x == ntrips % gridDim.x) {
                for (int64_t q = ntrips * per_trip + threadIdx.x; q < nq; q += kBlock)
                    quads<RT, ADAM, WRITE_G, TILED, 1>(a, rs, q, 0, sq, bad);
                const int64_t e = nq * 4 + threadIdx.x;
                if (e < a.S) one_elem<RT, ADAM, WRITE_G, TILED>(a, rs, e, sq, bad);
            }
        }
    } else if (!PRE && a.even_blocks > 0) {
        // A short table of long buckets: every bucket is cut into chunks of kChunk
        // elements (boundaries on 64-element lines) and the chunks are dealt over
        // the grid. Each workgroup reads the table and prefix-sums the chunk counts
        // in LDS: first[b] is bucket b's first chunk, first[n] the total.
        __shared__ int64_t first[kChunkTableMax + 1];
        __shared__ int64_t wave_sum[kBlock / 64];
        const int64_t nbk = a.n_buckets;
        const int64_t per = (nbk + kBlock - 1) / kBlock;
        const int64_t b0 = threadIdx.x * per;
        int64_t mine = 0;
        for (int64_t i = 0; i < per; ++i) {
            const int64_t b = b0 + i;
            if (b >= nbk) break;
            const zero_bucket bk = a.buckets[b];
            const int64_t lo = bk.shard_off, len = bk.len;
            int64_t c = 0;
            if (lo < 0 || len < 0 || lo > a.S || len > a.S - lo) {
                if (blockIdx.x == 0) badb += 1u;     // counted once, by workgroup 0
            } else {
                c = (len + kChunk - 1) / kChunk;
            }
            first[b] = c;
            mine += c;
        }
        const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
        int64_t incl = mine;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int64_t y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
        }
        if (lane == 63) wave_sum[wv] = incl;
        lds_barrier();
        int64_t run = incl - mine;
        for (int w = 0; w < wv; ++w) run += wave_sum[w];
        if (threadIdx.x == kBlock - 1) first[nbk] = run + mine;
        for (int64_t i = 0; i < per; ++i) {
            const int64_t b = b0 + i;
            if (b >= nbk) break;
            const int64_t c = first[b];
            first[b] = run;
            run += c;
        }
        lds_barrier();
        const int64_t total = first[nbk];
        for (int64_t j = xcd_trip(blockIdx.x, gridDim.x); j < total; j += gridDim.x) {
            // the bucket holding chunk j: first[lb] <= j < first[lb + 1]
            int64_t lb = 0, ub = nbk;
            while (ub - lb > 1) {
                const int64_t mid = (lb + ub) >> 1;
                if (first[mid] <= j) lb = mid;
                else ub = mid;
            }
            const zero_bucket bk = a.buckets[lb];
            const int64_t blo = bk.shard_off, bhi = blo + bk.len;
            const int64_t k = j - first[lb], last = first[lb + 1] - first[lb] - 1;
            int64_t lo = k == 0 ? blo : ((blo + k * kChunk) & ~int64_t(63));
            int64_t hi = k == last ? bhi : ((blo + (k + 1) * kChunk) & ~int64_t(63));
            if (lo < blo) lo = blo;
            if (hi < blo) hi = blo;
            range<RT, ADAM, WRITE_G, TILED>(a, rs, lo, hi, sq, bad);
        }
    } else {
        int64_t b = xcd_trip(blockIdx.x, gridDim.x);
        if constexpr (PRE) {
            // the first bucket, its first quad per lane loaded in the prologue
            if (b < a.n_buckets) {
                const zero_bucket bk = a.buckets[b];
                const int64_t lo = bk.shard_off, len = bk.len;
                if (lo < 0 || len < 0 || lo > a.S || len > a.S - lo) {
                    if (threadIdx.x == 0) badb += 1u;
                } else {
                    range<RT, ADAM, WRITE_G, TILED, true>(a, rs, lo, lo + len, sq, bad, &head);
                }
            }
            b += gridDim.x;
        }
        for (; b < a.n_buckets; b += gridDim.x) {
            const zero_bucket bk = a.buckets[b];
            const int64_t lo = bk.shard_off, len = bk.len;
            if (lo < 0 || len < 0 || lo > a.S || len > a.S - lo) {
                if (threadIdx.x == 0) badb += 1u;
                continue;
            }
            range<RT, ADAM, WRITE_G, TILED>(a, rs, lo, lo + len, sq, bad);
        }
    }
    block_reduce(sq, bad, badb);
    if constexpr (!CTRL) {
        if (threadIdx.x == 0) {
            Partial pt;
            pt.sumsq = sq;
            pt.bad = bad;
            pt.bad_buckets = badb;
            a.partials[blockIdx.x] = pt;
        }
    } else {
        // Each workgroup publishes its partial as three 64-bit agent-scope atomic
        // stores (written through to the coherence point all XCDs share), each
        // word tagged with this step's number, in the workspace half of the
        // number's parity, sets the step's flag word if it saw a non-finite
        // gradient, and leaves at once. 64-bit aligned stores and loads are
        // single-copy atomic, so no word is ever seen half written.
        if (threadIdx.x == 0) {
            const uint64_t tag = (uint64_t)rs.tag << 32;
            const uint64_t sqb = (uint64_t)__double_as_longlong(sq);
            uint64_t* w = a.ws_half[rs.tag & 1u] + 3 * ((int64_t)a.part_base + blockIdx.x);
            __hip_atomic_store(w + 0, tag | (sqb >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(w + 1, tag | (sqb & 0xffffffffull), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(w + 2, tag | (uint64_t)((bad ? 1u : 0u) | (badb << 1)), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            if (bad)
                __hip_atomic_store(a.ws_flags + (rs.tag & 1u), (uint64_t)rs.tag, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        if (blockIdx.x == 0 && a.collect_n > 0) finalize_launch(a, rs.tag);
    }
}

// Sum the per-workgroup partials in workgroup order and write the stats.
__global__ void __launch_bounds__(kFinalizeBlock) k_finalize(const Partial* parts, int n,
                                                            zero_stats* out) {
    double sq = 0.0;
    uint32_t bad = 0u, badb = 0u;
    for (int i = threadIdx.x; i < n; i += kFinalizeBlock) {
        const Partial pt = parts[i];
        sq += pt.sumsq;
        bad |= pt.bad;
        badb += pt.bad_buckets;
    }
    block_reduce(sq, bad, badb);
    if (threadIdx.x == 0) {
        out->overflow = bad ? 1u : 0u;
        out->bad_buckets = badb;
        out->sumsq = sq;
    }
}

// slot[i] = bf16(master[i]) over quads [0, S/4) by the whole grid, tail by workgroup
// 0; master is a p array (split) or a set buffer (tiled).
template <bool TILED>
__device__ __forceinline__ void cast_range(const float* master, int64_t S, uint16_t* slot) {
    const int64_t nq = S >> 2;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t q = (int64_t)blockIdx.x * kBlock + threadIdx.x; q < nq; q += stride) {
        const f32x4 x = ld(reinterpret_cast<const f32x4*>(master) + state_q<TILED>(q));
        u32x2 w;
        w.x = f2bf(x.x) | (f2bf(x.y) << 16);
        w.y = f2bf(x.z) | (f2bf(x.w) << 16);
        st(reinterpret_cast<u32x2*>(slot) + q, w);
    }
    if (blockIdx.x == 0) {
        const int64_t e = nq * 4 + threadIdx.x;
        if (e < S) slot[e] = (uint16_t)f2bf(master[state_e<TILED>(e)]);
    }
}

template <bool TILED>
__global__ void __launch_bounds__(kBlock) k_cast_slot(const float* master, int64_t S,
                                                     uint16_t* slot) {
    cast_range<TILED>(master, S, slot);
}

// After a device-resident step: if it overflowed, restore the slot from the
// committed master (the current set, which a skipped step leaves current).
// Every workgroup reads the verdict the step's commit wrote into the record and,
// on a clean step, exits at once.
template <bool TILED>
__global__ void __launch_bounds__(kBlock) k_restore(const zero_device_state* ctrl,
                                                   const uint64_t* flags, const float* set_p0,
                                                   const float* set_p1, uint16_t* slot, int64_t S) {
    // a frozen record: the slot stays as it is
    if (ctrl->error) return;
    // the step just run is pending in the record (or folded in by a flush)
    const uint32_t seq = ctrl->seq, pend = ctrl->pending_n;
    const bool overflow = pend ? flags[(seq + 1u) & 1u] == (uint64_t)(seq + 1u)
                               : ctrl->last_overflow != 0u;
    if (!overflow) return;
    // a skipped step leaves the current set of the record current
    cast_range<TILED>((ctrl->cur & 1u) ? set_p1 : set_p0, S, slot);
}

// zero_device_state_flush: one workgroup folds the pending step into the record.
__global__ void __launch_bounds__(kBlock) k_flush(zero_device_state* c, zero_stats* stats,
                                                 const uint64_t* half0, const uint64_t* half1,
                                                 const uint64_t* flags) {
    if (rd32(&c->error)) {
        // a frozen record: report it in the stats, change nothing
        if (threadIdx.x == 0) error_stats(stats);
        return;
    }
    const uint32_t seq = rd32(&c->seq), pend = rd32(&c->pending_n);
    if (!pend) return;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    double sq = 0.0;
    uint32_t bad = 0u, badb = 0u, tmo = 0u;
    collect(((seq + 1u) & 1u) ? half1 : half0, (int)pend, seq + 1u, t0, sq, bad, badb, tmo);
    tmo = block_or(tmo);
    if (threadIdx.x == 0) fold_pending(c, stats, flags, sq, badb, tmo, 0u);
}

// Conversion between three split arrays p, m, v [S] and one tiled set buffer;
// UNPACK copies tiled -> split (a NULL destination is skipped), else split -> tiled.
// Elements of the last tile at or beyond S are not touched.
template <bool UNPACK>
__global__ void __launch_bounds__(kBlock) k_state_convert(float* tiled, float* p, float* m, float* v,
                                                         int64_t S) {
    const int64_t nq = S >> 2;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    float* const sec[3] = {p, m, v};
    for (int64_t q = (int64_t)blockIdx.x * kBlock + threadIdx.x; q < nq; q += stride) {
        const int64_t t = state_q<true>(q);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            f32x4* tq = reinterpret_cast<f32x4*>(tiled) + t + k * kStateTileQuads;
            f32x4* sq = reinterpret_cast<f32x4*>(sec[k]) + q;
            if constexpr (UNPACK) {
                if (sec[k]) st(sq, ld(tq));
            } else {
                st(tq, ld(sq));
            }
        }
    }
    if (blockIdx.x == 0) {
        const int64_t e = nq * 4 + threadIdx.x;
        if (e < S) {
            const int64_t t = state_e<true>(e);
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                if constexpr (UNPACK) {
                    if (sec[k]) sec[k][e] = tiled[t + k * kStateTile];
                } else {
                    tiled[t + k * kStateTile] = sec[k][e];
                }
            }
        }
    }
}

// Writing a whole record (initial or restored), and clearing the workspace its
// steps will use (no partial may carry a tag before the record's next step).
__global__ void k_state_write(zero_device_state* s, zero_device_state rec, uint64_t* ws,
                              int64_t ws_words) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < ws_words; i += stride)
        ws[i] = 0ull;
    if (blockIdx.x == 0 && threadIdx.x == 0) *s = rec;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

// Quads per lane per trip: one row (one quad per lane per trip) by default; a
// build with ZERO_ROWS_FEW=2 gives launches with up to 16 replicas two rows,
// more bytes in flight per lane at a higher register count (one row measured
// faster with one trip per workgroup).
#ifndef ZERO_ROWS_FEW
#define ZERO_ROWS_FEW 1
#endif
int rows_for(int32_t n_rep) { return n_rep <= 16 ? ZERO_ROWS_FEW : 1; }

// Workgroups of the step kernel: many more than the chip holds at once (short
// workgroups, so faster CUs pick up more of the work and the tail is short;
// one trip each up to about 134M elements), at most kGridMax / 2 with two rows
// per lane and kGridMax with one, and balanced so that every workgroup makes
// the same number of full trips (no ragged last round).
// A whole-shard launch of kEvenMin .. kEvenMax - 1 trips (one trip per workgroup
// covers a workgroup's worth of quads) rounds its grid up to a multiple of
// kEvenUnit workgroups and splits the shard evenly over them: with few
// workgroups per compute unit, one more on some units than on others sets the
// launch's length. The split is in blocks of kEvenBlockQuads quads (128 bytes of
// a bf16 replica, 256 of fp32 state), so no cache line is fetched by two
// workgroups; workgroup b takes blocks [b*NB/G, (b+1)*NB/G). Returns NB, the
// number of blocks, or 0 for the usual grid.
constexpr int64_t kEvenUnit = 256, kEvenMin = 256, kEvenMax = 2048;
int64_t even_blocks_for(int64_t S, int64_t n_buckets, int32_t n_rep, int max_grid) {
    if (max_grid <= 0 || max_grid > kGridMax) max_grid = kGridMax;
    if (n_buckets > 0 || rows_for(n_rep) != 1) return 0;
    const int64_t trips = S / ((int64_t)kBlock * kVec);
    const int64_t grid = (trips + kEvenUnit - 1) / kEvenUnit * kEvenUnit;
    if (trips < kEvenMin || trips >= kEvenMax || grid > max_grid) return 0;
    const int64_t nq = S >> 2;
    return (nq + kEvenBlockQuads - 1) / kEvenBlockQuads;
}

bool bucket_chunks(int64_t S, int64_t n_buckets) {
    return n_buckets > 0 && n_buckets <= kChunkTableMax && n_buckets * 2 * kChunk <= S;
}

int grid_for(int64_t S, int64_t n_buckets, int32_t n_rep, int max_grid) {
    if (even_blocks_for(S, n_buckets, n_rep, max_grid) > 0) {
        const int64_t trips = S / ((int64_t)kBlock * kVec);
        return (int)((trips + kEvenUnit - 1) / kEvenUnit * kEvenUnit);
    }
    if (max_grid <= 0 || max_grid > kGridMax) max_grid = kGridMax;
    if (bucket_chunks(S, n_buckets)) {
        // enough workgroups for one chunk each when the buckets are disjoint
        const int64_t g = (S + kChunk - 1) / kChunk + n_buckets;
        const int64_t cap = grid_bound(S) < max_grid ? grid_bound(S) : max_grid;
        return (int)(g < cap ? g : cap);
    }
    if (n_buckets > 0) {
        // bucket launches stride over the table; at most grid_bound(S) workgroups
        int64_t g = n_buckets < max_grid ? n_buckets : max_grid;
        return (int)(g < grid_bound(S) ? g : grid_bound(S));
    }
    const int64_t per_trip = (int64_t)rows_for(n_rep) * kBlock * kVec;
    const int64_t trips = S / per_trip;
    if (trips < 1) return 1;
    const int64_t cap = rows_for(n_rep) == 2 ? (max_grid > 1 ? max_grid / 2 : 1) : max_grid;
    const int64_t rounds = (trips + cap - 1) / cap;
    return (int)((trips + rounds - 1) / rounds);
}

static int grid_stream(int64_t S) {
    const int64_t per = (int64_t)kBlock * kVec * 4;
    int64_t g = (S + per - 1) / per;
    if (g < 1) g = 1;
    if (g > kCommitGrid) g = kCommitGrid;
    return (int)g;
}

// One launch of the step kernel. With timing events the launch carries them
// (hipExtLaunchKernelGGL), so they take the kernel's own start and end and their
// interval is the kernel alone, not the stream's gaps around it.
template <typename RT, bool BUCKETS, bool ADAM, bool WRITE_G, bool CTRL, bool TILED, int ROWS,
          bool PRE = false>
static void launch_one(const StepDesc& d, const KParams& k, int grid, hipStream_t st) {
    if (d.ev_begin || d.ev_end)
        hipExtLaunchKernelGGL((k_step<RT, BUCKETS, ADAM, WRITE_G, CTRL, TILED, ROWS, PRE>), dim3(grid),
                              dim3(kBlock), 0, st, d.ev_begin, d.ev_end, 0, k);
    else
        hipLaunchKernelGGL((k_step<RT, BUCKETS, ADAM, WRITE_G, CTRL, TILED, ROWS, PRE>), dim3(grid),
                           dim3(kBlock), 0, st, k);
}

// Device-commit launches of at most this many workgroups, over the whole shard or
// a table of short buckets, take their first replica batch before the record
// (k_step's PRE): GPT-2-sized and smaller shards gain 1-3%; on the Llama shards it
// changes nothing or costs 0.1%.
constexpr int kPreGrid = 65536;

template <typename RT, bool BUCKETS, int ROWS>
static void launch_rows(const StepDesc& d, const KParams& k, int grid, hipStream_t st) {
    if (d.ctrl) {
        if constexpr (ROWS == 1) {
            if (grid <= kPreGrid && (!BUCKETS || k.even_blocks == 0)) {
                if (d.tiled) launch_one<RT, BUCKETS, true, false, true, true, 1, true>(d, k, grid, st);
                else launch_one<RT, BUCKETS, true, false, true, false, 1, true>(d, k, grid, st);
                return;
            }
        }
        if (d.tiled) launch_one<RT, BUCKETS, true, false, true, true, ROWS>(d, k, grid, st);
        else launch_one<RT, BUCKETS, true, false, true, false, ROWS>(d, k, grid, st);
    } else if (d.adam) {
        if (d.tiled) launch_one<RT, BUCKETS, true, false, false, true, ROWS>(d, k, grid, st);
        else launch_one<RT, BUCKETS, true, false, false, false, ROWS>(d, k, grid, st);
    } else if (d.g_out) {
        launch_one<RT, BUCKETS, false, true, false, false, ROWS>(d, k, grid, st);
    } else {
        launch_one<RT, BUCKETS, false, false, false, false, ROWS>(d, k, grid, st);
    }
}

template <typename RT, bool BUCKETS>
static void launch_typed(const StepDesc& d, const KParams& k, int grid, hipStream_t st) {
    if constexpr (ZERO_ROWS_FEW == 2) {
        if (rows_for(d.n_rep) == 2) return launch_rows<RT, BUCKETS, 2>(d, k, grid, st);
    }
    launch_rows<RT, BUCKETS, 1>(d, k, grid, st);
}

template <typename RT>
static void launch_dtype(const StepDesc& d, const KParams& k, int grid, hipStream_t st, bool buckets,
                         bool ext) {
    if (ext) {
        if (buckets) launch_typed<Ext<RT>, true>(d, k, grid, st);
        else launch_typed<Ext<RT>, false>(d, k, grid, st);
    } else {
        if (buckets) launch_typed<RT, true>(d, k, grid, st);
        else launch_typed<RT, false>(d, k, grid, st);
    }
}

// Writes n replica pointers (from the kernel arguments) into a device table.
struct PtrChunk {
    const void* p[kArgReplicas];
};

__global__ void __launch_bounds__(kArgReplicas) k_put_ptrs(const void** dst, const PtrChunk c, int n) {
    if ((int)threadIdx.x < n) dst[threadIdx.x] = c.p[threadIdx.x];
}

// More replicas than the kernel arguments hold: their pointers go into the
// device table d.rep_table first, kArgReplicas per launch, on the same stream.
static hipError_t put_replica_table(const StepDesc& d, hipStream_t st) {
    for (int32_t j0 = 0; j0 < d.n_rep; j0 += kArgReplicas) {
        const int n = d.n_rep - j0 < kArgReplicas ? d.n_rep - j0 : kArgReplicas;
        PtrChunk c{};
        for (int i = 0; i < n; ++i) c.p[i] = d.replicas[j0 + i];
        hipLaunchKernelGGL(k_put_ptrs, dim3(1), dim3(kArgReplicas), 0, st,
                           const_cast<const void**>(d.rep_table) + j0, c, n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_step(const StepDesc& d, hipStream_t st) {
    KParams k;
    const bool ext = d.n_rep > kArgReplicas;
    for (int j = 0; j < kArgReplicas; ++j) k.rep[j] = j < d.n_rep ? d.replicas[j] : nullptr;
    k.rep_ext = ext ? d.rep_table : nullptr;
    if (ext) {
        if (!d.rep_table) return hipErrorInvalidValue;
        const hipError_t e = put_replica_table(d, st);
        if (e != hipSuccess) return e;
    }
    k.n_rep = d.n_rep;
    k.even_blocks = 0;
    k.S = d.S;
    k.buckets = d.buckets;
    k.n_buckets = d.n_buckets;
    k.p_in = d.p_in;
    k.m_in = d.m_in;
    k.v_in = d.v_in;
    k.p_out = d.p_out;
    k.m_out = d.m_out;
    k.v_out = d.v_out;
    for (int i = 0; i < 2; ++i) {
        k.set_p[i] = d.set_p[i];
        k.set_m[i] = d.set_m[i];
        k.set_v[i] = d.set_v[i];
    }
    k.ctrl = d.ctrl;
    k.ctrl_rw = d.ctrl;
    k.stats = d.stats;
    k.slot = d.slot;
    k.set_slot[0] = d.set_slot[0];
    k.set_slot[1] = d.set_slot[1];
    k.g_out = d.g_out;
    k.partials = d.partials;
    for (int i = 0; i < 2; ++i) k.ws_half[i] = d.ws_half[i];
    k.ws_started = d.ws_started;
    k.ws_flags = d.ws_flags;
    k.sc = d.sc;
    const bool buckets = d.n_buckets > 0;
    const int grid = grid_for(d.S, d.n_buckets, d.n_rep, d.max_grid);
    k.even_blocks = buckets ? (bucket_chunks(d.S, d.n_buckets) ? 1 : 0)
                            : (int32_t)even_blocks_for(d.S, d.n_buckets, d.n_rep, d.max_grid);
    k.part_base = d.part_base;
    k.collect_n = d.collect_n == 0 ? grid : (d.collect_n > 0 ? d.collect_n : 0);
    if (d.dtype == ZERO_BF16) {
        launch_dtype<uint16_t>(d, k, grid, st, buckets, ext);
    } else if (d.dtype == ZERO_BF16_WIRE) {
        launch_dtype<WireBf16>(d, k, grid, st, buckets, ext);
    } else {
        launch_dtype<float>(d, k, grid, st, buckets, ext);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (d.ctrl) {
        if (d.slot && !d.set_slot[1] && !d.no_restore)
            return launch_restore(d.ctrl, d.ws_flags, d.set_p[0], d.set_p[1], d.slot, d.S, d.tiled, st);
    } else {
        hipLaunchKernelGGL(k_finalize, dim3(1), dim3(kFinalizeBlock), 0, st,
                           (const Partial*)d.partials, grid, d.stats);
    }
    return hipGetLastError();
}

hipError_t launch_restore(const zero_device_state* ctrl, const uint64_t* flags, const float* set_p0,
                          const float* set_p1, uint16_t* slot, int64_t S, bool tiled, hipStream_t st) {
    if (tiled)
        hipLaunchKernelGGL(k_restore<true>, dim3(grid_stream(S)), dim3(kBlock), 0, st, ctrl, flags,
                           set_p0, set_p1, slot, S);
    else
        hipLaunchKernelGGL(k_restore<false>, dim3(grid_stream(S)), dim3(kBlock), 0, st, ctrl, flags,
                           set_p0, set_p1, slot, S);
    return hipGetLastError();
}

hipError_t launch_flush(zero_device_state* ctrl, zero_stats* stats, const CommitWs& w,
                        hipStream_t st) {
    hipLaunchKernelGGL(k_flush, dim3(1), dim3(kBlock), 0, st, ctrl, stats, w.half[0], w.half[1],
                       w.flags);
    return hipGetLastError();
}

hipError_t launch_cast_slot(const float* master, int64_t S, bool tiled, uint16_t* slot,
                            hipStream_t st) {
    if (tiled)
        hipLaunchKernelGGL(k_cast_slot<true>, dim3(grid_stream(S)), dim3(kBlock), 0, st, master, S,
                           slot);
    else
        hipLaunchKernelGGL(k_cast_slot<false>, dim3(grid_stream(S)), dim3(kBlock), 0, st, master, S,
                           slot);
    return hipGetLastError();
}

hipError_t launch_state_convert(bool unpack, float* tiled, float* p, float* m, float* v, int64_t S,
                                hipStream_t st) {
    if (unpack)
        hipLaunchKernelGGL(k_state_convert<true>, dim3(grid_stream(S)), dim3(kBlock), 0, st, tiled, p,
                           m, v, S);
    else
        hipLaunchKernelGGL(k_state_convert<false>, dim3(grid_stream(S)), dim3(kBlock), 0, st, tiled,
                           p, m, v, S);
    return hipGetLastError();
}

hipError_t launch_state_write(zero_device_state* s, const zero_device_state& rec, void* ws,
                              size_t ws_bytes, hipStream_t st) {
    const int64_t words = (int64_t)(ws_bytes / 8);
    int64_t grid = (words + kBlock - 1) / kBlock;
    if (grid < 1) grid = 1;
    if (grid > 64) grid = 64;
    hipLaunchKernelGGL(k_state_write, dim3((unsigned)grid), dim3(kBlock), 0, st, s, rec,
                       static_cast<uint64_t*>(ws), words);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// scratch of the allocation-free entry point
// ---------------------------------------------------------------------------

// zero_adam_step_noalloc takes its workspace -- the per-workgroup partials of the
// flag and the squared norm, and the device table of replica pointers beyond
// the kernel arguments -- from this array instead of a caller's buffer. Every
// GPU the library runs on holds its own copy until the process ends. In host
// code the name stands for the symbol, not for device memory: kernels get the
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kNoallocBytes];

hipError_t noalloc_scratch(void** ptr) {
    static std::atomic<void*> addr[kNoallocMaxDevices];
    static std::mutex mu;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kNoallocMaxDevices) return hipErrorInvalidDevice;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(mu);
        p = addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace zk
