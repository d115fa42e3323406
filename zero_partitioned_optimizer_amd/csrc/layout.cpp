// layout.cpp -- flat layout, shard cut, segments, buckets and memory accounting
// (host only, C ABI half in abi.cpp).
//
// One contiguous flat buffer holds all tensors ("Why does not the stage 3
// implementation use broadcast and reduce-scatter?", the contiguous_gradients
// replies) and is cut into N equal shards so that each rank's gradient slice
// matches the optimizer-state and parameter slice it owns ("[REQUEST] Direct
// Correspondence between Gradient and Optimizer States to Reduce
// Communication", "Problem"); small tensors are grouped into buckets ("ZeRO
// Optimizer", "Communication Optimization"); the memory per device follows
// "ZeRO Optimizer", "Memory Components" and "Theoretical Reductions".
#include <stdint.h>

#include <algorithm>
#include <new>
#include <vector>

#include "zero.h"

struct zero_layout {
    std::vector<int64_t> numels;
    std::vector<int64_t> offsets;
    zero_layout_info info;
};

namespace zl {

void set_error(const char* fmt, ...);

static bool add_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_add_overflow(a, b, out); }
static bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

// smallest multiple of a that is >= x (x >= 0, a >= 1), overflow-checked
static bool align_up(int64_t x, int64_t a, int64_t* out) {
    int64_t r = x % a;
    if (r == 0) {
        *out = x;
        return true;
    }
    return add_ok(x, a - r, out);
}

int build(const int64_t* numels, int64_t T, int32_t N, int64_t A, int64_t B, zero_layout** out) {
    if (!out) {
        set_error("zero_layout_build: out is NULL");
        return ZERO_E_INVAL;
    }
    *out = nullptr;
    if (T < 0 || (T > 0 && !numels)) {
        set_error("zero_layout_build: n_tensors=%lld with numels=%p", (long long)T, (const void*)numels);
        return ZERO_E_INVAL;
    }
    if (N < 1 || N > (1 << 20) || A < 1 || A > (1 << 20) || B < 1 || B > (1 << 20)) {
        set_error("zero_layout_build: world_N=%d, tensor_align_A=%lld, shard_align_B=%lld out of [1, 2^20]",
                  (int)N, (long long)A, (long long)B);
        return ZERO_E_INVAL;
    }
    zero_layout* L = new (std::nothrow) zero_layout();
    if (!L) {
        set_error("zero_layout_build: out of host memory");
        return ZERO_E_NOMEM;
    }
    try {
        L->numels.assign(numels, numels + T);
        L->offsets.resize((size_t)T);
    } catch (...) {
        delete L;
        set_error("zero_layout_build: out of host memory");
        return ZERO_E_NOMEM;
    }
    int64_t end = 0, psi = 0;
    for (int64_t i = 0; i < T; ++i) {
        const int64_t n = numels[i];
        if (n < 0) {
            delete L;
            set_error("zero_layout_build: numels[%lld] = %lld is negative", (long long)i, (long long)n);
            return ZERO_E_INVAL;
        }
        int64_t o = 0;
        if (i > 0 && !align_up(end, A, &o)) goto overflow;
        L->offsets[(size_t)i] = o;
        if (!add_ok(o, n, &end) || !add_ok(psi, n, &psi)) goto overflow;
    }
    {
        const int64_t used = end;
        const int64_t per_rank = used / N + (used % N != 0);
        int64_t S = 0, padded = 0;
        if (!align_up(per_rank, B, &S) || !mul_ok(S, N, &padded)) goto overflow;
        zero_layout_info& I = L->info;
        I.n_tensors = T;
        I.psi = psi;
        I.used_L = used;
        I.padded_L = padded;
        I.shard_S = S;
        I.tensor_align_A = A;
        I.shard_align_B = B;
        I.world_N = N;
        I.reserved = 0;
    }
    *out = L;
    return ZERO_OK;
overflow:
    delete L;
    set_error("zero_layout_build: flat length overflows int64");
    return ZERO_E_RANGE;
}

// Segments of one rank, in tensor order (binary search for the first tensor).
static void collect_segments(const zero_layout* L, int32_t rank, std::vector<zero_segment>& segs) {
    const int64_t S = L->info.shard_S;
    const int64_t lo = (int64_t)rank * S, hi = lo + S;
    const int64_t T = L->info.n_tensors;
    // first tensor whose end is past lo: offsets are non-decreasing, ends too
    int64_t a = 0, b = T;
    while (a < b) {
        const int64_t mid = a + (b - a) / 2;
        if (L->offsets[(size_t)mid] + L->numels[(size_t)mid] <= lo) a = mid + 1;
        else b = mid;
    }
    for (int64_t i = a; i < T; ++i) {
        const int64_t o = L->offsets[(size_t)i];
        if (o >= hi) break;
        const int64_t s = std::max(o, lo);
        const int64_t e = std::min(o + L->numels[(size_t)i], hi);
        if (s < e) {
            zero_segment sg;
            sg.tensor = (int32_t)i;
            sg.reserved = 0;
            sg.tensor_off = s - o;
            sg.shard_off = s - lo;
            sg.len = e - s;
            segs.push_back(sg);
        }
    }
}

int segments(const zero_layout* L, int32_t rank, zero_segment* out, int64_t cap, int64_t* n_out) {
    if (!L || !n_out) {
        set_error("zero_layout_segments: NULL layout or n_out");
        return ZERO_E_INVAL;
    }
    if (rank < 0 || rank >= L->info.world_N) {
        set_error("zero_layout_segments: rank %d outside [0, %d)", (int)rank, (int)L->info.world_N);
        return ZERO_E_RANGE;
    }
    if (L->info.n_tensors > INT32_MAX) {
        set_error("zero_layout_segments: more than 2^31-1 tensors");
        return ZERO_E_RANGE;
    }
    std::vector<zero_segment> segs;
    collect_segments(L, rank, segs);
    *n_out = (int64_t)segs.size();
    if (!out) return ZERO_OK;
    if (cap < (int64_t)segs.size()) {
        set_error("zero_layout_segments: capacity %lld < %lld segments", (long long)cap,
                  (long long)segs.size());
        return ZERO_E_RANGE;
    }
    std::copy(segs.begin(), segs.end(), out);
    return ZERO_OK;
}

int buckets(const zero_layout* L, int32_t rank, int64_t be, zero_bucket* out, int64_t cap,
            int64_t* n_out) {
    if (!L || !n_out) {
        set_error("zero_layout_buckets: NULL layout or n_out");
        return ZERO_E_INVAL;
    }
    if (rank < 0 || rank >= L->info.world_N) {
        set_error("zero_layout_buckets: rank %d outside [0, %d)", (int)rank, (int)L->info.world_N);
        return ZERO_E_RANGE;
    }
    if (be < 1 || be > (int64_t(1) << 30)) {
        set_error("zero_layout_buckets: bucket_elems %lld outside [1, 2^30]", (long long)be);
        return ZERO_E_INVAL;
    }
    std::vector<zero_segment> segs;
    collect_segments(L, rank, segs);
    std::vector<zero_bucket> bks;
    bool open = false;
    int64_t start = 0, cur_end = 0;
    int32_t tensor = 0;
    auto close = [&](int64_t end) {
        zero_bucket b;
        b.shard_off = start;
        b.len = (int32_t)(end - start);
        b.tensor = tensor;
        bks.push_back(b);
        open = false;
    };
    for (const zero_segment& sg : segs) {
        const int64_t s = sg.shard_off, e = sg.shard_off + sg.len;
        if (open && s != cur_end) close(cur_end);        // padding between runs
        int64_t pos = s;
        while (pos < e) {
            if (!open) {
                open = true;
                start = pos;
                tensor = sg.tensor;
            }
            const int64_t next_cut = (pos / be + 1) * be;
            if (next_cut <= e) {
                close(next_cut);
                pos = next_cut;
            } else {
                pos = e;
            }
        }
        cur_end = e;
    }
    if (open) close(cur_end);
    *n_out = (int64_t)bks.size();
    if (!out) return ZERO_OK;
    if (cap < (int64_t)bks.size()) {
        set_error("zero_layout_buckets: capacity %lld < %lld buckets", (long long)cap,
                  (long long)bks.size());
        return ZERO_E_RANGE;
    }
    std::copy(bks.begin(), bks.end(), out);
    return ZERO_OK;
}

int mem(const zero_layout* L, int32_t stage, int64_t* v, bool bytes) {
    if (!L || !v) {
        set_error("zero_layout_mem: NULL argument");
        return ZERO_E_INVAL;
    }
    const int64_t P = L->info.padded_L, Pn = L->info.shard_S;
    // per-parameter widths: (parameters, gradients, optimizer state)
    const int64_t wp = bytes ? 2 : 1, wg = bytes ? 2 : 1, ws = bytes ? 12 : 2;
    int64_t np_, ng, ns;
    switch (stage) {
        case 0: np_ = P;  ng = P;  ns = P;  break;   // plain data parallel
        case 1: np_ = P;  ng = P;  ns = Pn; break;   // optimizer states partitioned
        case 2: np_ = P;  ng = Pn; ns = Pn; break;   // + gradients partitioned
        case 3: np_ = Pn; ng = Pn; ns = Pn; break;   // + parameters partitioned
        default:
            set_error("zero_layout_mem: stage %d outside [0, 3]", (int)stage);
            return ZERO_E_INVAL;
    }
    int64_t a, b, c, t1, t2;
    if (!mul_ok(np_, wp, &a) || !mul_ok(ng, wg, &b) || !mul_ok(ns, ws, &c) || !add_ok(a, b, &t1) ||
        !add_ok(t1, c, &t2)) {
        set_error("zero_layout_mem: overflow");
        return ZERO_E_RANGE;
    }
    v[0] = a;
    v[1] = b;
    v[2] = c;
    v[3] = t2;
    return ZERO_OK;
}

}  // namespace zl

extern "C" {

int zero_layout_build(const int64_t* numels, int64_t n_tensors, int32_t world_N,
                      int64_t tensor_align_A, int64_t shard_align_B, zero_layout** out) {
    return zl::build(numels, n_tensors, world_N, tensor_align_A, shard_align_B, out);
}

int zero_layout_info_get(const zero_layout* layout, zero_layout_info* out) {
    if (!layout || !out) {
        zl::set_error("zero_layout_info_get: NULL argument");
        return ZERO_E_INVAL;
    }
    *out = layout->info;
    return ZERO_OK;
}

int zero_layout_offsets(const zero_layout* layout, int64_t* out) {
    if (!layout || (!out && layout->info.n_tensors > 0)) {
        zl::set_error("zero_layout_offsets: NULL argument");
        return ZERO_E_INVAL;
    }
    std::copy(layout->offsets.begin(), layout->offsets.end(), out);
    return ZERO_OK;
}

int zero_layout_segments(const zero_layout* layout, int32_t rank, zero_segment* out, int64_t cap,
                         int64_t* n_out) {
    return zl::segments(layout, rank, out, cap, n_out);
}

int zero_layout_buckets(const zero_layout* layout, int32_t rank, int64_t bucket_elems,
                        zero_bucket* out, int64_t cap, int64_t* n_out) {
    return zl::buckets(layout, rank, bucket_elems, out, cap, n_out);
}

int zero_layout_mem_values(const zero_layout* layout, int32_t stage, int64_t* values) {
    return zl::mem(layout, stage, values, false);
}

int zero_layout_mem_bytes(const zero_layout* layout, int32_t stage, int64_t* values) {
    return zl::mem(layout, stage, values, true);
}

void zero_layout_free(zero_layout* layout) { delete layout; }

}  // extern "C"
