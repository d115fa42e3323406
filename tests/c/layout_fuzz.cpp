// Differential fuzz of the host layout code (layout.cpp) against the oracle's
// (oracle.c), meant to be built with AddressSanitizer and UBSan: random tensor
// lists, rank counts, alignments and bucket sizes; every offset, size, segment,
// bucket and memory figure must agree, and the error paths must not crash.
// Usage: layout_fuzz <iterations> <seed>; exit status 0 when all agree.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "zero.h"

namespace zl {
void set_error(const char*, ...) {}   // error text lives in abi.cpp, not built here
}

extern "C" {
int or_layout(const int64_t* numels, int64_t T, int64_t N, int64_t A, int64_t B, int64_t* offsets,
              int64_t* out3);
int64_t or_segments(const int64_t* numels, const int64_t* offsets, int64_t T, int64_t S, int64_t r,
                    int64_t* out, int64_t cap);
int64_t or_buckets(const int64_t* segs, int64_t nseg, int64_t S, int64_t bucket_elems, int64_t* out,
                   int64_t cap);
int or_mem_values(int64_t L_pad, int64_t S, int32_t stage, int64_t* out);
int or_mem_bytes(int64_t L_pad, int64_t S, int32_t stage, int64_t* out);
}

static uint64_t st;
static uint64_t rnd() {
    uint64_t z = (st += 0x9E3779B97F4A7C15ULL);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}
static int64_t pick(int64_t lo, int64_t hi) { return lo + (int64_t)(rnd() % (uint64_t)(hi - lo + 1)); }

#define REQUIRE(c)                                                              \
    do {                                                                        \
        if (!(c)) {                                                             \
            fprintf(stderr, "iteration %d: check failed at line %d: %s\n", it, __LINE__, #c); \
            return 1;                                                           \
        }                                                                       \
    } while (0)

int main(int argc, char** argv) {
    const int iters = argc > 1 ? atoi(argv[1]) : 2000;
    st = argc > 2 ? strtoull(argv[2], nullptr, 10) : 1;
    const int64_t aligns[] = {1, 2, 3, 8, 256};
    const int64_t grains[] = {1, 4, 8, 16};
    for (int it = 0; it < iters; ++it) {
        const int64_t T = pick(0, 40);
        std::vector<int64_t> numels((size_t)(T > 0 ? T : 1));
        for (int64_t i = 0; i < T; ++i) numels[(size_t)i] = (rnd() % 7 == 0) ? 0 : pick(1, 5000);
        const int32_t N = (int32_t)pick(1, 64);
        const int64_t A = aligns[rnd() % 5], B = grains[rnd() % 4];
        zero_layout* L = nullptr;
        REQUIRE(zero_layout_build(numels.data(), T, N, A, B, &L) == ZERO_OK);
        zero_layout_info info;
        REQUIRE(zero_layout_info_get(L, &info) == ZERO_OK);
        std::vector<int64_t> off((size_t)(T > 0 ? T : 1)), ooff((size_t)(T > 0 ? T : 1));
        int64_t out3[3];
        REQUIRE(or_layout(numels.data(), T, N, A, B, ooff.data(), out3) == 0);
        REQUIRE(zero_layout_offsets(L, off.data()) == ZERO_OK);
        for (int64_t i = 0; i < T; ++i) REQUIRE(off[(size_t)i] == ooff[(size_t)i]);
        REQUIRE(info.used_L == out3[0] && info.shard_S == out3[1] && info.padded_L == out3[2]);
        for (int stage = 0; stage < 4; ++stage) {
            int64_t a[4], b[4];
            REQUIRE(zero_layout_mem_values(L, stage, a) == ZERO_OK);
            REQUIRE(or_mem_values(out3[2], out3[1], stage, b) == 0);
            for (int k = 0; k < 4; ++k) REQUIRE(a[k] == b[k]);
            REQUIRE(zero_layout_mem_bytes(L, stage, a) == ZERO_OK);
            REQUIRE(or_mem_bytes(out3[2], out3[1], stage, b) == 0);
            for (int k = 0; k < 4; ++k) REQUIRE(a[k] == b[k]);
        }
        for (int rep = 0; rep < 3; ++rep) {
            const int32_t r = (int32_t)pick(0, N - 1);
            int64_t n = 0;
            REQUIRE(zero_layout_segments(L, r, nullptr, 0, &n) == ZERO_OK);
            std::vector<zero_segment> seg((size_t)(n + 1));
            REQUIRE(zero_layout_segments(L, r, seg.data(), n, &n) == ZERO_OK);
            std::vector<int64_t> oseg((size_t)(4 * (T + 1)));
            const int64_t on = or_segments(numels.data(), ooff.data(), T, out3[1], r, oseg.data(), T + 1);
            REQUIRE(on == n);
            for (int64_t k = 0; k < n; ++k) {
                REQUIRE(seg[(size_t)k].tensor == oseg[(size_t)(4 * k)]);
                REQUIRE(seg[(size_t)k].tensor_off == oseg[(size_t)(4 * k + 1)]);
                REQUIRE(seg[(size_t)k].shard_off == oseg[(size_t)(4 * k + 2)]);
                REQUIRE(seg[(size_t)k].len == oseg[(size_t)(4 * k + 3)]);
            }
            const int64_t be = pick(1, 3000);
            int64_t nb = 0;
            REQUIRE(zero_layout_buckets(L, r, be, nullptr, 0, &nb) == ZERO_OK);
            std::vector<zero_bucket> bk((size_t)(nb + 1));
            REQUIRE(zero_layout_buckets(L, r, be, bk.data(), nb, &nb) == ZERO_OK);
            const int64_t cap = on + out3[1] / be + 2;
            std::vector<int64_t> ob((size_t)(3 * cap));
            const int64_t onb = or_buckets(oseg.data(), on, out3[1], be, ob.data(), cap);
            REQUIRE(onb == nb);
            for (int64_t k = 0; k < nb; ++k) {
                REQUIRE(bk[(size_t)k].shard_off == ob[(size_t)(3 * k)]);
                REQUIRE(bk[(size_t)k].len == ob[(size_t)(3 * k + 1)]);
                REQUIRE(bk[(size_t)k].tensor == ob[(size_t)(3 * k + 2)]);
            }
            if (n > 0) {
                int64_t got = 0;
                REQUIRE(zero_layout_segments(L, r, seg.data(), n - 1, &got) == ZERO_E_RANGE && got == n);
            }
        }
        zero_layout_free(L);
    }
    // error paths
    const int64_t huge[2] = {INT64_C(1) << 62, INT64_C(1) << 62};
    zero_layout* L = nullptr;
    int it = -1;
    REQUIRE(zero_layout_build(huge, 2, 2, 1, 8, &L) == ZERO_E_RANGE && L == nullptr);
    const int64_t neg[2] = {5, -5};
    REQUIRE(zero_layout_build(neg, 2, 2, 1, 8, &L) == ZERO_E_INVAL);
    REQUIRE(zero_layout_build(nullptr, 3, 2, 1, 8, &L) == ZERO_E_INVAL);
    REQUIRE(zero_layout_build(nullptr, 0, 2, 1, 8, &L) == ZERO_OK);
    zero_layout_free(L);
    printf("layout_fuzz ok (%d iterations)\n", iters);
    return 0;
}
