/*
 * oracle.c -- plain, slow CPU oracle for the per-rank ZeRO stage-1/2 shard step.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the CPU-baseline
 * leg of the benchmark are the only code that may load this library. The GPU
 * product path never calls it and shares no code, header or table with it.
 *
 * Every function here is written from the method's definition, in the order the
 * sources give it, with no blocking, fusion or reordering beyond that order:
 *
 *   - flat layout and shard cut: the gradients are partitioned so that each
 *     rank's gradient slice lines up with the optimizer-state and parameter
 *     slice it owns ("[REQUEST] Direct Correspondence between Gradient and
 *     Optimizer States to Reduce Communication", section "Problem"); the
 *     gradients live in one contiguous buffer ("Why does not the stage 3
 *     implementation use broadcast and reduce-scatter?", the replies on
 *     contiguous_gradients); small tensors are grouped into buckets ("ZeRO
 *     Optimizer" wiki page, "Communication Optimization").
 *   - memory accounting: "ZeRO Optimizer", sections "Memory Components" and
 *     "Theoretical Reductions".
 *   - ring reduce-scatter / all-gather: "Why DeepSpeed ZeRO paper says
 *     reduce-scatter (or all-gather) has data movement of Psi elements?",
 *     the ring walk in GuanhuaWang's reply and the all-gather count in
 *     civat's follow-up.
 *   - the step: reduce-scatter of the gradients, update of the own partition,
 *     all-gather of the updated parameters ("[REQUEST] ...", "Problem"); Adam
 *     keeps m and v per parameter ("[REQUEST] ...", "Thoughts and viewpoints";
 *     "ZeRO Optimizer", "Memory Components"). The Adam formula itself is not on
 *     the pages: it is Kingma & Ba 2015 (Algorithm 1), with decoupled weight
 *     decay from Loshchilov & Hutter 2019 (AdamW).
 *
 * Numerics: the optimizer state is fp32 and the gradient replicas are bf16 (or
 * fp32); every floating-point operation below is one IEEE-754 operation in the
 * type of its operands, rounded to nearest-even.  Build with -ffp-contract=off
 * so that no multiply-add is contracted.  The reduction is a left fold in slot
 * order; a float64 exact-sum variant (or_reduce_f64) is provided to bound it.
 *
 * Parity pins (tests/test_oracle_*.py): hand-derived layout example, brute-force
 * element maps, page memory formulas, a message-passing ring simulation, the
 * Higham bound for recursive summation against math.fsum, torch.optim.Adam /
 * AdamW in float64, Adam closed forms, torch's float32->bfloat16 cast.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ECAP (-2)

/* ------------------------------------------------------------------------ */
/* Layout                                                                    */
/* ------------------------------------------------------------------------ */

static int64_t or_align_up(int64_t x, int64_t a) { return ((x + a - 1) / a) * a; }

/*
 * Flat layout of T tensors and the cut into N equal shards.
 *   offsets[0] = 0, offsets[i] = align_up(offsets[i-1] + numels[i-1], A)
 *   L     = offsets[T-1] + numels[T-1]      (0 when T == 0)
 *   S     = align_up(ceil(L / N), B)        (per-rank shard length)
 *   L_pad = N * S                           (padded flat length)
 * out3 = {L, S, L_pad}.
 */
int or_layout(const int64_t* numels, int64_t T, int64_t N, int64_t A, int64_t B,
              int64_t* offsets, int64_t* out3) {
    if (T < 0 || N < 1 || A < 1 || B < 1) return OR_EINVAL;
    int64_t end = 0;
    for (int64_t i = 0; i < T; i++) {
        if (numels[i] < 0) return OR_EINVAL;
        int64_t o = (i == 0) ? 0 : or_align_up(end, A);
        offsets[i] = o;
        end = o + numels[i];
    }
    int64_t L = end;
    int64_t per_rank = (L + N - 1) / N;
    int64_t S = or_align_up(per_rank, B);
    out3[0] = L;
    out3[1] = S;
    out3[2] = N * S;
    return OR_OK;
}

/*
 * Segments of rank r: for every tensor i (ascending) that meets the rank's
 * window [r*S, (r+1)*S), one record
 *   {i, a - offsets[i], a - r*S, b - a}  with a = max(offsets[i], r*S),
 *                                              b = min(offsets[i] + numels[i], (r+1)*S).
 * out holds 4 int64 per record. Returns the count, or OR_ECAP if cap is too small.
 */
int64_t or_segments(const int64_t* numels, const int64_t* offsets, int64_t T, int64_t S,
                    int64_t r, int64_t* out, int64_t cap) {
    int64_t lo = r * S, hi = (r + 1) * S, n = 0;
    for (int64_t i = 0; i < T; i++) {
        int64_t a = offsets[i] > lo ? offsets[i] : lo;
        int64_t e = offsets[i] + numels[i];
        int64_t b = e < hi ? e : hi;
        if (a < b) {
            if (n >= cap) return OR_ECAP;
            out[4 * n + 0] = i;
            out[4 * n + 1] = a - offsets[i];
            out[4 * n + 2] = a - lo;
            out[4 * n + 3] = b - a;
            n++;
        }
    }
    return n;
}

/*
 * Buckets of rank r: walk the shard element by element; an element belongs to a
 * bucket if some segment covers it. A bucket is a maximal run of covered
 * elements that does not cross a multiple of bucket_elems (shard-local); with
 * bucket_elems <= 0 runs are never cut. Each bucket is recorded as
 * {shard_off, len, tensor of its first element} (3 int64 per record).
 * This walks every element on purpose: it is the plain definition, for small S.
 */
int64_t or_buckets(const int64_t* segs, int64_t nseg, int64_t S, int64_t bucket_elems,
                   int64_t* out, int64_t cap) {
    int64_t* owner = (int64_t*)malloc(sizeof(int64_t) * (size_t)(S > 0 ? S : 1));
    if (!owner) return OR_EINVAL;
    for (int64_t k = 0; k < S; k++) owner[k] = -1;
    for (int64_t s = 0; s < nseg; s++)
        for (int64_t k = 0; k < segs[4 * s + 3]; k++) owner[segs[4 * s + 2] + k] = segs[4 * s + 0];
    int64_t n = 0, start = -1;
    for (int64_t k = 0; k <= S; k++) {
        int covered = (k < S) && owner[k] >= 0;
        int cut = (k < S) && bucket_elems > 0 && (k % bucket_elems) == 0;
        if (start >= 0 && (!covered || cut)) {
            if (n >= cap) { free(owner); return OR_ECAP; }
            out[3 * n + 0] = start;
            out[3 * n + 1] = k - start;
            out[3 * n + 2] = owner[start];
            n++;
            start = -1;
        }
        if (covered && start < 0) start = k;
    }
    free(owner);
    return n;
}

/*
 * Memory per device in "values" ("ZeRO Optimizer", "Memory Components" and
 * "Theoretical Reductions"), with P := L_pad and P/N := S.
 * out = {parameters, gradients, optimizer states (m and v), total}.
 * stage 0 = plain data parallelism: P, P, 2P.
 * stage 1 = optimizer states partitioned: P, P, 2P/N.
 * stage 2 = gradients partitioned too: P, P/N, 2P/N.
 * stage 3 = parameters partitioned too: P/N, P/N, 2P/N.
 */
int or_mem_values(int64_t L_pad, int64_t S, int32_t stage, int64_t* out) {
    int64_t P = L_pad, Pn = S, par, grd, st;
    switch (stage) {
        case 0: par = P;  grd = P;  st = 2 * P;  break;
        case 1: par = P;  grd = P;  st = 2 * Pn; break;
        case 2: par = P;  grd = Pn; st = 2 * Pn; break;
        case 3: par = Pn; grd = Pn; st = 2 * Pn; break;
        default: return OR_EINVAL;
    }
    out[0] = par; out[1] = grd; out[2] = st; out[3] = par + grd + st;
    return OR_OK;
}

/*
 * The same partitioning in bytes for this step's dtypes: bf16 parameters and
 * gradients (2 B each), fp32 master copy plus m plus v (12 B) per parameter.
 */
int or_mem_bytes(int64_t L_pad, int64_t S, int32_t stage, int64_t* out) {
    int64_t P = L_pad, Pn = S, par, grd, st;
    switch (stage) {
        case 0: par = 2 * P;  grd = 2 * P;  st = 12 * P;  break;
        case 1: par = 2 * P;  grd = 2 * P;  st = 12 * Pn; break;
        case 2: par = 2 * P;  grd = 2 * Pn; st = 12 * Pn; break;
        case 3: par = 2 * Pn; grd = 2 * Pn; st = 12 * Pn; break;
        default: return OR_EINVAL;
    }
    out[0] = par; out[1] = grd; out[2] = st; out[3] = par + grd + st;
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Ring collectives, simulated by message passing between N virtual ranks    */
/* ------------------------------------------------------------------------ */

static float or_hold(float x, int32_t wire_dtype);

/*
 * Standard ring reduce-scatter. Rank k holds its full local gradient
 * bufs[k*N*S ...], cut into N chunks of S. In step s = 0 .. N-2 every rank k
 * sends its running partial of chunk (k-1-s) mod N to rank k+1, which adds its
 * own local copy of that chunk to what it received (received + own, fp32).
 * After N-1 steps chunk c sits fully reduced at its owner c:
 *   out[c*S + e]. order[c*N + h] = the rank whose data was the h-th term of
 * chunk c. sent[k] / recv[k] count elements moved by rank k.
 * wire_dtype: the type the running partials are held and sent in. OR_F32
 * keeps them in fp32; OR_BF16 rounds every partial to bf16 (round to nearest
 * even) when it is formed, as a ring whose buffers and messages are bf16 does.
 */
int or_ring_rs_wire(const float* bufs, int64_t N, int64_t S, int32_t wire_dtype, float* out,
                    int64_t* sent, int64_t* recv, int64_t* order) {
    if (N < 1 || S < 0) return OR_EINVAL;
    /* partial[k] = the chunk rank k currently holds a running sum of */
    float* partial = (float*)malloc(sizeof(float) * (size_t)(N * (S > 0 ? S : 1)));
    float* msg = (float*)malloc(sizeof(float) * (size_t)(N * (S > 0 ? S : 1)));
    int64_t* pchunk = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    int64_t* nterms = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    int64_t* newchunk = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    if (!partial || !msg || !pchunk || !nterms || !newchunk) {
        free(partial); free(msg); free(pchunk); free(nterms); free(newchunk);
        return OR_EINVAL;
    }
    for (int64_t k = 0; k < N; k++) { sent[k] = 0; recv[k] = 0; }
    for (int64_t c = 0; c < N; c++) nterms[c] = 0;
    /* step "-1": rank k starts chunk (k-1) mod N with its own data */
    for (int64_t k = 0; k < N; k++) {
        int64_t c = ((k - 1) % N + N) % N;
        pchunk[k] = c;
        for (int64_t e = 0; e < S; e++) partial[k * S + e] = or_hold(bufs[k * N * S + c * S + e], wire_dtype);
        order[c * N + nterms[c]++] = k;
    }
    for (int64_t s = 0; s + 1 < N; s++) {
        /* every rank sends its partial to the right neighbour */
        for (int64_t k = 0; k < N; k++) {
            int64_t dst = (k + 1) % N;
            memcpy(msg + dst * S, partial + k * S, sizeof(float) * (size_t)S);
            sent[k] += S;
            recv[dst] += S;
        }
        /* every rank adds its own copy of the chunk it just received */
        for (int64_t k = 0; k < N; k++) newchunk[k] = pchunk[((k - 1) % N + N) % N];
        for (int64_t k = 0; k < N; k++) {
            int64_t c = newchunk[k];
            const float* own = bufs + k * N * S + c * S;
            for (int64_t e = 0; e < S; e++)
                partial[k * S + e] = or_hold(msg[k * S + e] + own[e], wire_dtype);
            pchunk[k] = c;
            order[c * N + nterms[c]++] = k;
        }
    }
    int rc = OR_OK;
    for (int64_t k = 0; k < N; k++) {
        if (pchunk[k] != k) { rc = OR_EINVAL; break; }
        memcpy(out + k * S, partial + k * S, sizeof(float) * (size_t)S);
    }
    free(partial); free(msg); free(pchunk); free(nterms); free(newchunk);
    return rc;
}

int or_ring_rs(const float* bufs, int64_t N, int64_t S, float* out, int64_t* sent,
               int64_t* recv, int64_t* order) {
    return or_ring_rs_wire(bufs, N, S, 0 /* fp32 */, out, sent, recv, order);
}

/*
 * The walk exactly as GuanhuaWang's reply tells it for the first chunk: chunk c
 * starts at rank c, travels c -> c+1 -> ... -> c-1 with every rank adding its
 * own copy, and the finished sum takes one more hop back to c. All N chunks
 * travel at once, one hop per step, N steps in total.
 */
int or_ring_rs_walk(const float* bufs, int64_t N, int64_t S, float* out, int64_t* sent,
                    int64_t* recv, int64_t* order) {
    if (N < 1 || S < 0) return OR_EINVAL;
    for (int64_t k = 0; k < N; k++) { sent[k] = 0; recv[k] = 0; }
    float* run = (float*)malloc(sizeof(float) * (size_t)(N * (S > 0 ? S : 1)));
    if (!run) return OR_EINVAL;
    for (int64_t c = 0; c < N; c++) {
        memcpy(run + c * S, bufs + c * N * S + c * S, sizeof(float) * (size_t)S);
        order[c * N + 0] = c;
    }
    for (int64_t h = 1; h <= N; h++) {
        for (int64_t c = 0; c < N; c++) {
            int64_t from = (c + h - 1) % N, to = (c + h) % N;
            sent[from] += S;
            recv[to] += S;
            if (h < N) {
                const float* own = bufs + to * N * S + c * S;
                for (int64_t e = 0; e < S; e++) run[c * S + e] = run[c * S + e] + own[e];
                order[c * N + h] = to;
            }
        }
    }
    memcpy(out, run, sizeof(float) * (size_t)(N * S));
    free(run);
    return OR_OK;
}

/*
 * Ring all-gather: rank k starts with its own chunk; in step s = 0 .. N-2 every
 * rank forwards the chunk it received last (first: its own) to rank k+1.
 * gathered[k*N*S ...] is rank k's full buffer afterwards.
 */
int or_ring_ag(const float* chunks, int64_t N, int64_t S, float* gathered, int64_t* sent,
               int64_t* recv) {
    if (N < 1 || S < 0) return OR_EINVAL;
    int64_t* holding = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    int64_t* next = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    for (int64_t k = 0; k < N; k++) {
        sent[k] = 0; recv[k] = 0;
        for (int64_t e = 0; e < N * S; e++) gathered[k * N * S + e] = NAN;
        memcpy(gathered + k * N * S + k * S, chunks + k * S, sizeof(float) * (size_t)S);
        holding[k] = k;
    }
    for (int64_t s = 0; s + 1 < N; s++) {
        for (int64_t k = 0; k < N; k++) {
            int64_t dst = (k + 1) % N, c = holding[k];
            memcpy(gathered + dst * N * S + c * S, gathered + k * N * S + c * S,
                   sizeof(float) * (size_t)S);
            sent[k] += S;
            recv[dst] += S;
            next[dst] = c;
        }
        for (int64_t k = 0; k < N; k++) holding[k] = next[k];
    }
    free(holding); free(next);
    return OR_OK;
}

/*
 * Stage-3 fetch of one tensor: the parameters are partitioned like the flat
 * buffer (rank r owns [r*S, (r+1)*S)) and gathered before the layer that uses
 * them ("ZeRO Optimizer", "ZeRO Stages" stage 3 and "Communication Patterns",
 * all-gather of only the required parameter subset). Element e of the tensor at
 * flat offset `offset` is element (offset + e) - r*S of rank r's shard, with
 * r = (offset + e) / S. elem_bytes is 2 (bf16 parameters) or 4; the copy is
 * bitwise.
 */
int or_gather_tensor(const void* const* shards, int64_t N, int64_t S, int32_t elem_bytes,
                     int64_t offset, int64_t n, void* out) {
    if (N < 1 || S < 1 || n < 0 || offset < 0 || offset + n > N * S ||
        (elem_bytes != 2 && elem_bytes != 4))
        return OR_EINVAL;
    for (int64_t e = 0; e < n; e++) {
        int64_t f = offset + e;
        int64_t r = f / S;
        const char* src = (const char*)shards[r] + (size_t)(f - r * S) * (size_t)elem_bytes;
        memcpy((char*)out + (size_t)e * (size_t)elem_bytes, src, (size_t)elem_bytes);
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* bfloat16                                                                  */
/* ------------------------------------------------------------------------ */

static uint32_t or_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float or_from_bits(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 pattern. */
float or_bf16_to_f32(uint16_t h) { return or_from_bits(((uint32_t)h) << 16); }

/*
 * fp32 -> bf16, round to nearest, ties to even, by definition: take the two
 * bf16 neighbours of x (truncation toward zero, and one bf16 ulp further from
 * zero), measure both distances exactly in double, keep the nearer, and on a
 * tie keep the one whose last mantissa bit is 0. Overflow goes to infinity
 * (the far neighbour of the largest finite bf16 is the infinity pattern, at
 * distance 2^128 - x). Any NaN becomes the quiet NaN 0x7FC0.
 */
uint16_t or_f32_to_bf16(float x) {
    if (isnan(x)) return 0x7FC0;
    uint32_t u = or_bits(x);
    uint32_t lo = u & 0xFFFF0000u;          /* toward zero */
    if (lo == u) return (uint16_t)(lo >> 16); /* exactly representable (incl. inf) */
    uint32_t hi = lo + 0x10000u;            /* away from zero (may be the inf pattern) */
    double ax = fabs((double)x);
    double alo = fabs((double)or_from_bits(lo));
    double ahi;
    if ((hi & 0x7FFFFFFFu) == 0x7F800000u) ahi = ldexp(1.0, 128);
    else ahi = fabs((double)or_from_bits(hi));
    double dlo = ax - alo, dhi = ahi - ax;
    if (dlo < dhi) return (uint16_t)(lo >> 16);
    if (dhi < dlo) return (uint16_t)(hi >> 16);
    return ((lo >> 16) & 1u) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);
}

void or_f32_to_bf16_array(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = or_f32_to_bf16(x[i]);
}

/* x as held in a buffer of wire_dtype: unchanged for fp32, rounded to bf16 for bf16. */
static float or_hold(float x, int32_t wire_dtype) {
    return wire_dtype == 0 ? x : or_bf16_to_f32(or_f32_to_bf16(x));
}

/* ------------------------------------------------------------------------ */
/* The step                                                                  */
/* ------------------------------------------------------------------------ */

#define OR_F32 0
#define OR_BF16 1
#define OR_BF16_WIRE 2    /* bf16 replicas summed as a bf16 ring does: each partial rounded */

static float or_load(const void* base, int32_t dtype, int64_t i) {
    if (dtype == OR_BF16 || dtype == OR_BF16_WIRE) return or_bf16_to_f32(((const uint16_t*)base)[i]);
    return ((const float*)base)[i];
}

/* One hop of the fold: the fp32 sum, held in bf16 when the wire is bf16. */
static float or_fold_add(float acc, float x, int32_t dtype) {
    return or_hold(acc + x, dtype == OR_BF16_WIRE ? OR_BF16 : OR_F32);
}

/* 1 / (N * loss_scale), computed in double and rounded once to fp32. */
float or_inv_scale(int32_t N, double loss_scale) {
    return (float)(1.0 / ((double)N * loss_scale));
}

/*
 * Average + unscale + overflow + squared norm of one shard (or of a sample of
 * its elements: every element is independent).
 *   acc   = R_0[i] + R_1[i] + ... + R_{N-1}[i]   left fold, fp32, slot order
 *   g[i]  = acc * inv,  inv = or_inv_scale(N, loss_scale)
 *   flag  = 1 if any g[i] is inf or NaN
 *   sumsq = sum of (double)g[i] * (double)g[i]
 * reps[j] is the j-th slot of the slot table (its own dtype-sized array of n).
 * dtype OR_BF16_WIRE: bf16 replicas whose running sum is rounded to bf16 after
 * every add, what each rank of the ring walk in GuanhuaWang's reply ("Why
 * DeepSpeed ZeRO paper says reduce-scatter ... Psi elements?") holds and sends
 * on when its buffers are bf16; the pages leave the precision open.
 */
void or_reduce(const void* const* reps, int32_t N, int32_t dtype, int64_t n,
               double loss_scale, float* g_out, uint32_t* flag_out, double* sumsq_out,
               int32_t nthreads) {
    float inv = or_inv_scale(N, loss_scale);
    uint32_t flag = 0;
    double sumsq = 0.0;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static) reduction(| : flag) reduction(+ : sumsq)
#endif
    for (int64_t i = 0; i < n; i++) {
        float acc = or_load(reps[0], dtype, i);
        for (int32_t j = 1; j < N; j++) acc = or_fold_add(acc, or_load(reps[j], dtype, i), dtype);
        float g = acc * inv;
        if (!isfinite(g)) flag |= 1u;
        sumsq += (double)g * (double)g;
        if (g_out) g_out[i] = g;
    }
    *flag_out = flag;
    *sumsq_out = sumsq;
}

/*
 * Exact-sum reference for the reduction: the replicas widened to double and
 * summed in double (exact for bf16 terms of similar magnitude), times
 * 1/(N*loss_scale) in double. Used only to bound the fp32 fold.
 */
void or_reduce_f64(const void* const* reps, int32_t N, int32_t dtype, int64_t n,
                   double loss_scale, double* g_out, double* abssum_out) {
    double inv = 1.0 / ((double)N * loss_scale);
    for (int64_t i = 0; i < n; i++) {
        double acc = 0.0, aacc = 0.0;
        for (int32_t j = 0; j < N; j++) {
            double x = (double)or_load(reps[j], dtype, i);
            acc += x;
            aacc += fabs(x);
        }
        g_out[i] = acc * inv;
        if (abssum_out) abssum_out[i] = aacc * inv;
    }
}

/*
 * The fp32 scalars of update number t (t >= 1), each computed in double and
 * rounded once: out = {b1, b2, 1-b1, 1-b2, bc1, bc2, lr, eps, decay}
 * with bc = 1 - beta^t where beta^t is the t-fold product beta*beta*...*beta
 * in double, and decay = 1 - lr*wd (decoupled weight decay).
 */
void or_adam_scalars(double lr, double beta1, double beta2, double eps, double wd,
                     int64_t t, float* out) {
    double p1 = 1.0, p2 = 1.0;
    for (int64_t k = 0; k < t; k++) { p1 = p1 * beta1; p2 = p2 * beta2; }
    out[0] = (float)beta1;
    out[1] = (float)beta2;
    out[2] = (float)(1.0 - beta1);
    out[3] = (float)(1.0 - beta2);
    out[4] = (float)(1.0 - p1);
    out[5] = (float)(1.0 - p2);
    out[6] = (float)lr;
    out[7] = (float)eps;
    out[8] = (float)(1.0 - lr * wd);
}

/*
 * Adam / AdamW update of n shard elements (Kingma & Ba 2015, Algorithm 1;
 * decoupled decay of Loshchilov & Hutter 2019), one fp32 operation per line:
 *   m'  = b1*m + (1-b1)*g
 *   v'  = b2*v + (1-b2)*(g*g)
 *   mh  = m'/bc1 ;  vh = v'/bc2
 *   den = sqrt(vh) + eps
 *   u   = mh/den
 *   p'  = p*decay - lr*u
 *   slot = bf16_rne(p')
 * Outputs may alias inputs element-for-element. slot_out may be NULL.
 */
void or_adam(const float* g, const float* p, const float* m, const float* v, int64_t n,
             double lr, double beta1, double beta2, double eps, double wd, int64_t t,
             float* p_out, float* m_out, float* v_out, uint16_t* slot_out, int32_t nthreads) {
    float sc[9];
    or_adam_scalars(lr, beta1, beta2, eps, wd, t, sc);
    const float b1 = sc[0], b2 = sc[1], omb1 = sc[2], omb2 = sc[3];
    const float bc1 = sc[4], bc2 = sc[5], lr_f = sc[6], eps_f = sc[7], decay = sc[8];
#ifdef _OPENMP
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t i = 0; i < n; i++) {
        float gi = g[i];
        float mt = b1 * m[i];
        float mg = omb1 * gi;
        float m1 = mt + mg;
        float gg = gi * gi;
        float vt = b2 * v[i];
        float vg = omb2 * gg;
        float v1 = vt + vg;
        float mh = m1 / bc1;
        float vh = v1 / bc2;
        float den = sqrtf(vh) + eps_f;
        float u = mh / den;
        float p1 = p[i] * decay;
        float lu = lr_f * u;
        float pn = p1 - lu;
        p_out[i] = pn;
        m_out[i] = m1;
        v_out[i] = v1;
        if (slot_out) slot_out[i] = or_f32_to_bf16(pn);
    }
}

/*
 * One full step of one rank (reduce -> average/unscale -> overflow check and
 * squared norm -> Adam on the shard -> bf16 into the own slot), with the skip
 * rule: when any g is non-finite nothing is written to p, m, v or the slot.
 * p, m, v and slot are updated in place. Returns the overflow flag (0/1);
 * *sumsq_out gets the shard's squared gradient norm.
 */
int or_step(const void* const* reps, int32_t N, int32_t dtype, int64_t n, double loss_scale,
            float* p, float* m, float* v, uint16_t* slot, double lr, double beta1, double beta2,
            double eps, double wd, int64_t t, double* sumsq_out, int32_t nthreads) {
    float* g = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    if (!g) return OR_EINVAL;
    uint32_t flag = 0;
    or_reduce(reps, N, dtype, n, loss_scale, g, &flag, sumsq_out, nthreads);
    if (!flag) or_adam(g, p, m, v, n, lr, beta1, beta2, eps, wd, t, p, m, v, slot, nthreads);
    free(g);
    return (int)flag;
}
