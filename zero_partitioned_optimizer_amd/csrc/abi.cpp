// abi.cpp -- the C entry points of libzero that launch device work: argument
// validation, the fp32 scalars of an update, error text, and the host-side
// commit rule. Kernels live in step_kernels.hip, the layout in layout.cpp.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <string>
#include <vector>

#include "zero.h"
#include "zero_internal.h"

namespace zl {

static thread_local std::string g_err;

void set_error(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
}

}  // namespace zl

namespace {

using zl::set_error;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    const char* name;
    uintptr_t lo, hi;               // [lo, hi)
};

Span span(const char* name, const void* p, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{name, lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlap(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi; }

int hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return ZERO_OK;
    set_error("%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
    return ZERO_E_HIP;
}

// beta^t as the t-fold product in double (1.0 * beta * beta * ...). A per-thread
// memo of the last (beta, t, beta^t) per beta lets consecutive steps extend the
// product by one multiply instead of t.
double pow_t(double beta, int64_t t) {
    struct Memo {
        double beta;
        int64_t t;
        double value;
    };
    static thread_local Memo memo[2] = {{-1.0, -1, 1.0}, {-1.0, -1, 1.0}};
    static thread_local int next = 0;
    Memo* m = nullptr;
    for (Memo& x : memo)
        if (x.beta == beta && x.t >= 0 && x.t <= t) m = &x;
    if (!m) {
        m = &memo[next];
        next ^= 1;
        *m = Memo{beta, 0, 1.0};
    }
    double v = m->value;
    for (int64_t k = m->t; k < t; ++k) v = v * beta;
    m->t = t;
    m->value = v;
    return v;
}

zk::Scalars adam_scalars(const zero_adam_args& a, int32_t n, double loss_scale) {
    zk::Scalars s;
    s.inv = (float)(1.0 / ((double)n * loss_scale));
    s.b1 = (float)a.beta1;
    s.b2 = (float)a.beta2;
    s.omb1 = (float)(1.0 - a.beta1);
    s.omb2 = (float)(1.0 - a.beta2);
    s.bc1 = (float)(1.0 - pow_t(a.beta1, a.step_t));
    s.bc2 = (float)(1.0 - pow_t(a.beta2, a.step_t));
    s.lr = (float)a.lr;
    s.eps = (float)a.eps;
    s.decay = (float)(1.0 - a.lr * a.weight_decay);
    return s;
}

int64_t elem_bytes(zero_dtype dt) { return dt == ZERO_F32 ? 4 : 2; }

// Floats of one tiled state set (three sections per tile of ZERO_STATE_TILE).
int64_t tiled_floats(int64_t S) {
    return 3 * ((S + ZERO_STATE_TILE - 1) / ZERO_STATE_TILE) * ZERO_STATE_TILE;
}

// state_layout must be split or tiled; a tiled state takes m and v from the p
// buffers, so their pointers must be NULL.
int check_layout(const char* fn, int32_t layout, const void* const* mv, int n_mv) {
    if (layout != ZERO_STATE_SPLIT && layout != ZERO_STATE_TILED) {
        set_error("%s: unknown state_layout %d", fn, (int)layout);
        return ZERO_E_INVAL;
    }
    if (layout == ZERO_STATE_TILED)
        for (int i = 0; i < n_mv; ++i)
            if (mv[i]) {
                set_error("%s: a tiled state keeps m and v in the p buffers; the m and v pointers "
                          "must be NULL", fn);
                return ZERO_E_INVAL;
            }
    return ZERO_OK;
}

int check_replicas(const char* fn, const void* const* replicas, int32_t n, zero_dtype dt,
                   int64_t S) {
    if (!replicas) {
        set_error("%s: replicas is NULL", fn);
        return ZERO_E_INVAL;
    }
    if (n < 1 || n > ZERO_MAX_REPLICAS) {
        set_error("%s: n_replicas=%d outside [1, %d]", fn, (int)n, ZERO_MAX_REPLICAS);
        return ZERO_E_RANGE;
    }
    if (dt != ZERO_F32 && dt != ZERO_BF16 && dt != ZERO_BF16_WIRE) {
        set_error("%s: grad_dtype %d is not ZERO_F32, ZERO_BF16 or ZERO_BF16_WIRE", fn, (int)dt);
        return ZERO_E_INVAL;
    }
    for (int32_t j = 0; j < n; ++j) {
        if (!replicas[j] && S > 0) {
            set_error("%s: replicas[%d] is NULL", fn, (int)j);
            return ZERO_E_INVAL;
        }
        if (!aligned16(replicas[j])) {
            set_error("%s: replicas[%d]=%p is not 16-byte aligned", fn, (int)j, replicas[j]);
            return ZERO_E_ALIGN;
        }
    }
    return ZERO_OK;
}

// lib_ws: the workspace is the library's own scratch (the allocation-free entry
// point): only its size is checked, against the launch capped at max_grid.
int check_common(const char* fn, int64_t S, const zero_bucket* buckets, int64_t n_buckets,
                 const zero_stats* stats, const void* ws, size_t ws_bytes, int32_t n_rep,
                 bool lib_ws = false, int max_grid = 0) {
    if (S < 0) {
        set_error("%s: shard_S=%lld is negative", fn, (long long)S);
        return ZERO_E_RANGE;
    }
    if (n_buckets < 0) {
        set_error("%s: n_buckets=%lld is negative", fn, (long long)n_buckets);
        return ZERO_E_RANGE;
    }
    if (n_buckets > 0 && !buckets) {
        set_error("%s: n_buckets=%lld with a NULL bucket table", fn, (long long)n_buckets);
        return ZERO_E_INVAL;
    }
    if (n_buckets > 0 && (reinterpret_cast<uintptr_t>(buckets) & 7u)) {
        set_error("%s: bucket table %p is not 8-byte aligned", fn, (const void*)buckets);
        return ZERO_E_ALIGN;
    }
    if (!stats || (!ws && !lib_ws)) {
        set_error("%s: stats_dev or workspace_dev is NULL", fn);
        return ZERO_E_INVAL;
    }
    if (!aligned16(stats) || !aligned16(ws)) {
        set_error("%s: stats_dev or workspace_dev is not 16-byte aligned", fn);
        return ZERO_E_ALIGN;
    }
    const size_t need = (size_t)zk::grid_for(S, n_buckets, n_rep, max_grid) * zk::kPartialBytes +
                        zk::rep_table_bytes(n_rep);
    if (ws_bytes < need) {
        if (lib_ws)
            set_error("%s: the launch needs %zu bytes of scratch, more than the %zu this entry "
                      "point holds", fn, need, ws_bytes);
        else
            set_error("%s: workspace of %zu bytes < %zu needed", fn, ws_bytes, need);
        return ZERO_E_RANGE;
    }
    return ZERO_OK;
}

bool finite_in(double x, double lo, double hi) { return isfinite(x) && x >= lo && x < hi; }

}  // namespace

namespace zl {

int hip_error(hipError_t e, const char* where) { return hip_status(e, where); }

zk::Scalars update_scalars(double lr, double beta1, double beta2, double eps, double wd,
                           int64_t t) {
    zero_adam_args a{};
    a.lr = lr;
    a.beta1 = beta1;
    a.beta2 = beta2;
    a.eps = eps;
    a.weight_decay = wd;
    a.step_t = t;
    return adam_scalars(a, 1, 1.0);
}

}  // namespace zl

extern "C" {

const char* zero_last_error(void) { return zl::g_err.c_str(); }

const char* zero_version(void) { return "libzero 1.0 (gfx950)"; }

size_t zero_workspace_bytes(int64_t shard_S) {
    // the device-commit layout (CommitWs) is the larger one; a host-commit call
    // uses its first grid * kPartialBytes bytes and the pointer table at the end
    return (size_t)zk::grid_bound(shard_S) * zk::kCommitSlotBytes + zk::kFlagBytes +
           zk::kRepTableMax;
}

int zero_reduce_shard(const void* const* replicas, int32_t n_replicas, zero_dtype grad_dtype,
                      int64_t shard_S, const zero_bucket* buckets_dev, int64_t n_buckets,
                      double loss_scale, float* grad_out_dev, zero_stats* stats_dev,
                      void* workspace_dev, size_t ws_bytes, void* stream) {
    static const char* fn = "zero_reduce_shard";
    int rc = check_replicas(fn, replicas, n_replicas, grad_dtype, shard_S);
    if (rc) return rc;
    rc = check_common(fn, shard_S, buckets_dev, n_buckets, stats_dev, workspace_dev, ws_bytes,
                      n_replicas);
    if (rc) return rc;
    if (!(isfinite(loss_scale) && loss_scale > 0.0)) {
        set_error("%s: loss_scale=%g must be finite and > 0", fn, loss_scale);
        return ZERO_E_INVAL;
    }
    if (grad_out_dev && !aligned16(grad_out_dev)) {
        set_error("%s: grad_out_dev is not 16-byte aligned", fn);
        return ZERO_E_ALIGN;
    }
    // Aliasing: the outputs (grad_out, stats, workspace) must be pairwise disjoint
    // and disjoint from every replica and from the bucket table.
    const int64_t gb = elem_bytes(grad_dtype);
    const Span outs[] = {span("grad_out", grad_out_dev, grad_out_dev ? 4 * shard_S : 0),
                         span("stats", stats_dev, 16),
                         span("workspace", workspace_dev, (int64_t)ws_bytes)};
    const int n_outs = 3;
    for (int i = 0; i < n_outs; ++i) {
        for (int k = i + 1; k < n_outs; ++k)
            if (overlap(outs[i], outs[k])) {
                set_error("%s: outputs %s and %s overlap", fn, outs[i].name, outs[k].name);
                return ZERO_E_INVAL;
            }
        for (int32_t j = 0; j < n_replicas; ++j)
            if (overlap(outs[i], span("replica", replicas[j], gb * shard_S))) {
                set_error("%s: %s overlaps replicas[%d]", fn, outs[i].name, (int)j);
                return ZERO_E_INVAL;
            }
        if (n_buckets > 0 && overlap(outs[i], span("buckets", buckets_dev, 16 * n_buckets))) {
            set_error("%s: %s overlaps the bucket table", fn, outs[i].name);
            return ZERO_E_INVAL;
        }
    }
    zk::StepDesc d{};
    d.replicas = replicas;
    d.n_rep = n_replicas;
    d.rep_table = zk::rep_table_at(workspace_dev, ws_bytes, n_replicas);
    d.dtype = grad_dtype;
    d.S = shard_S;
    d.buckets = n_buckets > 0 ? buckets_dev : nullptr;
    d.n_buckets = n_buckets;
    d.adam = false;
    d.g_out = grad_out_dev;
    d.sc = zk::Scalars{};
    d.sc.inv = (float)(1.0 / ((double)n_replicas * loss_scale));
    d.stats = stats_dev;
    d.partials = static_cast<zk::Partial*>(workspace_dev);
    return hip_status(zk::launch_step(d, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"

// zero_adam_step, with the workspace either the caller's (a.workspace_dev,
// a.ws_bytes) or, for noalloc, the library's scratch: then the checks see no
// workspace buffer, the launch's grid is capped at kNoallocGrid, and the scratch
// address is looked up only once every argument has passed.
static int adam_step(const char* fn, const zero_adam_args* args, bool noalloc, void* stream) {
    if (!args) {
        set_error("%s: args is NULL", fn);
        return ZERO_E_INVAL;
    }
    const zero_adam_args& a = *args;
    const bool fused = a.replicas != nullptr;
    if (fused == (a.grad_f32 != nullptr)) {
        set_error("%s: exactly one of replicas and grad_f32 must be given", fn);
        return ZERO_E_INVAL;
    }
    if (noalloc && (a.workspace_dev || a.ws_bytes)) {
        set_error("%s: takes no workspace (workspace_dev must be NULL and ws_bytes 0)", fn);
        return ZERO_E_INVAL;
    }
    const int max_grid = noalloc ? zk::kNoallocGrid : 0;
    const int64_t S = a.shard_S;
    int rc = check_common(fn, S, a.buckets_dev, a.n_buckets, a.stats_dev, a.workspace_dev,
                          noalloc ? zk::kNoallocBytes : a.ws_bytes, fused ? a.n_replicas : 1,
                          noalloc, max_grid);
    if (rc) return rc;
    if (fused) {
        rc = check_replicas(fn, a.replicas, a.n_replicas, a.grad_dtype, S);
        if (rc) return rc;
    }
    const void* mv[] = {a.m_in, a.v_in, a.m_out, a.v_out};
    rc = check_layout(fn, a.state_layout, mv, 4);
    if (rc) return rc;
    const bool tiled = a.state_layout == ZERO_STATE_TILED;
    const void* need[] = {fused ? (const void*)a.replicas : (const void*)a.grad_f32, a.p_in,
                          tiled ? a.p_in : a.m_in, tiled ? a.p_in : a.v_in, a.p_out,
                          tiled ? a.p_out : a.m_out, tiled ? a.p_out : a.v_out};
    for (const void* p : need) {
        if (!p && (S > 0 || p == (const void*)a.replicas)) {
            set_error("%s: a state or gradient buffer (p/m/v in/out, grad_f32) is NULL", fn);
            return ZERO_E_INVAL;
        }
        if (!aligned16(p) && p != (const void*)a.replicas) {
            set_error("%s: a state or gradient buffer is not 16-byte aligned", fn);
            return ZERO_E_ALIGN;
        }
    }
    if (a.slot_bf16 && !aligned16(a.slot_bf16)) {
        set_error("%s: slot_bf16 is not 16-byte aligned", fn);
        return ZERO_E_ALIGN;
    }
    if (!finite_in(a.beta1, 0.0, 1.0) || !finite_in(a.beta2, 0.0, 1.0) || !(isfinite(a.lr) && a.lr >= 0) ||
        !(isfinite(a.eps) && a.eps >= 0) || !(isfinite(a.weight_decay) && a.weight_decay >= 0) ||
        a.step_t < 1 || (fused && !(isfinite(a.loss_scale) && a.loss_scale > 0))) {
        set_error("%s: hyperparameters out of domain (lr=%g beta1=%g beta2=%g eps=%g wd=%g "
                  "loss_scale=%g t=%lld)", fn, a.lr, a.beta1, a.beta2, a.eps, a.weight_decay,
                  a.loss_scale, (long long)a.step_t);
        return ZERO_E_INVAL;
    }
    // Aliasing: outputs must be pairwise disjoint and disjoint from every input,
    // except that the unfused path may update p, m, v exactly in place.
    const int64_t b4 = 4 * S;
    const int64_t bp = tiled ? 4 * tiled_floats(S) : b4;   // p buffer: the whole set when tiled
    const int64_t bmv = tiled ? 0 : b4;
    const Span outs[] = {span("p_out", a.p_out, bp), span("m_out", a.m_out, bmv),
                         span("v_out", a.v_out, bmv),
                         span("slot", a.slot_bf16, a.slot_bf16 ? 2 * S : 0),
                         span("stats", a.stats_dev, 16),
                         span("workspace", a.workspace_dev, (int64_t)a.ws_bytes)};
    const int n_outs = 6;
    for (int i = 0; i < n_outs; ++i)
        for (int k = i + 1; k < n_outs; ++k)
            if (overlap(outs[i], outs[k])) {
                set_error("%s: outputs %s and %s overlap", fn, outs[i].name, outs[k].name);
                return ZERO_E_INVAL;
            }
    const Span ins_state[] = {span("p_in", a.p_in, bp), span("m_in", a.m_in, bmv),
                              span("v_in", a.v_in, bmv)};
    for (int i = 0; i < n_outs; ++i) {
        for (int k = 0; k < 3; ++k) {
            if (!overlap(outs[i], ins_state[k])) continue;
            const bool exact_alias = !fused && i == k && outs[i].lo == ins_state[k].lo;
            if (!exact_alias) {
                set_error("%s: output %s overlaps input %s%s", fn, outs[i].name, ins_state[k].name,
                          fused ? " (the fused step must be out of place)" : "");
                return ZERO_E_INVAL;
            }
        }
        if (fused) {
            const int64_t gb = elem_bytes(a.grad_dtype);
            for (int32_t j = 0; j < a.n_replicas; ++j)
                if (overlap(outs[i], span("replica", a.replicas[j], gb * S))) {
                    set_error("%s: output %s overlaps replicas[%d]", fn, outs[i].name, (int)j);
                    return ZERO_E_INVAL;
                }
        } else if (overlap(outs[i], span("grad_f32", a.grad_f32, b4))) {
            set_error("%s: output %s overlaps grad_f32", fn, outs[i].name);
            return ZERO_E_INVAL;
        }
        if (a.n_buckets > 0 &&
            overlap(outs[i], span("buckets", a.buckets_dev, 16 * a.n_buckets))) {
            set_error("%s: output %s overlaps the bucket table", fn, outs[i].name);
            return ZERO_E_INVAL;
        }
    }
    void* ws = a.workspace_dev;
    size_t ws_bytes = a.ws_bytes;
    if (noalloc) {
        rc = hip_status(zk::noalloc_scratch(&ws), fn);
        if (rc) return rc;
        ws_bytes = zk::kNoallocBytes;
    }
    const void* one_rep[1] = {a.grad_f32};
    zk::StepDesc d{};
    d.replicas = fused ? a.replicas : one_rep;
    d.n_rep = fused ? a.n_replicas : 1;
    d.rep_table = zk::rep_table_at(ws, ws_bytes, d.n_rep);
    d.dtype = fused ? a.grad_dtype : ZERO_F32;
    d.S = S;
    d.buckets = a.n_buckets > 0 ? a.buckets_dev : nullptr;
    d.n_buckets = a.n_buckets;
    d.adam = true;
    d.p_in = a.p_in;
    d.m_in = a.m_in;
    d.v_in = a.v_in;
    d.p_out = a.p_out;
    d.m_out = a.m_out;
    d.v_out = a.v_out;
    d.slot = a.slot_bf16;
    d.g_out = nullptr;
    d.tiled = tiled;
    // the unfused source is already averaged and unscaled: inv = 1 (x * 1 == x)
    d.sc = adam_scalars(a, fused ? a.n_replicas : 1, fused ? a.loss_scale : 1.0);
    d.stats = a.stats_dev;
    d.partials = static_cast<zk::Partial*>(ws);
    d.ev_begin = static_cast<hipEvent_t>(a.event_begin);
    d.ev_end = static_cast<hipEvent_t>(a.event_end);
    d.max_grid = max_grid;
    return hip_status(zk::launch_step(d, static_cast<hipStream_t>(stream)), fn);
}

extern "C" {

int zero_adam_step(const zero_adam_args* args, void* stream) {
    return adam_step("zero_adam_step", args, false, stream);
}

int zero_adam_step_noalloc(const zero_adam_args* args, void* stream) {
    return adam_step("zero_adam_step_noalloc", args, true, stream);
}

static int check_record_buffers(const char* fn, const zero_device_state* state_dev,
                                const void* workspace_dev, size_t ws_bytes) {
    if (!state_dev || !workspace_dev) {
        set_error("%s: state_dev or workspace_dev is NULL", fn);
        return ZERO_E_INVAL;
    }
    if (!aligned16(state_dev) || !aligned16(workspace_dev)) {
        set_error("%s: state_dev or workspace_dev is not 16-byte aligned", fn);
        return ZERO_E_ALIGN;
    }
    if (overlap(span("state", state_dev, (int64_t)sizeof(zero_device_state)),
                span("workspace", workspace_dev, (int64_t)ws_bytes))) {
        set_error("%s: state_dev and workspace_dev overlap", fn);
        return ZERO_E_INVAL;
    }
    return ZERO_OK;
}

static bool scales_ok(double beta1, double beta2, double loss_scale, double min_loss_scale) {
    return finite_in(beta1, 0.0, 1.0) && finite_in(beta2, 0.0, 1.0) && isfinite(loss_scale) &&
           loss_scale > 0 && isfinite(min_loss_scale) && min_loss_scale > 0 &&
           min_loss_scale <= loss_scale;
}

int zero_device_state_init(zero_device_state* state_dev, void* workspace_dev, size_t ws_bytes,
                           double beta1, double beta2, double loss_scale, double min_loss_scale,
                           int32_t dynamic, void* stream) {
    static const char* fn = "zero_device_state_init";
    int rc = check_record_buffers(fn, state_dev, workspace_dev, ws_bytes);
    if (rc) return rc;
    if (!scales_ok(beta1, beta2, loss_scale, min_loss_scale)) {
        set_error("%s: beta1=%g beta2=%g loss_scale=%g min_loss_scale=%g out of domain", fn, beta1,
                  beta2, loss_scale, min_loss_scale);
        return ZERO_E_INVAL;
    }
    zero_device_state rec{};
    rec.beta1 = beta1;
    rec.beta2 = beta2;
    rec.beta1_pow = 1.0;
    rec.beta2_pow = 1.0;
    rec.loss_scale = loss_scale;
    rec.min_loss_scale = min_loss_scale;
    rec.dynamic = dynamic ? 1u : 0u;
    return hip_status(zk::launch_state_write(state_dev, rec, workspace_dev, ws_bytes,
                                             static_cast<hipStream_t>(stream)),
                      fn);
}

int zero_device_state_load(zero_device_state* state_dev, void* workspace_dev, size_t ws_bytes,
                           const zero_device_state* saved, void* stream) {
    static const char* fn = "zero_device_state_load";
    int rc = check_record_buffers(fn, state_dev, workspace_dev, ws_bytes);
    if (rc) return rc;
    if (!saved) {
        set_error("%s: saved is NULL", fn);
        return ZERO_E_INVAL;
    }
    const zero_device_state& r = *saved;
    if (!scales_ok(r.beta1, r.beta2, r.loss_scale, r.min_loss_scale)) {
        set_error("%s: beta1=%g beta2=%g loss_scale=%g min_loss_scale=%g out of domain", fn,
                  r.beta1, r.beta2, r.loss_scale, r.min_loss_scale);
        return ZERO_E_INVAL;
    }
    const auto pow_ok = [](double x) { return x >= 0.0 && x <= 1.0; };   // false for NaN
    if (r.t < 0 || r.n_skipped < 0 || r.cur > 1u || r.last_overflow > 1u ||
        !pow_ok(r.beta1_pow) || !pow_ok(r.beta2_pow) ||
        (r.t == 0 && (r.beta1_pow != 1.0 || r.beta2_pow != 1.0))) {
        set_error("%s: inconsistent record (t=%lld n_skipped=%lld cur=%u last_overflow=%u "
                  "beta1_pow=%g beta2_pow=%g)",
                  fn, (long long)r.t, (long long)r.n_skipped, r.cur, r.last_overflow, r.beta1_pow,
                  r.beta2_pow);
        return ZERO_E_INVAL;
    }
    if (r.pending_n != 0u) {
        set_error("%s: the saved record has a pending step (pending_n=%u): flush before saving", fn,
                  r.pending_n);
        return ZERO_E_INVAL;
    }
    if (r.error != 0u) {
        set_error("%s: the saved record is frozen by error code %u (a bounded wait of a step ran "
                  "out); resume from a record saved before it", fn, r.error);
        return ZERO_E_INVAL;
    }
    zero_device_state rec = r;
    rec.dynamic = r.dynamic ? 1u : 0u;
    rec.seq = 0u;                    // the cleared workspace holds no tag of an earlier step
    return hip_status(zk::launch_state_write(state_dev, rec, workspace_dev, ws_bytes,
                                             static_cast<hipStream_t>(stream)),
                      fn);
}

int zero_device_state_flush(zero_device_state* state_dev, zero_stats* stats_dev, void* workspace_dev,
                            size_t ws_bytes, void* stream) {
    static const char* fn = "zero_device_state_flush";
    int rc = check_record_buffers(fn, state_dev, workspace_dev, ws_bytes);
    if (rc) return rc;
    if (!stats_dev) {
        set_error("%s: stats_dev is NULL", fn);
        return ZERO_E_INVAL;
    }
    if (!aligned16(stats_dev)) {
        set_error("%s: stats_dev is not 16-byte aligned", fn);
        return ZERO_E_ALIGN;
    }
    const zk::CommitWs cw = zk::commit_ws(workspace_dev, ws_bytes);
    if (cw.cap < 1) {
        set_error("%s: ws_bytes=%zu is smaller than any step's workspace", fn, ws_bytes);
        return ZERO_E_RANGE;
    }
    const Span b[] = {span("state", state_dev, (int64_t)sizeof(zero_device_state)),
                      span("stats", stats_dev, 16),
                      span("workspace", workspace_dev, (int64_t)ws_bytes)};
    for (int i = 0; i < 3; ++i)
        for (int k = i + 1; k < 3; ++k)
            if (overlap(b[i], b[k])) {
                set_error("%s: %s and %s overlap", fn, b[i].name, b[k].name);
                return ZERO_E_INVAL;
            }
    return hip_status(zk::launch_flush(state_dev, stats_dev, cw, static_cast<hipStream_t>(stream)),
                      fn);
}

// Every check of zero_train_step, shared with zero_train_step_part.
static int check_train_args(const char* fn, const zero_train_args* args) {
    if (!args) {
        set_error("%s: args is NULL", fn);
        return ZERO_E_INVAL;
    }
    const zero_train_args& a = *args;
    const int64_t S = a.shard_S;
    int rc = check_replicas(fn, a.replicas, a.n_replicas, a.grad_dtype, S);
    if (rc) return rc;
    rc = check_common(fn, S, a.buckets_dev, a.n_buckets, a.stats_dev, a.workspace_dev, a.ws_bytes,
                      a.n_replicas);
    if (rc) return rc;
    if (!a.state_dev) {
        set_error("%s: state_dev is NULL", fn);
        return ZERO_E_INVAL;
    }
    if (!aligned16(a.state_dev)) {
        set_error("%s: state_dev is not 16-byte aligned", fn);
        return ZERO_E_ALIGN;
    }
    const void* mv[] = {a.m[0], a.m[1], a.v[0], a.v[1]};
    rc = check_layout(fn, a.state_layout, mv, 4);
    if (rc) return rc;
    const bool tiled = a.state_layout == ZERO_STATE_TILED;
    const float* sets[6] = {a.p[0], a.p[1], tiled ? a.p[0] : a.m[0], tiled ? a.p[1] : a.m[1],
                            tiled ? a.p[0] : a.v[0], tiled ? a.p[1] : a.v[1]};
    for (const float* p : sets) {
        if (!p && S > 0) {
            set_error("%s: a state buffer is NULL", fn);
            return ZERO_E_INVAL;
        }
        if (!aligned16(p)) {
            set_error("%s: a state buffer is not 16-byte aligned", fn);
            return ZERO_E_ALIGN;
        }
    }
    if ((a.slot[0] && !aligned16(a.slot[0])) || (a.slot[1] && !aligned16(a.slot[1]))) {
        set_error("%s: a slot buffer is not 16-byte aligned", fn);
        return ZERO_E_ALIGN;
    }
    if (a.slot[1] && !a.slot[0]) {
        set_error("%s: slot[1] given without slot[0]", fn);
        return ZERO_E_INVAL;
    }
    if (!(isfinite(a.lr) && a.lr >= 0) || !(isfinite(a.eps) && a.eps >= 0) ||
        !(isfinite(a.weight_decay) && a.weight_decay >= 0)) {
        set_error("%s: lr=%g eps=%g weight_decay=%g out of domain", fn, a.lr, a.eps, a.weight_decay);
        return ZERO_E_INVAL;
    }
    const int64_t b4 = 4 * S;
    const int64_t bp = tiled ? 4 * tiled_floats(S) : b4;   // p buffer: the whole set when tiled
    const int64_t bmv = tiled ? 0 : b4;
    const Span bufs[] = {span("p[0]", a.p[0], bp), span("p[1]", a.p[1], bp),
                         span("m[0]", a.m[0], bmv), span("m[1]", a.m[1], bmv),
                         span("v[0]", a.v[0], bmv), span("v[1]", a.v[1], bmv),
                         span("slot[0]", a.slot[0], a.slot[0] ? 2 * S : 0),
                         span("slot[1]", a.slot[1], a.slot[1] ? 2 * S : 0),
                         span("stats", a.stats_dev, 16),
                         span("workspace", a.workspace_dev, (int64_t)a.ws_bytes),
                         span("state", a.state_dev, (int64_t)sizeof(zero_device_state))};
    const int nb = 11;
    for (int i = 0; i < nb; ++i) {
        for (int k = i + 1; k < nb; ++k)
            if (overlap(bufs[i], bufs[k])) {
                set_error("%s: buffers %s and %s overlap", fn, bufs[i].name, bufs[k].name);
                return ZERO_E_INVAL;
            }
        const int64_t gb = elem_bytes(a.grad_dtype);
        for (int32_t j = 0; j < a.n_replicas; ++j)
            if (overlap(bufs[i], span("replica", a.replicas[j], gb * S))) {
                set_error("%s: %s overlaps replicas[%d]", fn, bufs[i].name, (int)j);
                return ZERO_E_INVAL;
            }
        if (a.n_buckets > 0 && overlap(bufs[i], span("buckets", a.buckets_dev, 16 * a.n_buckets))) {
            set_error("%s: %s overlaps the bucket table", fn, bufs[i].name);
            return ZERO_E_INVAL;
        }
    }
    return ZERO_OK;
}

// The step descriptor of a whole-shard device-commit launch.
static zk::StepDesc train_desc(const zero_train_args& a) {
    zk::StepDesc d{};
    d.replicas = a.replicas;
    d.n_rep = a.n_replicas;
    d.rep_table = zk::rep_table_at(a.workspace_dev, a.ws_bytes, a.n_replicas);
    d.dtype = a.grad_dtype;
    d.S = a.shard_S;
    d.buckets = a.n_buckets > 0 ? a.buckets_dev : nullptr;
    d.n_buckets = a.n_buckets;
    d.adam = true;
    for (int i = 0; i < 2; ++i) {
        d.set_p[i] = a.p[i];
        d.set_m[i] = a.m[i];
        d.set_v[i] = a.v[i];
    }
    d.ctrl = a.state_dev;
    d.tiled = a.state_layout == ZERO_STATE_TILED;
    d.slot = a.slot[0];
    if (a.slot[1]) {
        d.set_slot[0] = a.slot[0];
        d.set_slot[1] = a.slot[1];
    }
    d.sc = zk::Scalars{};
    d.sc.lr = (float)a.lr;
    d.sc.eps = (float)a.eps;
    d.sc.decay = (float)(1.0 - a.lr * a.weight_decay);
    d.stats = a.stats_dev;
    d.partials = static_cast<zk::Partial*>(a.workspace_dev);
    const zk::CommitWs cw = zk::commit_ws(a.workspace_dev, a.ws_bytes);
    d.ws_half[0] = cw.half[0];
    d.ws_half[1] = cw.half[1];
    d.ws_started = cw.started;
    d.ws_flags = cw.flags;
    d.ev_begin = static_cast<hipEvent_t>(a.event_begin);
    d.ev_end = static_cast<hipEvent_t>(a.event_end);
    return d;
}

int zero_train_step(const zero_train_args* args, void* stream) {
    static const char* fn = "zero_train_step";
    const int rc = check_train_args(fn, args);
    if (rc) return rc;
    const zero_train_args& a = *args;
    const int64_t cap = zk::commit_ws(a.workspace_dev, a.ws_bytes).cap;
    const int grid = zk::grid_for(a.shard_S, a.n_buckets, a.n_replicas);
    if (cap < grid) {
        set_error("%s: ws_bytes=%zu holds %lld workgroup slots of a device-committed step, %d "
                  "needed (zero_workspace_bytes)", fn, a.ws_bytes, (long long)cap, grid);
        return ZERO_E_RANGE;
    }
    const zk::StepDesc d = train_desc(*args);
    return hip_status(zk::launch_step(d, static_cast<hipStream_t>(stream)), fn);
}

int zero_train_step_part(const zero_train_args* args, const int64_t* part_ends, int32_t n_parts,
                         int32_t part, void* stream) {
    static const char* fn = "zero_train_step_part";
    int rc = check_train_args(fn, args);
    if (rc) return rc;
    const zero_train_args& a = *args;
    const int64_t S = a.shard_S;
    if (a.n_buckets > 0) {
        set_error("%s: parts cover element ranges; a bucket table is not supported", fn);
        return ZERO_E_UNSUPPORTED;
    }
    if (!part_ends) {
        set_error("%s: part_ends is NULL", fn);
        return ZERO_E_INVAL;
    }
    if (n_parts < 1 || n_parts > zk::kMaxParts || part < 0 || part >= n_parts) {
        set_error("%s: part %d of n_parts=%d out of range", fn, (int)part, (int)n_parts);
        return ZERO_E_RANGE;
    }
    // boundaries: non-decreasing, multiples of 8 elements (16 bytes; of ZERO_STATE_TILE
    // with a tiled state, so that a part starts on a tile), the last one S;
    // every part gets at most kGridMax / n_parts workgroups, so the partial slots
    // of all parts fit the workspace of a whole-shard step
    const int part_cap = zk::kGridMax / n_parts;
    const bool tiled = a.state_layout == ZERO_STATE_TILED;
    const int64_t gran = tiled ? ZERO_STATE_TILE : 8;
    int64_t prev = 0, total = 0, base = 0;
    for (int32_t k = 0; k < n_parts; ++k) {
        const int64_t e = part_ends[k];
        const bool last = k == n_parts - 1;
        if (e < prev || e > S || (last ? e != S : (e % gran) != 0)) {
            set_error("%s: part_ends[%d]=%lld invalid (previous %lld, shard_S %lld; inner ends "
                      "must be multiples of %lld, the last must equal shard_S)",
                      fn, (int)k, (long long)e, (long long)prev, (long long)S, (long long)gran);
            return ZERO_E_RANGE;
        }
        const int64_t g = zk::grid_for(e - prev, 0, a.n_replicas, part_cap);
        if (k == part) base = total;
        total += g;
        prev = e;
    }
    const int64_t cap = zk::commit_ws(a.workspace_dev, a.ws_bytes).cap;
    if (total > cap || total > INT32_MAX) {
        set_error("%s: the %d parts need %lld workgroup slots, ws_bytes=%zu holds %lld", fn,
                  (int)n_parts, (long long)total, a.ws_bytes, (long long)cap);
        return ZERO_E_RANGE;
    }
    const int64_t lo = part == 0 ? 0 : part_ends[part - 1], hi = part_ends[part];
    const bool last = part == n_parts - 1;
    zk::StepDesc d = train_desc(a);
    const int64_t gb = elem_bytes(a.grad_dtype);
    const void* shifted[ZERO_MAX_REPLICAS];
    for (int32_t j = 0; j < a.n_replicas; ++j)
        shifted[j] = static_cast<const char*>(a.replicas[j]) + lo * gb;
    d.replicas = shifted;
    d.S = hi - lo;
    for (int i = 0; i < 2; ++i) {
        if (tiled) {
            d.set_p[i] = a.p[i] + lo / ZERO_STATE_TILE * 3 * ZERO_STATE_TILE;   // lo starts a tile
        } else {
            d.set_p[i] = a.p[i] + lo;
            d.set_m[i] = a.m[i] + lo;
            d.set_v[i] = a.v[i] + lo;
        }
        if (d.set_slot[i]) d.set_slot[i] = d.set_slot[i] + lo;
    }
    if (d.slot) d.slot = d.slot + lo;
    d.part_base = (int32_t)base;
    d.max_grid = part_cap;
    d.collect_n = last ? (int32_t)total : -1;
    d.no_restore = true;
    rc = hip_status(zk::launch_step(d, static_cast<hipStream_t>(stream)), fn);
    if (rc || !last || !a.slot[0] || a.slot[1]) return rc;
    return hip_status(zk::launch_restore(a.state_dev, zk::commit_ws(a.workspace_dev, a.ws_bytes).flags,
                                         a.p[0], a.p[1], a.slot[0], S, tiled,
                                         static_cast<hipStream_t>(stream)),
                      fn);
}

int zero_gather_tensors(const void* const* shards, int32_t n_shards, int64_t shard_S,
                        int32_t elem_bytes, const int64_t* offsets, const int64_t* numels,
                        void* const* outs, int32_t n_tensors, void* stream) {
    static const char* fn = "zero_gather_tensors";
    if (n_tensors < 0) {
        set_error("%s: n_tensors=%d is negative", fn, (int)n_tensors);
        return ZERO_E_RANGE;
    }
    if (!shards || (n_tensors > 0 && (!offsets || !numels || !outs))) {
        set_error("%s: shards, offsets, numels or outs is NULL", fn);
        return ZERO_E_INVAL;
    }
    if (n_shards < 1 || n_shards > zk::kGatherMaxShards || shard_S < 1 ||
        shard_S > (int64_t(1) << 40)) {
        set_error("%s: n_shards=%d shard_S=%lld out of range", fn, (int)n_shards,
                  (long long)shard_S);
        return ZERO_E_RANGE;
    }
    if (elem_bytes != 2 && elem_bytes != 4) {
        set_error("%s: elem_bytes=%d is neither 2 nor 4", fn, (int)elem_bytes);
        return ZERO_E_INVAL;
    }
    const int64_t L_pad = (int64_t)n_shards * shard_S;
    const uintptr_t eb = (uintptr_t)elem_bytes;
    for (int32_t r = 0; r < n_shards; ++r) {
        if (!shards[r] || (reinterpret_cast<uintptr_t>(shards[r]) % eb) != 0) {
            set_error("%s: shards[%d]=%p is NULL or not element-aligned", fn, (int)r, shards[r]);
            return shards[r] ? ZERO_E_ALIGN : ZERO_E_INVAL;
        }
    }
    for (int32_t k = 0; k < n_tensors; ++k) {
        const int64_t o = offsets[k], n = numels[k];
        if (o < 0 || n < 0 || o > L_pad || n > L_pad - o) {
            set_error("%s: tensor %d at offset %lld with %lld elements leaves the %lld-element "
                      "buffer", fn, (int)k, (long long)o, (long long)n, (long long)L_pad);
            return ZERO_E_RANGE;
        }
        if (n > 0 && !outs[k]) {
            set_error("%s: outs[%d] is NULL", fn, (int)k);
            return ZERO_E_INVAL;
        }
        if ((reinterpret_cast<uintptr_t>(outs[k]) % eb) != 0) {
            set_error("%s: outs[%d]=%p is not element-aligned", fn, (int)k, outs[k]);
            return ZERO_E_ALIGN;
        }
        const Span sk = span("out", outs[k], n * elem_bytes);
        for (int32_t r = 0; r < n_shards && n > 0; ++r)
            if (overlap(sk, span("shard", shards[r], shard_S * elem_bytes))) {
                set_error("%s: outs[%d] overlaps shards[%d]", fn, (int)k, (int)r);
                return ZERO_E_INVAL;
            }
    }
    // outputs pairwise disjoint: sorted by start, two non-empty outputs overlap
    // exactly when some output starts before its predecessor in that order ends
    std::vector<int32_t> order;
    order.reserve((size_t)n_tensors);
    for (int32_t k = 0; k < n_tensors; ++k)
        if (numels[k] > 0) order.push_back(k);
    std::sort(order.begin(), order.end(), [outs](int32_t x, int32_t y) {
        return reinterpret_cast<uintptr_t>(outs[x]) < reinterpret_cast<uintptr_t>(outs[y]);
    });
    for (size_t i = 1; i < order.size(); ++i) {
        const int32_t j = order[i - 1], k = order[i];
        if (overlap(span("out", outs[j], numels[j] * elem_bytes),
                    span("out", outs[k], numels[k] * elem_bytes))) {
            set_error("%s: outs[%d] overlaps outs[%d]", fn, (int)(j > k ? j : k), (int)(j < k ? j : k));
            return ZERO_E_INVAL;
        }
    }
    return hip_status(zk::launch_gather(shards, n_shards, shard_S, elem_bytes, offsets, numels, outs,
                                        n_tensors, static_cast<hipStream_t>(stream)),
                      fn);
}

static int gather_slot(const char* fn, const float* master_dev, int64_t shard_S, bool tiled,
                       uint16_t* slot_bf16_dev, void* stream) {
    if (shard_S < 0) {
        set_error("%s: shard_S=%lld is negative", fn, (long long)shard_S);
        return ZERO_E_RANGE;
    }
    if (shard_S > 0 && (!master_dev || !slot_bf16_dev)) {
        set_error("%s: NULL buffer", fn);
        return ZERO_E_INVAL;
    }
    if (!aligned16(master_dev) || !aligned16(slot_bf16_dev)) {
        set_error("%s: buffers must be 16-byte aligned", fn);
        return ZERO_E_ALIGN;
    }
    const int64_t mb = 4 * (tiled ? tiled_floats(shard_S) : shard_S);
    if (overlap(span("master", master_dev, mb), span("slot", slot_bf16_dev, 2 * shard_S))) {
        set_error("%s: master and slot overlap", fn);
        return ZERO_E_INVAL;
    }
    if (shard_S == 0) return ZERO_OK;
    return hip_status(zk::launch_cast_slot(master_dev, shard_S, tiled, slot_bf16_dev,
                                           static_cast<hipStream_t>(stream)), fn);
}

int zero_gather_slot(const float* master_dev, int64_t shard_S, uint16_t* slot_bf16_dev,
                     void* stream) {
    return gather_slot("zero_gather_slot", master_dev, shard_S, false, slot_bf16_dev, stream);
}

int zero_gather_slot_tiled(const float* set_dev, int64_t shard_S, uint16_t* slot_bf16_dev,
                           void* stream) {
    return gather_slot("zero_gather_slot_tiled", set_dev, shard_S, true, slot_bf16_dev, stream);
}

int64_t zero_state_set_floats(int64_t shard_S, int32_t state_layout) {
    if (shard_S < 0) return -1;
    if (state_layout == ZERO_STATE_SPLIT) return 3 * shard_S;
    if (state_layout == ZERO_STATE_TILED) return tiled_floats(shard_S);
    return -1;
}

static int state_convert(const char* fn, bool unpack, float* set_dev, int64_t S, float* p, float* m,
                         float* v, void* stream) {
    if (S < 0) {
        set_error("%s: shard_S=%lld is negative", fn, (long long)S);
        return ZERO_E_RANGE;
    }
    if (S > 0 && (!set_dev || (!unpack && (!p || !m || !v)))) {
        set_error("%s: NULL buffer", fn);
        return ZERO_E_INVAL;
    }
    if (!aligned16(set_dev) || !aligned16(p) || !aligned16(m) || !aligned16(v)) {
        set_error("%s: buffers must be 16-byte aligned", fn);
        return ZERO_E_ALIGN;
    }
    const Span b[] = {span("set", set_dev, 4 * tiled_floats(S)), span("p", p, p ? 4 * S : 0),
                      span("m", m, m ? 4 * S : 0), span("v", v, v ? 4 * S : 0)};
    for (int i = 0; i < 4; ++i)
        for (int k = i + 1; k < 4; ++k)
            if (overlap(b[i], b[k])) {
                set_error("%s: buffers %s and %s overlap", fn, b[i].name, b[k].name);
                return ZERO_E_INVAL;
            }
    if (S == 0) return ZERO_OK;
    return hip_status(zk::launch_state_convert(unpack, set_dev, p, m, v, S,
                                               static_cast<hipStream_t>(stream)), fn);
}

int zero_state_pack(const float* p_dev, const float* m_dev, const float* v_dev, int64_t shard_S,
                    float* set_dev, void* stream) {
    return state_convert("zero_state_pack", false, set_dev, shard_S, const_cast<float*>(p_dev),
                         const_cast<float*>(m_dev), const_cast<float*>(v_dev), stream);
}

int zero_state_unpack(const float* set_dev, int64_t shard_S, float* p_dev, float* m_dev,
                      float* v_dev, void* stream) {
    return state_convert("zero_state_unpack", true, const_cast<float*>(set_dev), shard_S, p_dev, m_dev,
                         v_dev, stream);
}

int zero_commit_rule(zero_train_state* state, const zero_stats* stats_host) {
    if (!state || !stats_host) {
        set_error("zero_commit_rule: NULL argument");
        return ZERO_E_INVAL;
    }
    if (stats_host->overflow == 0u) {
        state->t += 1;
        return ZERO_COMMIT;
    }
    state->n_skipped += 1;
    if (state->dynamic) {
        const double floor = state->min_loss_scale > 0 ? state->min_loss_scale : 1.0;
        const double half = state->loss_scale / 2.0;
        state->loss_scale = half > floor ? half : floor;
    }
    return ZERO_SKIP;
}

}  // extern "C"
