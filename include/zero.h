/*
 * zero.h -- C ABI of libzero: the per-rank ZeRO stage-1/2 optimizer step on one
 * GPU's share of the work (AMD Instinct MI355X, gfx950).
 *
 * What the step computes. After forward and backward, the gradients of all
 * data-parallel ranks are partitioned so that each rank's gradient slice lines
 * up with the optimizer-state and parameter slice it owns; a reduce-scatter
 * delivers to every rank the sum of its slice over all ranks; the rank updates
 * its slice of the parameters with its slice of the optimizer state; an
 * all-gather then hands the updated parameters to everyone ("[REQUEST] Direct
 * Correspondence between Gradient and Optimizer States to Reduce
 * Communication", section "Problem"). The sum arrives in ring order: the
 * partial sum of a slice is passed from rank to rank, each adding its own copy
 * ("Why DeepSpeed ZeRO paper says reduce-scatter (or all-gather) has data
 * movement of Psi elements?", GuanhuaWang's reply). The optimizer is Adam, whose
 * two moments m and v live only on the owning rank ("ZeRO Optimizer",
 * "Memory Components" and "ZeRO Stages"; the Adam formula is Kingma & Ba 2015,
 * Algorithm 1, with decoupled weight decay after Loshchilov & Hutter 2019).
 *
 * On one GPU the N gradient replicas of this rank's shard are already resident
 * in HBM (one per simulated rank, in slot order); the library folds them,
 * averages and unscales, checks for overflow, updates fp32 master / m / v and
 * writes the bf16 result into this rank's slot of the gathered parameter buffer.
 *
 * Conventions (all entry points):
 *  - Element counts and offsets are int64. Device pointers are plain pointers
 *    to memory on the current HIP device; the caller owns all device memory and
 *    the library never allocates device memory.
 *  - Every call returns a zero_status. Argument checks are synchronous and
 *    happen before any launch; no C++ exception crosses the ABI. On a non-OK
 *    return, zero_last_error() gives a thread-local description.
 *  - Kernels are enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *    the default stream). No entry point synchronizes, except the offloaded
 *    step zero_offload_step, which waits for its own copies and host updates.
 *    zero_layout_*, zero_commit_rule and zero_host_adam are host-only and
 *    synchronous.
 *  - Device buffers must be 16-byte aligned (dwordx4 access).
 */
#ifndef ZERO_SHARD_STEP_H
#define ZERO_SHARD_STEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_ABI_VERSION 1
#define ZERO_MAX_REPLICAS 1024

typedef enum {
    ZERO_OK = 0,
    ZERO_E_INVAL = -1,        /* a required pointer is NULL, a value is out of its domain, or buffers overlap */
    ZERO_E_ALIGN = -2,        /* a device pointer is not 16-byte aligned */
    ZERO_E_RANGE = -3,        /* a size, rank or capacity is out of range */
    ZERO_E_NOMEM = -4,        /* host allocation failed (layout objects only) */
    ZERO_E_HIP = -5,          /* the HIP runtime reported an error at launch */
    ZERO_E_UNSUPPORTED = -6   /* a valid but unsupported combination */
} zero_status;

/*
 * Element type of the gradient replicas, and how the fold holds its running sum:
 *   ZERO_F32       fp32 replicas, fp32 running sum;
 *   ZERO_BF16      bf16 replicas, fp32 running sum (never rounded between adds);
 *   ZERO_BF16_WIRE bf16 replicas, the running sum rounded to bf16 (nearest,
 *                  ties to even) after every add: what each GPU of the ring walk
 *                  in GuanhuaWang's reply ("Why DeepSpeed ZeRO paper says
 *                  reduce-scatter (or all-gather) has data movement of Psi
 *                  elements?") holds and passes on when its buffers are bf16.
 *                  The pages leave that precision open; ZERO_BF16 is the default
 *                  reading, this one reproduces a bf16 ring bit for bit.
 */
typedef enum { ZERO_F32 = 0, ZERO_BF16 = 1, ZERO_BF16_WIRE = 2 } zero_dtype;

/*
 * How the fp32 state of a shard (master p, Adam moments m and v; "ZeRO
 * Optimizer", "Memory Components") sits in device memory. The pages fix no
 * layout; the step reads and writes all three together, element by element.
 *   ZERO_STATE_SPLIT  three arrays p, m, v of shard_S floats each.
 *   ZERO_STATE_TILED  one buffer per state set of
 *                     zero_state_set_floats(shard_S, ZERO_STATE_TILED) floats:
 *                     tiles of ZERO_STATE_TILE elements, tile k holding p, then
 *                     m, then v of shard elements [k*T, (k+1)*T) (T =
 *                     ZERO_STATE_TILE), i.e. element e of p, m, v at floats
 *                     (e / T)*3T + e % T + {0, T, 2T}. Elements of the last tile
 *                     at or beyond shard_S are never read or written. A step then
 *                     streams one state buffer in and one out instead of three
 *                     and three, which HBM serves faster on this GPU.
 * Entry points taking a state_layout field read m and v from the p buffers
 * when it is ZERO_STATE_TILED, and then require the m and v pointers to be NULL.
 */
#define ZERO_STATE_TILE 8192
typedef enum { ZERO_STATE_SPLIT = 0, ZERO_STATE_TILED = 1 } zero_state_layout;

/* ------------------------------------------------------------------------ */
/* Flat layout and shard cut (host only)                                      */
/* ------------------------------------------------------------------------ */

/* Opaque, immutable once built; safe to share between threads. */
typedef struct zero_layout zero_layout;

typedef struct {
    int64_t n_tensors;
    int64_t psi;              /* sum of the tensors' element counts */
    int64_t used_L;           /* end of the last tensor in the flat buffer */
    int64_t padded_L;         /* N * shard_S */
    int64_t shard_S;          /* elements per rank */
    int64_t tensor_align_A;
    int64_t shard_align_B;
    int32_t world_N;
    int32_t reserved;
} zero_layout_info;

/* One tensor's piece inside one rank's shard. */
typedef struct {
    int32_t tensor;
    int32_t reserved;
    int64_t tensor_off;       /* first element of the piece, inside the tensor */
    int64_t shard_off;        /* first element of the piece, inside the shard */
    int64_t len;
} zero_segment;

/* A padding-free run of shard elements, 16 bytes, copied to the device as is. */
typedef struct {
    int64_t shard_off;
    int32_t len;
    int32_t tensor;           /* tensor holding the bucket's first element */
} zero_bucket;

/*
 * Build the flat layout of n_tensors tensors and cut it into world_N shards.
 * The gradient, parameter and optimizer-state buffers all share this one flat
 * layout, so every rank's gradient slice matches its state slice ("[REQUEST]
 * Direct Correspondence ...", "Problem"; one contiguous gradient buffer as in
 * the contiguous_gradients replies of "Why does not the stage 3 implementation
 * use broadcast and reduce-scatter?"):
 *   offset[0] = 0, offset[i] = align_up(offset[i-1] + numels[i-1], tensor_align_A)
 *   used_L    = offset[T-1] + numels[T-1]        (0 for T = 0)
 *   shard_S   = align_up(ceil(used_L / world_N), shard_align_B)
 *   padded_L  = world_N * shard_S
 * numels: host array of n_tensors counts (>= 0). world_N in [1, 2^20];
 * tensor_align_A, shard_align_B in [1, 2^20]. On success *out owns a new layout
 * (release with zero_layout_free). Errors: ZERO_E_INVAL (NULL, negative count,
 * out-of-domain argument), ZERO_E_RANGE (int64 overflow), ZERO_E_NOMEM.
 */
int zero_layout_build(const int64_t* numels, int64_t n_tensors, int32_t world_N,
                      int64_t tensor_align_A, int64_t shard_align_B, zero_layout** out);

/* Copy the layout's sizes into *out. Errors: ZERO_E_INVAL on NULL. */
int zero_layout_info_get(const zero_layout* layout, zero_layout_info* out);

/* Copy the n_tensors flat offsets into out (host array, n_tensors entries). */
int zero_layout_offsets(const zero_layout* layout, int64_t* out);

/*
 * Segments of rank `rank`: one per tensor that meets [rank*S, (rank+1)*S), in
 * tensor order. With out == NULL only *n_out is set (the count). If cap is
 * smaller than the count, nothing is written, *n_out is the count and the
 * call returns ZERO_E_RANGE. Errors: ZERO_E_RANGE for rank outside [0, N).
 */
int zero_layout_segments(const zero_layout* layout, int32_t rank, zero_segment* out,
                         int64_t cap, int64_t* n_out);

/*
 * Buckets of rank `rank`: the maximal runs of shard elements covered by some
 * tensor (no alignment padding inside), cut where the shard-local index is a
 * multiple of bucket_elems. Small tensors are grouped this way ("ZeRO
 * Optimizer", "Communication Optimization"), and the table lets a step skip
 * padding. bucket_elems in [1, 2^30]. Capacity protocol as for segments.
 */
int zero_layout_buckets(const zero_layout* layout, int32_t rank, int64_t bucket_elems,
                        zero_bucket* out, int64_t cap, int64_t* n_out);

/*
 * Per-device memory under each stage ("ZeRO Optimizer", "Memory Components"
 * and "Theoretical Reductions"), with P := padded_L and P/N := shard_S.
 * values[0..3] = parameters, gradients, optimizer states (m + v), total, in
 * values (elements): stage 0 (plain data parallel) P, P, 2P; stage 1 P, P, 2P/N;
 * stage 2 P, P/N, 2P/N; stage 3 P/N, P/N, 2P/N. Errors: ZERO_E_INVAL.
 */
int zero_layout_mem_values(const zero_layout* layout, int32_t stage, int64_t* values);

/*
 * The same accounting in bytes for this library's dtypes: bf16 parameters and
 * gradients (2 B), fp32 master + m + v (12 B) per parameter of the state.
 */
int zero_layout_mem_bytes(const zero_layout* layout, int32_t stage, int64_t* values);

void zero_layout_free(zero_layout* layout);

/* ------------------------------------------------------------------------ */
/* Device step                                                               */
/* ------------------------------------------------------------------------ */

/* Written (not accumulated) by every reduce / Adam call; 16 bytes, device. */
typedef struct {
    uint32_t overflow;        /* 1 if any averaged gradient element is inf or NaN */
    uint32_t bad_buckets;     /* buckets skipped because they leave [0, shard_S) */
    double sumsq;             /* sum over the processed elements of g*g, in fp64 */
} zero_stats;

/*
 * Bytes of device workspace a reduce, Adam or train-step call on a shard of
 * shard_S elements needs. Per workgroup slot (one workgroup per 1,024 elements
 * plus one per part of a split step, at most 4,096, capped at 4,194,304 slots):
 * 24 bytes of fp64 partials for a host-commit call; for a device-committed
 * record 56 bytes (the partials of two consecutive steps and a start mark, about
 * 46 MB for a 842M-element shard) and 64 bytes of flag words. At the end, 8 KB +
 * 16 for the device table of replica pointers that a call with more than 256
 * replicas uses (the first 256 pointers travel in the kernel arguments). The
 * same workspace may be reused by consecutive calls on one stream; calls that
 * run concurrently need their own.
 */
size_t zero_workspace_bytes(int64_t shard_S);

/*
 * Reduce the N gradient replicas of this rank's shard ("[REQUEST] Direct
 * Correspondence ...", "Problem": the reduce-scatter half of the step; the
 * order is the ring walk of "Why DeepSpeed ZeRO paper says reduce-scatter (or
 * all-gather) has data movement of Psi elements?"), average over the N ranks
 * and unscale by the loss scale, flag overflow and form the squared norm:
 *   acc = R_0[i] + R_1[i] + ... + R_{N-1}[i]   fp32, left to right in slot order
 *   g   = acc * inv,  inv = fp32(1 / (N * loss_scale)) rounded once from double
 *   stats->overflow = any g non-finite; stats->sumsq = sum (double)g * g
 * replicas: host array of n_replicas device pointers (slot order), each shard_S
 *   elements of grad_dtype. n_replicas in [1, ZERO_MAX_REPLICAS]. Up to 256
 *   pointers travel in the kernel arguments; beyond that the call first writes
 *   all n_replicas pointers into the last 8 * n_replicas (+ up to 16) bytes of
 *   the workspace with a small kernel on `stream`, and the step reads them
 *   there (the workspace must then hold that table after its partials).
 * buckets_dev, n_buckets: device bucket table; only elements inside buckets are
 *   written and count towards the flag and the norm (NULL, 0 = the whole
 *   shard). A group of four elements (4k .. 4k+3) cut by a bucket edge is read
 *   whole, so up to three elements beyond each edge, inside the shard, are read
 *   and never written. Buckets must not overlap; one that leaves [0, shard_S)
 *   is skipped and counted in stats->bad_buckets.
 * grad_out_dev: fp32 [shard_S] output of g, or NULL.
 * stats_dev: device zero_stats. workspace_dev/ws_bytes: >= zero_workspace_bytes.
 * The outputs (grad_out, stats, workspace) must not overlap one another, a
 * replica or the bucket table (ZERO_E_INVAL).
 * Errors: ZERO_E_INVAL, ZERO_E_ALIGN, ZERO_E_RANGE, ZERO_E_HIP.
 */
int zero_reduce_shard(const void* const* replicas, int32_t n_replicas, zero_dtype grad_dtype,
                      int64_t shard_S, const zero_bucket* buckets_dev, int64_t n_buckets,
                      double loss_scale, float* grad_out_dev, zero_stats* stats_dev,
                      void* workspace_dev, size_t ws_bytes, void* stream);

typedef struct {
    /* gradient source: exactly one of the two */
    const void* const* replicas;   /* fused: host array of n_replicas device pointers */
    int32_t n_replicas;
    zero_dtype grad_dtype;
    const float* grad_f32;         /* unfused: averaged, unscaled g from zero_reduce_shard */
    /* fp32 state of the shard, [shard_S] each */
    const float* p_in;
    const float* m_in;
    const float* v_in;
    float* p_out;
    float* m_out;
    float* v_out;
    uint16_t* slot_bf16;           /* this rank's slot of the gathered bf16 parameters, or NULL */
    int64_t shard_S;
    const zero_bucket* buckets_dev;
    int64_t n_buckets;
    double lr, beta1, beta2, eps, weight_decay;
    double loss_scale;             /* fused source only */
    int64_t step_t;                /* number of this update, >= 1 */
    zero_stats* stats_dev;
    void* workspace_dev;
    size_t ws_bytes;
    /* optional hipEvent_t handles (NULL: none), created by the caller: the main
       step kernel's launch carries them (hipExtLaunchKernel), so they take that
       kernel's own start and end time on `stream`, apart from the finalize.
       For eager launches; leave them NULL for a launch under stream capture */
    void* event_begin;
    void* event_end;
    /* zero_state_layout of p_in/m_in/v_in and p_out/m_out/v_out (0: split). Tiled:
       p_in and p_out are set buffers, m and v pointers NULL */
    int32_t state_layout;
} zero_adam_args;

/*
 * Adam / AdamW update of this rank's shard and the bf16 write of the result
 * into its slot of the gathered parameter buffer ("[REQUEST] Direct
 * Correspondence ...", "Problem": update the owned partition, then all-gather
 * the updated parameters; the local part of the all-gather is this slot write,
 * as in civat's all-gather count in "Why DeepSpeed ZeRO paper says ...").
 * Per element, one fp32 operation per line, no fused multiply-add:
 *   m' = b1*m + (1-b1)*g          v' = b2*v + (1-b2)*(g*g)
 *   mh = m'/bc1   vh = v'/bc2     den = sqrt(vh) + eps     u = mh/den
 *   p' = p*decay - lr*u           slot = bf16 round-to-nearest-even(p')
 * with b1, b2, 1-b1, 1-b2, lr, eps, decay = 1 - lr*weight_decay and
 * bc = 1 - beta^t (beta^t the t-fold product) each computed in double and
 * rounded once to fp32.
 * Fused source (replicas): g is formed as in zero_reduce_shard inside the same
 *   pass; the state must be out of place (p_out != p_in etc., ZERO_E_INVAL
 *   otherwise), because the overflow verdict is only known after the whole
 *   shard: on overflow the caller keeps the *_in buffers and restores the slot
 *   with zero_gather_slot(p_in) (see zero_commit_rule).
 * Unfused source (grad_f32): g is read as is; each *_out may equal its *_in
 *   (in place); partial overlaps are rejected.
 * Outputs and stats are written on every call, overflow or not. Alignment and
 * error rules as for zero_reduce_shard; hyperparameters must be finite with
 * beta1, beta2 in [0, 1), lr, eps, weight_decay >= 0, loss_scale > 0, step_t >= 1.
 */
int zero_adam_step(const zero_adam_args* args, void* stream);

/*
 * zero_adam_step for callers that cannot allocate device memory: code under
 * stream or graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, arithmetic and errors as zero_adam_step, and the
 * same p, m, v and slot bit for bit (the squared norm equal within rounding: its
 * per-workgroup partials are grouped differently), except:
 *  - workspace_dev must be NULL and ws_bytes 0 (ZERO_E_INVAL otherwise);
 *  - the per-workgroup partial sums and, for more than 256 replicas, the device
 *    table of replica pointers go into a scratch array compiled into the
 *    library: ZERO_NOALLOC_SCRATCH_BYTES bytes on each GPU the library runs on,
 *    held until the process ends. A launch uses at most 65,536 workgroups
 *    (shards beyond 64M elements stride over their 1,024-element trips), so
 *    every shard size and replica count the other checks accept fits; a launch
 *    that would need more scratch is refused with ZERO_E_RANGE;
 *  - the first call on a device looks the scratch address up
 *    (hipGetSymbolAddress, no allocation): make it outside any stream capture;
 *  - calls on one GPU share its scratch, which keeps what the last call wrote:
 *    calls that overlap in time (other streams, other threads) race, so order
 *    them on one stream. Nothing in it needs to start at zero: a launch writes
 *    every partial its finalize reads, and the pointer table before its use.
 * No hipMalloc, hipFree or allocating library routine is called.
 */
#define ZERO_NOALLOC_SCRATCH_BYTES 1581072
int zero_adam_step_noalloc(const zero_adam_args* args, void* stream);

/*
 * slot[i] = bf16 round-to-nearest-even(master[i]) for i in [0, shard_S): the
 * local part of the all-gather of updated parameters ("[REQUEST] Direct
 * Correspondence ...", "Problem"), used to initialise the slot and to restore
 * it after a skipped step. NaN becomes 0x7FC0.
 */
int zero_gather_slot(const float* master_dev, int64_t shard_S, uint16_t* slot_bf16_dev,
                     void* stream);

/*
 * zero_gather_slot with the master read from a tiled state set (the p sections
 * of set_dev, ZERO_STATE_TILED). Same errors.
 */
int zero_gather_slot_tiled(const float* set_dev, int64_t shard_S, uint16_t* slot_bf16_dev,
                           void* stream);

/*
 * Floats of one state set for a shard of shard_S elements: 3 * shard_S for
 * ZERO_STATE_SPLIT (three arrays), 3 * shard_S rounded up to a multiple of
 * 3 * ZERO_STATE_TILE for ZERO_STATE_TILED (one buffer). -1 for a negative
 * shard_S or an unknown layout.
 */
int64_t zero_state_set_floats(int64_t shard_S, int32_t state_layout);

/*
 * Conversion between the split arrays p, m, v [shard_S] and one tiled set buffer
 * (zero_state_set_floats(shard_S, ZERO_STATE_TILED) floats), bit for bit, for
 * initialising a tiled state and for reading it back (checkpoints, inspection).
 * Not part of a step. zero_state_unpack skips a NULL destination. The split
 * arrays must not overlap the set buffer or each other.
 * Errors: ZERO_E_INVAL (NULL buffers when shard_S > 0, overlap), ZERO_E_ALIGN,
 * ZERO_E_RANGE (negative shard_S), ZERO_E_HIP.
 */
int zero_state_pack(const float* p_dev, const float* m_dev, const float* v_dev, int64_t shard_S,
                    float* set_dev, void* stream);
int zero_state_unpack(const float* set_dev, int64_t shard_S, float* p_dev, float* m_dev,
                      float* v_dev, void* stream);

/*
 * The commit rule of a mixed-precision step, host side. The pages name mixed
 * precision ("ZeRO Optimizer", "Hybrid Approaches") but give no rule; this is
 * the common one. Given the stats of a fused step:
 *   clean    -> state->t += 1; return ZERO_COMMIT (caller swaps in/out buffers)
 *   overflow -> t unchanged; state->n_skipped += 1; if state->dynamic, the loss
 *               scale halves, never below state->min_loss_scale; return
 *               ZERO_SKIP (caller keeps the *_in buffers and restores its slot).
 * Returns ZERO_E_INVAL for NULL arguments.
 */
typedef struct {
    int64_t t;                     /* committed updates so far */
    int64_t n_skipped;
    double loss_scale;
    double min_loss_scale;         /* 1.0 by default */
    int32_t dynamic;               /* nonzero: halve the loss scale on overflow */
    int32_t reserved;
} zero_train_state;

enum { ZERO_COMMIT = 1, ZERO_SKIP = 2 };

int zero_commit_rule(zero_train_state* state, const zero_stats* stats_host);

/* ------------------------------------------------------------------------ */
/* Device-resident step: commit on the GPU, no host round trip per step       */
/* ------------------------------------------------------------------------ */

/*
 * The committed-state record of one rank's shard, in device memory (96 bytes,
 * 16-byte aligned, caller-owned). It holds the state after its `seq` finalized
 * steps. The step that a zero_train_step runs is not folded into the record by
 * its own launch but by the next one (or by zero_device_state_flush): until then
 * it is pending (pending_n > 0), its overflow flag and partial sums in the
 * workspace. Every launch derives the committed state from the record and the
 * pending step's flag with the skip rule of zero_commit_rule, so consecutive
 * steps need no host synchronization and no launch waits for its own last
 * workgroup (and steps can be graph-captured). To read the record on the host,
 * enqueue zero_device_state_flush, synchronize, then copy it: the flushed record
 * describes every step enqueued before the flush, and so do the stats.
 */
typedef struct {
    double beta1, beta2;           /* fixed for the life of the record */
    double beta1_pow, beta2_pow;   /* beta^t of the committed t (t-fold products) */
    double loss_scale;
    double min_loss_scale;
    double last_sumsq;             /* squared norm of the last step's averaged gradient */
    int64_t t;                     /* committed updates */
    int64_t n_skipped;             /* steps skipped on overflow */
    uint32_t cur;                  /* 0/1: which state set holds the committed state */
    uint32_t dynamic;              /* nonzero: halve the loss scale on overflow */
    uint32_t last_overflow;
    uint32_t seq;                  /* steps folded into this record (committed or skipped) */
    uint32_t pending_n;            /* > 0: one more step has run and awaits folding in (its
                                      partial count); 0 after init, load and flush */
    uint32_t error;                /* 0, or a ZERO_RECORD_E_* code: the record is frozen */
} zero_device_state;

/*
 * Sticky error codes of a record (zero_device_state.error). The folding of a
 * pending step waits, bounded by 2 s of the GPU's real-time counter, for two
 * things: the pending step's partials (written by the previous launch, so
 * present at once in a correct run) and the start marks of every workgroup of
 * its own launch (which must all have read the record before it changes).
 * Should either wait run out, which a correct launch never does, the folding
 * workgroup leaves every other field of the record as it is and stores one of
 * these codes instead; the stats read overflow = 1, bad_buckets = 0xFFFFFFFF,
 * sumsq = NaN. From then on every step launch on the record returns at once
 * without reading replicas or writing state, slot, partials or stats, the
 * restore kernel leaves the slot alone and a flush only writes the error stats,
 * so no update can land on state that a late workgroup may still be reading.
 * The state set that the frozen record's pending step names (as the skip rule
 * would apply it) is not written by the failed launch, but the caller should
 * treat the run as failed and resume from a checkpoint: zero_device_state_load
 * and zero_device_state_init clear the code. zero_device_state_load refuses a
 * saved record that carries one.
 */
enum { ZERO_RECORD_OK = 0, ZERO_RECORD_E_COLLECT = 1, ZERO_RECORD_E_MARKS = 2 };

/*
 * Enqueue the initialisation of a device state record (a small kernel, no
 * memset): t = 0, seq = 0, beta^0 = 1, set 0 current; and the clearing of the
 * workspace (workspace_dev, ws_bytes) that the record's steps will use. That
 * workspace belongs to the record from then on: the record's steps tag the
 * partials they leave in it with their step number, and another call using the
 * same workspace in between could leave stale words behind. beta1, beta2 in
 * [0, 1); loss_scale finite > 0; min_loss_scale in (0, loss_scale].
 * Errors: ZERO_E_INVAL, ZERO_E_ALIGN, ZERO_E_HIP.
 */
int zero_device_state_init(zero_device_state* state_dev, void* workspace_dev, size_t ws_bytes,
                           double beta1, double beta2, double loss_scale, double min_loss_scale,
                           int32_t dynamic, void* stream);

/*
 * Resume from a checkpoint. The committed state of a shard is p, m, v of the
 * current set plus this record; the pages define the per-rank optimizer state
 * as the fp32 master copy with the two Adam moments ("ZeRO Optimizer", stage 1
 * memory terms) and nothing else, so saving those and the record is a complete
 * checkpoint. This enqueues the writing of *saved (a host copy of a record
 * taken after synchronizing its stream) into state_dev and the clearing of the
 * workspace, as zero_device_state_init does; seq restarts at 0 and the other
 * fields are kept bit for bit, so the steps that follow are identical to those
 * of an uninterrupted run. The caller puts the saved p, m, v into set
 * saved->cur of the zero_train_args it will pass, and rewrites its slot with
 * zero_gather_slot from that master (into slot[saved->cur] when the slot is
 * double-buffered). The host record is read before return.
 * Errors: ZERO_E_INVAL (NULL, betas or loss scales as for zero_device_state_init,
 * t or n_skipped negative, cur or last_overflow not 0/1, beta powers outside
 * [0, 1] or not 1 at t = 0, a pending step, a nonzero error code),
 * ZERO_E_ALIGN, ZERO_E_HIP.
 */
int zero_device_state_load(zero_device_state* state_dev, void* workspace_dev, size_t ws_bytes,
                           const zero_device_state* saved, void* stream);

/*
 * Fold the pending step of a device-committed record into it (one small kernel
 * on `stream`): t, the loss scale, beta^t, the current set, n_skipped,
 * last_overflow and last_sumsq then describe every step enqueued before the
 * flush, and *stats_dev holds that last step's overflow flag, bucket count and
 * squared norm. No-op if nothing is pending. On a record frozen by a
 * ZERO_RECORD_E_* code it changes nothing in the record and writes the error
 * stats (overflow = 1, bad_buckets = 0xFFFFFFFF, sumsq = NaN); the caller finds
 * the code in the record it copies back. The workspace must be the record's.
 * Errors: ZERO_E_INVAL (NULL, overlapping buffers), ZERO_E_ALIGN, ZERO_E_RANGE
 * (workspace too small for any step), ZERO_E_HIP.
 */
int zero_device_state_flush(zero_device_state* state_dev, zero_stats* stats_dev, void* workspace_dev,
                            size_t ws_bytes, void* stream);

typedef struct {
    const void* const* replicas;   /* host array of n_replicas device pointers, slot order */
    int32_t n_replicas;
    zero_dtype grad_dtype;
    float* p[2];                   /* the two fp32 state sets, [shard_S] each */
    float* m[2];
    float* v[2];
    /* this rank's slot of the gathered bf16 parameters: slot[0] alone (slot[1] = NULL),
       or a double-buffered pair in which slot[cur] holds the committed parameters */
    uint16_t* slot[2];
    int64_t shard_S;
    const zero_bucket* buckets_dev;
    int64_t n_buckets;
    double lr, eps, weight_decay;  /* may change from step to step; betas live in the record */
    zero_device_state* state_dev;
    zero_stats* stats_dev;
    void* workspace_dev;
    size_t ws_bytes;
    void* event_begin;             /* optional hipEvent_t handles: the start and end */
    void* event_end;               /* time of the step kernel itself, as above */
    /* zero_state_layout of the two sets (0: split). Tiled: p[0], p[1] are the set
       buffers, m and v NULL; inner part ends of zero_train_step_part must then be
       multiples of ZERO_STATE_TILE */
    int32_t state_layout;
} zero_train_args;

/*
 * One whole step of this rank's shard with the commit on the device: the fused
 * pass of zero_adam_step (fold in slot order, average and unscale, overflow flag
 * and squared norm, Adam/AdamW, bf16 slot), reading the committed set and writing
 * the other set. Every workgroup first derives the committed state from the
 * record and the previous step's overflow flag (the skip rule of
 * zero_commit_rule: clean -> t += 1 and the written set became current;
 * overflow -> nothing committed, dynamic loss scale halved), leaves a start mark,
 * and at its end a partial tagged with the step's number (and the step's flag
 * word if it saw a non-finite gradient). Workgroup 0 sums the previous step's
 * partials in workgroup order and, once every workgroup of the launch has left
 * its start mark, folds that step into *state_dev; this step stays pending until
 * the next step or zero_device_state_flush. The waits are bounded (2 s); should
 * one run out, which a correct launch never does, the record is frozen with a
 * ZERO_RECORD_E_* code and every later step on it does nothing (see
 * zero_device_state.error). The workspace must be the one given to
 * zero_device_state_init, of at least zero_workspace_bytes(shard_S) bytes. With
 * a single slot the candidate bf16 values go straight into it and a second kernel
 * restores it from the committed master after an overflow;
 * with a double-buffered slot the candidate goes into slot[1 - cur] and the
 * commit flips it with the state sets, so a step is one kernel. Same arithmetic
 * as zero_adam_step, bit for bit.
 * Source of the step: "[REQUEST] Direct Correspondence between Gradient and
 * Optimizer States to Reduce Communication", "Problem"; ring order as in
 * GuanhuaWang's reply in "Why DeepSpeed ZeRO paper says reduce-scatter (or
 * all-gather) has data movement of Psi elements?".
 * The six state buffers, the slot, stats, workspace and record must not overlap
 * each other or the replicas. Errors as for zero_adam_step.
 */
int zero_train_step(const zero_train_args* args, void* stream);

/*
 * One part of a device-committed step split into consecutive element ranges,
 * so that each range can be stepped as soon as its gradients are ready while
 * the rest are still being produced. The pages list overlap with computation
 * and bucketing of small gradient groups among ZeRO's communication
 * optimizations ("ZeRO Optimizer", "Communication Optimization" and
 * "Communication Patterns", all-reduce for gradients) without fixing a
 * mechanism; stepping each range once its gradients are in place is this
 * library's reading of that overlap for the fused step.
 * part_ends: host array of n_parts non-decreasing shard offsets; part k covers
 * [part_ends[k-1], part_ends[k]) with part_ends[-1] = 0; inner ends are multiples
 * of 8 elements and part_ends[n_parts - 1] == shard_S (empty parts are allowed).
 * Call part = 0, 1, ..., n_parts - 1 in that order on ONE stream: every part reads
 * the same committed record and leaves tagged partials, and the last part's
 * workgroup 0 folds the previous step into the record once the last part's
 * workgroups have read it, as zero_train_step does; the step whose parts these
 * are then stays pending (its partials, in part then workgroup order, are summed
 * by the next step or flush); with a single slot the restore kernel
 * follows the last part. p, m, v and the slot come out bit-identical to
 * zero_train_step's; the squared norm is summed in another grouping (equal
 * within rounding). The workspace of zero_workspace_bytes(shard_S) suffices.
 * args must carry no bucket table (ZERO_E_UNSUPPORTED); parts cover padding like
 * a whole-shard step.
 * Errors: as zero_train_step; ZERO_E_INVAL for a NULL part_ends; ZERO_E_RANGE for
 * n_parts outside [1, 4096], part outside [0, n_parts) or a bad boundary.
 */
int zero_train_step_part(const zero_train_args* args, const int64_t* part_ends, int32_t n_parts,
                         int32_t part, void* stream);

/* ------------------------------------------------------------------------ */
/* Stage-3 fetch: whole tensors out of the rank shards                        */
/* ------------------------------------------------------------------------ */

/*
 * Stage 3 partitions the parameters like the gradients and optimizer state and
 * gathers the ones a layer needs just before it runs, freeing them afterwards
 * ("ZeRO Optimizer", "ZeRO Stages" stage 3 and "Communication Patterns",
 * all-gather of the required parameter subset; "Why does not the stage 3
 * implementation use broadcast and reduce-scatter?": all-gather rather than
 * broadcast). Tensor k occupies flat elements [offsets[k], offsets[k] + numels[k])
 * (zero_layout_offsets) and rank r's shard holds flat elements [r*shard_S,
 * (r+1)*shard_S); this copies every listed tensor, bit for bit, from the
 * n_shards device shards into outs[k] (device, numels[k] contiguous elements),
 * on `stream`. elem_bytes: 2 (bf16 parameters) or 4. The caller owns outs and
 * frees them after the layer. shards and outs must be element-aligned; outs must
 * not overlap the shards or each other. Empty tensors are skipped.
 * Errors: ZERO_E_INVAL (NULL pointer, elem_bytes not 2 or 4, overlap),
 * ZERO_E_ALIGN, ZERO_E_RANGE (n_shards outside [1, 256], shard_S outside
 * [1, 2^40], n_tensors < 0, a tensor leaving the n_shards * shard_S buffer),
 * ZERO_E_HIP.
 */
int zero_gather_tensors(const void* const* shards, int32_t n_shards, int64_t shard_S,
                        int32_t elem_bytes, const int64_t* offsets, const int64_t* numels,
                        void* const* outs, int32_t n_tensors, void* stream);

/* ------------------------------------------------------------------------ */
/* Optimizer state offloaded to host memory                                   */
/* ------------------------------------------------------------------------ */

/*
 * The "ZeRO Optimizer" page ("Advanced Optimizations", ZeRO-Offload) moves the
 * optimizer states to CPU memory and balances the GPU-CPU transfers against the
 * work; it gives no algorithm. Read plainly: the shard's fp32 master, m and v
 * live in host memory, the GPU folds and checks the gradients as in
 * zero_reduce_shard, the averaged fp32 gradient crosses to the host, the host
 * runs the same Adam/AdamW (one fp32 operation per source operation, correctly
 * rounded division and square root, no contraction, so the result is bit for
 * bit that of zero_adam_step), and the bf16 result crosses back into the
 * rank's slot.
 */

/*
 * Adam/AdamW on the host, in place on p, m, v over n elements, optionally
 * writing bf16 (nearest even) into slot_bf16. Same operation sequence and fp32
 * scalars as zero_adam_step (step_t >= 1; beta^t as a t-fold product in double).
 * All pointers are host memory; the arrays must not overlap (not checked).
 * nthreads: worker threads (0: one per CPU in the calling process's affinity mask,
 * at most 256). Synchronous.
 * Errors: ZERO_E_INVAL (NULL pointer with n > 0, a parameter out of domain),
 * ZERO_E_RANGE (n < 0).
 */
typedef struct {
    const float* g;
    float* p;
    float* m;
    float* v;
    uint16_t* slot_bf16;           /* may be NULL */
    int64_t n;
    double lr, beta1, beta2, eps, weight_decay;
    int64_t step_t;
    int32_t nthreads;
    int32_t reserved;
} zero_host_adam_args;

int zero_host_adam(const zero_host_adam_args* args);

/*
 * One offloaded step of this rank's shard, synchronous on the host:
 *  1. on `stream`: fold the replicas into g_dev (fp32 [shard_S], device),
 *     ×1/(N·loss_scale), overflow flag and squared norm into stats_dev
 *     (zero_reduce_shard); copy the 16-byte stats back and wait for them;
 *  2. overflow: no state or slot buffer is touched, the commit rule skips
 *     (state->n_skipped += 1,
 *     dynamic loss scale halved), return ZERO_SKIP;
 *  3. clean: g_dev is copied to g_host in chunks of chunk_elems elements, one
 *     event per chunk; as soon as a chunk has landed every host thread updates
 *     its stripe of it (the zero_host_adam arithmetic, update number
 *     state->t + 1), and the thread that finishes the chunk uploads its bf16
 *     values from slot_host to slot_dev on stream_h2d (or on `stream` if NULL)
 *     while later chunks are still crossing; after both streams are
 *     synchronized, state->t += 1 and ZERO_COMMIT is returned.
 * *stats_out (may be NULL) gets the step's stats. Host buffers: p_host, m_host,
 * v_host any host memory; g_host and slot_host pinned (hipHostMalloc) for
 * asynchronous copies, and not reused by the caller until the call returns.
 * The library creates its chunk events per call and frees them. Errors: as
 * zero_reduce_shard and zero_host_adam; ZERO_E_RANGE for chunk_elems < 0.
 */
typedef struct {
    const void* const* replicas;   /* host array of n_replicas device pointers, slot order */
    int32_t n_replicas;
    zero_dtype grad_dtype;
    int64_t shard_S;
    float* g_dev;                  /* device [shard_S] */
    float* g_host;                 /* pinned host [shard_S] */
    float* p_host;                 /* host [shard_S], the committed state, updated in place */
    float* m_host;
    float* v_host;
    uint16_t* slot_host;           /* pinned host [shard_S] staging */
    uint16_t* slot_dev;            /* device [shard_S], this rank's slot */
    double lr, beta1, beta2, eps, weight_decay;
    zero_train_state* state;       /* host: t, skips, loss scale; the commit rule updates it */
    zero_stats* stats_dev;
    void* workspace_dev;
    size_t ws_bytes;
    int64_t chunk_elems;           /* 0: 1,048,576 */
    int32_t nthreads;              /* host worker threads, 0: one per CPU of the affinity mask */
    int32_t reserved;
    void* stream_h2d;              /* optional second stream for the slot uploads */
} zero_offload_args;

int zero_offload_step(const zero_offload_args* args, void* stream, zero_stats* stats_out);

/* Thread-local text for the last non-OK return on this thread ("" if none). */
const char* zero_last_error(void);

/* Library version string, e.g. "libzero 1.0 (gfx950)". */
const char* zero_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_SHARD_STEP_H */
