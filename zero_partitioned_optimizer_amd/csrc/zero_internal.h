// zero_internal.h -- internal interface between the C ABI layer (abi.cpp) and
// the gfx950 kernels (step_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero.h"

namespace zk {

#ifndef ZERO_GRID_MAX
#define ZERO_GRID_MAX 4194304
#endif

#ifndef ZERO_BLOCK
#define ZERO_BLOCK 256
#endif

constexpr int kBlock = ZERO_BLOCK;  // threads per workgroup: 4 wave64s
constexpr int kVec = 4;             // elements per lane per row (one quad)
constexpr int kGridMax = ZERO_GRID_MAX;  // workgroups of the grid-stride step kernel
constexpr int kMaxParts = 4096;          // parts of one step split over launches
constexpr int kArgReplicas = 256;        // replica pointers carried in the kernel arguments
constexpr int64_t kEvenBlockQuads = 16;  // quads per block of an evenly split small launch
// A bucket launch over a table of at most kChunkTableMax buckets that average at
// least two chunks each cuts the buckets into chunks of kChunk elements.
constexpr int64_t kChunk = (int64_t)kBlock * kVec;
constexpr int64_t kChunkTableMax = 2048;

// Bytes at the end of the workspace that a launch with n_rep replicas uses for
// its device table of replica pointers (only beyond kArgReplicas replicas; 16
// bytes of slack for alignment), and where that table starts.
inline size_t rep_table_bytes(int32_t n_rep) {
    return n_rep > kArgReplicas ? 8 * (size_t)n_rep + 16 : 0;
}
inline const void** rep_table_at(void* ws, size_t ws_bytes, int32_t n_rep) {
    if (n_rep <= kArgReplicas) return nullptr;
    const uintptr_t end = reinterpret_cast<uintptr_t>(ws) + ws_bytes;
    return reinterpret_cast<const void**>((end - 8 * (uintptr_t)n_rep) & ~uintptr_t(15));
}

// Upper bound on the workgroups of any step launch over a shard of S elements
// (one trip of kBlock * kVec elements each, plus one per part of a split step),
// which sizes the workspace of partials.
inline int64_t grid_bound(int64_t S) {
    const int64_t trips = S > 0 ? (S + (int64_t)kBlock * kVec - 1) / ((int64_t)kBlock * kVec) : 1;
    const int64_t g = trips + kMaxParts;
    return g < kGridMax ? g : kGridMax;
}
// Tiled state layout: tiles of kStateTile elements, each [p | m | v].
constexpr int kStateTileLog2 = 13;
constexpr int64_t kStateTile = int64_t(1) << kStateTileLog2;
constexpr int kStateTileQuadsLog2 = kStateTileLog2 - 2;
constexpr int64_t kStateTileQuads = int64_t(1) << kStateTileQuadsLog2;
static_assert(kStateTile == ZERO_STATE_TILE, "the tile of the ABI");
constexpr int kCommitGrid = 512;    // workgroups of the commit / cast kernels
constexpr int kFinalizeBlock = 256;

// Workspace of a device-committed record: two halves of tagged partials (three
// 64-bit words per workgroup slot; steps with odd and even numbers alternate, so
// a launch can fold the previous step's partials while writing its own), one
// start mark per workgroup slot, the two overflow flag words (by step number
// parity, padded to 64 bytes), and the replica pointer table reserved at the end.
// Slots = cap, derived from the workspace size alone, so every launch on a
// record sees the same layout.
constexpr size_t kRepTableMax = 8 * (size_t)ZERO_MAX_REPLICAS + 16;
constexpr size_t kCommitSlotBytes = 2 * 24 + 8;
constexpr size_t kFlagBytes = 64;
struct CommitWs {
    uint64_t* half[2];
    uint64_t* started;
    uint64_t* flags;
    int64_t cap;                    // workgroup slots
};
inline CommitWs commit_ws(void* ws, size_t ws_bytes) {
    CommitWs w{};
    if (!ws || ws_bytes < kRepTableMax + kFlagBytes) return w;
    const int64_t cap = (int64_t)((ws_bytes - kRepTableMax - kFlagBytes) / kCommitSlotBytes);
    uint64_t* b = static_cast<uint64_t*>(ws);
    w.half[0] = b;
    w.half[1] = b + 3 * cap;
    w.started = b + 6 * cap;
    w.flags = b + 7 * cap;
    w.cap = cap;
    return w;
}

// Per-workgroup partial result of the overflow flag and the squared norm.
struct Partial {
    double sumsq;
    uint32_t bad;
    uint32_t bad_buckets;
};
static_assert(sizeof(Partial) == 16, "partials are 16 bytes");

// Workspace bytes per workgroup: a 16-byte Partial (host commit), or three
// tagged 64-bit words (device commit).
constexpr size_t kPartialBytes = 24;

// The allocation-free entry point's scratch (a file-scope device array in
// step_kernels.hip, one copy per GPU): the partials of at most kNoallocGrid
// workgroups and the replica pointer table at its end. Its launches cap their
// grid at kNoallocGrid, so longer shards stride over their trips.
constexpr int kNoallocGrid = 65536;
constexpr size_t kNoallocBytes = (size_t)kNoallocGrid * kPartialBytes + kRepTableMax;
constexpr int kNoallocMaxDevices = 64;
static_assert(kNoallocBytes == ZERO_NOALLOC_SCRATCH_BYTES, "the scratch size of the ABI");

// fp32 scalars of one update, each rounded once from double on the host.
struct Scalars {
    float inv;                      // 1 / (N * loss_scale)
    float b1, b2, omb1, omb2;       // beta1, beta2, 1 - beta1, 1 - beta2
    float bc1, bc2;                 // 1 - beta1^t, 1 - beta2^t
    float lr, eps, decay;           // decay = 1 - lr * weight_decay
};

// What one launch of the step kernel does.
struct StepDesc {
    const void* const* replicas;    // host array of n_rep device pointers
    int32_t n_rep;
    const void** rep_table;         // workspace table for n_rep > kArgReplicas, else nullptr
    zero_dtype dtype;
    int64_t S;
    const zero_bucket* buckets;     // device, or nullptr for the whole shard
    int64_t n_buckets;
    bool adam;                      // false: reduce only
    const float* p_in;
    const float* m_in;
    const float* v_in;
    float* p_out;
    float* m_out;
    float* v_out;
    uint16_t* slot;                 // may be nullptr
    float* g_out;                   // may be nullptr
    Scalars sc;
    float* set_p[2];                // device-commit path: both state sets
    float* set_m[2];
    float* set_v[2];
    zero_device_state* ctrl;        // device-commit path, else nullptr
    uint16_t* set_slot[2];          // device-commit path, double-buffered slot (else nullptr)
    zero_stats* stats;
    Partial* partials;              // workspace, >= grid_for() entries
    hipEvent_t ev_begin;            // optional, around the main kernel only
    hipEvent_t ev_end;
    // device commit split over several launches (parts of one step):
    int32_t part_base;              // partial slot of this launch's workgroup 0
    int32_t collect_n;              // 0: a whole step (its own grid of partials); > 0: the last
                                    // part of a split step, n partials over all parts; either
                                    // way workgroup 0 folds the pending step into the record and
                                    // this step becomes pending; < 0: a part before the last
                                    // (publish only)
    bool no_restore;                // single slot: leave the restore kernel to the caller
    bool tiled;                     // state sets in the tiled layout (m, v pointers unused)
    uint64_t* ws_half[2];           // device-commit path: the workspace regions of CommitWs
    uint64_t* ws_started;
    uint64_t* ws_flags;
    int max_grid;                   // cap on the workgroups (0: kGridMax)
};

int rows_for(int32_t n_rep);
int grid_for(int64_t S, int64_t n_buckets, int32_t n_rep, int max_grid = 0);
int64_t even_blocks_for(int64_t S, int64_t n_buckets, int32_t n_rep, int max_grid = 0);
bool bucket_chunks(int64_t S, int64_t n_buckets);
hipError_t launch_step(const StepDesc& d, hipStream_t stream);
hipError_t launch_cast_slot(const float* master, int64_t S, bool tiled, uint16_t* slot,
                            hipStream_t stream);
// Split p, m, v [S] <-> one tiled set buffer (unpack: tiled -> split; NULL
// destinations skipped).
hipError_t launch_state_convert(bool unpack, float* tiled, float* p, float* m, float* v, int64_t S,
                                hipStream_t stream);
// Stage-3 fetch (gather_kernels.hip), over at most kGatherMaxShards shards.
constexpr int kGatherMaxShards = 256;
hipError_t launch_gather(const void* const* shards, int32_t n_shards, int64_t S, int32_t elem_bytes,
                         const int64_t* offsets, const int64_t* numels, void* const* outs,
                         int32_t n_tensors, hipStream_t stream);
// After a device-committed step with a single slot: recast the slot from the
// current master if the step was skipped (no-op kernel otherwise).
hipError_t launch_restore(const zero_device_state* ctrl, const uint64_t* flags, const float* set_p0,
                          const float* set_p1, uint16_t* slot, int64_t S, bool tiled,
                          hipStream_t stream);
// Fold the pending step of a device-committed record into it (one workgroup).
hipError_t launch_flush(zero_device_state* ctrl, zero_stats* stats, const CommitWs& w,
                        hipStream_t stream);
// Write rec to *s and clear the workspace (ws_bytes / 8 words), on st.
hipError_t launch_state_write(zero_device_state* s, const zero_device_state& rec, void* ws,
                              size_t ws_bytes, hipStream_t st);
// Device address of the allocation-free scratch on the current device
// (kNoallocBytes bytes), looked up once per device.
hipError_t noalloc_scratch(void** ptr);

}  // namespace zk

namespace zl {
// Thread-local error text of the last failing call (zero_last_error).
void set_error(const char* fmt, ...);
// ZERO_OK, or ZERO_E_HIP with the error text set.
int hip_error(hipError_t e, const char* where);
// The fp32 scalars of update number t (inv = 1), as the device steps use them.
zk::Scalars update_scalars(double lr, double beta1, double beta2, double eps, double wd, int64_t t);
}  // namespace zl
