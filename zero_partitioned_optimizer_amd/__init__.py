"""zero_partitioned_optimizer_amd -- the per-rank ZeRO stage-1/2 optimizer step on one
MI355X (gfx950): N resident gradient replicas of this rank's shard are folded in
ring order, averaged and unscaled, checked for overflow, used for an Adam/AdamW
update of fp32 master / m / v, and the bf16 result lands in this rank's slot of
the gathered parameter buffer.

The compute lives in ``libzero.so`` (hand-written HIP for gfx950 behind a C ABI,
``include/zero.h``); this package is its ctypes binding (same function names)
plus ``ShardStep``, which owns buffers and applies the commit rule. There is no
CPU fallback: without the built library every call raises.
"""
from ._binding import (  # noqa: F401
    ZERO_BF16, ZERO_BF16_WIRE, ZERO_COMMIT, ZERO_F32, ZERO_MAX_REPLICAS, ZERO_SKIP, ZeroError, lib,
    make_adam_args, stats_from_tensor, zero_adam_args, zero_adam_step, zero_bucket,
    zero_commit_rule, zero_gather_slot, zero_last_error, zero_layout_buckets,
    zero_layout_buckets_raw, zero_layout_build, zero_layout_free, zero_layout_info,
    zero_layout_info_get, zero_layout_mem_bytes, zero_layout_mem_values, zero_layout_offsets,
    zero_layout_segments, zero_reduce_shard, zero_segment, zero_stats, zero_train_state,
    zero_version, zero_workspace_bytes, zero_device_state, zero_device_state_init,
    zero_device_state_load, zero_train_step_part, part_table, zero_host_adam,
    zero_offload_step, zero_offload_args, zero_host_adam_args, zero_gather_tensors, GatherPlan,
    zero_train_args, zero_train_step, make_train_args, device_state_from_tensor,
    ZERO_STATE_SPLIT, ZERO_STATE_TILED, ZERO_STATE_TILE, zero_gather_slot_tiled,
    zero_state_set_floats, zero_state_pack, zero_state_unpack, zero_device_state_flush,
    ZeroRecordError, ZERO_RECORD_OK, ZERO_RECORD_E_COLLECT, ZERO_RECORD_E_MARKS,
    zero_adam_step_noalloc, ZERO_NOALLOC_SCRATCH_BYTES)
from .shard_step import DeviceShardStep, OffloadShardStep, ShardStep  # noqa: F401
