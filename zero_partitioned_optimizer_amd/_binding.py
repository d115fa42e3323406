"""ctypes binding of libzero's C ABI (include/zero.h), argument marshalling only.

Every function keeps the C name. Device buffers are passed as torch tensors (or
raw integer addresses); torch provides device memory and streams, nothing else.
torch is imported before the library is opened so that libzero binds to the
HIP runtime torch already loaded (both carry the soname libamdhip64.so.7).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch  # noqa: F401  (must come before the library is opened)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libzero.so")

i32, i64, u32, f64, vp, sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_double,
                              ctypes.c_void_p, ctypes.c_size_t)

ZERO_OK, ZERO_E_INVAL, ZERO_E_ALIGN, ZERO_E_RANGE, ZERO_E_NOMEM, ZERO_E_HIP, ZERO_E_UNSUPPORTED = \
    0, -1, -2, -3, -4, -5, -6
ZERO_F32, ZERO_BF16, ZERO_BF16_WIRE = 0, 1, 2
ZERO_COMMIT, ZERO_SKIP = 1, 2
ZERO_MAX_REPLICAS = 1024
ZERO_STATE_SPLIT, ZERO_STATE_TILED = 0, 1
ZERO_STATE_TILE = 8192
ZERO_NOALLOC_SCRATCH_BYTES = 1581072
ZERO_RECORD_OK, ZERO_RECORD_E_COLLECT, ZERO_RECORD_E_MARKS = 0, 1, 2

_STATUS = {0: "ZERO_OK", -1: "ZERO_E_INVAL", -2: "ZERO_E_ALIGN", -3: "ZERO_E_RANGE",
           -4: "ZERO_E_NOMEM", -5: "ZERO_E_HIP", -6: "ZERO_E_UNSUPPORTED"}


class ZeroError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class ZeroRecordError(RuntimeError):
    """A device-committed record frozen by a ZERO_RECORD_E_* code: a bounded wait
    inside a step ran out, and every later step on the record did nothing."""

    _WHAT = {ZERO_RECORD_E_COLLECT: "the previous step's partial sums did not arrive",
             ZERO_RECORD_E_MARKS: "a workgroup of the step did not read the record in time"}

    def __init__(self, code: int):
        super().__init__(f"device record frozen by error code {code} "
                         f"({self._WHAT.get(code, 'unknown code')}); resume from a checkpoint")
        self.code = code


class zero_layout_info(ctypes.Structure):
    _fields_ = [("n_tensors", i64), ("psi", i64), ("used_L", i64), ("padded_L", i64),
                ("shard_S", i64), ("tensor_align_A", i64), ("shard_align_B", i64),
                ("world_N", i32), ("reserved", i32)]


class zero_segment(ctypes.Structure):
    _fields_ = [("tensor", i32), ("reserved", i32), ("tensor_off", i64), ("shard_off", i64),
                ("len", i64)]


class zero_bucket(ctypes.Structure):
    _fields_ = [("shard_off", i64), ("len", i32), ("tensor", i32)]


class zero_stats(ctypes.Structure):
    _fields_ = [("overflow", u32), ("bad_buckets", u32), ("sumsq", f64)]


class zero_adam_args(ctypes.Structure):
    _fields_ = [("replicas", ctypes.POINTER(vp)), ("n_replicas", i32), ("grad_dtype", i32),
                ("grad_f32", vp),
                ("p_in", vp), ("m_in", vp), ("v_in", vp), ("p_out", vp), ("m_out", vp),
                ("v_out", vp), ("slot_bf16", vp), ("shard_S", i64), ("buckets_dev", vp),
                ("n_buckets", i64), ("lr", f64), ("beta1", f64), ("beta2", f64), ("eps", f64),
                ("weight_decay", f64), ("loss_scale", f64), ("step_t", i64),
                ("stats_dev", vp), ("workspace_dev", vp), ("ws_bytes", sz),
                ("event_begin", vp), ("event_end", vp), ("state_layout", i32)]


class zero_train_state(ctypes.Structure):
    _fields_ = [("t", i64), ("n_skipped", i64), ("loss_scale", f64), ("min_loss_scale", f64),
                ("dynamic", i32), ("reserved", i32)]


class zero_device_state(ctypes.Structure):
    _fields_ = [("beta1", f64), ("beta2", f64), ("beta1_pow", f64), ("beta2_pow", f64),
                ("loss_scale", f64), ("min_loss_scale", f64), ("last_sumsq", f64),
                ("t", i64), ("n_skipped", i64), ("cur", u32), ("dynamic", u32),
                ("last_overflow", u32), ("seq", u32), ("pending_n", u32), ("error", u32)]


class zero_train_args(ctypes.Structure):
    _fields_ = [("replicas", ctypes.POINTER(vp)), ("n_replicas", i32), ("grad_dtype", i32),
                ("p", vp * 2), ("m", vp * 2), ("v", vp * 2), ("slot", vp * 2), ("shard_S", i64),
                ("buckets_dev", vp), ("n_buckets", i64), ("lr", f64), ("eps", f64),
                ("weight_decay", f64), ("state_dev", vp), ("stats_dev", vp),
                ("workspace_dev", vp), ("ws_bytes", sz), ("event_begin", vp), ("event_end", vp),
                ("state_layout", i32)]


class zero_host_adam_args(ctypes.Structure):
    _fields_ = [("g", vp), ("p", vp), ("m", vp), ("v", vp), ("slot_bf16", vp), ("n", i64),
                ("lr", f64), ("beta1", f64), ("beta2", f64), ("eps", f64), ("weight_decay", f64),
                ("step_t", i64), ("nthreads", i32), ("reserved", i32)]


class zero_offload_args(ctypes.Structure):
    _fields_ = [("replicas", ctypes.POINTER(vp)), ("n_replicas", i32), ("grad_dtype", i32),
                ("shard_S", i64), ("g_dev", vp), ("g_host", vp), ("p_host", vp), ("m_host", vp),
                ("v_host", vp), ("slot_host", vp), ("slot_dev", vp), ("lr", f64), ("beta1", f64),
                ("beta2", f64), ("eps", f64), ("weight_decay", f64),
                ("state", ctypes.POINTER(zero_train_state)), ("stats_dev", vp),
                ("workspace_dev", vp), ("ws_bytes", sz), ("chunk_elems", i64), ("nthreads", i32),
                ("reserved", i32), ("stream_h2d", vp)]


assert ctypes.sizeof(zero_device_state) == 96
assert ctypes.sizeof(zero_bucket) == 16 and ctypes.sizeof(zero_stats) == 16
assert ctypes.sizeof(zero_segment) == 32

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Open libzero.so (building it first only if it does not exist)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.zero_layout_build.argtypes = [P(i64), i64, i32, i64, i64, P(vp)]
    L.zero_layout_info_get.argtypes = [vp, P(zero_layout_info)]
    L.zero_layout_offsets.argtypes = [vp, P(i64)]
    L.zero_layout_segments.argtypes = [vp, i32, P(zero_segment), i64, P(i64)]
    L.zero_layout_buckets.argtypes = [vp, i32, i64, P(zero_bucket), i64, P(i64)]
    L.zero_layout_mem_values.argtypes = [vp, i32, P(i64)]
    L.zero_layout_mem_bytes.argtypes = [vp, i32, P(i64)]
    L.zero_layout_free.argtypes = [vp]
    L.zero_layout_free.restype = None
    L.zero_workspace_bytes.argtypes = [i64]
    L.zero_workspace_bytes.restype = sz
    L.zero_reduce_shard.argtypes = [P(vp), i32, i32, i64, vp, i64, f64, vp, vp, vp, sz, vp]
    L.zero_adam_step.argtypes = [P(zero_adam_args), vp]
    L.zero_adam_step_noalloc.argtypes = [P(zero_adam_args), vp]
    L.zero_gather_slot.argtypes = [vp, i64, vp, vp]
    L.zero_gather_slot_tiled.argtypes = [vp, i64, vp, vp]
    L.zero_state_set_floats.argtypes = [i64, i32]
    L.zero_state_set_floats.restype = i64
    L.zero_state_pack.argtypes = [vp, vp, vp, i64, vp, vp]
    L.zero_state_unpack.argtypes = [vp, i64, vp, vp, vp, vp]
    L.zero_commit_rule.argtypes = [P(zero_train_state), P(zero_stats)]
    L.zero_device_state_init.argtypes = [vp, vp, sz, f64, f64, f64, f64, i32, vp]
    L.zero_device_state_load.argtypes = [vp, vp, sz, P(zero_device_state), vp]
    L.zero_device_state_flush.argtypes = [vp, vp, vp, sz, vp]
    L.zero_train_step.argtypes = [P(zero_train_args), vp]
    L.zero_train_step_part.argtypes = [P(zero_train_args), vp, i32, i32, vp]
    L.zero_gather_tensors.argtypes = [P(vp), i32, i64, i32, P(i64), P(i64), P(vp), i32, vp]
    L.zero_host_adam.argtypes = [P(zero_host_adam_args)]
    L.zero_offload_step.argtypes = [P(zero_offload_args), vp, P(zero_stats)]
    L.zero_last_error.argtypes = []
    L.zero_last_error.restype = ctypes.c_char_p
    L.zero_version.argtypes = []
    L.zero_version.restype = ctypes.c_char_p
    for name in ("zero_layout_build", "zero_layout_info_get", "zero_layout_offsets",
                 "zero_layout_segments", "zero_layout_buckets", "zero_layout_mem_values",
                 "zero_layout_mem_bytes", "zero_reduce_shard", "zero_adam_step", "zero_adam_step_noalloc",
                 "zero_gather_slot", "zero_gather_slot_tiled", "zero_state_pack",
                 "zero_state_unpack", "zero_commit_rule", "zero_device_state_init",
                 "zero_device_state_load", "zero_device_state_flush", "zero_train_step", "zero_train_step_part",
                 "zero_host_adam", "zero_offload_step", "zero_gather_tensors"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int) -> int:
    if rc < 0:
        raise ZeroError(rc, lib().zero_last_error().decode())
    return rc


def _addr(x) -> int:
    """Device address of a tensor (or an int address, or None -> 0)."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# layout (host only)
# ---------------------------------------------------------------------------

def zero_layout_build(numels: Sequence[int], world_N: int, tensor_align_A: int = 1,
                      shard_align_B: int = 8) -> int:
    """Returns an opaque layout handle (free with zero_layout_free)."""
    arr = (i64 * max(len(numels), 1))(*[int(n) for n in numels])
    h = vp()
    _check(lib().zero_layout_build(arr, len(numels), int(world_N), int(tensor_align_A),
                                   int(shard_align_B), ctypes.byref(h)))
    return h.value


def zero_layout_info_get(h: int) -> zero_layout_info:
    info = zero_layout_info()
    _check(lib().zero_layout_info_get(h, ctypes.byref(info)))
    return info


def zero_layout_offsets(h: int) -> list:
    n = zero_layout_info_get(h).n_tensors
    out = (i64 * max(n, 1))()
    _check(lib().zero_layout_offsets(h, out))
    return list(out)[:n]


def zero_layout_segments(h: int, rank: int) -> list:
    """List of (tensor, tensor_off, shard_off, len)."""
    n = i64()
    _check(lib().zero_layout_segments(h, int(rank), None, 0, ctypes.byref(n)))
    out = (zero_segment * max(n.value, 1))()
    _check(lib().zero_layout_segments(h, int(rank), out, n.value, ctypes.byref(n)))
    return [(s.tensor, s.tensor_off, s.shard_off, s.len) for s in out[:n.value]]


def zero_layout_buckets_raw(h: int, rank: int, bucket_elems: int):
    """The bucket table as a ctypes array of zero_bucket (16 bytes each) and its length."""
    n = i64()
    _check(lib().zero_layout_buckets(h, int(rank), int(bucket_elems), None, 0, ctypes.byref(n)))
    out = (zero_bucket * max(n.value, 1))()
    _check(lib().zero_layout_buckets(h, int(rank), int(bucket_elems), out, n.value, ctypes.byref(n)))
    return out, n.value


def zero_layout_buckets(h: int, rank: int, bucket_elems: int) -> list:
    """List of (shard_off, len, tensor)."""
    out, n = zero_layout_buckets_raw(h, rank, bucket_elems)
    return [(b.shard_off, b.len, b.tensor) for b in out[:n]]


def zero_layout_mem_values(h: int, stage: int) -> list:
    out = (i64 * 4)()
    _check(lib().zero_layout_mem_values(h, int(stage), out))
    return list(out)


def zero_layout_mem_bytes(h: int, stage: int) -> list:
    out = (i64 * 4)()
    _check(lib().zero_layout_mem_bytes(h, int(stage), out))
    return list(out)


def zero_layout_free(h: int) -> None:
    lib().zero_layout_free(h)


# ---------------------------------------------------------------------------
# device step
# ---------------------------------------------------------------------------

def zero_workspace_bytes(shard_S: int) -> int:
    return int(lib().zero_workspace_bytes(int(shard_S)))


def _replica_table(replicas):
    return (vp * max(len(replicas), 1))(*[_addr(r) for r in replicas])


def zero_reduce_shard(replicas, grad_dtype: int, shard_S: int, stats, workspace, *,
                      buckets=None, n_buckets: int = 0, loss_scale: float = 1.0,
                      grad_out=None, stream=None) -> None:
    table = _replica_table(replicas)
    ws = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    _check(lib().zero_reduce_shard(table, len(replicas), int(grad_dtype), int(shard_S),
                                   _addr(buckets), int(n_buckets), float(loss_scale),
                                   _addr(grad_out), _addr(stats), _addr(workspace), ws,
                                   _stream(stream)))


def make_adam_args(*, replicas=None, grad_dtype: int = ZERO_BF16, grad_f32=None, p_in, m_in, v_in,
                   p_out, m_out, v_out, slot=None, shard_S: int, buckets=None, n_buckets: int = 0,
                   lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
                   loss_scale: float = 1.0, step_t: int, stats, workspace, event_begin=None,
                   event_end=None, state_layout: int = 0):
    a = zero_adam_args()
    keep = []
    if replicas is not None:
        table = _replica_table(replicas)
        keep.append(table)
        a.replicas = ctypes.cast(table, ctypes.POINTER(vp))
        a.n_replicas = len(replicas)
    a.grad_dtype = int(grad_dtype)
    a.grad_f32 = _addr(grad_f32) or None
    for name, t in (("p_in", p_in), ("m_in", m_in), ("v_in", v_in), ("p_out", p_out),
                    ("m_out", m_out), ("v_out", v_out), ("slot_bf16", slot)):
        setattr(a, name, _addr(t) or None)
    a.shard_S = int(shard_S)
    a.buckets_dev = _addr(buckets) or None
    a.n_buckets = int(n_buckets)
    a.lr, a.beta1, a.beta2, a.eps = float(lr), float(beta1), float(beta2), float(eps)
    a.weight_decay, a.loss_scale, a.step_t = float(weight_decay), float(loss_scale), int(step_t)
    a.stats_dev = _addr(stats) or None
    a.workspace_dev = _addr(workspace) or None
    a.ws_bytes = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    a.event_begin = _event(event_begin)
    a.event_end = _event(event_end)
    a.state_layout = int(state_layout)
    a._keep = keep
    return a


def _event(ev):
    """hipEvent_t handle of a torch.cuda.Event (created on first record if needed)."""
    if ev is None:
        return None
    if isinstance(ev, int):
        return ev
    h = ev.cuda_event
    if not h:
        ev.record()
        h = ev.cuda_event
    return h


def zero_adam_step(args: zero_adam_args, stream=None) -> None:
    _check(lib().zero_adam_step(ctypes.byref(args), _stream(stream)))


def zero_adam_step_noalloc(args: zero_adam_args, stream=None) -> None:
    """zero_adam_step with the library's own scratch: args carry no workspace
    (make_adam_args(..., workspace=None))."""
    _check(lib().zero_adam_step_noalloc(ctypes.byref(args), _stream(stream)))


def zero_gather_slot(master, shard_S: int, slot, stream=None) -> None:
    _check(lib().zero_gather_slot(_addr(master), int(shard_S), _addr(slot), _stream(stream)))


def zero_gather_slot_tiled(set_buf, shard_S: int, slot, stream=None) -> None:
    _check(lib().zero_gather_slot_tiled(_addr(set_buf), int(shard_S), _addr(slot), _stream(stream)))


def zero_state_set_floats(shard_S: int, state_layout: int) -> int:
    n = lib().zero_state_set_floats(int(shard_S), int(state_layout))
    if n < 0:
        raise ZeroError(ZERO_E_INVAL, f"zero_state_set_floats: shard_S={shard_S}, "
                                      f"state_layout={state_layout}")
    return n


def zero_state_pack(p, m, v, shard_S: int, set_buf, stream=None) -> None:
    _check(lib().zero_state_pack(_addr(p), _addr(m), _addr(v), int(shard_S), _addr(set_buf),
                                 _stream(stream)))


def zero_state_unpack(set_buf, shard_S: int, p=None, m=None, v=None, stream=None) -> None:
    _check(lib().zero_state_unpack(_addr(set_buf), int(shard_S), _addr(p), _addr(m), _addr(v),
                                   _stream(stream)))


def zero_commit_rule(state: zero_train_state, stats_host: zero_stats) -> int:
    return _check(lib().zero_commit_rule(ctypes.byref(state), ctypes.byref(stats_host)))


def zero_device_state_init(state, workspace, beta1: float, beta2: float, loss_scale: float,
                           min_loss_scale: float = 1.0, dynamic: bool = False, stream=None) -> None:
    ws = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    _check(lib().zero_device_state_init(_addr(state), _addr(workspace), ws, float(beta1),
                                        float(beta2), float(loss_scale), float(min_loss_scale),
                                        int(bool(dynamic)), _stream(stream)))


def zero_device_state_load(state, workspace, saved: zero_device_state, stream=None) -> None:
    ws = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    _check(lib().zero_device_state_load(_addr(state), _addr(workspace), ws, ctypes.byref(saved),
                                        _stream(stream)))


def zero_device_state_flush(state, stats, workspace, stream=None) -> None:
    ws = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    _check(lib().zero_device_state_flush(_addr(state), _addr(stats), _addr(workspace), ws,
                                         _stream(stream)))


def make_train_args(*, replicas, grad_dtype: int, p, m, v, slot=None, shard_S: int, buckets=None,
                    n_buckets: int = 0, lr: float, eps: float, weight_decay: float, state, stats,
                    workspace, event_begin=None, event_end=None,
                    state_layout: int = 0) -> zero_train_args:
    a = zero_train_args()
    table = _replica_table(replicas)
    a.replicas = ctypes.cast(table, ctypes.POINTER(vp))
    a.n_replicas = len(replicas)
    a.grad_dtype = int(grad_dtype)
    for name, pair in (("p", p), ("m", m), ("v", v)):
        setattr(a, name, (vp * 2)(_addr(pair[0]) or None, _addr(pair[1]) or None))
    if isinstance(slot, (list, tuple)):
        a.slot = (vp * 2)(_addr(slot[0]) or None, _addr(slot[1]) or None)
    else:
        a.slot = (vp * 2)(_addr(slot) or None, None)
    a.shard_S = int(shard_S)
    a.buckets_dev = _addr(buckets) or None
    a.n_buckets = int(n_buckets)
    a.lr, a.eps, a.weight_decay = float(lr), float(eps), float(weight_decay)
    a.state_dev = _addr(state) or None
    a.stats_dev = _addr(stats) or None
    a.workspace_dev = _addr(workspace) or None
    a.ws_bytes = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    a.event_begin = _event(event_begin)
    a.event_end = _event(event_end)
    a.state_layout = int(state_layout)
    a._keep = [table]
    return a


def zero_train_step(args: zero_train_args, stream=None) -> None:
    _check(lib().zero_train_step(ctypes.byref(args), _stream(stream)))


def _host_addr(x) -> int:
    """Address of a host buffer: a CPU torch tensor, a numpy array, an int or None."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        assert not x.is_cuda, "host buffer expected"
        return x.data_ptr()
    return x.ctypes.data


def zero_host_adam(g, p, m, v, n: int, *, lr: float, beta1: float, beta2: float, eps: float,
                   weight_decay: float, step_t: int, slot=None, nthreads: int = 0) -> None:
    """Adam/AdamW on host buffers (in place on p, m, v)."""
    a = zero_host_adam_args(g=_host_addr(g), p=_host_addr(p), m=_host_addr(m), v=_host_addr(v),
                            slot_bf16=_host_addr(slot) or None, n=int(n), lr=float(lr),
                            beta1=float(beta1), beta2=float(beta2), eps=float(eps),
                            weight_decay=float(weight_decay), step_t=int(step_t),
                            nthreads=int(nthreads))
    _check(lib().zero_host_adam(ctypes.byref(a)))


def zero_offload_step(args: zero_offload_args, stream=None) -> tuple:
    """Returns (ZERO_COMMIT or ZERO_SKIP, zero_stats)."""
    st = zero_stats()
    rc = _check(lib().zero_offload_step(ctypes.byref(args), _stream(stream), ctypes.byref(st)))
    return rc, st


class GatherPlan:
    """The marshalled arguments of one zero_gather_tensors call, reusable: calling
    the plan enqueues the copies again (same shards, tensors and outputs)."""

    def __init__(self, shards, shard_S: int, offsets, numels, outs):
        self.k = len(numels)
        self.outs = outs
        self._keep = (shards, outs)
        self.args = (_replica_table(shards), len(shards), int(shard_S), shards[0].element_size(),
                     (i64 * max(self.k, 1))(*[int(o) for o in offsets]),
                     (i64 * max(self.k, 1))(*[int(n) for n in numels]),
                     (vp * max(self.k, 1))(*[_addr(o) for o in outs]), self.k)

    def __call__(self, stream=None):
        _check(lib().zero_gather_tensors(*self.args, _stream(stream)))
        return self.outs


def zero_gather_tensors(shards, shard_S: int, offsets, numels, outs=None, stream=None):
    """Copy whole tensors out of the rank shards (device tensors of shard_S elements,
    2- or 4-byte elements). outs: device tensors to fill, or None to allocate them
    (same dtype as the shards). Returns the outputs."""
    numels = [int(n) for n in numels]
    if outs is None:
        outs = [torch.empty(n, dtype=shards[0].dtype, device=shards[0].device) for n in numels]
    return GatherPlan(shards, shard_S, offsets, numels, outs)(stream)


def part_table(part_ends):
    """A host int64 array of part boundaries for zero_train_step_part."""
    ends = [int(e) for e in part_ends]
    return (ctypes.c_int64 * len(ends))(*ends), len(ends)


def zero_train_step_part(args: zero_train_args, table, n_parts: int, part: int, stream=None) -> None:
    _check(lib().zero_train_step_part(ctypes.byref(args), ctypes.addressof(table), int(n_parts),
                                      int(part), _stream(stream)))


def device_state_from_tensor(t) -> zero_device_state:
    """Read a device zero_device_state (uint8 tensor of 96+ bytes) to the host (synchronizes)."""
    raw = bytes(t.detach().to("cpu").numpy().tobytes())[: ctypes.sizeof(zero_device_state)]
    return zero_device_state.from_buffer_copy(raw)


def zero_last_error() -> str:
    return lib().zero_last_error().decode()


def zero_version() -> str:
    return lib().zero_version().decode()


def stats_from_tensor(t) -> zero_stats:
    """Read a 16-byte device zero_stats (uint8 tensor) into a host struct (synchronizes)."""
    raw = bytes(t.detach().to("cpu").numpy().tobytes())
    return zero_stats.from_buffer_copy(raw)
