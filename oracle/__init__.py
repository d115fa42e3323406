"""Plain CPU oracle for the per-rank ZeRO stage-1/2 shard step.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check (``smoke()``) and the
``cpu_baseline`` leg of ``bench.py`` are the only callers. The GPU product path
(``zero_partitioned_optimizer_amd``) never imports this package, and this package
never imports it: the two share no code.

This module is argument marshalling (ctypes over ``liboracle.so``, built from
``oracle.c`` with gcc) plus the multi-step commit rule, which is host logic:

* the step and its skip rule -- reduce-scatter the gradients so each rank's slice
  matches its optimizer-state partition, update that partition, all-gather the
  updated parameters ("[REQUEST] Direct Correspondence between Gradient and
  Optimizer States to Reduce Communication", section "Problem");
* the dynamic loss scale (halve on overflow, never below 1) and the rule that a
  skipped step leaves the state and the step counter untouched are the standard
  mixed-precision recipe ("ZeRO Optimizer" wiki page, "Hybrid Approaches" names
  mixed precision; the pages give no further detail, so this is the plainest
  reading).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1
BF16_WIRE = 2      # bf16 replicas, running sum rounded to bf16 after every add

GCC_FLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
             "-fopenmp", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = load(_LIB_PATH)
    return _lib


def load(path: str) -> ctypes.CDLL:
    """Open an oracle build at ``path`` and declare its C signatures."""
    L = ctypes.CDLL(path)
    i64, i32, vp, dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double
    L.or_layout.argtypes = [vp, i64, i64, i64, i64, vp, vp]
    L.or_layout.restype = ctypes.c_int
    L.or_segments.argtypes = [vp, vp, i64, i64, i64, vp, i64]
    L.or_segments.restype = i64
    L.or_buckets.argtypes = [vp, i64, i64, i64, vp, i64]
    L.or_buckets.restype = i64
    L.or_mem_values.argtypes = [i64, i64, i32, vp]
    L.or_mem_values.restype = ctypes.c_int
    L.or_mem_bytes.argtypes = [i64, i64, i32, vp]
    L.or_mem_bytes.restype = ctypes.c_int
    for name in ("or_ring_rs", "or_ring_rs_walk"):
        getattr(L, name).argtypes = [vp, i64, i64, vp, vp, vp, vp]
        getattr(L, name).restype = ctypes.c_int
    L.or_ring_rs_wire.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp]
    L.or_ring_rs_wire.restype = ctypes.c_int
    L.or_gather_tensor.argtypes = [vp, i64, i64, i32, i64, i64, vp]
    L.or_gather_tensor.restype = ctypes.c_int
    L.or_ring_ag.argtypes = [vp, i64, i64, vp, vp, vp]
    L.or_ring_ag.restype = ctypes.c_int
    L.or_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.or_bf16_to_f32.restype = ctypes.c_float
    L.or_f32_to_bf16.argtypes = [ctypes.c_float]
    L.or_f32_to_bf16.restype = ctypes.c_uint16
    L.or_f32_to_bf16_array.argtypes = [vp, i64, vp]
    L.or_f32_to_bf16_array.restype = None
    L.or_inv_scale.argtypes = [i32, dbl]
    L.or_inv_scale.restype = ctypes.c_float
    L.or_reduce.argtypes = [vp, i32, i32, i64, dbl, vp, vp, vp, i32]
    L.or_reduce.restype = None
    L.or_reduce_f64.argtypes = [vp, i32, i32, i64, dbl, vp, vp]
    L.or_reduce_f64.restype = None
    L.or_adam_scalars.argtypes = [dbl, dbl, dbl, dbl, dbl, i64, vp]
    L.or_adam_scalars.restype = None
    L.or_adam.argtypes = [vp, vp, vp, vp, i64, dbl, dbl, dbl, dbl, dbl, i64,
                          vp, vp, vp, vp, i32]
    L.or_adam.restype = None
    L.or_step.argtypes = [vp, i32, i32, i64, dbl, vp, vp, vp, vp, dbl, dbl, dbl, dbl, dbl,
                          i64, vp, i32]
    L.or_step.restype = ctypes.c_int
    return L


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


# ---------------------------------------------------------------------------
# layout and memory accounting
# ---------------------------------------------------------------------------

class Layout:
    """Flat layout + shard cut, as the oracle computes it (all int64)."""

    def __init__(self, numels, N: int, A: int = 1, B: int = 8):
        self.numels = np.ascontiguousarray(np.asarray(numels, dtype=np.int64))
        self.T = int(self.numels.size)
        self.N, self.A, self.B = int(N), int(A), int(B)
        self.offsets = np.zeros(max(self.T, 1), dtype=np.int64)
        out3 = np.zeros(3, dtype=np.int64)
        rc = lib().or_layout(_ptr(self.numels), self.T, self.N, self.A, self.B,
                             _ptr(self.offsets), _ptr(out3))
        if rc != 0:
            raise ValueError(f"or_layout rejected the arguments (rc={rc})")
        self.offsets = self.offsets[: self.T]
        self.L, self.S, self.L_pad = (int(x) for x in out3)
        self.psi = int(self.numels.sum())

    def segments(self, r: int) -> np.ndarray:
        """(k, 4) int64: tensor, tensor_off, shard_off, len."""
        cap = self.T + 1
        out = np.zeros((cap, 4), dtype=np.int64)
        n = lib().or_segments(_ptr(self.numels), _ptr(np.ascontiguousarray(self.offsets)),
                              self.T, self.S, int(r), _ptr(out), cap)
        if n < 0:
            raise RuntimeError("or_segments failed")
        return out[:n].copy()

    def buckets(self, r: int, bucket_elems: int) -> np.ndarray:
        """(k, 3) int64: shard_off, len, tensor of the first element."""
        seg = np.ascontiguousarray(self.segments(r))
        cap = len(seg) + (self.S // bucket_elems if bucket_elems > 0 else 0) + 2
        out = np.zeros((cap, 3), dtype=np.int64)
        n = lib().or_buckets(_ptr(seg) if len(seg) else 0, len(seg), self.S, int(bucket_elems),
                             _ptr(out), cap)
        if n < 0:
            raise RuntimeError("or_buckets failed")
        return out[:n].copy()

    def mem_values(self, stage: int) -> np.ndarray:
        out = np.zeros(4, dtype=np.int64)
        if lib().or_mem_values(self.L_pad, self.S, int(stage), _ptr(out)) != 0:
            raise ValueError("bad stage")
        return out

    def mem_bytes(self, stage: int) -> np.ndarray:
        out = np.zeros(4, dtype=np.int64)
        if lib().or_mem_bytes(self.L_pad, self.S, int(stage), _ptr(out)) != 0:
            raise ValueError("bad stage")
        return out


# ---------------------------------------------------------------------------
# ring collectives (message-passing simulation)
# ---------------------------------------------------------------------------

def ring_reduce_scatter(bufs: np.ndarray, walk: bool = False, wire: str = "f32"):
    """bufs: (N, N*S) float32, rank k's full local buffer in row k.

    Returns (chunks (N, S) float32 -- chunk c as held by its owner c,
    sent (N,), recv (N,), order (N, N) -- order[c] = ranks in the order their
    data entered chunk c). walk=True runs the literal one-extra-hop walk.
    wire="bf16" holds and sends every running partial in bf16 (standard ring)."""
    bufs = np.ascontiguousarray(bufs, dtype=np.float32)
    N = bufs.shape[0]
    S = bufs.shape[1] // N
    assert bufs.shape[1] == N * S
    out = np.zeros((N, S), dtype=np.float32)
    sent = np.zeros(N, dtype=np.int64)
    recv = np.zeros(N, dtype=np.int64)
    order = np.full((N, N), -1, dtype=np.int64)
    assert wire in ("f32", "bf16") and not (walk and wire != "f32")
    if walk:
        rc = lib().or_ring_rs_walk(_ptr(bufs), N, S, _ptr(out), _ptr(sent), _ptr(recv), _ptr(order))
    else:
        rc = lib().or_ring_rs_wire(_ptr(bufs), N, S, 1 if wire == "bf16" else 0, _ptr(out),
                                   _ptr(sent), _ptr(recv), _ptr(order))
    if rc != 0:
        raise RuntimeError("ring simulation failed")
    return out, sent, recv, order


def ring_all_gather(chunks: np.ndarray):
    """chunks: (N, S) float32. Returns (gathered (N, N*S), sent, recv)."""
    chunks = np.ascontiguousarray(chunks, dtype=np.float32)
    N, S = chunks.shape
    gathered = np.zeros((N, N * S), dtype=np.float32)
    sent = np.zeros(N, dtype=np.int64)
    recv = np.zeros(N, dtype=np.int64)
    if lib().or_ring_ag(_ptr(chunks), N, S, _ptr(gathered), _ptr(sent), _ptr(recv)) != 0:
        raise RuntimeError("ring all-gather simulation failed")
    return gathered, sent, recv


def gather_tensor(shards, offset: int, n: int) -> np.ndarray:
    """Stage-3 fetch: tensor elements [offset, offset + n) of the flat buffer,
    read from the N rank shards (arrays of S uint16 or float32 each)."""
    shards = [np.ascontiguousarray(x) for x in shards]
    N, S = len(shards), shards[0].size
    assert all(x.size == S and x.dtype == shards[0].dtype for x in shards)
    eb = shards[0].dtype.itemsize
    out = np.zeros(int(n), dtype=shards[0].dtype)
    table = (ctypes.c_void_p * N)(*[_ptr(x) for x in shards])
    if lib().or_gather_tensor(table, N, S, eb, int(offset), int(n), _ptr(out)) != 0:
        raise ValueError("gather_tensor: bad arguments")
    return out


# ---------------------------------------------------------------------------
# numerics
# ---------------------------------------------------------------------------

def f32_to_bf16(x) -> np.ndarray:
    """float32 array -> uint16 bf16 patterns (round to nearest even)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).reshape(-1)
    out = np.zeros(x.size, dtype=np.uint16)
    lib().or_f32_to_bf16_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(h) -> np.ndarray:
    h = np.asarray(h, dtype=np.uint16).reshape(-1)
    return (h.astype(np.uint32) << 16).view(np.float32)


def inv_scale(N: int, loss_scale: float) -> np.float32:
    return np.float32(lib().or_inv_scale(int(N), float(loss_scale)))


def adam_scalars(lr, beta1, beta2, eps, wd, t) -> np.ndarray:
    out = np.zeros(9, dtype=np.float32)
    lib().or_adam_scalars(lr, beta1, beta2, eps, wd, int(t), _ptr(out))
    return out


def _rep_table(reps, wire: bool = False):
    """wire=True: bf16 replicas folded as a bf16 ring does (each partial rounded)."""
    reps = [np.ascontiguousarray(r) for r in reps]
    dt = {np.dtype(np.float32): F32, np.dtype(np.uint16): BF16}
    kinds = {dt[r.dtype] for r in reps}
    assert len(kinds) == 1, "all replicas must share one dtype (float32 or uint16 bf16)"
    n = reps[0].size
    assert all(r.size == n for r in reps)
    table = (ctypes.c_void_p * len(reps))(*[_ptr(r) for r in reps])
    kind = kinds.pop()
    if wire:
        assert kind == BF16, "the bf16 wire applies to bf16 replicas"
        kind = BF16_WIRE
    return reps, table, kind, n


def reduce(reps, loss_scale: float = 1.0, nthreads: int = 1, wire: bool = False):
    """Slot-ordered fp32 left fold, times 1/(N*loss_scale).

    reps: list of N arrays (float32, or uint16 holding bf16 patterns).
    wire=True rounds the running sum to bf16 after every add.
    Returns (g float32, overflow flag int, sumsq float)."""
    reps, table, dtype, n = _rep_table(reps, wire)
    g = np.zeros(n, dtype=np.float32)
    flag = ctypes.c_uint32(0)
    sumsq = ctypes.c_double(0.0)
    lib().or_reduce(table, len(reps), dtype, n, float(loss_scale), _ptr(g),
                    ctypes.addressof(flag), ctypes.addressof(sumsq), int(nthreads))
    return g, int(flag.value), float(sumsq.value)


def reduce_f64(reps, loss_scale: float = 1.0):
    """Exact double-precision sum (and sum of magnitudes), times 1/(N*loss_scale)."""
    reps, table, dtype, n = _rep_table(reps)
    g = np.zeros(n, dtype=np.float64)
    a = np.zeros(n, dtype=np.float64)
    lib().or_reduce_f64(table, len(reps), dtype, n, float(loss_scale), _ptr(g), _ptr(a))
    return g, a


def adam(g, p, m, v, *, lr, beta1, beta2, eps, wd, t, nthreads: int = 1):
    """Adam/AdamW update (out of place). Returns (p', m', v', slot uint16)."""
    g, p, m, v = (np.ascontiguousarray(np.asarray(a, dtype=np.float32)) for a in (g, p, m, v))
    n = g.size
    po, mo, vo = (np.zeros(n, dtype=np.float32) for _ in range(3))
    slot = np.zeros(n, dtype=np.uint16)
    lib().or_adam(_ptr(g), _ptr(p), _ptr(m), _ptr(v), n, float(lr), float(beta1), float(beta2),
                  float(eps), float(wd), int(t), _ptr(po), _ptr(mo), _ptr(vo), _ptr(slot),
                  int(nthreads))
    return po, mo, vo, slot


def step(reps, p, m, v, slot, *, loss_scale, lr, beta1, beta2, eps, wd, t, nthreads: int = 1,
         wire: bool = False):
    """One step with the skip rule, in place on p, m, v, slot. Returns (flag, sumsq)."""
    reps, table, dtype, n = _rep_table(reps, wire)
    for a, want in ((p, np.float32), (m, np.float32), (v, np.float32), (slot, np.uint16)):
        assert a.dtype == want and a.flags["C_CONTIGUOUS"] and a.size == n
    sumsq = ctypes.c_double(0.0)
    flag = lib().or_step(table, len(reps), dtype, n, float(loss_scale), _ptr(p), _ptr(m),
                         _ptr(v), _ptr(slot), float(lr), float(beta1), float(beta2), float(eps),
                         float(wd), int(t), ctypes.addressof(sumsq), int(nthreads))
    if flag < 0:
        raise RuntimeError("or_step failed")
    return int(flag), float(sumsq.value)


class Trainer:
    """The multi-step rule around ``step``: a clean step commits and advances the
    update counter t; an overflowed step leaves p, m, v, the slot and t as they
    were and, with a dynamic loss scale, halves the scale (never below 1)."""

    def __init__(self, p, m, v, slot, *, lr, beta1, beta2, eps, wd, loss_scale=1.0,
                 dynamic=False, nthreads=1, wire=False):
        self.p, self.m, self.v, self.slot = p, m, v, slot
        self.wire = bool(wire)
        self.hyper = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, wd=wd)
        self.loss_scale = float(loss_scale)
        self.dynamic = bool(dynamic)
        self.t = 0
        self.nthreads = nthreads
        self.history = []

    def step(self, reps):
        flag, sumsq = step(reps, self.p, self.m, self.v, self.slot, loss_scale=self.loss_scale,
                           t=self.t + 1, nthreads=self.nthreads, wire=self.wire, **self.hyper)
        self.history.append((flag, sumsq, self.loss_scale, self.t))
        if flag:
            if self.dynamic:
                self.loss_scale = max(self.loss_scale / 2.0, 1.0)
        else:
            self.t += 1
        return flag, sumsq
