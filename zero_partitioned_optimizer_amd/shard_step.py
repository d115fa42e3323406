"""ShardStep: one rank's ZeRO stage-1/2 optimizer step around libzero.

Device work runs in libzero's kernels; this class only owns buffers (through
torch) and applies the host commit rule:

* the fused step reads the N resident gradient replicas and the committed state
  (p, m, v "in"), and writes the candidate state (p, m, v "out") plus the bf16
  slot, with the overflow flag and squared norm in a 16-byte stats record;
* ``zero_commit_rule`` decides: a clean step swaps the in/out buffers and advances
  t; an overflowed step keeps the in buffers, restores the slot from the
  committed master copy and (dynamic scaling) halves the loss scale.

The step and its data flow follow "[REQUEST] Direct Correspondence between
Gradient and Optimizer States to Reduce Communication", "Problem"; mixed
precision is named in "ZeRO Optimizer", "Hybrid Approaches".
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _binding as B


class ShardStep:
    def __init__(self, shard_S: int, n_replicas: int, grad_dtype: int, p0: torch.Tensor, *,
                 lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
                 loss_scale: float = 1.0, dynamic: bool = False, min_loss_scale: float = 1.0,
                 slot: Optional[torch.Tensor] = None, buckets: Optional[torch.Tensor] = None,
                 n_buckets: int = 0):
        dev = p0.device
        S = int(shard_S)
        assert p0.dtype == torch.float32 and p0.numel() == S and p0.is_contiguous()
        self.S, self.N, self.grad_dtype = S, int(n_replicas), int(grad_dtype)
        self.hyper = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay)
        # zeros: bucket-table steps leave padding untouched
        self.p = [p0.clone(), torch.zeros_like(p0)]
        self.m = [torch.zeros_like(p0), torch.zeros_like(p0)]
        self.v = [torch.zeros_like(p0), torch.zeros_like(p0)]
        self.cur = 0
        self.slot = slot if slot is not None else torch.empty(S, dtype=torch.int16, device=dev)
        assert self.slot.numel() == S and self.slot.element_size() == 2
        self.buckets, self.n_buckets = buckets, int(n_buckets)
        self.stats = torch.zeros(16, dtype=torch.uint8, device=dev)
        self.stats_host = torch.zeros(16, dtype=torch.uint8, pin_memory=True)
        self.ws = torch.empty(B.zero_workspace_bytes(S), dtype=torch.uint8, device=dev)
        self.state = B.zero_train_state(t=0, n_skipped=0, loss_scale=float(loss_scale),
                                        min_loss_scale=float(min_loss_scale), dynamic=int(dynamic))
        B.zero_gather_slot(self.p[0], S, self.slot)
        self._args = [None, None]
        self._args_key = None

    # committed state
    @property
    def master(self) -> torch.Tensor:
        return self.p[self.cur]

    @property
    def exp_avg(self) -> torch.Tensor:
        return self.m[self.cur]

    @property
    def exp_avg_sq(self) -> torch.Tensor:
        return self.v[self.cur]

    @property
    def t(self) -> int:
        return int(self.state.t)

    @property
    def loss_scale(self) -> float:
        return float(self.state.loss_scale)

    def _args_for(self, replicas: Sequence[torch.Tensor]):
        """The argument block for the current direction (in -> out). Two blocks are
        built once per replica set and reused; only t, the loss scale and the
        events change from step to step."""
        key = tuple(r.data_ptr() for r in replicas)
        if self._args_key != key:
            self._args = [None, None]
            self._args_key = key
        i, o = self.cur, 1 - self.cur
        a = self._args[i]
        if a is None:
            a = B.make_adam_args(replicas=list(replicas), grad_dtype=self.grad_dtype,
                                 p_in=self.p[i], m_in=self.m[i], v_in=self.v[i], p_out=self.p[o],
                                 m_out=self.m[o], v_out=self.v[o], slot=self.slot, shard_S=self.S,
                                 buckets=self.buckets, n_buckets=self.n_buckets,
                                 loss_scale=self.state.loss_scale, step_t=self.state.t + 1,
                                 stats=self.stats, workspace=self.ws, **self.hyper)
            self._args[i] = a
        a.step_t = self.state.t + 1
        a.loss_scale = self.state.loss_scale
        return a

    def launch(self, replicas: Sequence[torch.Tensor], stream=None, events=None) -> None:
        """Enqueue the fused step (no synchronization). ``events`` = optional pair of
        torch.cuda.Event that the main kernel's launch carries (its start and end)."""
        a = self._args_for(replicas)
        if events is not None:
            a.event_begin = B._event(events[0])
            a.event_end = B._event(events[1])
        else:
            a.event_begin = a.event_end = None
        B.zero_adam_step(a, stream)

    def read_stats(self, stream=None) -> B.zero_stats:
        self.stats_host.copy_(self.stats, non_blocking=True)
        (stream or torch.cuda.current_stream()).synchronize()
        return B.zero_stats.from_buffer_copy(self.stats_host.numpy().tobytes())

    def commit(self, st: B.zero_stats, stream=None) -> int:
        verdict = B.zero_commit_rule(self.state, st)
        if verdict == B.ZERO_COMMIT:
            self.cur = 1 - self.cur
        else:
            B.zero_gather_slot(self.p[self.cur], self.S, self.slot, stream)
        return verdict

    def state_dict(self) -> dict:
        """The committed state on the host: master copy, moments and the commit
        record (t, skips, loss scale). Hyperparameters are the caller's."""
        st = self.state
        return {"p": self.master.cpu(), "m": self.exp_avg.cpu(), "v": self.exp_avg_sq.cpu(),
                "t": int(st.t), "n_skipped": int(st.n_skipped), "loss_scale": float(st.loss_scale),
                "min_loss_scale": float(st.min_loss_scale), "dynamic": int(st.dynamic)}

    def load_state_dict(self, sd: dict) -> None:
        """Resume from ``state_dict()``: the next step continues the saved run."""
        c = self.cur
        for dst, key in ((self.p[c], "p"), (self.m[c], "m"), (self.v[c], "v")):
            assert sd[key].numel() == self.S and sd[key].dtype == torch.float32
            dst.copy_(sd[key])
        self.state = B.zero_train_state(t=sd["t"], n_skipped=sd["n_skipped"],
                                        loss_scale=sd["loss_scale"],
                                        min_loss_scale=sd["min_loss_scale"], dynamic=sd["dynamic"])
        B.zero_gather_slot(self.p[c], self.S, self.slot)

    def step(self, replicas: Sequence[torch.Tensor], stream=None, events=None):
        """One full step: fused kernel, read the 16-byte stats, apply the commit rule."""
        self.launch(replicas, stream, events)
        st = self.read_stats(stream)
        verdict = self.commit(st, stream)
        return st, verdict


class DeviceShardStep:
    """The same step with the commit on the device (``zero_train_step``): each
    launch derives the committed state from the record and the previous step's
    overflow flag, and its workgroup 0 folds the previous step into the record,
    so steps queue back to back with no host synchronization. The host reads the
    record (t, loss scale, current set) only when it wants to, after a flush
    (``state()``, ``last_stats()`` and the methods built on them do that)."""

    def __init__(self, shard_S: int, n_replicas: int, grad_dtype: int, p0: torch.Tensor, *,
                 lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
                 loss_scale: float = 1.0, dynamic: bool = False, min_loss_scale: float = 1.0,
                 slot: Optional[torch.Tensor] = None, buckets: Optional[torch.Tensor] = None,
                 n_buckets: int = 0, double_slot: bool = False,
                 state_layout: int = B.ZERO_STATE_SPLIT):
        """double_slot: keep a second slot buffer so that the candidate bf16 values
        land in the non-current one and a skipped step needs no restore kernel;
        ``slot`` is then the pair's first buffer and ``current_slot()`` the
        committed one. state_layout: ZERO_STATE_SPLIT keeps p, m, v of each set in
        three arrays (``self.p[k]``, ``self.m[k]``, ``self.v[k]``);
        ZERO_STATE_TILED keeps each set in one tiled buffer (``self.sets[k]``)."""
        dev = p0.device
        S = int(shard_S)
        assert p0.dtype == torch.float32 and p0.numel() == S and p0.is_contiguous()
        self.S, self.N, self.grad_dtype = S, int(n_replicas), int(grad_dtype)
        self.lr, self.eps, self.weight_decay = float(lr), float(eps), float(weight_decay)
        self.double_slot = bool(double_slot)
        self.tiled = int(state_layout) == B.ZERO_STATE_TILED
        assert int(state_layout) in (B.ZERO_STATE_SPLIT, B.ZERO_STATE_TILED)
        if self.tiled:
            n = B.zero_state_set_floats(S, B.ZERO_STATE_TILED)
            self.sets = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(2)]
            zm, zv = torch.zeros_like(p0), torch.zeros_like(p0)
            B.zero_state_pack(p0, zm, zv, S, self.sets[0])
            torch.cuda.current_stream(dev).synchronize()
            del zm, zv
            self.p = self.m = self.v = None
        else:
            self.sets = None
            self.p = [p0.clone(), torch.zeros_like(p0)]
            self.m = [torch.zeros_like(p0), torch.zeros_like(p0)]
            self.v = [torch.zeros_like(p0), torch.zeros_like(p0)]
        self.slot = slot if slot is not None else torch.empty(S, dtype=torch.int16, device=dev)
        assert self.slot.numel() == S and self.slot.element_size() == 2
        self.slot_alt = torch.zeros(S, dtype=torch.int16, device=dev) if self.double_slot else None
        self.buckets, self.n_buckets = buckets, int(n_buckets)
        self.stats = torch.zeros(16, dtype=torch.uint8, device=dev)
        self.record = torch.zeros(128, dtype=torch.uint8, device=dev)
        self.ws = torch.empty(B.zero_workspace_bytes(S), dtype=torch.uint8, device=dev)
        B.zero_device_state_init(self.record, self.ws, beta1, beta2, loss_scale, min_loss_scale,
                                 dynamic)
        self._cast_slot(0, self.slot)
        self._args = None
        self._args_key = None

    def _args_for(self, replicas):
        key = tuple(r.data_ptr() for r in replicas)
        if self._args_key != key:
            slot = (self.slot, self.slot_alt) if self.double_slot else self.slot
            if self.tiled:
                p, m, v = self.sets, (None, None), (None, None)
            else:
                p, m, v = self.p, self.m, self.v
            self._args = B.make_train_args(replicas=list(replicas), grad_dtype=self.grad_dtype,
                                           p=p, m=m, v=v, slot=slot,
                                           shard_S=self.S, buckets=self.buckets,
                                           n_buckets=self.n_buckets, lr=self.lr, eps=self.eps,
                                           weight_decay=self.weight_decay, state=self.record,
                                           stats=self.stats, workspace=self.ws,
                                           state_layout=B.ZERO_STATE_TILED if self.tiled
                                           else B.ZERO_STATE_SPLIT)
            self._args_key = key
        a = self._args
        a.lr, a.eps, a.weight_decay = self.lr, self.eps, self.weight_decay
        return a

    def step(self, replicas: Sequence[torch.Tensor], stream=None, events=None) -> None:
        """Enqueue one whole step (fused kernel + device commit); no synchronization."""
        a = self._args_for(replicas)
        if events is not None:
            a.event_begin = B._event(events[0])
            a.event_end = B._event(events[1])
        else:
            a.event_begin = a.event_end = None
        B.zero_train_step(a, stream)

    def step_parts(self, replicas: Sequence[torch.Tensor], part_ends: Sequence[int],
                   ready=None, stream=None, events=None) -> None:
        """Enqueue one step as consecutive element ranges (``zero_train_step_part``),
        all on one stream; ``ready[k]`` (a torch.cuda.Event, optional) is waited on
        before part k, so each range is stepped as soon as its gradients are
        written. ``events[k]`` (optional pair) times part k's kernel."""
        a = self._args_for(replicas)
        key = tuple(int(e) for e in part_ends)
        if getattr(self, "_parts_key", None) != key:
            self._parts, self._parts_n = B.part_table(key)
            self._parts_key = key
        st = stream if stream is not None else torch.cuda.current_stream()
        for k in range(self._parts_n):
            if ready is not None and ready[k] is not None:
                st.wait_event(ready[k])
            ev = events[k] if events is not None else None
            a.event_begin = B._event(ev[0]) if ev is not None else None
            a.event_end = B._event(ev[1]) if ev is not None else None
            B.zero_train_step_part(a, self._parts, self._parts_n, k, st)
        a.event_begin = a.event_end = None

    def flush(self, stream=None) -> None:
        """Enqueue the folding of the last step into the record and the stats."""
        B.zero_device_state_flush(self.record, self.stats, self.ws, stream)

    def state(self, check: bool = True) -> B.zero_device_state:
        """Flush, then copy the committed-state record back (synchronizes). A record
        frozen by a ZERO_RECORD_E_* code raises ZeroRecordError unless check is
        False."""
        self.flush()
        rec = B.device_state_from_tensor(self.record)
        if check and rec.error:
            raise B.ZeroRecordError(int(rec.error))
        return rec

    def last_stats(self) -> B.zero_stats:
        """Flush, then copy the last step's stats back (synchronizes). Raises
        ZeroRecordError on a frozen record."""
        self.state()
        return B.stats_from_tensor(self.stats)

    def _cast_slot(self, k: int, slot: torch.Tensor) -> None:
        """Cast set k's master into ``slot`` (bf16)."""
        if self.tiled:
            B.zero_gather_slot_tiled(self.sets[k], self.S, slot)
        else:
            B.zero_gather_slot(self.p[k], self.S, slot)

    def set_state(self, k: int):
        """(master, m, v) of state set k as flat fp32 tensors: views of the split
        arrays, or copies unpacked from the tiled buffer (on the current stream)."""
        if not self.tiled:
            return self.p[k], self.m[k], self.v[k]
        out = [torch.empty(self.S, dtype=torch.float32, device=self.sets[k].device)
               for _ in range(3)]
        B.zero_state_unpack(self.sets[k], self.S, *out)
        return tuple(out)

    def set_state_at(self, k: int, idx: torch.Tensor):
        """(master, m, v) of state set k at the element indices ``idx`` (an int64
        device tensor), without unpacking the whole set."""
        if not self.tiled:
            return self.p[k][idx], self.m[k][idx], self.v[k][idx]
        T = B.ZERO_STATE_TILE
        base = (idx // T) * (3 * T) + idx % T
        s = self.sets[k]
        return s[base], s[base + T], s[base + 2 * T]

    def committed(self):
        """(master, m, v) of the committed state (synchronizes)."""
        return self.set_state(self.state().cur & 1)

    def committed_at(self, idx: torch.Tensor):
        """(master, m, v) of the committed state at element indices ``idx``
        (synchronizes)."""
        return self.set_state_at(self.state().cur & 1, idx)

    def state_dict(self) -> dict:
        """The committed state on the host (synchronizes): the record's bytes and
        the master copy and moments of its current set, as flat fp32 arrays in
        either layout."""
        rec = self.state()
        p, m, v = self.set_state(rec.cur & 1)
        return {"record": bytes(rec), "p": p.cpu(), "m": m.cpu(), "v": v.cpu()}

    def load_state_dict(self, sd: dict) -> None:
        """Resume from ``state_dict()``: the saved set goes back into the set the
        record names, libzero rewrites the record (clearing the workspace) and
        the slot is cast again from the master copy."""
        rec = B.zero_device_state.from_buffer_copy(sd["record"])
        c = rec.cur & 1
        for key in ("p", "m", "v"):
            assert sd[key].numel() == self.S and sd[key].dtype == torch.float32
        if self.tiled:
            dev = self.sets[c].device
            p, m, v = (sd[key].to(dev).contiguous() for key in ("p", "m", "v"))
            B.zero_state_pack(p, m, v, self.S, self.sets[c])
            torch.cuda.current_stream(dev).synchronize()
        else:
            for dst, key in ((self.p[c], "p"), (self.m[c], "m"), (self.v[c], "v")):
                dst.copy_(sd[key])
        B.zero_device_state_load(self.record, self.ws, rec)
        slot = self.slot_alt if (self.double_slot and c) else self.slot
        self._cast_slot(c, slot)

    def current_slot(self) -> torch.Tensor:
        """The slot buffer holding the committed bf16 parameters (synchronizes)."""
        if not self.double_slot:
            return self.slot
        return self.slot_alt if self.state().cur & 1 else self.slot


class OffloadShardStep:
    """The step with the shard's fp32 master, m and v in host memory
    (``zero_offload_step``): the GPU folds and checks the replicas, the averaged
    gradient crosses to the host in chunks, host threads run Adam on each chunk
    as it lands, and the bf16 values go back into the slot on the GPU. The
    commit rule runs on the host, as in ``ShardStep``; a skipped step touches
    nothing. Only the replicas, one fp32 gradient buffer and the slot stay in
    device memory."""

    def __init__(self, shard_S: int, n_replicas: int, grad_dtype: int, p0: torch.Tensor, *,
                 lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
                 loss_scale: float = 1.0, dynamic: bool = False, min_loss_scale: float = 1.0,
                 slot: Optional[torch.Tensor] = None, chunk_elems: int = 0, nthreads: int = 0,
                 upload_stream: bool = True, device=None):
        S = int(shard_S)
        assert p0.dtype == torch.float32 and p0.numel() == S
        dev = torch.device(device) if device is not None else torch.device(
            "cuda", torch.cuda.current_device())
        self.S, self.N, self.grad_dtype = S, int(n_replicas), int(grad_dtype)
        self.hyper = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay)
        self.p = p0.detach().to("cpu", copy=True).contiguous()
        self.m = torch.zeros(S, dtype=torch.float32)
        self.v = torch.zeros(S, dtype=torch.float32)
        self.g_dev = torch.empty(S, dtype=torch.float32, device=dev)
        self.g_host = torch.empty(S, dtype=torch.float32, pin_memory=True)
        self.slot_host = torch.empty(S, dtype=torch.int16, pin_memory=True)
        self.slot = slot if slot is not None else torch.empty(S, dtype=torch.int16, device=dev)
        assert self.slot.numel() == S and self.slot.element_size() == 2 and self.slot.is_cuda
        self.stats = torch.zeros(16, dtype=torch.uint8, device=dev)
        self.ws = torch.empty(B.zero_workspace_bytes(S), dtype=torch.uint8, device=dev)
        self.state = B.zero_train_state(t=0, n_skipped=0, loss_scale=float(loss_scale),
                                        min_loss_scale=float(min_loss_scale), dynamic=int(dynamic))
        self.chunk_elems, self.nthreads = int(chunk_elems), int(nthreads)
        self.upload = torch.cuda.Stream(device=dev) if upload_stream else None
        self._args = None
        self._args_key = None
        self._recast_slot()

    def _recast_slot(self):
        master = self.p.to(self.g_dev.device)
        B.zero_gather_slot(master, self.S, self.slot)
        torch.cuda.current_stream().synchronize()

    @property
    def t(self) -> int:
        return int(self.state.t)

    @property
    def loss_scale(self) -> float:
        return float(self.state.loss_scale)

    def _args_for(self, replicas: Sequence[torch.Tensor]) -> B.zero_offload_args:
        key = tuple(r.data_ptr() for r in replicas)
        if self._args_key != key:
            table = B._replica_table(list(replicas))
            a = B.zero_offload_args()
            a.replicas = ctypes.cast(table, ctypes.POINTER(ctypes.c_void_p))
            a.n_replicas = len(replicas)
            a.grad_dtype = self.grad_dtype
            a.shard_S = self.S
            a.g_dev, a.g_host = self.g_dev.data_ptr(), self.g_host.data_ptr()
            a.p_host, a.m_host, a.v_host = self.p.data_ptr(), self.m.data_ptr(), self.v.data_ptr()
            a.slot_host, a.slot_dev = self.slot_host.data_ptr(), self.slot.data_ptr()
            a.state = ctypes.pointer(self.state)
            a.stats_dev = self.stats.data_ptr()
            a.workspace_dev = self.ws.data_ptr()
            a.ws_bytes = self.ws.numel()
            a.chunk_elems, a.nthreads = self.chunk_elems, self.nthreads
            a.stream_h2d = self.upload.cuda_stream if self.upload is not None else None
            self._args, self._table, self._args_key = a, table, key
        a = self._args
        a.lr, a.beta1, a.beta2 = self.hyper["lr"], self.hyper["beta1"], self.hyper["beta2"]
        a.eps, a.weight_decay = self.hyper["eps"], self.hyper["weight_decay"]
        return a

    def step(self, replicas: Sequence[torch.Tensor], stream=None):
        """One offloaded step (synchronous). Returns (stats, ZERO_COMMIT or ZERO_SKIP)."""
        verdict, st = B.zero_offload_step(self._args_for(replicas), stream)
        return st, verdict

    def state_dict(self) -> dict:
        st = self.state
        return {"p": self.p.clone(), "m": self.m.clone(), "v": self.v.clone(), "t": int(st.t),
                "n_skipped": int(st.n_skipped), "loss_scale": float(st.loss_scale),
                "min_loss_scale": float(st.min_loss_scale), "dynamic": int(st.dynamic)}

    def load_state_dict(self, sd: dict) -> None:
        for dst, key in ((self.p, "p"), (self.m, "m"), (self.v, "v")):
            assert sd[key].numel() == self.S and sd[key].dtype == torch.float32
            dst.copy_(sd[key])
        self.state.t, self.state.n_skipped = sd["t"], sd["n_skipped"]
        self.state.loss_scale, self.state.min_loss_scale = sd["loss_scale"], sd["min_loss_scale"]
        self.state.dynamic = sd["dynamic"]
        self._recast_slot()
