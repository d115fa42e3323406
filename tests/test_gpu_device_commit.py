"""GPU parity of the device-commit step (zero_train_step) against the oracle.

The commit rule runs on the GPU: the fused kernel reads the committed-state
record (current set, t, loss scale, beta^t) and its last workgroup applies the
skip rule. These tests compare the committed state after every step with the
oracle's multi-step rule (bit for bit), queue many steps with no host
synchronization in between (an overflow injected mid-chain), and check that the
device path equals the host-commit path.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import NTHREADS, check_state, say, sumsq_close, to_dev, to_host

pytestmark = pytest.mark.gpu


def layout_of(w, rank):
    lay = oracle.Layout(w.numels, N=w.N, A=w.A, B=w.B)
    return lay, [(int(s[2]), int(s[3])) for s in lay.segments(rank)]


def bucket_table(Z, w, rank, bucket_elems):
    h = Z.zero_layout_build(list(w.numels), w.N, w.A, w.B)
    raw, nb = Z.zero_layout_buckets_raw(h, rank, bucket_elems)
    Z.zero_layout_free(h)
    return torch.frombuffer(bytearray(bytes(raw)[: 16 * nb]), dtype=torch.uint8).to("cuda"), nb


def run_device_protocol(Z, w, rank, bucket_elems=0, steps=None, double_slot=False, wire=False,
                        tiled=False):
    lay, covered = layout_of(w, rank)
    S = lay.S
    gdt = Z.ZERO_BF16 if w.grad_dtype == "bf16" else Z.ZERO_F32
    if wire:
        gdt = Z.ZERO_BF16_WIRE
    p0 = W.host_params(w, S, covered, rank)
    bt, nb = bucket_table(Z, w, rank, bucket_elems) if bucket_elems else (None, 0)
    step = Z.DeviceShardStep(S, w.N, gdt, to_dev(p0), lr=w.lr, beta1=w.beta1, beta2=w.beta2,
                             eps=w.eps, weight_decay=w.wd, loss_scale=w.loss_scale,
                             dynamic=w.dynamic_loss_scale, buckets=bt, n_buckets=nb,
                             double_slot=double_slot,
                             state_layout=Z.ZERO_STATE_TILED if tiled else Z.ZERO_STATE_SPLIT)
    tr = oracle.Trainer(p0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32),
                        oracle.f32_to_bf16(p0), loss_scale=w.loss_scale, dynamic=w.dynamic_loss_scale,
                        nthreads=NTHREADS, wire=wire, **w.hyper())
    flags = []
    for s in range(w.steps if steps is None else steps):
        say(f"device {w.name} rank={rank} step={s} buckets={nb} wire={wire} tiled={tiled}")
        reps = W.host_replicas(w, S, covered, rank, s)
        step.step([to_dev(r) for r in reps])
        flag, sumsq = tr.step(reps)
        flags.append(flag)
        rec = step.state()
        st = step.last_stats()
        assert st.overflow == flag == rec.last_overflow and st.bad_buckets == 0
        assert rec.t == tr.t and rec.loss_scale == tr.loss_scale
        assert rec.n_skipped == sum(flags)
        assert sumsq_close(st.sumsq, sumsq) and sumsq_close(rec.last_sumsq, sumsq)
        P, M, V = step.committed()
        check_state(f"device {w.name} r{rank} s{s}", to_host(P), to_host(M), to_host(V),
                    to_host(step.current_slot()), tr.p, tr.m, tr.v, tr.slot)
    return flags


@pytest.mark.parametrize("double_slot", [False, True])
@pytest.mark.parametrize("tiled", [False, True])
def test_tiny_every_rank(Z, double_slot, tiled):
    w = W.get("tiny")
    for rank in range(w.N):
        assert run_device_protocol(Z, w, rank, double_slot=double_slot, tiled=tiled) == [0, 0, 0]


@pytest.mark.parametrize("rank,bucket_elems,double_slot,tiled", [
    (0, 0, False, False), (63, 0, True, False), (0, 4096, True, False), (31, 1000, False, False),
    (0, 0, False, True), (63, 0, True, True), (0, 4096, True, True), (31, 1000, False, True),
    (5, 65536, False, True), (40, 1 << 20, True, False)])
def test_ragged_injection(Z, rank, bucket_elems, double_slot, tiled):
    w = W.get("ragged")
    lay, covered = layout_of(w, rank)
    inj = W.injection(w, lay.S, covered, rank)
    flags = run_device_protocol(Z, w, rank, bucket_elems, double_slot=double_slot, tiled=tiled)
    assert flags == [1 if s == inj[0] else 0 for s in range(w.steps)]


@pytest.mark.parametrize("name,rank,double_slot,tiled", [("ragged", 63, True, False),
                                                         ("gpt2s", 0, False, False),
                                                         ("ragged", 0, False, True)])
def test_wire_device_commit(Z, name, rank, double_slot, tiled):
    w = W.get(name)
    run_device_protocol(Z, w, rank, double_slot=double_slot, wire=True,
                        steps=None if name == "ragged" else 2, tiled=tiled)


@pytest.mark.parametrize("rank", [0, 7])
def test_gpt2_tiled_device_commit(Z, rank):
    """The benchmark's configuration (GPT-2-small shard, tiled state, two slots)
    against the oracle for three steps, on the first and last rank."""
    run_device_protocol(Z, W.get("gpt2s"), rank, double_slot=True, tiled=True, steps=3)


def test_gpt2_bench_launch_all_steps(Z):
    """The bench's own launch and inputs -- GPT-2-small shard, rank 0, replicas and
    master filled on the device by the bench's generators, device commit, tiled
    state, two slots -- against the oracle for all 10 of the workload's steps,
    every element."""
    w = W.get("gpt2s")
    rank = 0
    lay, covered = layout_of(w, rank)
    S = lay.S
    p0 = torch.empty(S, dtype=torch.float32, device="cuda")
    W.device_fill_params(p0, w, covered, rank)
    ph = to_host(p0)
    step = Z.DeviceShardStep(S, w.N, Z.ZERO_BF16, p0, lr=w.lr, beta1=w.beta1, beta2=w.beta2,
                             eps=w.eps, weight_decay=w.wd, loss_scale=w.loss_scale,
                             dynamic=w.dynamic_loss_scale, double_slot=True,
                             state_layout=Z.ZERO_STATE_TILED)
    tr = oracle.Trainer(ph.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32),
                        oracle.f32_to_bf16(ph), loss_scale=w.loss_scale,
                        dynamic=w.dynamic_loss_scale, nthreads=NTHREADS, **w.hyper())
    reps = [torch.empty(S, dtype=torch.bfloat16, device="cuda") for _ in range(w.N)]
    assert w.steps == 10
    for s in range(w.steps):
        say(f"gpt2s bench launch step {s}")
        for j, r in enumerate(reps):
            W.device_fill_replica(r, w, covered, rank, s, j)
        dreps = [r.view(torch.int16) for r in reps]
        step.step(dreps)
        flag, sumsq = tr.step([to_host(r) for r in dreps])
        rec = step.state()
        st = step.last_stats()
        assert flag == 0 and st.overflow == 0 and rec.t == tr.t == s + 1
        assert sumsq_close(st.sumsq, sumsq), (st.sumsq, sumsq)
        P, M, V = step.committed()
        check_state(f"gpt2s bench launch s{s}", to_host(P), to_host(M), to_host(V),
                    to_host(step.current_slot()), tr.p, tr.m, tr.v, tr.slot)


def test_gpt2_device_equals_host_commit(Z):
    w = W.get("gpt2s")
    lay, covered = layout_of(w, 0)
    S = lay.S
    p0 = to_dev(W.host_params(w, S, covered, 0))
    kw = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.wd,
              loss_scale=w.loss_scale)
    hs = Z.ShardStep(S, w.N, Z.ZERO_BF16, p0, **kw)
    ds = Z.DeviceShardStep(S, w.N, Z.ZERO_BF16, p0, **kw)
    for s in range(3):
        say(f"gpt2s device vs host step {s}")
        dreps = [to_dev(r) for r in W.host_replicas(w, S, covered, 0, s)]
        st_h, _ = hs.step(dreps)
        ds.step(dreps)
        torch.cuda.synchronize()
        P, M, V = ds.committed()
        assert torch.equal(P, hs.master) and torch.equal(M, hs.exp_avg) and torch.equal(V, hs.exp_avg_sq)
        assert torch.equal(ds.slot, hs.slot)
        assert ds.last_stats().sumsq == st_h.sumsq
        assert ds.state().t == hs.t == s + 1


@pytest.mark.parametrize("double_slot", [False, True])
def test_queued_chain_with_overflow(Z, double_slot):
    """20 steps enqueued back to back with no host synchronization; step 7 carries
    a NaN and step 13 an +inf. The final state equals the oracle's trajectory."""
    S, N, K = 300_007, 8, 20
    rng = np.random.default_rng(77)
    sets = []
    for k in range(K):
        reps = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-4 * 1024.0))
                for _ in range(N)]
        if k == 7:
            reps[3][12345] = 0x7FC0
        if k == 13:
            reps[0][S - 1] = 0x7F80
        sets.append(reps)
    p0 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    step = Z.DeviceShardStep(S, N, Z.ZERO_BF16, to_dev(p0), weight_decay=0.01, loss_scale=1024.0,
                             dynamic=True, double_slot=double_slot, **hy)
    dsets = [[to_dev(r) for r in reps] for reps in sets]
    torch.cuda.synchronize()
    say("queued chain: enqueue 20 steps")
    for k in range(K):
        step.step(dsets[k])
    tr = oracle.Trainer(p0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32),
                        oracle.f32_to_bf16(p0), loss_scale=1024.0, dynamic=True, wd=0.01,
                        nthreads=NTHREADS, **hy)
    flags = [tr.step(reps)[0] for reps in sets]
    assert flags == [1 if k in (7, 13) else 0 for k in range(K)]
    rec = step.state()
    assert rec.t == tr.t == K - 2 and rec.n_skipped == 2 and rec.loss_scale == tr.loss_scale == 256.0
    P, M, V = step.committed()
    check_state("queued chain", to_host(P), to_host(M), to_host(V), to_host(step.current_slot()),
                tr.p, tr.m, tr.v, tr.slot)


def test_record_init_and_validation(Z):
    rec = torch.full((128,), 0x5A, dtype=torch.uint8, device="cuda")
    ws = torch.full((Z.zero_workspace_bytes(1 << 20),), 0x77, dtype=torch.uint8, device="cuda")
    Z.zero_device_state_init(rec, ws, 0.8, 0.95, 512.0, 2.0, True)
    r = Z.device_state_from_tensor(rec)
    assert (r.beta1, r.beta2, r.beta1_pow, r.beta2_pow) == (0.8, 0.95, 1.0, 1.0)
    assert (r.loss_scale, r.min_loss_scale, r.t, r.n_skipped, r.cur, r.dynamic) == (512.0, 2.0, 0, 0, 0, 1)
    assert (r.seq, r.last_overflow) == (0, 0)
    assert not bool(ws.any().item()), "the workspace is cleared"
    with pytest.raises(Z.ZeroError):
        Z.zero_device_state_init(rec, ws, 1.0, 0.9, 1.0)
    with pytest.raises(Z.ZeroError):
        Z.zero_device_state_init(rec[8:], ws, 0.9, 0.9, 1.0)
    with pytest.raises(Z.ZeroError):
        Z.zero_device_state_init(rec, ws, 0.9, 0.9, 1.0, min_loss_scale=2.0)


def test_stale_workspace_from_an_earlier_record(Z):
    """A workspace that an earlier record left holding partials tagged 1, 2, ... is
    cleared by the next record's init, so its first step cannot take them for its
    own: two records run back to back on one workspace match the oracle."""
    S, N = 200_003, 4
    rng = np.random.default_rng(3)
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    ws = torch.empty(Z.zero_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    for run in range(2):
        reps = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3)) for _ in range(N)]
        p0 = (rng.standard_normal(S) * 0.02).astype(np.float32)
        step = Z.DeviceShardStep(S, N, Z.ZERO_BF16, to_dev(p0), weight_decay=0.0, **hy)
        step.ws = ws
        Z.zero_device_state_init(step.record, ws, 0.9, 0.999, 1.0)
        dreps = [to_dev(r) for r in reps]
        tr = oracle.Trainer(p0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32),
                            oracle.f32_to_bf16(p0), wd=0.0, nthreads=NTHREADS, **hy)
        for k in range(2):
            step.step(dreps)
            tr.step(reps)
        P, M, V = step.committed()
        check_state(f"record {run}", to_host(P), to_host(M), to_host(V), to_host(step.current_slot()),
                    tr.p, tr.m, tr.v, tr.slot)
        assert step.state().seq == 2


@pytest.mark.parametrize("double_slot", [False, True])
def test_deferred_commit_overflow_on_last_step(Z, double_slot):
    """A step is folded into the record by the next launch or by a flush. Queue
    five steps with no host read in between, the last one carrying a +inf: the
    flush folds that skipped step in (t stays 4, the loss scale halves, the slot
    holds the committed master), and a second flush changes nothing."""
    S, N, K = 50_001, 3, 5
    rng = np.random.default_rng(21)
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    p0 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    sets = []
    for k in range(K):
        reps = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3 * 64.0)) for _ in range(N)]
        if k == K - 1:
            reps[1][S // 2] = W._bf16_bits_from_f32(np.array([np.inf]))[0]
        sets.append(reps)
    step = Z.DeviceShardStep(S, N, Z.ZERO_BF16, to_dev(p0), weight_decay=0.0, loss_scale=64.0,
                             dynamic=True, double_slot=double_slot, **hy)
    for reps in sets:
        step.step([to_dev(r) for r in reps])
    torch.cuda.synchronize()
    raw = Z.device_state_from_tensor(step.record)
    assert raw.pending_n > 0 and raw.seq == K - 1      # the last step is still pending
    tr = oracle.Trainer(p0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32),
                        oracle.f32_to_bf16(p0), loss_scale=64.0, dynamic=True, wd=0.0,
                        nthreads=NTHREADS, **hy)
    flags = [tr.step(reps)[0] for reps in sets]
    assert flags == [0, 0, 0, 0, 1]
    rec = step.state()
    assert (rec.seq, rec.pending_n, rec.t, rec.n_skipped, rec.last_overflow) == (K, 0, 4, 1, 1)
    assert rec.loss_scale == tr.loss_scale == 32.0
    assert step.last_stats().overflow == 1
    P, M, V = step.committed()
    check_state("deferred overflow", to_host(P), to_host(M), to_host(V),
                to_host(step.current_slot()), tr.p, tr.m, tr.v, tr.slot)
    again = step.state()
    assert bytes(again) == bytes(rec)
