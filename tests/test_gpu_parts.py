"""A device-committed step split into consecutive element ranges.

zero_train_step_part steps one range of the shard at a time, so a range can be
stepped as soon as its gradients are written while later ones are still being
produced (overlap with the gradient producer, "ZeRO Optimizer", "Communication
Optimization"). The last part collects every part's partials and commits. The
committed state must equal a whole-shard zero_train_step bit for bit whatever
the split (empty parts, one part, many parts, a ragged last part), across an
overflow step, with single and double-buffered slots, and when the parts wait on
events of a producer stream; and it must equal the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import NTHREADS, check_state, say, sumsq_close, to_dev, to_host

pytestmark = pytest.mark.gpu

S, N = 1_000_003, 8
HY = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, loss_scale=256.0,
          dynamic=True)


def replicas_for(step, n=N, size=S):
    rng = np.random.default_rng(5000 + step)
    reps = [to_dev(np.asarray(W._bf16_bits_from_f32(rng.standard_normal(size) * 1e-3 * 256.0)))
            for _ in range(n)]
    if step == 2:
        reps[3][777_777] = 0x7F80          # overflow inside a later part
    return reps


def tables():
    rng = np.random.default_rng(77)
    inner = np.sort(rng.choice(S // 8, size=6, replace=False)) * 8
    return {"one": [S], "tiny_first": [8, S], "empty": [0, 0, 504, 504, S],
            "random7": [int(x) for x in inner] + [S],
            "forty": [int(x) for x in np.linspace(0, S, 41)[1:-1] // 8 * 8] + [S]}


@pytest.fixture(scope="module")
def steps():
    return [replicas_for(k) for k in range(4)]


@pytest.fixture(scope="module")
def p0():
    return to_dev((np.random.default_rng(5100).standard_normal(S) * 0.02).astype(np.float32))


def same(a, b, tag):
    ra, rb = a.state(), b.state()
    for f in ("t", "n_skipped", "cur", "loss_scale", "beta1_pow", "beta2_pow", "last_overflow"):
        assert getattr(ra, f) == getattr(rb, f), (tag, f)
    assert sumsq_close(ra.last_sumsq, rb.last_sumsq), (tag, ra.last_sumsq, rb.last_sumsq)
    for x, y in zip(a.committed(), b.committed()):
        assert torch.equal(x, y), tag
    assert torch.equal(a.current_slot(), b.current_slot()), tag


@pytest.mark.parametrize("double_slot", [False, True])
@pytest.mark.parametrize("name", ["one", "tiny_first", "empty", "random7", "forty"])
def test_parts_equal_whole_step(Z, steps, p0, name, double_slot):
    ends = tables()[name]
    say(f"parts {name} ({len(ends)} parts) double_slot={double_slot}")
    whole = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, double_slot=double_slot, **HY)
    parts = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, double_slot=double_slot, **HY)
    for k, reps in enumerate(steps):
        whole.step(reps)
        parts.step_parts(reps, ends)
        same(whole, parts, (name, k))
    assert parts.state().n_skipped == 1 and parts.state().t == 3


def test_parts_wait_on_a_producer_stream(Z, p0):
    """A producer stream writes each range of the replicas (from a pool) and
    records an event; part k waits on event k. Three steps with new data each."""
    say("parts with a producer stream")
    ends = tables()["random7"]
    pool = [replicas_for(10 + k) for k in range(3)]
    bufs = [torch.empty(S, dtype=torch.int16, device="cuda") for _ in range(N)]
    ref = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, **HY)
    run = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, double_slot=True, **HY)
    producer, stepper = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for k in range(3):
        producer.wait_stream(stepper)       # the previous step has read the buffers
        ready = []
        lo = 0
        with torch.cuda.stream(producer):
            for hi in ends:
                for j in range(N):
                    bufs[j][lo:hi].copy_(pool[k][j][lo:hi])
                ev = torch.cuda.Event()
                ev.record(producer)
                ready.append(ev)
                lo = hi
        run.step_parts(bufs, ends, ready=ready, stream=stepper)
        ref.step(pool[k])
        torch.cuda.synchronize()
        same(ref, run, k)


@pytest.mark.parametrize("rank", [0, 63])
def test_parts_ragged_against_oracle(Z, rank):
    w = W.get("ragged")
    lay = oracle.Layout(w.numels, N=w.N, A=w.A, B=w.B)
    covered = [(int(s[2]), int(s[3])) for s in lay.segments(rank)]
    SS = lay.S
    ends = [SS // 5 // 8 * 8 * i for i in range(1, 5)] + [SS]
    p0h = W.host_params(w, SS, covered, rank)
    step = Z.DeviceShardStep(SS, w.N, Z.ZERO_BF16, to_dev(p0h), lr=w.lr, beta1=w.beta1,
                             beta2=w.beta2, eps=w.eps, weight_decay=w.wd, loss_scale=w.loss_scale,
                             dynamic=w.dynamic_loss_scale)
    tr = oracle.Trainer(p0h.copy(), np.zeros(SS, np.float32), np.zeros(SS, np.float32),
                        oracle.f32_to_bf16(p0h), loss_scale=w.loss_scale,
                        dynamic=w.dynamic_loss_scale, nthreads=NTHREADS, **w.hyper())
    flags = []
    for s in range(w.steps):
        say(f"parts ragged rank={rank} step={s}")
        reps = W.host_replicas(w, SS, covered, rank, s)
        step.step_parts([to_dev(r) for r in reps], ends)
        flag, sumsq = tr.step(reps)
        flags.append(flag)
        rec = step.state()
        assert rec.last_overflow == flag and rec.t == tr.t and rec.loss_scale == tr.loss_scale
        assert sumsq_close(rec.last_sumsq, sumsq)
        P, M, V = step.committed()
        check_state(f"parts ragged r{rank} s{s}", to_host(P), to_host(M), to_host(V),
                    to_host(step.current_slot()), tr.p, tr.m, tr.v, tr.slot)
    assert sum(flags) == 1


@pytest.mark.parametrize("tiled", [False, True])
def test_parts_multi_trip_grid_stride(Z, tiled):
    """4,096 parts cap each part's grid at 4,194,304 / 4,096 = 1,024 workgroups.
    The last part, 1,537,037 elements (1,501 trips of 1,024 elements, then 3
    quads and 1 element), runs on 751 workgroups that stride over two trips
    each; the one with a single trip (1,501 mod 751 = 750) also takes the quads
    after the last trip and the S % 4 tail. 4,094 empty parts come first, then an
    8,192-element part. Against the whole-shard step and the oracle, two steps."""
    first = 8192
    SS = first + 1501 * 1024 + 13
    ends = [0] * 4094 + [first, SS]
    n = 8
    rng = np.random.default_rng(99)
    p0h = (rng.standard_normal(SS) * 0.02).astype(np.float32)
    kw = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, loss_scale=1.0,
              double_slot=True, state_layout=Z.ZERO_STATE_TILED if tiled else Z.ZERO_STATE_SPLIT)
    parts = Z.DeviceShardStep(SS, n, Z.ZERO_BF16, to_dev(p0h), **kw)
    whole = Z.DeviceShardStep(SS, n, Z.ZERO_BF16, to_dev(p0h), **kw)
    tr = oracle.Trainer(p0h.copy(), np.zeros(SS, np.float32), np.zeros(SS, np.float32),
                        oracle.f32_to_bf16(p0h), loss_scale=1.0, dynamic=False, nthreads=NTHREADS,
                        lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)
    for s in range(2):
        say(f"parts multi-trip tiled={tiled} step {s}")
        hreps = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(SS) * 1e-3))
                 for _ in range(n)]
        dreps = [to_dev(r) for r in hreps]
        parts.step_parts(dreps, ends)
        whole.step(dreps)
        flag, sumsq = tr.step(hreps)
        assert flag == 0
        same(whole, parts, ("multi-trip", tiled, s))
        rec = parts.state()
        assert rec.t == s + 1 and sumsq_close(rec.last_sumsq, sumsq)
        P, M, V = parts.committed()
        check_state(f"parts multi-trip tiled={tiled} s{s}", to_host(P), to_host(M), to_host(V),
                    to_host(parts.current_slot()), tr.p, tr.m, tr.v, tr.slot)
