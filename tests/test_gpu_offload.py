"""The offloaded step (optimizer state in host memory) against the oracle.

zero_offload_step folds and checks the replicas on the GPU, moves the averaged
fp32 gradient to the host in chunks, runs the host Adam on each chunk as it
lands and uploads the bf16 values into the slot on the GPU ("ZeRO Optimizer",
"Advanced Optimizations", ZeRO-Offload). The committed host state and the
device slot must equal the oracle's multi-step rule bit for bit, across an
injected overflow with a dynamic loss scale, for every chunking, and equal the
all-GPU step on the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import NTHREADS, check_state, say, sumsq_close, to_dev, to_host

pytestmark = pytest.mark.gpu


def run_offload_protocol(Z, w, rank, steps=None, chunk_elems=0, upload_stream=True, nthreads=0):
    lay = oracle.Layout(w.numels, N=w.N, A=w.A, B=w.B)
    covered = [(int(s[2]), int(s[3])) for s in lay.segments(rank)]
    S = lay.S
    gdt = Z.ZERO_BF16 if w.grad_dtype == "bf16" else Z.ZERO_F32
    p0 = W.host_params(w, S, covered, rank)
    step = Z.OffloadShardStep(S, w.N, gdt, torch.from_numpy(p0.copy()), lr=w.lr, beta1=w.beta1,
                              beta2=w.beta2, eps=w.eps, weight_decay=w.wd,
                              loss_scale=w.loss_scale, dynamic=w.dynamic_loss_scale,
                              chunk_elems=chunk_elems, upload_stream=upload_stream,
                              nthreads=nthreads)
    tr = oracle.Trainer(p0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32),
                        oracle.f32_to_bf16(p0), loss_scale=w.loss_scale, dynamic=w.dynamic_loss_scale,
                        nthreads=NTHREADS, **w.hyper())
    flags = []
    for s in range(w.steps if steps is None else steps):
        say(f"offload {w.name} rank={rank} step={s} chunk={chunk_elems}")
        reps = W.host_replicas(w, S, covered, rank, s)
        st, verdict = step.step([to_dev(r) for r in reps])
        flag, sumsq = tr.step(reps)
        flags.append(flag)
        assert st.overflow == flag and verdict == (Z.ZERO_SKIP if flag else Z.ZERO_COMMIT)
        assert step.t == tr.t and step.loss_scale == tr.loss_scale
        assert sumsq_close(st.sumsq, sumsq)
        check_state(f"offload {w.name} r{rank} s{s}", step.p.numpy(), step.m.numpy(),
                    step.v.numpy(), to_host(step.slot), tr.p, tr.m, tr.v, tr.slot)
    return step, flags


def test_tiny_every_rank(Z):
    w = W.get("tiny")
    for rank in range(w.N):
        assert run_offload_protocol(Z, w, rank, chunk_elems=1000)[1] == [0, 0, 0]


@pytest.mark.parametrize("rank,chunk,upload", [(63, 100_003, True), (0, 0, False), (31, 8, True)])
def test_ragged_injection(Z, rank, chunk, upload):
    w = W.get("ragged")
    lay = oracle.Layout(w.numels, N=w.N, A=w.A, B=w.B)
    covered = [(int(s[2]), int(s[3])) for s in lay.segments(rank)]
    inj = W.injection(w, lay.S, covered, rank)
    steps = w.steps if chunk != 8 else 2
    _, flags = run_offload_protocol(Z, w, rank, steps=steps, chunk_elems=chunk,
                                    upload_stream=upload, nthreads=4)
    assert flags == [1 if s == inj[0] else 0 for s in range(steps)]


def test_gpt2_small_two_steps(Z):
    run_offload_protocol(Z, W.get("gpt2s"), 0, steps=2)


def test_offload_equals_gpu_step_and_resumes(Z):
    """Same inputs through the all-GPU step and the offloaded step; then a
    checkpoint of the offloaded run resumes bit for bit."""
    S, N = 300_007, 8
    rng = np.random.default_rng(606)
    p0 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, loss_scale=1024.0,
              dynamic=True)
    gpu = Z.DeviceShardStep(S, N, Z.ZERO_BF16, to_dev(p0), double_slot=True, **hy)
    off = Z.OffloadShardStep(S, N, Z.ZERO_BF16, torch.from_numpy(p0.copy()), chunk_elems=65_536, **hy)
    batches = [[to_dev(np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3 * 1024.0)))
                for _ in range(N)] for _ in range(4)]
    batches[1][2][9] = 0x7F80
    sd = None
    for k, reps in enumerate(batches):
        gpu.step(reps)
        off.step(reps)
        P, M, V = gpu.committed()
        assert torch.equal(P.cpu(), off.p) and torch.equal(M.cpu(), off.m) and torch.equal(V.cpu(), off.v)
        assert torch.equal(gpu.current_slot(), off.slot), k
        rec = gpu.state()
        assert (rec.t, rec.n_skipped, rec.loss_scale) == (off.t, off.state.n_skipped, off.loss_scale)
        if k == 1:
            sd = off.state_dict()
    res = Z.OffloadShardStep(S, N, Z.ZERO_BF16, torch.zeros(S), chunk_elems=65_536, **hy)
    res.load_state_dict(sd)
    for reps in batches[2:]:
        res.step(reps)
    assert torch.equal(res.p, off.p) and torch.equal(res.slot, off.slot) and res.t == off.t
