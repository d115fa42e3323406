"""Checkpoint and resume of one rank's shard state.

The committed state of the shard is the fp32 master copy, the two Adam moments
and the commit record (t, skipped steps, loss scale, beta powers): the per-rank
optimizer state of "ZeRO Optimizer" (stage 1 memory terms). A run stopped after
k steps, saved to the host, and resumed in a fresh object (or in the same object
after it has run further) must continue bit for bit like an uninterrupted run,
including a skipped overflow step and the loss scale it halved.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu

S, N, K = 300_007, 8, 6
HY = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, loss_scale=1024.0,
          dynamic=True)


def replicas_for(step):
    """Seeded bf16 replicas of one step; step 3 carries a +inf in slot 5."""
    rng = np.random.default_rng(4000 + step)
    reps = [to_dev(np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3 * 1024.0)))
            for _ in range(N)]
    if step == 3:
        reps[5][12345] = 0x7F80
    return reps


@pytest.fixture(scope="module")
def steps():
    return [replicas_for(k) for k in range(K)]


@pytest.fixture(scope="module")
def p0():
    rng = np.random.default_rng(4100)
    return to_dev((rng.standard_normal(S) * 0.02).astype(np.float32))


def same_device(a, b, k):
    ra, rb = a.state(), b.state()
    for f in ("t", "n_skipped", "cur", "loss_scale", "beta1_pow", "beta2_pow", "last_overflow",
              "last_sumsq"):
        assert getattr(ra, f) == getattr(rb, f), (k, f, getattr(ra, f), getattr(rb, f))
    for x, y in zip(a.committed(), b.committed()):
        assert torch.equal(x, y), k
    assert torch.equal(a.current_slot(), b.current_slot()), k


@pytest.mark.parametrize("double_slot", [False, True])
@pytest.mark.parametrize("cut", [2, 4])
def test_device_resume_in_fresh_object(Z, steps, p0, double_slot, cut):
    say(f"device resume: cut={cut} double_slot={double_slot}")
    ref = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, double_slot=double_slot, **HY)
    run = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, double_slot=double_slot, **HY)
    for k in range(cut):
        ref.step(steps[k])
        run.step(steps[k])
    sd = run.state_dict()
    del run
    torch.cuda.synchronize()
    zeros = torch.zeros(S, dtype=torch.float32, device="cuda")
    res = Z.DeviceShardStep(S, N, Z.ZERO_BF16, zeros, double_slot=double_slot, **HY)
    res.load_state_dict(sd)
    same_device(ref, res, cut)
    for k in range(cut, K):
        ref.step(steps[k])
        res.step(steps[k])
        same_device(ref, res, k)
    st = res.state()
    assert st.t == K - 1 and st.n_skipped == 1 and st.loss_scale == 512.0


def test_device_resume_in_same_object_after_running_ahead(Z, steps, p0):
    """Loading clears the workspace: partials tagged by the steps run after the
    checkpoint cannot be taken for the resumed steps' own."""
    say("device resume in the same object")
    ref = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, **HY)
    run = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, **HY)
    for k in range(2):
        ref.step(steps[k])
        run.step(steps[k])
    sd = run.state_dict()
    for k in range(2, K):
        run.step(steps[k])
    run.load_state_dict(sd)
    assert run.state().seq == 0 and run.state().t == 2
    for k in range(2, K):
        ref.step(steps[k])
        run.step(steps[k])
        same_device(ref, run, k)


def test_host_commit_resume(Z, steps, p0):
    say("host-commit resume")
    ref = Z.ShardStep(S, N, Z.ZERO_BF16, p0, **HY)
    run = Z.ShardStep(S, N, Z.ZERO_BF16, p0, **HY)
    for k in range(3):
        ref.step(steps[k])
        run.step(steps[k])
    sd = run.state_dict()
    res = Z.ShardStep(S, N, Z.ZERO_BF16, torch.zeros_like(p0), **HY)
    res.load_state_dict(sd)
    for k in range(3, K):
        ref.step(steps[k])
        res.step(steps[k])
        assert (ref.t, ref.loss_scale, ref.state.n_skipped) == (res.t, res.loss_scale,
                                                                res.state.n_skipped)
        for x, y in ((ref.master, res.master), (ref.exp_avg, res.exp_avg),
                     (ref.exp_avg_sq, res.exp_avg_sq), (ref.slot, res.slot)):
            assert torch.equal(x, y), k
    assert res.t == K - 1 and res.loss_scale == 512.0
