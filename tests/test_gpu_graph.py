"""The device-commit step under HIP graph capture.

zero_train_step takes every per-step decision on the device (current state set,
t, loss scale, skip), so one captured step can be replayed as the next step.
The graph holds no memset node (the library issues none). Each replay is
followed by eager work and a synchronization, and every replay's committed state
is compared with an eager run of the same steps on separate buffers, including
a step whose replicas carry an injected +inf.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("double_slot", [True, False])
def test_captured_step_replays_like_eager(Z, double_slot):
    S, N, K = 1_000_003, 8, 6
    rng = np.random.default_rng(31)
    reps_h = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3 * 256.0))
              for _ in range(N)]
    p0 = to_dev((rng.standard_normal(S) * 0.02).astype(np.float32))
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, loss_scale=256.0,
              dynamic=True, double_slot=double_slot)
    reps_g = [to_dev(r) for r in reps_h]
    reps_e = [to_dev(r) for r in reps_h]
    sg = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, **hy)
    se = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, **hy)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        sg._args_for(reps_g)            # build the argument block outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            sg.step(reps_g)
    torch.cuda.synchronize()
    # capturing does not execute: the record still says t = 0
    assert sg.state().t == 0

    scratch = torch.empty(1 << 20, device="cuda")
    for k in range(K):
        if k == 3:      # overflow on the fourth step, in both runs
            reps_g[2][77] = 0x7F80
            reps_e[2][77] = 0x7F80
        say(f"graph replay {k} (double_slot={double_slot})")
        graph.replay()
        se.step(reps_e)
        scratch.normal_()                # the program's own eager work between replays
        torch.cuda.synchronize()
        if k == 3:
            reps_g[2][77] = int(reps_h[2][77].view(np.int16))
            reps_e[2][77] = int(reps_h[2][77].view(np.int16))
        rg, re = sg.state(), se.state()
        assert (rg.t, rg.n_skipped, rg.cur, rg.loss_scale) == (re.t, re.n_skipped, re.cur, re.loss_scale)
        assert rg.last_overflow == (1 if k == 3 else 0)
        assert sg.last_stats().sumsq == se.last_stats().sumsq or k == 3
        for a, b in zip(sg.committed(), se.committed()):
            assert torch.equal(a, b)
        assert torch.equal(sg.current_slot(), se.current_slot())
    assert sg.state().t == K - 1 and sg.state().loss_scale == 128.0


@pytest.mark.parametrize("tiled", [False, True])
def test_graph_of_two_steps_replayed_back_to_back(Z, tiled):
    """A graph of two steps replayed three times with no host read in between:
    each launch folds the previous step into the record on the device, a replay's
    first launch folding in the previous replay's last step. Both steps of the
    second replay see an injected +inf. After one flush the record, the committed
    state and the slot equal six eager steps with the same inputs."""
    S, N = 300_007, 4
    rng = np.random.default_rng(41)
    reps_h = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3 * 64.0))
              for _ in range(N)]
    p0 = to_dev((rng.standard_normal(S) * 0.02).astype(np.float32))
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, loss_scale=64.0,
              dynamic=True, state_layout=Z.ZERO_STATE_TILED if tiled else Z.ZERO_STATE_SPLIT)
    reps_g = [to_dev(r) for r in reps_h]
    reps_e = [to_dev(r) for r in reps_h]
    sg = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, **hy)
    se = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, **hy)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        sg._args_for(reps_g)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            sg.step(reps_g)
            sg.step(reps_g)
    torch.cuda.synchronize()
    bad = int(reps_h[1][5].view(np.int16))
    for r in range(3):
        say(f"two-step graph replay {r} (tiled={tiled})")
        if r == 1:
            reps_g[1][5] = 0x7F80
            reps_e[1][5] = 0x7F80
        graph.replay()
        se.step(reps_e)
        se.step(reps_e)
        if r == 1:
            reps_g[1][5] = bad
            reps_e[1][5] = bad
    torch.cuda.synchronize()
    rg, re = sg.state(), se.state()
    assert (rg.t, rg.n_skipped, rg.seq, rg.loss_scale) == (re.t, re.n_skipped, re.seq, re.loss_scale)
    assert (rg.t, rg.n_skipped, rg.seq, rg.loss_scale) == (4, 2, 6, 16.0)
    for a, b in zip(sg.committed(), se.committed()):
        assert torch.equal(a, b)
    assert torch.equal(sg.current_slot(), se.current_slot())


@pytest.mark.parametrize("bucket_len", [1000, 70_000])
def test_graph_over_a_bucket_table(Z, bucket_len):
    """Steps over a bucket table under graph capture: short buckets (one workgroup
    each, the first replica batch loaded before the record) and long ones (cut
    into chunks). A graph of two steps replayed three times, an injected +inf
    inside a bucket on the second replay, against eager steps over the same
    table; the committed state must be equal everywhere (outside the buckets both
    keep the initial values)."""
    S, N = 300_007, 4
    rng = np.random.default_rng(43)
    reps_h = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3 * 64.0))
              for _ in range(N)]
    p0 = to_dev((rng.standard_normal(S) * 0.02).astype(np.float32))
    offs = np.arange(3, S - bucket_len, bucket_len + 5, dtype=np.int64)
    raw = np.zeros(len(offs), dtype=np.dtype([("off", "<i8"), ("len", "<i4"), ("t", "<i4")]))
    raw["off"] = offs
    raw["len"] = bucket_len
    buckets = torch.from_numpy(raw.view(np.uint8).copy()).to("cuda")
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, loss_scale=64.0,
              dynamic=True, state_layout=Z.ZERO_STATE_TILED, double_slot=True, buckets=buckets,
              n_buckets=len(offs))
    reps_g = [to_dev(r) for r in reps_h]
    reps_e = [to_dev(r) for r in reps_h]
    sg = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, **hy)
    se = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, **hy)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        sg._args_for(reps_g)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            sg.step(reps_g)
            sg.step(reps_g)
    torch.cuda.synchronize()
    inside = int(offs[len(offs) // 2]) + 7
    good = int(reps_h[2][inside].view(np.int16))
    for r in range(3):
        say(f"graph over buckets of {bucket_len}: replay {r}")
        if r == 1:
            reps_g[2][inside] = 0x7F80
            reps_e[2][inside] = 0x7F80
        graph.replay()
        se.step(reps_e)
        se.step(reps_e)
        torch.cuda.synchronize()
        if r == 1:
            reps_g[2][inside] = good
            reps_e[2][inside] = good
    rg, re = sg.state(), se.state()
    assert (rg.t, rg.n_skipped, rg.seq, rg.loss_scale) == (re.t, re.n_skipped, re.seq, re.loss_scale)
    assert (rg.t, rg.n_skipped) == (4, 2)
    for a, b in zip(sg.committed(), se.committed()):
        assert torch.equal(a, b)
    assert torch.equal(sg.current_slot(), se.current_slot())
