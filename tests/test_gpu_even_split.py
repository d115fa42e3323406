"""GPU parity at the edges of the even split of small whole-shard launches: a
shard of 256 to 2,047 workgroups' worth of 1,024 elements is split over a grid
rounded up to a multiple of 256 workgroups, each taking whole 64-element blocks,
the last one also the S % 4 tail. Sizes at both ends of that range, one whose
workgroups take 257 quads (more than one per lane), ragged tails, and the first
size past the range; every step bit for bit against the oracle, through the
host commit and the device commit in both state layouts. Also launches in the
range with 16 to 64 replicas (bf16, fp32 and the bf16 wire), one step skipped.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import NTHREADS, assert_bitexact, say, sumsq_close, to_dev, to_host

pytestmark = pytest.mark.gpu

SIZES = [262_143, 262_144, 263_167, 263_171, 1_000_003, 2_097_151, 2_097_152]


@pytest.mark.parametrize("S", SIZES)
@pytest.mark.parametrize("path", ["host", "split", "tiled"])
def test_even_split_edges(Z, S, path):
    N, steps = 3, 2
    rng = np.random.default_rng(S % 9973)
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)
    zhy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    p0 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    say(f"even split S={S} path={path}")
    if path == "host":
        st = Z.ShardStep(S, N, Z.ZERO_BF16, to_dev(p0), loss_scale=16.0, **zhy)
    else:
        st = Z.DeviceShardStep(S, N, Z.ZERO_BF16, to_dev(p0), loss_scale=16.0, double_slot=True,
                               state_layout=Z.ZERO_STATE_TILED if path == "tiled"
                               else Z.ZERO_STATE_SPLIT, **zhy)
    tr = oracle.Trainer(p0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32),
                        oracle.f32_to_bf16(p0), loss_scale=16.0, nthreads=NTHREADS, **hy)
    for s in range(steps):
        reps = [W._bf16_bits_from_f32(rng.standard_normal(S) * 16e-3) for _ in range(N)]
        flag, sumsq = tr.step(reps)
        assert flag == 0
        dreps = [to_dev(r) for r in reps]
        if path == "host":
            stats, _ = st.step(dreps)
            torch.cuda.synchronize()
            got = (st.master, st.exp_avg, st.exp_avg_sq, st.slot)
            got_sumsq = stats.sumsq
        else:
            st.step(dreps)
            rec = st.state()
            assert rec.t == s + 1 and rec.last_overflow == 0
            got = (*st.committed(), st.current_slot())
            got_sumsq = rec.last_sumsq
        assert sumsq_close(got_sumsq, sumsq), (got_sumsq, sumsq)
        for name, g, want in zip(("p", "m", "v", "slot"), got, (tr.p, tr.m, tr.v, tr.slot)):
            assert_bitexact(f"S={S} {path} step {s} {name}", to_host(g), want)


@pytest.mark.parametrize("N", [16, 24, 25, 39, 64])
@pytest.mark.parametrize("kind", ["bf16", "f32", "wire"])
@pytest.mark.parametrize("path", ["host", "tiled"])
def test_even_split_wide_batches(Z, N, kind, path):
    """Evenly split launches with many replicas, in every replica type: N = 16,
    24, 25, 39 and 64 take the fold's first batch of 8, further batches of 8 and
    tails of 1 and 7 slots. Three steps of a ragged shard; the second carries a
    NaN in the last replica, which must skip the step."""
    S, steps = 263_171, 3
    rng = np.random.default_rng(7 * N + len(kind))
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)
    zhy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    gdt = {"bf16": Z.ZERO_BF16, "f32": Z.ZERO_F32, "wire": Z.ZERO_BF16_WIRE}[kind]
    p0 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    say(f"even split, wide batches: S={S} N={N} {kind} {path}")
    if path == "host":
        st = Z.ShardStep(S, N, gdt, to_dev(p0), loss_scale=8.0, **zhy)
    else:
        st = Z.DeviceShardStep(S, N, gdt, to_dev(p0), loss_scale=8.0, double_slot=True,
                               state_layout=Z.ZERO_STATE_TILED, **zhy)
    tr = oracle.Trainer(p0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32),
                        oracle.f32_to_bf16(p0), loss_scale=8.0, nthreads=NTHREADS,
                        wire=(kind == "wire"), **hy)
    for s in range(steps):
        sample = [rng.standard_normal(S) * 8e-3 for _ in range(N)]
        if kind == "f32":
            reps = [x.astype(np.float32) for x in sample]
        else:
            reps = [W._bf16_bits_from_f32(x) for x in sample]
        if s == 1:
            reps[N - 1][4 * 1000 + 2] = (np.float32(np.nan) if kind == "f32"
                                         else W._bf16_bits_from_f32(np.array([np.nan]))[0])
        flag, sumsq = tr.step(reps)
        assert flag == (1 if s == 1 else 0)
        dreps = [to_dev(r) for r in reps]
        if path == "host":
            stats, _ = st.step(dreps)
            torch.cuda.synchronize()
            assert stats.overflow == flag
            got = (st.master, st.exp_avg, st.exp_avg_sq, st.slot)
            got_sumsq = stats.sumsq
        else:
            st.step(dreps)
            rec = st.state()
            assert rec.last_overflow == flag and rec.t == tr.t
            got = (*st.committed(), st.current_slot())
            got_sumsq = rec.last_sumsq
        if not flag:
            assert sumsq_close(got_sumsq, sumsq), (got_sumsq, sumsq)
        for name, g, want in zip(("p", "m", "v", "slot"), got, (tr.p, tr.m, tr.v, tr.slot)):
            assert_bitexact(f"S={S} N={N} {kind} {path} step {s} {name}", to_host(g), want)
