"""GPU parity at the edges of the even split of small whole-shard launches: a
shard of 256 to 2,047 workgroups' worth of 1,024 elements is split over a grid
rounded up to a multiple of 256 workgroups, each taking whole 64-element blocks,
the last one also the S % 4 tail. Sizes at both ends of that range, one whose
workgroups take 257 quads (more than one per lane), ragged tails, and the first
size past the range; every step bit for bit against the oracle, through the
host commit and the device commit in both state layouts.
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
