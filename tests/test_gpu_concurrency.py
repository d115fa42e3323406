"""Two shards stepped at the same time on two streams.

Each rank's step owns its record and workspace, so independent steps may run
concurrently on one GPU (two ranks' shards sharing a device, or a step beside
other work). Every step of both runs, interleaved on two streams with no
synchronization between them, must commit exactly what the same steps commit
one after the other.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def batches(seed, S, N, K):
    rng = np.random.default_rng(seed)
    return [[to_dev(np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3 * 64.0)))
             for _ in range(N)] for _ in range(K)]


@pytest.mark.parametrize("double_slot", [True, False])
def test_two_streams_equal_sequential(Z, double_slot):
    S1, S2, N, K = 2_000_003, 700_001, 8, 5
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, loss_scale=64.0,
              dynamic=True, double_slot=double_slot)
    rng = np.random.default_rng(77)
    p1 = to_dev((rng.standard_normal(S1) * 0.02).astype(np.float32))
    p2 = to_dev((rng.standard_normal(S2) * 0.02).astype(np.float32))
    b1, b2 = batches(1, S1, N, K), batches(2, S2, N, K)
    b2[2][4][1234] = 0x7F80                              # one overflow in the second run
    say(f"concurrent steps, double_slot={double_slot}")
    c1 = Z.DeviceShardStep(S1, N, Z.ZERO_BF16, p1, **hy)
    c2 = Z.DeviceShardStep(S2, N, Z.ZERO_BF16, p2, **hy)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for k in range(K):
        c1.step(b1[k], stream=s1)
        c2.step(b2[k], stream=s2)
    torch.cuda.synchronize()
    q1 = Z.DeviceShardStep(S1, N, Z.ZERO_BF16, p1, **hy)
    q2 = Z.DeviceShardStep(S2, N, Z.ZERO_BF16, p2, **hy)
    for k in range(K):
        q1.step(b1[k])
    for k in range(K):
        q2.step(b2[k])
    torch.cuda.synchronize()
    for c, q in ((c1, q1), (c2, q2)):
        rc, rq = c.state(), q.state()
        assert (rc.t, rc.n_skipped, rc.loss_scale, rc.cur) == (rq.t, rq.n_skipped, rq.loss_scale, rq.cur)
        assert rc.last_sumsq == rq.last_sumsq
        for x, y in zip(c.committed(), q.committed()):
            assert torch.equal(x, y)
        assert torch.equal(c.current_slot(), q.current_slot())
    assert c1.state().t == K and c2.state().t == K - 1 and c2.state().loss_scale == 32.0
