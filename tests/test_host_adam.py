"""libzero's host Adam (the update of an offloaded step) against the oracle.

zero_host_adam is product code that runs on the CPU: the update of a shard
whose optimizer state lives in host memory ("ZeRO Optimizer", "Advanced
Optimizations", ZeRO-Offload). It must equal the oracle's Adam/AdamW bit for
bit: same fp32 operation sequence, correctly rounded division and square root.
No GPU is needed, so these run with the host tests.
"""
import numpy as np
import pytest

import oracle
from gpu_util import assert_bitexact

HY = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


@pytest.fixture(scope="module")
def Z():
    import zero_partitioned_optimizer_amd as Z
    Z.lib()
    return Z


def inputs(n, seed, t):
    rng = np.random.default_rng(seed)
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-8, 2, n)).astype(np.float32)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    if t > 1:
        m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v = ((rng.standard_normal(n) * 1e-4) ** 2).astype(np.float32)
    else:
        m = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
    if n > 16:
        g[:4] = [0.0, -0.0, 1e-30, 3e38]            # zero, tiny, huge gradients
        v[4:8] = [0.0, 1e-38, 1e-45, 3e38]            # subnormal and extreme second moments
        p[8:12] = g[8:12] = m[8:12] = v[8:12] = 0.0   # padding: stays +0
    return g, p, m, v


@pytest.mark.parametrize("n,t,wd,nthreads", [(0, 1, 0.0, 1), (1, 1, 0.0, 1), (17, 2, 0.01, 1),
                                             (4099, 3, 0.0, 4), (1_000_003, 1000, 0.01, 0),
                                             (262_147, 100_000, 0.01, 3)])
def test_host_adam_matches_oracle(Z, n, t, wd, nthreads):
    g, p, m, v = inputs(n, seed=n + t, t=t)
    po, mo, vo, so = oracle.adam(g, p, m, v, t=t, wd=wd, **HY)
    P, M, V = p.copy(), m.copy(), v.copy()
    slot = np.zeros(n, np.uint16)
    Z.zero_host_adam(g, P, M, V, n, weight_decay=wd, step_t=t, slot=slot, nthreads=nthreads, **HY)
    for name, got, want in (("p", P, po), ("m", M, mo), ("v", V, vo), ("slot", slot, so)):
        assert_bitexact(f"host adam {name} n={n} t={t}", got, want)
    if n > 16:
        assert np.all(P[8:12].view(np.uint32) == 0) and np.all(slot[8:12] == 0)


def test_host_adam_without_slot_and_repeated_steps(Z):
    n = 50_001
    g, p, m, v = inputs(n, seed=5, t=1)
    P, M, V = p.copy(), m.copy(), v.copy()
    ps, ms, vs = p.copy(), m.copy(), v.copy()
    for t in range(1, 6):
        Z.zero_host_adam(g, P, M, V, n, weight_decay=0.01, step_t=t, **HY)
        ps, ms, vs, _ = oracle.adam(g, ps, ms, vs, t=t, wd=0.01, **HY)
    assert_bitexact("p after 5", P, ps)
    assert_bitexact("m after 5", M, ms)
    assert_bitexact("v after 5", V, vs)


def test_host_adam_validation(Z):
    a = np.zeros(8, np.float32)
    for kw, status in ((dict(step_t=0), -1), (dict(beta1=1.0), -1), (dict(lr=float("nan")), -1),
                       (dict(eps=-1.0), -1)):
        args = dict(HY, weight_decay=0.0, step_t=1)
        args.update(kw)
        with pytest.raises(Z.ZeroError) as e:
            Z.zero_host_adam(a, a.copy(), a.copy(), a.copy(), 8, **args)
        assert e.value.status == status
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_host_adam(a, a.copy(), a.copy(), a.copy(), -1, weight_decay=0.0, step_t=1, **HY)
    assert e.value.status == -3
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_host_adam(None, a.copy(), a.copy(), a.copy(), 8, weight_decay=0.0, step_t=1, **HY)
    assert e.value.status == -1
