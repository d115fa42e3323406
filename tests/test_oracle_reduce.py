"""Pins of the oracle's replica reduction, averaging/unscaling and overflow check.

The reduction is the reduce half of the step ("[REQUEST] Direct Correspondence
between Gradient and Optimizer States to Reduce Communication", "Problem"), in
the ring order of the 8-GPU walk ("Why DeepSpeed ZeRO paper says reduce-scatter
(or all-gather) has data movement of Psi elements?", GuanhuaWang's reply). The
result is averaged over the N replicas (the averaging step named in "Why does not
the stage 3 implementation use broadcast and reduce-scatter?") and unscaled by
the loss scale.

Pins: N = 1 identity, an order-sensitive closed form, the recursive-summation
error bound |fl(sum) - sum| <= gamma_{N-1} * sum|x| (Higham, "Accuracy and
Stability of Numerical Algorithms", 2nd ed., eq. 4.4) against math.fsum, the
IEEE classes for the overflow flag, and math.fsum for the squared norm.
"""
import math

import numpy as np
import pytest

U = 2.0 ** -24


def gamma(k):
    return k * U / (1 - k * U)


def bf16(x):
    import torch
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def test_single_replica_is_identity(orc):
    rng = np.random.default_rng(0)
    x = rng.standard_normal(1000).astype(np.float32)
    g, flag, sumsq = orc.reduce([x], loss_scale=1.0)
    assert flag == 0 and np.array_equal(g.view(np.uint32), x.view(np.uint32))
    g, _, _ = orc.reduce([x], loss_scale=4.0)                 # power of two: exact
    assert np.array_equal(g, x * np.float32(0.25))


def test_left_fold_order_closed_form(orc):
    one, e = np.float32(1.0), np.float32(2.0 ** -24)
    a = [np.array([one]), np.array([e]), np.array([e])]
    # (1 + 2^-24) rounds to 1 (tie to even), + 2^-24 -> 1 again
    g, _, _ = orc.reduce(a, loss_scale=1.0 / 3.0)
    assert g[0] == np.float32(1.0) * orc.inv_scale(3, 1.0 / 3.0)
    # the other order: 2^-24 + 2^-24 = 2^-23, + 1 = 1 + 2^-23 (exact)
    g2, _, _ = orc.reduce(a[::-1], loss_scale=1.0 / 3.0)
    assert g2[0] == np.float32(1.0 + 2.0 ** -23) * orc.inv_scale(3, 1.0 / 3.0)
    assert g[0] != g2[0]


def test_inv_scale_rounding(orc):
    assert orc.inv_scale(8, 65536.0) == np.float32(2.0 ** -19)
    assert orc.inv_scale(64, 65536.0) == np.float32(2.0 ** -22)
    assert orc.inv_scale(3, 1.0) == np.float32(1.0 / 3.0)
    assert orc.inv_scale(1, 1.0) == np.float32(1.0)


@pytest.mark.parametrize("N,dtype", [(2, "f32"), (8, "bf16"), (64, "bf16"), (32, "f32")])
def test_higham_bound_against_fsum(orc, N, dtype):
    rng = np.random.default_rng(N)
    n = 300
    xs = [(rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3, n)).astype(np.float32)
          for _ in range(N)]
    reps = [bf16(x) for x in xs] if dtype == "bf16" else xs
    vals = [orc.bf16_to_f32(r) if dtype == "bf16" else r for r in reps]
    ls = 1.0 / N                                  # makes inv = 1: compare the raw fold
    assert N * ls == 1.0
    g, flag, _ = orc.reduce(reps, loss_scale=ls)
    gd, ad = orc.reduce_f64(reps, loss_scale=ls)
    assert flag == 0
    for i in range(n):
        terms = [float(v[i]) for v in vals]
        exact = math.fsum(terms)
        # the double variant is exact for bf16 terms, within N ulps of double otherwise
        assert abs(gd[i] - exact) <= (0.0 if dtype == "bf16" else N * 2.0 ** -53 * ad[i])
        assert abs(ad[i] - math.fsum(abs(t) for t in terms)) <= N * 2.0 ** -53 * ad[i]
        assert abs(float(g[i]) - exact) <= gamma(N - 1) * ad[i]


def test_overflow_classes(orc):
    base = [np.zeros(4, dtype=np.float32) for _ in range(3)]
    _, flag, _ = orc.reduce(base)
    assert flag == 0
    for val in (np.inf, -np.inf, np.nan):
        reps = [b.copy() for b in base]
        reps[1][2] = val
        _, flag, _ = orc.reduce(reps)
        assert flag == 1
    reps = [b.copy() for b in base]
    reps[0][0], reps[2][0] = np.inf, -np.inf      # inf + (-inf) = NaN
    g, flag, _ = orc.reduce(reps)
    assert flag == 1 and np.isnan(g[0])
    # finite terms whose fp32 sum overflows
    big = [np.full(2, 3.0e38, dtype=np.float32) for _ in range(2)]
    g, flag, _ = orc.reduce(big, loss_scale=0.5)
    assert flag == 1 and np.isinf(g[0])
    # bf16: the largest finite bf16 alone is finite, but two of them overflow the fp32
    # fold before the 1/N scale is applied, although their mean is finite
    mx = np.full(3, 0x7F7F, dtype=np.uint16)
    _, flag, _ = orc.reduce([mx])
    assert flag == 0
    _, flag, _ = orc.reduce([mx] * 2)
    assert flag == 1


def test_sumsq_against_fsum(orc):
    rng = np.random.default_rng(5)
    reps = [bf16(rng.standard_normal(5000) * 1e-3) for _ in range(8)]
    g, _, sumsq = orc.reduce(reps, loss_scale=1.0)
    want = math.fsum(float(x) * float(x) for x in g)
    assert abs(sumsq - want) <= 1e-12 * want
    _, _, sumsq4 = orc.reduce(reps, loss_scale=1.0, nthreads=4)
    assert abs(sumsq4 - want) <= 1e-12 * want


def test_threads_do_not_change_elements(orc):
    rng = np.random.default_rng(9)
    reps = [bf16(rng.standard_normal(10007)) for _ in range(5)]
    g1, f1, _ = orc.reduce(reps, loss_scale=2.0, nthreads=1)
    g4, f4, _ = orc.reduce(reps, loss_scale=2.0, nthreads=4)
    assert f1 == f4 == 0 and np.array_equal(g1.view(np.uint32), g4.view(np.uint32))
