"""Pins of the oracle's whole step and its multi-step rule.

The step: reduce-scatter of the gradients, update of the own partition, then the
updated parameters go out through the all-gather ("[REQUEST] Direct
Correspondence between Gradient and Optimizer States to Reduce Communication",
"Problem"). Mixed precision ("ZeRO Optimizer", "Hybrid Approaches") brings a loss
scale; the pages give no overflow rule, so the plainest one is taken: a step
whose averaged gradient holds inf or NaN changes nothing and halves a dynamic
loss scale (never below 1); the update counter t advances only on clean steps.
"""
import numpy as np
import pytest

import workloads as W

from test_oracle_adam import HY, check_against_torch


def tiny_inputs(orc, w, rank=0):
    lay = orc.Layout(w.numels, N=w.N, A=w.A, B=w.B)
    covered = [(int(s[2]), int(s[3])) for s in lay.segments(rank)]
    return lay, covered


def test_overflow_skips_everything(orc):
    w = W.get("ragged")
    S, N = 512, 8
    rng = np.random.default_rng(1)
    reps = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 6.5)) for _ in range(N)]
    reps[3][100] = 0x7F80                                    # +inf
    p = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m = (rng.standard_normal(S) * 1e-4).astype(np.float32)
    v = ((rng.standard_normal(S) * 1e-4) ** 2).astype(np.float32)
    slot = np.full(S, 0x1234, np.uint16)
    before = [a.copy() for a in (p, m, v, slot)]
    flag, sumsq = orc.step(reps, p, m, v, slot, loss_scale=65536.0, t=3, wd=0.0, **HY)
    assert flag == 1 and not np.isfinite(sumsq)
    for a, b in zip((p, m, v, slot), before):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_trainer_dynamic_scale_and_counter(orc):
    w = W.get("ragged")
    S, N = 256, 4
    rng = np.random.default_rng(2)
    p = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m, v = np.zeros(S, np.float32), np.zeros(S, np.float32)
    slot = orc.f32_to_bf16(p)
    tr = orc.Trainer(p, m, v, slot, loss_scale=65536.0, dynamic=True, wd=0.0, **HY)
    for step in range(5):
        reps = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 6.5)) for _ in range(N)]
        if step in (1, 2):
            reps[0][7] = 0x7F80 if step == 1 else 0x7FC0       # +inf, then NaN
        p_before = tr.p.copy()
        flag, _ = tr.step(reps)
        assert flag == (1 if step in (1, 2) else 0)
        if flag:
            assert np.array_equal(tr.p, p_before)
    assert [h[2] for h in tr.history] == [65536.0, 65536.0, 32768.0, 16384.0, 16384.0]
    assert [h[3] for h in tr.history] == [0, 1, 1, 1, 2]
    assert tr.t == 3 and tr.loss_scale == 16384.0


def test_scale_never_below_one(orc):
    S = 8
    p = np.zeros(S, np.float32)
    tr = orc.Trainer(p, p.copy(), p.copy(), np.zeros(S, np.uint16), loss_scale=2.0,
                     dynamic=True, wd=0.0, **HY)
    bad = [np.full(S, 0x7F80, np.uint16)]
    for _ in range(4):
        tr.step(bad)
    assert tr.loss_scale == 1.0 and tr.t == 0


def test_tiny_three_steps_against_torch(orc):
    """Tiny workload, both ranks: every step equals torch.optim.Adam (float64) applied
    to the oracle's own pre-step state and reduced gradient, within the fp32 bound."""
    w = W.get("tiny")
    lay = orc.Layout(w.numels, N=w.N, A=w.A, B=w.B)
    for rank in range(w.N):
        covered = [(int(s[2]), int(s[3])) for s in lay.segments(rank)]
        p = W.host_params(w, lay.S, covered, rank)
        m, v = np.zeros(lay.S, np.float32), np.zeros(lay.S, np.float32)
        slot = orc.f32_to_bf16(p)
        tr = orc.Trainer(p, m, v, slot, loss_scale=w.loss_scale, dynamic=False, **w.hyper())
        for step in range(w.steps):
            reps = W.host_replicas(w, lay.S, covered, rank, step)
            g, flag, _ = orc.reduce(reps, loss_scale=w.loss_scale)
            assert flag == 0
            pre = (tr.p.copy(), tr.m.copy(), tr.v.copy())
            tr.step(reps)
            po, mo, vo, so = check_against_torch(orc, g, *pre, t=step + 1, wd=w.wd)
            assert np.array_equal(po, tr.p) and np.array_equal(mo, tr.m)
            assert np.array_equal(vo, tr.v) and np.array_equal(so, tr.slot)
        assert tr.t == w.steps


def test_loss_scale_invariance(orc):
    """bf16(K x) = K bf16(x) for a power-of-two K, so unscaling recovers the same g."""
    rng = np.random.default_rng(4)
    xs = [(rng.standard_normal(1000) * 1e-4).astype(np.float32) for _ in range(8)]
    r1 = [np.asarray(W._bf16_bits_from_f32(x)) for x in xs]
    rk = [np.asarray(W._bf16_bits_from_f32(x * np.float32(65536.0))) for x in xs]
    g1, _, s1 = orc.reduce(r1, loss_scale=1.0)
    gk, _, sk = orc.reduce(rk, loss_scale=65536.0)
    assert np.array_equal(g1, gk) and s1 == sk


@pytest.mark.parametrize("nthreads", [1, 3])
def test_step_threads_bit_identical(orc, nthreads):
    rng = np.random.default_rng(6)
    S = 3001
    reps = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3)) for _ in range(8)]
    def run(nt):
        p = (np.arange(S, dtype=np.float32) * 1e-5)
        m, v, slot = np.zeros(S, np.float32), np.zeros(S, np.float32), np.zeros(S, np.uint16)
        flag, sumsq = orc.step(reps, p, m, v, slot, loss_scale=1.0, t=1, wd=0.01,
                               nthreads=nt, **HY)
        return p, m, v, slot, sumsq
    a, b = run(1), run(nthreads)
    for x, y in zip(a[:4], b[:4]):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
    assert abs(a[4] - b[4]) <= 1e-12 * a[4]
