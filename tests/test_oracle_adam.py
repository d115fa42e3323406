"""Pins of the oracle's Adam / AdamW update on the shard.

The pages name Adam's two moments m and v as the optimizer state each rank keeps
for its own partition ("[REQUEST] Direct Correspondence between Gradient and
Optimizer States to Reduce Communication", "Thoughts and viewpoints"; "ZeRO
Optimizer", "Memory Components") but print no formula. The oracle follows Adam
(Kingma & Ba 2015, Algorithm 1) with decoupled weight decay (Loshchilov & Hutter
2019). Pins, none of which retypes the oracle's arithmetic:

* the library routine: torch.optim.Adam / AdamW on the CPU in float64, with a
  first-order error bound for the oracle's fp32 operation sequence;
* closed forms: at t = 1 from zero moments the bias corrections cancel exactly,
  so the step is lr * g / (|g| + eps); a constant gradient keeps m_hat = g and
  v_hat = g^2 at every t; a zero gradient with zero moments leaves p unchanged
  (or only decays it);
* padding (all zeros) stays +0 bit for bit.
"""
import math

import numpy as np
import pytest
import torch

U = 2.0 ** -24
HY = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def torch_step(g, p, m, v, t, lr, beta1, beta2, eps, wd):
    """One torch.optim step in float64 from state (m, v) after t-1 updates."""
    P = torch.nn.Parameter(torch.tensor(np.asarray(p, dtype=np.float64)))
    if wd:
        opt = torch.optim.AdamW([P], lr=lr, betas=(beta1, beta2), eps=eps, weight_decay=wd,
                                foreach=False)
    else:
        opt = torch.optim.Adam([P], lr=lr, betas=(beta1, beta2), eps=eps, weight_decay=0.0,
                               foreach=False)
    opt.state[P] = {"step": torch.tensor(float(t - 1), dtype=torch.float64),
                    "exp_avg": torch.tensor(np.asarray(m, dtype=np.float64)),
                    "exp_avg_sq": torch.tensor(np.asarray(v, dtype=np.float64))}
    P.grad = torch.tensor(np.asarray(g, dtype=np.float64))
    opt.step()
    st = opt.state[P]
    return P.detach().numpy().copy(), st["exp_avg"].numpy().copy(), st["exp_avg_sq"].numpy().copy()


def error_bounds(g, p, m, v, t, lr, beta1, beta2, eps, wd, pr, mr, vr):
    """First-order bounds on |fp32 sequence - exact| for m', v', p' (safety factor 2)."""
    g, p, m, v = (np.asarray(a, dtype=np.float64) for a in (g, p, m, v))
    bc1, bc2 = 1 - beta1 ** t, 1 - beta2 ** t
    em = 4 * U * (abs(beta1 * m) + abs((1 - beta1) * g)) + 1e-45
    ev = 8 * U * np.abs(vr) + 1e-45
    mh = mr / bc1
    vh = vr / bc2
    den = np.sqrt(vh) + eps
    u = mh / den
    emh = em / bc1 + 3 * U * np.abs(mh)
    rel_den = 7 * U
    eu = emh / den + np.abs(u) * (rel_den + U)
    decay = 1 - lr * wd
    ep = 2 * U * np.abs(p * decay) + lr * eu + 2 * U * lr * np.abs(u) + U * np.abs(pr) + 1e-45
    return 2 * em, 2 * ev, 2 * ep


def check_against_torch(orc, g, p, m, v, t, wd):
    po, mo, vo, slot = orc.adam(g, p, m, v, t=t, wd=wd, **HY)
    pr, mr, vr = torch_step(g, p, m, v, t, wd=wd, **HY)
    em, ev, ep = error_bounds(g, p, m, v, t, wd=wd, pr=pr, mr=mr, vr=vr, **HY)
    assert np.all(np.abs(mo - mr) <= em), np.max(np.abs(mo - mr) / em)
    assert np.all(np.abs(vo - vr) <= ev), np.max(np.abs(vo - vr) / ev)
    assert np.all(np.abs(po - pr) <= ep), np.max(np.abs(po - pr) / ep)
    return po, mo, vo, slot


def rand_state(seed, n, t):
    rng = np.random.default_rng(seed)
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, -2, n)).astype(np.float32)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    if t == 1:
        m = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
    else:
        m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v = (rng.standard_normal(n) * 1e-4).astype(np.float32) ** 2
    return g, p, m, v


@pytest.mark.parametrize("t", [1, 2, 3, 10, 1000, 100000])
@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_matches_torch_float64(orc, t, wd):
    g, p, m, v = rand_state(t, 4000, t)
    check_against_torch(orc, g, p, m, v, t, wd)


def test_first_step_closed_form(orc):
    # m = v = 0, t = 1, wd = 0: m_hat = g and v_hat = g^2 exactly in real arithmetic,
    # so p' = p - lr * g / (|g| + eps)
    g, p, _, _ = rand_state(11, 5000, 1)
    z = np.zeros_like(g)
    po, mo, vo, _ = orc.adam(g, p, z, z, t=1, wd=0.0, **HY)
    gd = g.astype(np.float64)
    want = p.astype(np.float64) - HY["lr"] * gd / (np.abs(gd) + HY["eps"])
    assert np.all(np.abs(po - want) <= 8 * U * (np.abs(p) + HY["lr"]))
    assert np.allclose(mo, 0.1 * gd, rtol=4 * U, atol=0)
    assert np.allclose(vo, 0.001 * gd * gd, rtol=8 * U, atol=0)


def test_constant_gradient_moves_lr_per_step(orc):
    # constant g: m_t = (1 - b1^t) g and v_t = (1 - b2^t) g^2, so every step moves
    # p by lr * g / (|g| + eps) -- about lr * sign(g) when |g| >> eps
    n = 64
    g = np.linspace(-1e-2, 1e-2, n).astype(np.float32)
    g[n // 2] = np.float32(3e-3)
    p0 = np.full(n, 0.5, np.float32)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    T = 50
    for t in range(1, T + 1):
        p, m, v, _ = orc.adam(g, p, m, v, t=t, wd=0.0, **HY)
    gd = g.astype(np.float64)
    want = p0 - T * HY["lr"] * gd / (np.abs(gd) + HY["eps"])
    assert np.all(np.abs(p - want) <= 1e-5 * T * HY["lr"] + 4e-6)
    assert np.all(np.sign(p0 - p) == np.sign(g))


def test_zero_gradient(orc):
    rng = np.random.default_rng(3)
    p = (rng.standard_normal(100) * 0.02).astype(np.float32)
    z = np.zeros_like(p)
    po, mo, vo, _ = orc.adam(z, p, z, z, t=1, wd=0.0, **HY)
    assert np.array_equal(po.view(np.uint32), p.view(np.uint32))
    assert not mo.view(np.uint32).any() and not vo.view(np.uint32).any()
    po, _, _, _ = orc.adam(z, p, z, z, t=7, wd=0.1, **HY)
    decay = np.float32(1.0 - HY["lr"] * 0.1)
    assert np.all(np.abs(po - p.astype(np.float64) * (1 - HY["lr"] * 0.1)) <= 2 * U * np.abs(p))
    assert np.array_equal(po, p * decay)


def test_padding_stays_positive_zero(orc):
    z = np.zeros(16, np.float32)
    for t, wd in ((1, 0.0), (5, 0.01)):
        po, mo, vo, slot = orc.adam(z, z, z, z, t=t, wd=wd, **HY)
        for a in (po, mo, vo):
            assert not a.view(np.uint32).any()
        assert not slot.any()


def test_scalars_use_t_fold_product(orc):
    for t in (1, 2, 17, 5000):
        s = orc.adam_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, t)
        assert s[4] == np.float32(1.0 - 0.9 ** t)
        assert abs(float(s[5]) - (1.0 - 0.999 ** t)) <= U * (1.0 - 0.999 ** t)
        assert s[8] == np.float32(1.0 - 1e-3 * 0.01)
        assert (s[0], s[2]) == (np.float32(0.9), np.float32(1.0 - 0.9))


def test_slot_is_rounded_master(orc):
    g, p, m, v = rand_state(21, 3000, 4)
    po, _, _, slot = orc.adam(g, p, m, v, t=4, wd=0.01, **HY)
    want = torch.from_numpy(po).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(slot, want)
