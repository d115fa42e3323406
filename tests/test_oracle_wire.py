"""Pins of the bf16-wire fold (each running partial rounded to bf16).

The pages leave open the precision in which the ring's partial sums travel.
GuanhuaWang's reply in "Why DeepSpeed ZeRO paper says reduce-scatter (or
all-gather) has data movement of Psi elements?" has each GPU add its own copy to
the partial it received and pass the result on; when the buffers and messages
are bf16, every such partial is a bf16 value. The oracle's wire mode rounds the
fp32 sum to bf16 (nearest, ties to even) after every add. Pinned here against:
hand-computed ties, torch's own bf16 tensor additions (fp32 add, one rounding to
bf16), the ring simulator with bf16 messages, and the cases where no rounding
can occur (the plain fp32 fold).
"""
import numpy as np
import pytest
import torch


def bf16(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_hand_computed_ties(orc):
    one, h = 1.0, 2.0 ** -8           # h is half a bf16 ulp at 1
    # 1 + h is a tie between 1 (even) and 1 + 2h (odd): stays 1, twice over
    g, flag, _ = orc.reduce([bf16([one]), bf16([h]), bf16([h])], loss_scale=1.0 / 3, wire=True)
    assert flag == 0 and g[0] == np.float32(1.0)
    g32, _, _ = orc.reduce([bf16([one]), bf16([h]), bf16([h])], loss_scale=1.0 / 3)
    assert g32[0] == np.float32(1.0 + 2 * h)          # the fp32 fold keeps both halves
    # (1 + 2h) + h is a tie between 1 + 2h (odd) and 1 + 4h (even): goes up
    g, _, _ = orc.reduce([bf16([one + 2 * h]), bf16([h])], loss_scale=0.5, wire=True)
    assert g[0] == np.float32(1.0 + 4 * h)
    # negative values mirror
    g, _, _ = orc.reduce([bf16([-(one + 2 * h)]), bf16([-h])], loss_scale=0.5, wire=True)
    assert g[0] == np.float32(-(1.0 + 4 * h))


@pytest.mark.parametrize("N", [2, 3, 8, 64])
def test_matches_torch_bf16_tensor_adds(orc, N):
    rng = np.random.default_rng(700 + N)
    n = 4096
    mags = 10.0 ** rng.uniform(-4, 4, size=(N, n))
    x = rng.standard_normal((N, n)) * mags
    x[:, :8] = 3.0e38 * np.sign(x[:, :8])                # sums that leave bf16 range
    reps_t = [torch.from_numpy(x[j].astype(np.float32)).to(torch.bfloat16) for j in range(N)]
    reps = [r.view(torch.int16).numpy().view(np.uint16).copy() for r in reps_t]
    acc = reps_t[0].clone()
    for j in range(1, N):
        acc = acc + reps_t[j]                           # torch: fp32 add, RNE to bf16
    ls = 4.0
    want = acc.to(torch.float32) * torch.tensor(orc.inv_scale(N, ls), dtype=torch.float32)
    g, flag, _ = orc.reduce(reps, loss_scale=ls, wire=True)
    w = want.numpy()
    fin = np.isfinite(w)
    assert np.array_equal(np.isfinite(g), fin)
    assert np.array_equal(g[fin].view(np.uint32), w[fin].view(np.uint32))
    assert np.array_equal(np.sign(g[np.isinf(g)]), np.sign(w[np.isinf(w)]))
    assert flag == int(not fin.all())


@pytest.mark.parametrize("N", [2, 3, 8])
def test_ring_with_bf16_messages_equals_wire_fold(orc, N):
    S = 257
    rng = np.random.default_rng(800 + N)
    raw = (rng.standard_normal((N, N * S)) * 10.0 ** rng.uniform(-3, 3, size=(N, N * S)))
    bufs = orc.bf16_to_f32(orc.f32_to_bf16(raw.astype(np.float32))).reshape(N, N * S)
    out, sent, recv, order = orc.ring_reduce_scatter(bufs, wire="bf16")
    out32, _, _, _ = orc.ring_reduce_scatter(bufs)
    assert sent.tolist() == [(N - 1) * S] * N
    differ = 0
    for c in range(N):
        ring_order = order[c].tolist()
        reps = [orc.f32_to_bf16(np.ascontiguousarray(bufs[k, c * S:(c + 1) * S])) for k in ring_order]
        g, _, _ = orc.reduce(reps, loss_scale=1.0 / N, wire=True)
        assert np.array_equal(g.view(np.uint32), out[c].view(np.uint32))
        # every partial is a bf16 value
        assert np.array_equal(orc.bf16_to_f32(orc.f32_to_bf16(out[c])).view(np.uint32),
                              out[c].view(np.uint32))
        differ += int(np.sum(out[c] != out32[c]))
    assert differ > 0                                   # the wire does round on these inputs


def test_no_rounding_when_sums_are_bf16_exact(orc):
    rng = np.random.default_rng(901)
    N, n = 8, 2048
    ints = rng.integers(-15, 16, size=(N, n))          # partial sums stay below 2^8
    reps = [bf16(ints[j].astype(np.float32)) for j in range(N)]
    g, _, _ = orc.reduce(reps, loss_scale=1.0, wire=True)
    g32, _, _ = orc.reduce(reps, loss_scale=1.0)
    assert np.array_equal(g.view(np.uint32), g32.view(np.uint32))
    one = [bf16(rng.standard_normal(n).astype(np.float32))]
    assert np.array_equal(orc.reduce(one, wire=True)[0], orc.reduce(one)[0])   # N = 1


def test_wire_rounding_can_decide_the_skip(orc):
    """bf16 max plus half its ulp: finite in fp32, a tie that rounds to the even
    neighbour -- the infinity pattern -- on a bf16 wire."""
    bmax = np.array([0x7F7F], dtype=np.uint16)
    half_ulp = bf16([2.0 ** 119])
    for wire, want_flag in ((False, 0), (True, 1)):
        p = np.array([0.5], dtype=np.float32)
        m = np.zeros(1, np.float32)
        v = np.zeros(1, np.float32)
        slot = orc.f32_to_bf16(p)
        p0, slot0 = p.copy(), slot.copy()
        flag, _ = orc.step([bmax, half_ulp], p, m, v, slot, loss_scale=2.0 ** 100, lr=1e-3,
                           beta1=0.9, beta2=0.999, eps=1e-8, wd=0.0, t=1, wire=wire)
        assert flag == want_flag
        if flag:
            assert p.tobytes() == p0.tobytes() and slot.tobytes() == slot0.tobytes()
        else:
            assert p[0] != p0[0]
