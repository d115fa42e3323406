"""GPU parity of the tiled state layout (ZERO_STATE_TILED): each state set is one
buffer of tiles of ZERO_STATE_TILE elements, tile k holding that range of p, then
of m, then of v.

* pack / unpack: every element lands at the position include/zero.h documents
  (checked by index arithmetic on the host), nothing else in the set buffer and
  nothing outside it is written (sentinel bytes), and the round trip is bit-exact,
  ragged tails included.
* zero_adam_step (host commit) with tiled state, fused from replicas and unfused
  in place from the fp32 gradient, against the oracle, bit for bit.
* a step split into tile-aligned parts, with a skipped step and a single slot
  (restore kernel), equals the whole step; a checkpoint taken from a tiled step
  resumes bit for bit.
The device-commit step in this layout is also covered on the Tiny, GPT-2-small
and ragged workloads (tests/test_gpu_device_commit.py) and in the random cases
(tests/test_gpu_random.py).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import Guarded, NTHREADS, check_state, say, to_dev, to_host

pytestmark = pytest.mark.gpu

SENT = np.uint32(0xA5A5A5A5)        # Guarded's fill byte, as a float's bits


def tiled_pos(e, k, T):
    return (e // T) * 3 * T + e % T + k * T


@pytest.mark.parametrize("S", [1, 3, 4, 5, 8191, 8192, 8193, 3 * 8192 + 1000, 100_003])
def test_pack_unpack_positions(Z, S):
    T = Z.ZERO_STATE_TILE
    n = Z.zero_state_set_floats(S, Z.ZERO_STATE_TILED)
    say(f"pack/unpack S={S} set floats={n}")
    rng = np.random.default_rng(S)
    src = [rng.standard_normal(S).astype(np.float32) for _ in range(3)]
    dsrc = [to_dev(x) for x in src]
    buf = Guarded(4 * n, torch.float32)
    Z.zero_state_pack(*dsrc, S, buf.t)
    torch.cuda.synchronize()
    got = to_host(buf.t).view(np.uint32)
    assert buf.intact()
    e = np.arange(S, dtype=np.int64)
    want = np.full(n, SENT, dtype=np.uint32)
    for k in range(3):
        want[tiled_pos(e, k, T)] = src[k].view(np.uint32)
    assert np.array_equal(got, want)
    outs = [Guarded(4 * S, torch.float32) for _ in range(3)]
    Z.zero_state_unpack(buf.t, S, outs[0].t, outs[1].t, outs[2].t)
    torch.cuda.synchronize()
    for o, x in zip(outs, src):
        assert o.intact()
        assert np.array_equal(to_host(o.t).view(np.uint32), x.view(np.uint32))
    # a NULL destination is skipped
    only_v = Guarded(4 * S, torch.float32)
    Z.zero_state_unpack(buf.t, S, None, None, only_v.t)
    torch.cuda.synchronize()
    assert only_v.intact() and np.array_equal(to_host(only_v.t), src[2])
    # the slot cast from a tiled set equals the cast of the master
    slot = Guarded(2 * S, torch.int16)
    Z.zero_gather_slot_tiled(buf.t, S, slot.t)
    torch.cuda.synchronize()
    assert slot.intact() and np.array_equal(to_host(slot.t), oracle.f32_to_bf16(src[0]))


def pack(Z, p, m, v):
    S = p.size
    buf = torch.empty(Z.zero_state_set_floats(S, Z.ZERO_STATE_TILED), dtype=torch.float32,
                      device="cuda")
    Z.zero_state_pack(to_dev(p), to_dev(m), to_dev(v), S, buf)
    return buf


def unpack(Z, buf, S):
    out = [torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(3)]
    Z.zero_state_unpack(buf, S, *out)
    torch.cuda.synchronize()
    return [to_host(x) for x in out]


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("S,N,t", [(1000, 3, 1), (3 * 8192 + 5, 8, 4), (200_003, 5, 2)])
def test_adam_step_tiled(Z, fused, S, N, t):
    """Host-commit step on a tiled state with nonzero moments and t > 1."""
    say(f"adam_step tiled fused={fused} S={S} N={N} t={t}")
    rng = np.random.default_rng(S + N)
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)
    ls = 1024.0
    reps = [W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3 * ls) for _ in range(N)]
    p = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m = (rng.standard_normal(S) * 1e-4).astype(np.float32)
    v = (np.abs(rng.standard_normal(S)) * 1e-7).astype(np.float32)
    sin = pack(Z, p, m, v)
    dreps = [to_dev(r) for r in reps]
    stats = torch.zeros(16, dtype=torch.uint8, device="cuda")
    ws = torch.empty(Z.zero_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    slot = Guarded(2 * S, torch.int16)
    kw = dict(lr=hy["lr"], beta1=hy["beta1"], beta2=hy["beta2"], eps=hy["eps"],
              weight_decay=hy["wd"], step_t=t, stats=stats, workspace=ws,
              state_layout=Z.ZERO_STATE_TILED, m_in=None, v_in=None, m_out=None, v_out=None)
    if fused:
        sout = torch.empty_like(sin)
        a = Z.make_adam_args(replicas=dreps, grad_dtype=Z.ZERO_BF16, p_in=sin, p_out=sout,
                             slot=slot.t, shard_S=S, loss_scale=ls, **kw)
    else:
        g = torch.empty(S, dtype=torch.float32, device="cuda")
        Z.zero_reduce_shard(dreps, Z.ZERO_BF16, S, stats, ws, loss_scale=ls, grad_out=g)
        sout = sin                                      # in place
        a = Z.make_adam_args(grad_f32=g, p_in=sin, p_out=sout, slot=slot.t, shard_S=S, **kw)
    Z.zero_adam_step(a)
    torch.cuda.synchronize()
    st = Z.stats_from_tensor(stats)
    want_slot = oracle.f32_to_bf16(p)
    flag, _ = oracle.step(reps, p, m, v, want_slot, loss_scale=ls, t=t, nthreads=NTHREADS, **hy)
    assert flag == 0 and st.overflow == 0
    P, M, V = unpack(Z, sout, S)
    assert slot.intact()
    check_state(f"tiled adam fused={fused} S={S}", P, M, V, to_host(slot.t), p, m, v, want_slot)


def test_parts_and_restore_tiled(Z):
    """Tile-aligned parts, a single slot and an overflow on the second step: the
    split step equals the whole step, and the skipped step restores the slot from
    the tiled master."""
    T = Z.ZERO_STATE_TILE
    S, N = 5 * T + 100, 4
    rng = np.random.default_rng(3)
    p0 = to_dev((rng.standard_normal(S) * 0.02).astype(np.float32))
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, loss_scale=256.0,
              dynamic=True)
    whole = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, state_layout=Z.ZERO_STATE_TILED, **hy)
    parts = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, state_layout=Z.ZERO_STATE_TILED, **hy)
    ends = [T, 3 * T, 3 * T, S]
    for s in range(4):
        reps = [W._bf16_bits_from_f32(rng.standard_normal(S) * 256e-3) for _ in range(N)]
        if s == 1:
            reps[2][4 * T + 7] = W._bf16_bits_from_f32(np.array([np.inf]))[0]
        say(f"tiled parts step {s}")
        dreps = [to_dev(r) for r in reps]
        whole.step(dreps)
        parts.step_parts(dreps, ends)
        a, b = whole.state(), parts.state()
        assert a.last_overflow == b.last_overflow == (1 if s == 1 else 0)
        assert a.t == b.t and a.loss_scale == b.loss_scale
        for x, y in zip(whole.committed(), parts.committed()):
            assert torch.equal(x, y)
        assert torch.equal(whole.current_slot(), parts.current_slot())
        P = whole.committed()[0]
        want = oracle.f32_to_bf16(to_host(P))
        assert np.array_equal(to_host(whole.current_slot()), want)


@pytest.mark.parametrize("into_tiled", [True, False])
def test_checkpoint_tiled(Z, into_tiled):
    """state_dict of a tiled step resumes, in either layout, bit for bit."""
    S, N = 70_001, 8
    rng = np.random.default_rng(11)
    p0 = to_dev((rng.standard_normal(S) * 0.02).astype(np.float32))
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, double_slot=True)
    steps = [[to_dev(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3)) for _ in range(N)]
             for _ in range(4)]
    ref = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, state_layout=Z.ZERO_STATE_TILED, **hy)
    run = Z.DeviceShardStep(S, N, Z.ZERO_BF16, p0, state_layout=Z.ZERO_STATE_TILED, **hy)
    for s in range(4):
        ref.step(steps[s])
    for s in range(2):
        run.step(steps[s])
    sd = run.state_dict()
    res = Z.DeviceShardStep(S, N, Z.ZERO_BF16, torch.zeros_like(p0),
                            state_layout=Z.ZERO_STATE_TILED if into_tiled else Z.ZERO_STATE_SPLIT,
                            **hy)
    res.load_state_dict(sd)
    for s in range(2, 4):
        res.step(steps[s])
    assert res.state().t == ref.state().t == 4
    for x, y in zip(ref.committed(), res.committed()):
        assert torch.equal(x, y)
    assert torch.equal(ref.current_slot(), res.current_slot())
