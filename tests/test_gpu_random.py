"""Randomized GPU parity: seeded random cases against the oracle, bit for bit.

Each seed draws a replica count (1 to 256), a shard size (1 to 2M elements,
ragged), the gradient type (bf16, fp32, bf16 wire), the path (host commit,
device commit with one or two slots, a step split into random parts), Adam
hyperparameters, a power-of-two loss scale with or without dynamic halving,
value magnitudes over six decades (seeds 40 and up keep the device paths' state
in the tiled layout, with tile-aligned parts), and, on about a quarter of the steps, one
injected +inf, -inf, NaN or 3e38. Every step's overflow flag, t, loss scale and
squared norm (1e-9 relative) are checked, and the committed p, m, v and slot are
compared bit for bit with the oracle's. Inputs come from numpy's seeded
generator (bf16 storage through workloads' cast); expected values from oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import NTHREADS, assert_bitexact, say, sumsq_close, to_dev, to_host

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(10_000 + seed)
    if rng.random() < 0.9:
        N = int(rng.choice([1, 2, 3, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 64]))
    else:
        N = int(rng.choice([100, 128, 200, 255, 256]))
    smax = 2_000_000 if N <= 16 else (400_000 if N <= 64 else 60_000)
    S = int(rng.integers(1, smax)) if rng.random() < 0.7 else int(rng.integers(1, 5000))
    kind = str(rng.choice(["bf16", "f32", "wire"])) if rng.random() < 0.8 else "bf16"
    path = str(rng.choice(["host", "dev1", "dev2", "parts"]))
    if kind == "f32" and path == "parts":
        path = "dev2"
    return rng, N, S, kind, path


@pytest.mark.parametrize("seed", range(64))
def test_random_case(Z, seed):
    rng, N, S, kind, path = draw(seed)
    tiled = seed >= 40 and path != "host"
    steps = int(rng.integers(2, 5))
    ls = float(2.0 ** int(rng.integers(0, 17)))
    dynamic = bool(rng.random() < 0.5)
    hy = dict(lr=float(10 ** rng.uniform(-5, -1)), beta1=float(rng.choice([0.9, 0.8, 0.0, 0.99])),
              beta2=float(rng.choice([0.999, 0.95, 0.5])),
              eps=float(rng.choice([1e-8, 1e-6, 1e-12])), wd=float(rng.choice([0.0, 0.01, 0.1])))
    sigma = float(10 ** rng.uniform(-6, 0))
    p0 = (rng.standard_normal(S) * 10 ** rng.uniform(-3, 0)).astype(np.float32)
    gdt = {"bf16": Z.ZERO_BF16, "f32": Z.ZERO_F32, "wire": Z.ZERO_BF16_WIRE}[kind]
    tr = oracle.Trainer(p0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32),
                        oracle.f32_to_bf16(p0), loss_scale=ls, dynamic=dynamic, nthreads=NTHREADS,
                        wire=(kind == "wire"), **hy)
    zhy = dict(lr=hy["lr"], beta1=hy["beta1"], beta2=hy["beta2"], eps=hy["eps"],
               weight_decay=hy["wd"])
    if path == "host":
        st = Z.ShardStep(S, N, gdt, to_dev(p0), loss_scale=ls, dynamic=dynamic, **zhy)
    else:
        st = Z.DeviceShardStep(S, N, gdt, to_dev(p0), loss_scale=ls, dynamic=dynamic,
                               double_slot=(path != "dev1"),
                               state_layout=Z.ZERO_STATE_TILED if tiled else Z.ZERO_STATE_SPLIT,
                               **zhy)
    ends = None
    if path == "parts":
        k = int(rng.integers(1, 9))
        g = Z.ZERO_STATE_TILE if tiled else 8
        ends = sorted(int(x) // g * g for x in rng.integers(0, S + 1, size=k - 1)) + [S]
    desc = (f"seed={seed} N={N} S={S} {kind} {path} steps={steps} loss_scale={ls} "
            f"dynamic={dynamic} parts={ends} tiled={tiled}")
    say(desc)
    for s in range(steps):
        sample = [rng.standard_normal(S) * sigma * ls for _ in range(N)]
        if kind == "f32":
            reps = [x.astype(np.float32) for x in sample]
        else:
            reps = [W._bf16_bits_from_f32(x) for x in sample]
        if rng.random() < 0.25:
            j, i = int(rng.integers(0, N)), int(rng.integers(0, S))
            v = float(rng.choice([np.inf, -np.inf, np.nan, 3e38]))
            reps[j][i] = v if kind == "f32" else W._bf16_bits_from_f32(np.array([v]))[0]
        dreps = [to_dev(r) for r in reps]
        flag, sumsq = tr.step(reps)
        if path == "host":
            stt, _ = st.step(dreps)
            torch.cuda.synchronize()
            assert stt.overflow == flag, (desc, s)
            got_sumsq, t, scale = stt.sumsq, st.t, st.loss_scale
            got = (st.master, st.exp_avg, st.exp_avg_sq, st.slot)
        else:
            if ends is not None:
                st.step_parts(dreps, ends)
            else:
                st.step(dreps)
            rec = st.state()
            assert rec.last_overflow == flag, (desc, s)
            got_sumsq, t, scale = rec.last_sumsq, rec.t, rec.loss_scale
            got = (*st.committed(), st.current_slot())
        assert t == tr.t and scale == tr.loss_scale, (desc, s)
        if not flag:
            assert sumsq_close(got_sumsq, sumsq), (desc, s, got_sumsq, sumsq)
        for name, g, w in zip(("p", "m", "v", "slot"), got, (tr.p, tr.m, tr.v, tr.slot)):
            assert_bitexact(f"{desc} step {s} {name}", to_host(g), w)
