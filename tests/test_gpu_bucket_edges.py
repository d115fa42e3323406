"""GPU parity at bucket edges that cut quads (4-element groups).

A bucket-table launch updates exactly the elements inside its buckets ("ZeRO
Optimizer", Communication Optimization: gradients are reduced and applied in
buckets). The kernel takes a quad cut by a bucket edge with the same vector
loads as a whole one and keeps only the bucket's elements, so these tests put
the edges everywhere a quad can be cut:
- buckets of 1, 2 and 3 elements, both edges inside one quad;
- neighbouring buckets sharing a quad (two workgroups writing one quad);
- a bucket that ends at S with S % 4 != 0 (the shard's last partial quad);
- an empty bucket.
NaN and inf sit in the excluded elements of cut quads (in every replica slot the
case draws); they must neither raise the overflow flag nor reach the norm.
Elements outside the buckets keep their sentinel.

The short table (11 buckets over 4,003 elements) runs one workgroup per bucket;
a generated table of about 10,000 buckets of 1-5 elements has more buckets than
workgroups, one of about 70,000 buckets of 950 elements a grid above the
65,536 workgroups up to which device-commit launches load their first replica
batch before the committed-state record, and one of short buckets runs under
300 replicas, whose pointers the kernel reads from the workspace.
Tables of a few long buckets are cut into chunks dealt over the grid: the long
table (and the same table in reverse order), the mid table over 3,000,003
elements, and a 70,000,003-element shard through the allocation-free entry
point, whose grid cap makes every workgroup take several chunks.
Checked: the fused step (p, m, v, slot bit for bit), the reduce-only launch (g
bit for bit), the device-commit step in the tiled layout (committed state inside
the buckets). Inputs from numpy's seeded generator; expected values from oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import NTHREADS, assert_bitexact, say, sumsq_close, to_dev, to_host

pytestmark = pytest.mark.gpu

# (offset, length) tables; S % 4 == 3 in all of them
SHORT_S = 4003
SHORT = [(1, 1), (2, 2), (5, 2), (8, 4), (13, 10), (30, 900), (50 + 900, 0), (1000, 3),
         (3990, 9), (3999, 1), (4000, 3)]
SHORT_BAD = [0, 4, 7, 12, 23, 1003]                       # outside, in cut quads
LONG_S = 300_003
LONG = [(3, 100_000), (100_005, 150_001), (250_007, 49_993), (300_000, 3)]
LONG_BAD = [0, 2, 100_003, 100_004, 250_006]
MID_S = 3_000_003
MID = [(2, 1_000_000), (1_000_006, 999_990), (2_000_064, 999_936), (3_000_000, 3)]
MID_BAD = [0, 1, 1_000_002, 1_000_005, 1_999_996, 2_000_000, 2_000_063]


def _generated(S, seed, first, sizes, gaps):
    """A table of buckets from `first` on, lengths and gaps drawn from the given
    ranges (a gap of 0 puts two buckets in one quad), the last bucket the shard's
    last 3 elements; the bad positions are gap elements spread over the shard."""
    rng = np.random.default_rng(seed)
    table, pos, gap_at = [], first, []
    while True:
        ln = int(rng.integers(*sizes))
        if pos + ln > S - 4:
            break
        table.append((pos, ln))
        pos += ln
        gp = int(rng.integers(*gaps))
        gap_at.extend(range(pos, pos + gp))
        pos += gp
    gap_at.extend(range(pos, S - 3))
    table.append((S - 3, 3))
    pick = np.linspace(0, len(gap_at) - 1, 7).astype(np.int64)
    return S, table, [gap_at[i] for i in pick]


TABLES = {"short": (SHORT_S, SHORT, SHORT_BAD), "long": (LONG_S, LONG, LONG_BAD),
          "long_rev": (LONG_S, LONG[::-1], LONG_BAD), "mid": (MID_S, MID, MID_BAD),
          # about 10,000 buckets of 1-5 elements over 40,003: more buckets than the
          # grid's 4,136 workgroups, so a workgroup takes two or three in turn
          "many": _generated(40_003, 71, 1, (1, 6), (0, 3)),
          # about 70,000 buckets of 950 elements over 67,000,003: a grid of 69,526
          # workgroups, past the 65,536 up to which the first replica batch is
          # loaded before the committed-state record
          "wide": _generated(67_000_003, 72, 2, (950, 951), (0, 3)),
          # short buckets under 300 replicas: the replica pointers come from the
          # workspace table instead of the kernel arguments
          "ptr": _generated(9001, 73, 3, (5, 40), (0, 4))}

CASES = [("short", "bf16", 5), ("short", "f32", 3), ("short", "bf16", 20), ("short", "wire", 9),
         ("many", "bf16", 5), ("ptr", "bf16", 300),
         ("long", "bf16", 5), ("long", "bf16", 20), ("long", "f32", 3), ("long_rev", "bf16", 5),
         ("mid", "bf16", 5), ("mid", "wire", 9), ("mid", "f32", 3), ("mid", "bf16", 33)]


def _case(Z, table_kind, kind, N):
    S, table, bad = TABLES[table_kind]
    rng = np.random.default_rng(4000 + N + len(kind) + S)
    sample = [rng.standard_normal(S) * 4e-3 for _ in range(N)]
    for i, e in enumerate(bad):
        sample[(3 * i) % N][e] = (np.nan, np.inf, -np.inf)[i % 3]
    if kind == "f32":
        reps = [x.astype(np.float32) for x in sample]
    else:
        reps = [np.asarray(W._bf16_bits_from_f32(x)) for x in sample]
    inside = np.zeros(S, bool)
    for o, ln in table:
        inside[o:o + ln] = True
    assert not inside[bad].any()
    raw = np.array([(o, ln, 0) for o, ln in table],
                   dtype=np.dtype([("off", "<i8"), ("len", "<i4"), ("t", "<i4")]))
    buckets = torch.from_numpy(raw.view(np.uint8).copy()).to("cuda")
    gdt = {"bf16": Z.ZERO_BF16, "f32": Z.ZERO_F32, "wire": Z.ZERO_BF16_WIRE}[kind]
    g, _, _ = oracle.reduce(reps, wire=(kind == "wire"))
    return S, table, rng, reps, inside, buckets, gdt, g


def _stats(Z, t):
    torch.cuda.synchronize()
    return Z.stats_from_tensor(t)


@pytest.mark.parametrize("table_kind,kind,N", CASES)
def test_bucket_edges_fused_and_reduce(Z, table_kind, kind, N):
    S, table, rng, reps, inside, buckets, gdt, g = _case(Z, table_kind, kind, N)
    say(f"bucket edges {table_kind} {kind} N={N} S={S} buckets={len(table)}")
    want_sumsq = float(np.sum(g[inside].astype(np.float64) ** 2))
    assert np.isfinite(g[inside]).all()
    p = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m = (rng.standard_normal(S) * 1e-4).astype(np.float32)
    v = ((rng.standard_normal(S) * 1e-4) ** 2).astype(np.float32)
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    po, mo, vo, so = oracle.adam(g, p, m, v, t=3, wd=0.01, **hy)
    dreps = [to_dev(r) for r in reps]
    sent = np.full(S, 0x7FBADBAD, np.uint32).view(np.float32)
    P_out, M_out, V_out = (to_dev(sent.copy()) for _ in range(3))
    slot = to_dev(np.full(S, 0x5A5A, np.uint16))
    stats = torch.zeros(16, dtype=torch.uint8, device="cuda")
    ws = torch.empty(Z.zero_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    a = Z.make_adam_args(replicas=dreps, grad_dtype=gdt, p_in=to_dev(p), m_in=to_dev(m),
                         v_in=to_dev(v), p_out=P_out, m_out=M_out, v_out=V_out, slot=slot,
                         shard_S=S, buckets=buckets, n_buckets=len(table), loss_scale=1.0,
                         step_t=3, weight_decay=0.01, stats=stats, workspace=ws, **hy)
    Z.zero_adam_step(a)
    st = _stats(Z, stats)
    assert st.overflow == 0 and st.bad_buckets == 0
    assert sumsq_close(st.sumsq, want_sumsq, rel=1e-12), (st.sumsq, want_sumsq)
    for name, got, want in (("p", P_out, po), ("m", M_out, mo), ("v", V_out, vo), ("slot", slot, so)):
        h = to_host(got)
        assert_bitexact(f"{table_kind} {kind} N={N} {name}", h[inside], want[inside])
        if name == "slot":
            assert np.all(h[~inside] == 0x5A5A)
        else:
            assert np.all(h[~inside].view(np.uint32) == 0x7FBADBAD), name
    # reduce-only launch over the same table: g inside, sentinel outside
    G = to_dev(sent.copy())
    stats.zero_()
    Z.zero_reduce_shard(dreps, gdt, S, stats, ws, buckets=buckets, n_buckets=len(table), grad_out=G)
    st = _stats(Z, stats)
    assert st.overflow == 0 and st.bad_buckets == 0
    assert sumsq_close(st.sumsq, want_sumsq, rel=1e-12)
    gh = to_host(G)
    assert_bitexact(f"{table_kind} {kind} N={N} g", gh[inside], g[inside])
    assert np.all(gh[~inside].view(np.uint32) == 0x7FBADBAD)


@pytest.mark.parametrize("table_kind", ["short", "long", "mid", "many", "wide", "ptr"])
def test_bucket_edges_device_commit_tiled(Z, table_kind):
    """Three device-commit steps over the table in the tiled layout; the second
    step's replicas carry an inf inside a bucket, so it is skipped. Tables of short
    buckets (short, many) load each workgroup's first replica batch before the
    committed-state record; the wide table's grid is past that bound."""
    N = {"wide": 2, "ptr": 300}.get(table_kind, 6)
    S, table, rng, reps, inside, buckets, gdt, g = _case(Z, table_kind, "bf16", N)
    say(f"bucket edges device commit tiled {table_kind} S={S}")
    p0 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    zhy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    st = Z.DeviceShardStep(S, N, gdt, to_dev(p0), loss_scale=1.0, double_slot=True,
                           state_layout=Z.ZERO_STATE_TILED, buckets=buckets, n_buckets=len(table),
                           **zhy)
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)
    tr = oracle.Trainer(p0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32),
                        oracle.f32_to_bf16(p0), loss_scale=1.0, nthreads=NTHREADS, **hy)
    first_inside = int(np.flatnonzero(inside)[17])
    for s in range(3):
        if s == 0:
            rs = reps
        else:
            rs = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 4e-3)) for _ in range(N)]
        if s == 1:
            rs[N - 1][first_inside] = np.asarray(W._bf16_bits_from_f32(np.array([np.inf])))[0]
        # the oracle sees only the buckets' elements: outside them the step reads nothing
        masked = [np.where(inside, r, np.uint16(0)) for r in rs]
        flag, sumsq = tr.step(masked)
        assert flag == (1 if s == 1 else 0)
        st.step([to_dev(r) for r in rs])
        rec = st.state()
        assert rec.last_overflow == flag and rec.t == tr.t
        if not flag:
            assert sumsq_close(rec.last_sumsq, sumsq), (rec.last_sumsq, sumsq)
        got = (*st.committed(), st.current_slot())
        for name, gv, want in zip(("p", "m", "v", "slot"), got, (tr.p, tr.m, tr.v, tr.slot)):
            assert_bitexact(f"{table_kind} step {s} {name}", to_host(gv)[inside], want[inside])


def test_chunks_over_a_capped_grid_noalloc(Z):
    """The allocation-free entry point caps the grid at 65,536 workgroups, so the
    68,361 chunks of a 70,000,003-element shard's four buckets are dealt over it
    more than once. Bucket edges cut quads, a NaN sits in a 64-element gap
    between buckets, the last bucket ends at S (S % 4 == 3)."""
    S, N = 70_000_003, 2
    table = [(0, 10_000_001), (10_000_005, 30_000_000), (40_000_069, 29_999_931), (70_000_000, 3)]
    bad = [10_000_002, 10_000_004, 40_000_040, 40_000_068]
    rng = np.random.default_rng(4242)
    say(f"chunks over a capped grid: S={S} N={N} buckets={len(table)}")
    sample = [rng.standard_normal(S, dtype=np.float32) * np.float32(4e-3) for _ in range(N)]
    for i, e in enumerate(bad):
        sample[i % N][e] = np.nan
    reps = [np.asarray(W._bf16_bits_from_f32(x)) for x in sample]
    del sample
    inside = np.zeros(S, bool)
    for o, ln in table:
        inside[o:o + ln] = True
    assert not inside[bad].any()
    raw = np.array([(o, ln, 0) for o, ln in table],
                   dtype=np.dtype([("off", "<i8"), ("len", "<i4"), ("t", "<i4")]))
    buckets = torch.from_numpy(raw.view(np.uint8).copy()).to("cuda")
    p = rng.standard_normal(S, dtype=np.float32) * np.float32(0.02)
    z = np.zeros(S, np.float32)
    g, _, _ = oracle.reduce(reps, nthreads=NTHREADS)
    want_sumsq = float(np.sum(g[inside].astype(np.float64) ** 2))
    po, mo, vo, so = oracle.adam(g, p, z, z, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01,
                                 t=1, nthreads=NTHREADS)
    del g
    sent = torch.full((S,), 0x7FBADBAD, dtype=torch.int32, device="cuda")
    P, M, V = (sent.clone().view(torch.float32) for _ in range(3))
    slot = torch.full((S,), 0x5A5A, dtype=torch.int16, device="cuda")
    stats = torch.zeros(16, dtype=torch.uint8, device="cuda")
    zd = torch.zeros(S, dtype=torch.float32, device="cuda")
    a = Z.make_adam_args(replicas=[to_dev(r) for r in reps], grad_dtype=Z.ZERO_BF16,
                         p_in=to_dev(p), m_in=zd, v_in=zd, p_out=P, m_out=M, v_out=V, slot=slot,
                         shard_S=S, buckets=buckets, n_buckets=len(table), loss_scale=1.0, step_t=1,
                         lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, stats=stats,
                         workspace=None)
    Z.zero_adam_step_noalloc(a)
    st = _stats(Z, stats)
    assert st.overflow == 0 and st.bad_buckets == 0
    assert sumsq_close(st.sumsq, want_sumsq), (st.sumsq, want_sumsq)
    for name, got, want in (("p", P, po), ("m", M, mo), ("v", V, vo), ("slot", slot, so)):
        h = to_host(got)
        assert_bitexact(f"capped grid {name}", h[inside], want[inside])
        if name == "slot":
            assert np.all(h[~inside] == 0x5A5A)
        else:
            assert np.all(h[~inside].view(np.uint32) == 0x7FBADBAD), name
