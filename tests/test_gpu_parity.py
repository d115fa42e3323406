"""GPU parity: libzero's HIP path against the CPU oracle, element by element.

Acceptance (per element): p', m', v' within 1e-6 relative and the bf16 slot within
1 bf16 ulp; the overflow flag and the bucket-error count exactly; the squared
norm within 1e-9 relative (fp64 sums in different orders). Both sides use the
same fp32 operation sequence, so the p/m/v/slot checks also demand bit equality.

Cases: the Tiny workload on every rank for its 3 steps; the GPT-2-small shard;
the ragged 10,000-tensor workload with its injected +inf and dynamic loss scale,
whole-shard and bucket-table launches; ragged sizes and tails; every replica
count class; extreme values for the division and square root; the unfused path;
the bf16 cast; slot-only writes with guard bands; determinism.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import (NTHREADS, Guarded, assert_bitexact, check_state, say, sumsq_close, to_dev,
                      to_host)

pytestmark = pytest.mark.gpu


def layout_of(w, rank):
    lay = oracle.Layout(w.numels, N=w.N, A=w.A, B=w.B)
    covered = [(int(s[2]), int(s[3])) for s in lay.segments(rank)]
    return lay, covered


def read_stats(Z, stats_t):
    torch.cuda.synchronize()
    return Z.stats_from_tensor(stats_t)


def run_protocol(Z, w, rank, steps=None, bucket_elems=0, device_gen=False, wire=False):
    """Run the workload's steps on the GPU (ShardStep) and in the oracle (Trainer),
    comparing the committed state after every step. wire: fold on a bf16 wire."""
    lay, covered = layout_of(w, rank)
    S = lay.S
    gdt = Z.ZERO_BF16 if w.grad_dtype == "bf16" else Z.ZERO_F32
    if wire:
        gdt = Z.ZERO_BF16_WIRE
    p0 = W.host_params(w, S, covered, rank)
    buckets_t, nb = None, 0
    if bucket_elems:
        h = Z.zero_layout_build(list(w.numels), w.N, w.A, w.B)
        raw, nb = Z.zero_layout_buckets_raw(h, rank, bucket_elems)
        Z.zero_layout_free(h)
        buckets_t = torch.frombuffer(bytearray(bytes(raw)[: 16 * nb]), dtype=torch.uint8).to("cuda")
    step = Z.ShardStep(S, w.N, gdt, to_dev(p0), lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                       weight_decay=w.wd, loss_scale=w.loss_scale, dynamic=w.dynamic_loss_scale,
                       buckets=buckets_t, n_buckets=nb)
    tr = oracle.Trainer(p0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32),
                        oracle.f32_to_bf16(p0), loss_scale=w.loss_scale, dynamic=w.dynamic_loss_scale,
                        nthreads=NTHREADS, wire=wire, **w.hyper())
    flags = []
    for s in range(w.steps if steps is None else steps):
        say(f"{w.name} rank={rank} step={s} S={S} N={w.N} buckets={nb} wire={wire}")
        reps = W.host_replicas(w, S, covered, rank, s)
        dreps = [to_dev(r) for r in reps]
        st, verdict = step.step(dreps)
        flag, sumsq = tr.step(reps)
        flags.append(flag)
        assert st.overflow == flag and st.bad_buckets == 0
        assert verdict == (Z.ZERO_SKIP if flag else Z.ZERO_COMMIT)
        assert step.t == tr.t and step.loss_scale == tr.loss_scale
        if not flag:
            assert sumsq_close(st.sumsq, sumsq), (st.sumsq, sumsq)
        else:
            assert not np.isfinite(st.sumsq)
        torch.cuda.synchronize()
        check_state(f"{w.name} r{rank} s{s}", to_host(step.master), to_host(step.exp_avg),
                    to_host(step.exp_avg_sq), to_host(step.slot), tr.p, tr.m, tr.v, tr.slot)
    return flags


def test_tiny_every_rank_all_steps(Z):
    w = W.get("tiny")
    for rank in range(w.N):
        flags = run_protocol(Z, w, rank)
        assert flags == [0, 0, 0]


@pytest.mark.parametrize("rank", [0, 7])
def test_gpt2_small_shard(Z, rank):
    w = W.get("gpt2s")
    run_protocol(Z, w, rank, steps=3 if rank == 0 else 1)


@pytest.mark.parametrize("rank,bucket_elems", [(0, 0), (0, 4096), (63, 0), (63, 1000), (31, 2048),
                                               (17, 65536)])
def test_ragged_inf_injection_and_dynamic_scale(Z, rank, bucket_elems):
    w = W.get("ragged")
    lay, covered = layout_of(w, rank)
    inj = W.injection(w, lay.S, covered, rank)
    flags = run_protocol(Z, w, rank, bucket_elems=bucket_elems)
    want = [1 if s == inj[0] else 0 for s in range(w.steps)]
    assert flags == want


def single_step_case(Z, S, N, dtype, seed, *, loss_scale=1.0, t=1, wd=0.01, scale=1e-3,
                     slot=True, fused=True, buckets=None, wire=False, reps=None):
    """One fused (or reduce + unfused) step on random inputs; returns GPU and oracle results.
    wire: bf16 replicas folded on a bf16 wire; reps: replicas to use instead of random ones."""
    rng = np.random.default_rng(seed)
    if reps is not None:
        pass
    elif dtype == "bf16" and wire:     # magnitudes spread over 8 decades: the wire rounds
        reps = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * scale * loss_scale
                                                 * 10.0 ** rng.uniform(-4, 4, size=S)))
                for _ in range(N)]
    elif dtype == "bf16":
        reps = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * scale * loss_scale))
                for _ in range(N)]
    else:
        reps = [(rng.standard_normal(S) * scale * loss_scale).astype(np.float32) for _ in range(N)]
    p = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m = (rng.standard_normal(S) * 1e-4).astype(np.float32) if t > 1 else np.zeros(S, np.float32)
    v = ((rng.standard_normal(S) * 1e-4) ** 2).astype(np.float32) if t > 1 else np.zeros(S, np.float32)
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    g, flag, sumsq = oracle.reduce(reps, loss_scale=loss_scale, nthreads=NTHREADS, wire=wire)
    po, mo, vo, so = oracle.adam(g, p, m, v, t=t, wd=wd, nthreads=NTHREADS, **hy)
    dreps = [to_dev(r) for r in reps]
    P_in, M_in, V_in = to_dev(p), to_dev(m), to_dev(v)
    P_out, M_out, V_out = (torch.empty(max(S, 1), dtype=torch.float32, device="cuda")[:S] for _ in range(3))
    slot_t = torch.empty(max(S, 1), dtype=torch.int16, device="cuda")[:S] if slot else None
    stats = torch.zeros(16, dtype=torch.uint8, device="cuda")
    ws = torch.empty(Z.zero_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    gdt = (Z.ZERO_BF16_WIRE if wire else Z.ZERO_BF16) if dtype == "bf16" else Z.ZERO_F32
    if fused:
        a = Z.make_adam_args(replicas=dreps, grad_dtype=gdt, p_in=P_in, m_in=M_in, v_in=V_in,
                             p_out=P_out, m_out=M_out, v_out=V_out, slot=slot_t, shard_S=S,
                             loss_scale=loss_scale, step_t=t, weight_decay=wd, stats=stats,
                             workspace=ws, **hy)
        Z.zero_adam_step(a)
    else:
        G = torch.empty(max(S, 1), dtype=torch.float32, device="cuda")[:S]
        Z.zero_reduce_shard(dreps, gdt, S, stats, ws, loss_scale=loss_scale, grad_out=G)
        st = read_stats(Z, stats)
        assert st.overflow == flag and sumsq_close(st.sumsq, sumsq)
        assert_bitexact("g", to_host(G), g)
        a = Z.make_adam_args(grad_f32=G, p_in=P_in, m_in=M_in, v_in=V_in, p_out=P_out, m_out=M_out,
                             v_out=V_out, slot=slot_t, shard_S=S, step_t=t, weight_decay=wd,
                             stats=stats, workspace=ws, **hy)
        Z.zero_adam_step(a)
    st = read_stats(Z, stats)
    assert st.overflow == flag, (st.overflow, flag)
    if flag == 0:
        assert sumsq_close(st.sumsq, sumsq), (st.sumsq, sumsq)
        check_state(f"S={S} N={N} {dtype}", to_host(P_out), to_host(M_out), to_host(V_out),
                    to_host(slot_t) if slot else None, po, mo, vo, so if slot else None)
    return st


SIZES = [0, 1, 2, 3, 4, 5, 7, 8, 9, 1023, 1024, 1025, 2047, 2048, 2049, 4095, 4096, 4099,
         3 * 2048 + 5, 100_003]


@pytest.mark.parametrize("S", SIZES)
def test_ragged_sizes_bf16(Z, S):
    say(f"fused bf16 S={S} N=8")
    st = single_step_case(Z, S, 8, "bf16", seed=S)
    if S == 0:
        assert st.overflow == 0 and st.sumsq == 0.0


@pytest.mark.parametrize("N", [1, 2, 3, 7, 8, 9, 16, 17, 32, 64, 65, 255, 256])
def test_replica_counts(Z, N):
    say(f"fused bf16 S=5003 N={N}")
    single_step_case(Z, 5003, N, "bf16", seed=1000 + N, loss_scale=65536.0, t=3, wd=0.0)


@pytest.mark.parametrize("N", [257, 300, 511, 512, 1000, 1024])
def test_replica_counts_beyond_argument_block(Z, N):
    """More replicas than the kernel arguments carry: the pointers go through a
    device table at the end of the workspace, written ahead of the step."""
    say(f"fused bf16 S=5003 N={N} (pointer table)")
    single_step_case(Z, 5003, N, "bf16", seed=2000 + N, loss_scale=65536.0, t=2, wd=0.01)


@pytest.mark.parametrize("N,dtype,fused,wire", [(300, "f32", True, False), (300, "bf16", True, True),
                                                (1024, "bf16", False, False),
                                                (700, "bf16", False, True)])
def test_pointer_table_other_paths(Z, N, dtype, fused, wire):
    say(f"{dtype} N={N} fused={fused} wire={wire} (pointer table)")
    single_step_case(Z, 4101, N, dtype, seed=3000 + N, scale=1e-2, fused=fused, wire=wire, t=3)


@pytest.mark.parametrize("double_slot,parts", [(False, None), (True, [1000, 1000, 4096, 9001])])
def test_device_commit_with_pointer_table(Z, double_slot, parts):
    """Device-committed steps (one or two slots, whole or split into parts) with
    N = 300 replicas, an overflow on the second step, against the oracle."""
    S, N = 9001, 300
    rng = np.random.default_rng(41)
    p0 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    tr = oracle.Trainer(p0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32),
                        oracle.f32_to_bf16(p0), loss_scale=256.0, dynamic=True, nthreads=NTHREADS,
                        wd=0.01, **hy)
    st = Z.DeviceShardStep(S, N, Z.ZERO_BF16, to_dev(p0), loss_scale=256.0, dynamic=True,
                           double_slot=double_slot, weight_decay=0.01, **hy)
    for k in range(3):
        say(f"device commit N={N} step {k} double_slot={double_slot} parts={parts}")
        reps = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3 * 256.0))
                for _ in range(N)]
        if k == 1:
            reps[N - 1][S // 2] = 0x7F80            # +inf in the last slot
        flag, sumsq = tr.step(reps)
        dreps = [to_dev(r) for r in reps]
        if parts:
            st.step_parts(dreps, parts)
        else:
            st.step(dreps)
        rec = st.state()
        assert rec.last_overflow == flag == (1 if k == 1 else 0)
        assert rec.t == tr.t and rec.loss_scale == tr.loss_scale
        if not flag:
            assert sumsq_close(rec.last_sumsq, sumsq), (rec.last_sumsq, sumsq)
        p, m, v = st.committed()
        check_state(f"N={N} step {k}", to_host(p), to_host(m), to_host(v),
                    to_host(st.current_slot()), tr.p, tr.m, tr.v, tr.slot)


@pytest.mark.parametrize("N,S", [(1, 999), (2, 2024), (5, 4101)])
def test_fp32_replicas(Z, N, S):
    say(f"fused f32 S={S} N={N}")
    single_step_case(Z, S, N, "f32", seed=N * 7, scale=1e-2, wd=0.0)


@pytest.mark.parametrize("S", [1, 4097, 262_147])
def test_unfused_matches_oracle(Z, S):
    say(f"reduce + unfused adam S={S}")
    single_step_case(Z, S, 8, "bf16", seed=S + 5, fused=False, t=2)


def test_unfused_in_place(Z):
    S, N = 70_001, 4
    rng = np.random.default_rng(17)
    reps = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3)) for _ in range(N)]
    p = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m = (rng.standard_normal(S) * 1e-4).astype(np.float32)
    v = ((rng.standard_normal(S) * 1e-4) ** 2).astype(np.float32)
    hy = dict(lr=2e-3, beta1=0.8, beta2=0.99, eps=1e-6)
    g, _, _ = oracle.reduce(reps)
    po, mo, vo, so = oracle.adam(g, p, m, v, t=9, wd=0.1, **hy)
    P, M, V, G = to_dev(p), to_dev(m), to_dev(v), to_dev(g)
    slot = torch.empty(S, dtype=torch.int16, device="cuda")
    stats = torch.zeros(16, dtype=torch.uint8, device="cuda")
    ws = torch.empty(Z.zero_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    a = Z.make_adam_args(grad_f32=G, p_in=P, m_in=M, v_in=V, p_out=P, m_out=M, v_out=V, slot=slot,
                         shard_S=S, step_t=9, weight_decay=0.1, stats=stats, workspace=ws, **hy)
    Z.zero_adam_step(a)
    torch.cuda.synchronize()
    check_state("in place", to_host(P), to_host(M), to_host(V), to_host(slot), po, mo, vo, so)


def test_division_and_sqrt_extremes(Z):
    """Wide-range g, m, v (v down to fp32 subnormals) through the unfused path:
    exercises the correctly rounded division and square root against the CPU."""
    S = 1 << 20
    rng = np.random.default_rng(99)
    def logu(lo, hi, n, signed=True):
        x = np.exp2(rng.uniform(lo, hi, n)) * rng.uniform(1.0, 2.0, n)
        if signed:
            x *= rng.choice([-1.0, 1.0], n)
        return x.astype(np.float32)
    g = logu(-60, 60, S)
    m = logu(-60, 60, S)
    v = logu(-149, 100, S, signed=False)
    v[:1000] = np.arange(1000, dtype=np.uint32).view(np.float32)   # +0 and the smallest subnormals
    p = logu(-30, 10, S)
    for t in (1, 2, 10, 10_000):
        hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
        po, mo, vo, so = oracle.adam(g, p, m, v, t=t, wd=0.01, nthreads=NTHREADS, **hy)
        finite = np.isfinite(po) & np.isfinite(mo) & np.isfinite(vo)
        P_out, M_out, V_out = (torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(3))
        slot = torch.empty(S, dtype=torch.int16, device="cuda")
        stats = torch.zeros(16, dtype=torch.uint8, device="cuda")
        ws = torch.empty(Z.zero_workspace_bytes(S), dtype=torch.uint8, device="cuda")
        a = Z.make_adam_args(grad_f32=to_dev(g), p_in=to_dev(p), m_in=to_dev(m), v_in=to_dev(v),
                             p_out=P_out, m_out=M_out, v_out=V_out, slot=slot, shard_S=S, step_t=t,
                             weight_decay=0.01, stats=stats, workspace=ws, **hy)
        say(f"extremes t={t}")
        Z.zero_adam_step(a)
        torch.cuda.synchronize()
        gp, gm, gv, gs = to_host(P_out), to_host(M_out), to_host(V_out), to_host(slot)
        assert finite.mean() > 0.99
        for name, x, y in (("p", gp, po), ("m", gm, mo), ("v", gv, vo)):
            assert_bitexact(f"extremes t={t} {name}", x[finite], y[finite])
        assert_bitexact(f"extremes t={t} slot", gs[finite], so[finite])


def test_overflow_classes(Z):
    S, N = 4099, 8
    rng = np.random.default_rng(3)
    base = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3)) for _ in range(N)]
    cases = {"+inf": [(2, 17, 0x7F80)], "-inf": [(0, 4098, 0xFF80)], "nan": [(7, 0, 0x7FC0)],
             "inf-inf": [(1, 100, 0x7F80), (5, 100, 0xFF80)],
             "finite overflow": [(j, 3000, 0x7F7F) for j in range(N)]}
    stats = torch.zeros(16, dtype=torch.uint8, device="cuda")
    ws = torch.empty(Z.zero_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    for name, edits in list(cases.items()) + [("clean", [])]:
        reps = [r.copy() for r in base]
        for j, i, val in edits:
            reps[j][i] = val
        _, flag, sumsq = oracle.reduce(reps)
        say(f"overflow case {name}")
        Z.zero_reduce_shard([to_dev(r) for r in reps], Z.ZERO_BF16, S, stats, ws)
        st = read_stats(Z, stats)
        assert st.overflow == flag == (0 if name == "clean" else 1), name
        assert sumsq_close(st.sumsq, sumsq), (name, st.sumsq, sumsq)


@pytest.mark.parametrize("S", [0, 1, 3, 4, 5, 1_000_003])
def test_gather_slot(Z, S):
    rng = np.random.default_rng(S)
    x = (rng.standard_normal(S) * 10.0 ** rng.uniform(-40, 38, S)).astype(np.float32)
    if S > 20:
        x[:8] = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, 3.4e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8],
                         dtype=np.float32)
        x[8:20] = np.array([0x3F808000, 0x3F818000, 0x7F7F8000, 0x00008000, 0x80018000, 0x7FC00001,
                            0xFFFFFFFF, 0x00000001, 0x3F80FFFF, 0x3F807FFF, 0xBF808000, 0x7F7FFFFF],
                           dtype=np.uint32).view(np.float32)
    want = oracle.f32_to_bf16(x)
    slot = Guarded(2 * S, torch.int16)
    say(f"gather_slot S={S}")
    Z.zero_gather_slot(to_dev(x), S, slot.t)
    torch.cuda.synchronize()
    assert_bitexact("slot", to_host(slot.t), want)
    assert slot.intact()


def test_slot_only_writes_and_guard_bands(Z):
    """The step writes this rank's slot and nothing else of the gathered buffer, and
    no byte outside any output buffer."""
    N, S, rank = 8, 10_000, 5
    rng = np.random.default_rng(8)
    reps = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3)) for _ in range(N)]
    p = (rng.standard_normal(S) * 0.02).astype(np.float32)
    z = np.zeros(S, np.float32)
    g, _, _ = oracle.reduce(reps)
    po, mo, vo, so = oracle.adam(g, p, z, z, t=1, wd=0.0, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    gathered = Guarded(2 * N * S, torch.int16)
    gathered.t.fill_(0x5A5A)
    gr = [Guarded(2 * S, torch.int16, to_dev(r)) for r in reps]
    P_in, M_in, V_in = (Guarded(4 * S, torch.float32, to_dev(a)) for a in (p, z, z))
    P_out, M_out, V_out = (Guarded(4 * S, torch.float32) for _ in range(3))
    stats = Guarded(16, torch.uint8)
    ws = Guarded(Z.zero_workspace_bytes(S), torch.uint8)
    slot = gathered.t[rank * S:(rank + 1) * S]
    a = Z.make_adam_args(replicas=[r.t for r in gr], grad_dtype=Z.ZERO_BF16, p_in=P_in.t, m_in=M_in.t,
                         v_in=V_in.t, p_out=P_out.t, m_out=M_out.t, v_out=V_out.t, slot=slot,
                         shard_S=S, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                         loss_scale=1.0, step_t=1, stats=stats.t, workspace=ws.t)
    Z.zero_adam_step(a)
    torch.cuda.synchronize()
    allg = to_host(gathered.t)
    for r in range(N):
        if r != rank:
            assert np.all(allg[r * S:(r + 1) * S] == 0x5A5A), f"slot {r} was written"
    check_state("slot-only", to_host(P_out.t), to_host(M_out.t), to_host(V_out.t),
                allg[rank * S:(rank + 1) * S], po, mo, vo, so)
    for buf in [gathered, *gr, P_in, M_in, V_in, P_out, M_out, V_out, stats, ws]:
        assert buf.intact()
    # the inputs are untouched
    assert_bitexact("p_in", to_host(P_in.t), p)


@pytest.mark.parametrize("N,S,n_cuts", [(6, 20_011, 400), (300, 20_011, 400), (6, 300_007, 40),
                                         (65, 300_007, 40), (8, 300_007, 1)])
def test_bucket_table_random(Z, N, S, n_cuts):
    """Random disjoint buckets at arbitrary (unaligned) offsets: elements inside are
    updated as the oracle says, elements outside keep their sentinel, a bucket
    that leaves the shard is skipped and counted (N = 300: replica pointers from
    the workspace table). S = 300,007 with few cuts: a short table of long
    buckets, cut into chunks spread over the grid."""
    say(f"bucket table N={N} S={S} cuts={n_cuts}")
    rng = np.random.default_rng(12)
    reps = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3)) for _ in range(N)]
    p = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m = (rng.standard_normal(S) * 1e-4).astype(np.float32)
    v = ((rng.standard_normal(S) * 1e-4) ** 2).astype(np.float32)
    cuts = np.sort(rng.choice(np.arange(1, S), size=n_cuts, replace=False))
    edges = np.concatenate([[0], cuts, [S]])
    table = []
    for a0, b0 in zip(edges[:-1], edges[1:]):
        if (rng.random() < 0.6 or n_cuts < 2) and b0 > a0:
            table.append((int(a0), int(b0 - a0), 0))
    inside = np.zeros(S, bool)
    for o, ln, _ in table:
        inside[o:o + ln] = True
    table_bad = table + [(S - 5, 10, 0), (-4, 2, 0), (10, -3, 0)]
    raw = np.array(table_bad, dtype=np.dtype([("off", "<i8"), ("len", "<i4"), ("t", "<i4")]))
    buckets = torch.from_numpy(raw.view(np.uint8).copy()).to("cuda")
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    g, _, _ = oracle.reduce(reps)
    po, mo, vo, so = oracle.adam(g, p, m, v, t=4, wd=0.0, **hy)
    want_sumsq = float(np.sum(g[inside].astype(np.float64) ** 2))
    sent = np.full(S, 0x7FBADBAD, np.uint32).view(np.float32)
    P_out, M_out, V_out = (to_dev(sent.copy()) for _ in range(3))
    slot = to_dev(np.full(S, 0x5A5A, np.uint16))
    stats = torch.zeros(16, dtype=torch.uint8, device="cuda")
    ws = torch.empty(Z.zero_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    a = Z.make_adam_args(replicas=[to_dev(r) for r in reps], grad_dtype=Z.ZERO_BF16, p_in=to_dev(p),
                         m_in=to_dev(m), v_in=to_dev(v), p_out=P_out, m_out=M_out, v_out=V_out,
                         slot=slot, shard_S=S, buckets=buckets, n_buckets=len(table_bad),
                         loss_scale=1.0, step_t=4, weight_decay=0.0, stats=stats, workspace=ws, **hy)
    Z.zero_adam_step(a)
    st = read_stats(Z, stats)
    assert st.bad_buckets == 3 and st.overflow == 0
    assert sumsq_close(st.sumsq, want_sumsq, rel=1e-12)
    gp, gm, gv, gs = to_host(P_out), to_host(M_out), to_host(V_out), to_host(slot)
    check_state("buckets", gp[inside], gm[inside], gv[inside], gs[inside], po[inside], mo[inside],
                vo[inside], so[inside])
    assert np.all(gp[~inside].view(np.uint32) == 0x7FBADBAD)
    assert np.all(gs[~inside] == 0x5A5A)


def test_rerun_is_bit_identical(Z):
    S, N = 3_000_017, 8
    rng = np.random.default_rng(21)
    dreps = [to_dev(np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3))) for _ in range(N)]
    P_in = to_dev((rng.standard_normal(S) * 0.02).astype(np.float32))
    Z0 = torch.zeros(S, dtype=torch.float32, device="cuda")
    outs, sums = [], []
    for _ in range(2):
        P_out, M_out, V_out = (torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(3))
        slot = torch.empty(S, dtype=torch.int16, device="cuda")
        stats = torch.zeros(16, dtype=torch.uint8, device="cuda")
        ws = torch.empty(Z.zero_workspace_bytes(S), dtype=torch.uint8, device="cuda")
        a = Z.make_adam_args(replicas=dreps, grad_dtype=Z.ZERO_BF16, p_in=P_in, m_in=Z0, v_in=Z0,
                             p_out=P_out, m_out=M_out, v_out=V_out, slot=slot, shard_S=S, lr=1e-3,
                             beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, loss_scale=1.0,
                             step_t=1, stats=stats, workspace=ws)
        Z.zero_adam_step(a)
        st = read_stats(Z, stats)
        outs.append((P_out, M_out, V_out, slot))
        sums.append(st.sumsq)
    assert sums[0] == sums[1]
    for x, y in zip(*outs):
        assert torch.equal(x, y)
    # reduce-only and fused share the partition of the work: identical norm
    stats = torch.zeros(16, dtype=torch.uint8, device="cuda")
    ws = torch.empty(Z.zero_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    Z.zero_reduce_shard(dreps, Z.ZERO_BF16, S, stats, ws)
    assert read_stats(Z, stats).sumsq == sums[0]


# --- bf16 wire: the running sum rounded to bf16 after every add ---------------

@pytest.mark.parametrize("N,S", [(2, 4099), (3, 1), (8, 100_003), (8, 1_000_003), (17, 5),
                                 (64, 262_147)])
def test_wire_fused(Z, N, S):
    say(f"wire fused N={N} S={S}")
    single_step_case(Z, S, N, "bf16", seed=9000 + N, wire=True, t=3)


@pytest.mark.parametrize("S", [1, 4097, 262_147])
def test_wire_unfused_g_bit_exact(Z, S):
    say(f"wire unfused S={S}")
    single_step_case(Z, S, 8, "bf16", seed=9100 + S, wire=True, fused=False)


def test_wire_changes_the_result_and_decides_overflow(Z):
    """The kernel really takes the wire path: on spread magnitudes its g differs
    from the fp32 fold's; bf16 max plus half its ulp overflows on the wire only,
    and the NaN of an inf - inf pair is the same quiet NaN on both sides."""
    S, N = 4096, 8
    rng = np.random.default_rng(9200)
    reps = [np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S)
                                             * 10.0 ** rng.uniform(-4, 4, size=S))) for _ in range(N)]
    g_w = oracle.reduce(reps, wire=True)[0]
    g_f = oracle.reduce(reps)[0]
    assert np.sum(g_w != g_f) > S // 4
    stats = torch.zeros(16, dtype=torch.uint8, device="cuda")
    ws = torch.empty(Z.zero_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    G = torch.empty(S, dtype=torch.float32, device="cuda")
    Z.zero_reduce_shard([to_dev(r) for r in reps], Z.ZERO_BF16_WIRE, S, stats, ws, grad_out=G)
    assert_bitexact("g wire", to_host(G), g_w)
    # overflow on the wire only
    r0 = np.zeros(S, np.uint16)
    r1 = np.zeros(S, np.uint16)
    r0[10], r1[10] = 0x7F7F, np.asarray(W._bf16_bits_from_f32(np.array([2.0 ** 119])))[0]
    r0[20], r1[20] = 0x7F80, 0xFF80            # +inf + -inf -> NaN
    for wire in (False, True):
        g, flag, _ = oracle.reduce([r0, r1], wire=wire)
        gdt = Z.ZERO_BF16_WIRE if wire else Z.ZERO_BF16
        Z.zero_reduce_shard([to_dev(r0), to_dev(r1)], gdt, S, stats, ws, grad_out=G)
        st = read_stats(Z, stats)
        assert st.overflow == flag == 1
        got = to_host(G)
        assert np.isfinite(got[10]) == (not wire) and np.isfinite(g[10]) == (not wire)
        # NaN sign and payload are the hardware's (x86 and gfx950 differ for inf - inf)
        nan = np.isnan(g)
        assert np.array_equal(np.isnan(got), nan) and nan[20]
        assert_bitexact(f"g wire={wire}", got[~nan], g[~nan])


@pytest.mark.parametrize("rank,bucket_elems", [(0, 0), (63, 1000)])
def test_wire_ragged_protocol(Z, rank, bucket_elems):
    w = W.get("ragged")
    run_protocol(Z, w, rank, bucket_elems=bucket_elems, wire=True)
