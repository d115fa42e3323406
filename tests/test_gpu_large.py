"""GPU parity at full shard sizes, in the launch configuration bench.py times
(device commit, double-buffered slot, whole-shard grid, tiled state; the
Llama-7B shard also with split state):

* every element of the Llama-7B shard (S = 842,301,952, N = 8, loss scale
  65536) through its 5 steps and of the Llama-70B shard (S = 2,155,520,256,
  N = 32, AdamW) through its 3 steps, rank 0: after each step the committed p,
  m, v and slot come back chunk by chunk and the oracle steps the same chunk of
  its own state with the same replica values; every element must agree bit for
  bit (test_*_shard_every_element);
* rank 0 (Llama-7B) and rank N - 1 (both shards), whose standard-ring order is
  the ascending walk rank0 + rank1 + ... + rank(N-1), on sampled elements: the
  oracle follows the trajectory of the first and last 64 Ki elements, every
  tensor boundary of the shard and random positions (each element's update
  depends only on its own inputs; the overflow flag is global and is checked to
  be 0 on both sides). Whole-shard properties close the gap: the fused step
  equals the unfused path (reduce, then Adam from the fp32 gradient) bit for
  bit, the unfused gradient equals the oracle on the samples, and the fused
  squared norm equals an fp64 sum of that gradient's squares.

A box with too little free device memory for a shard fails the test with a
message rather than skipping it.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import NTHREADS, assert_bitexact, check_state, say, sumsq_close, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


GIB = 1 << 30


def require_device_memory(gib: float, what: str):
    """Fail (not skip) when the device has less free memory than a shard needs."""
    free, total = torch.cuda.mem_get_info()
    if free < gib * GIB:
        pytest.fail(f"{what} needs about {gib:.0f} GiB of free device memory; this device has "
                    f"{free / GIB:.0f} of {total / GIB:.0f} GiB free")


def sample_index(S, covered, rng, n_random):
    idx = [np.arange(0, min(S, 65536)), np.arange(max(0, S - 65536), S)]
    for off, ln in covered:
        for e in (off, off + 1, off + ln - 2, off + ln - 1):
            if 0 <= e < S:
                idx.append(np.array([e]))
    idx.append(rng.integers(0, S, n_random))
    return np.unique(np.concatenate(idx)).astype(np.int64)


def gather(t, idx_t):
    return t[idx_t]


def new_step(Z, w, S, covered, rank, tiled=True):
    """Rank ``rank``'s initial fp32 master, filled on the device, and the keyword
    arguments of the bench's DeviceShardStep (device commit, double slot)."""
    p0 = torch.empty(S, dtype=torch.float32, device="cuda")
    W.device_fill_params(p0, w, covered, rank)
    return p0, dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.wd,
                    loss_scale=w.loss_scale, dynamic=w.dynamic_loss_scale, double_slot=True,
                    state_layout=Z.ZERO_STATE_TILED if tiled else Z.ZERO_STATE_SPLIT)


def run_large(Z, name, steps, n_random, sub_elems, tiled=True, rank=0):
    w = W.get(name)
    lay = oracle.Layout(w.numels, N=w.N, A=w.A, B=w.B)
    S = lay.S
    covered = [(int(s[2]), int(s[3])) for s in lay.segments(rank)]
    rng = np.random.default_rng(5 + rank)
    idx = sample_index(S, covered, rng, n_random)
    idx_t = torch.from_numpy(idx).cuda()
    say(f"{name}: rank {rank} S={S} N={w.N}, {idx.size} samples, tiled={tiled}, allocating")
    p0, kw = new_step(Z, w, S, covered, rank, tiled)
    p0_s = to_host(gather(p0, idx_t))
    p0_head = p0[:min(S, sub_elems)].clone()
    step = Z.DeviceShardStep(S, w.N, Z.ZERO_BF16, p0, **kw)
    del p0
    torch.cuda.empty_cache()
    reps = [torch.empty(S, dtype=torch.bfloat16, device="cuda") for _ in range(w.N)]
    tr = oracle.Trainer(p0_s.copy(), np.zeros(idx.size, np.float32), np.zeros(idx.size, np.float32),
                        oracle.f32_to_bf16(p0_s), loss_scale=w.loss_scale,
                        dynamic=w.dynamic_loss_scale, nthreads=NTHREADS, **w.hyper())
    for s in range(steps):
        say(f"{name}: rank {rank} generating step {s} replicas")
        for j, r in enumerate(reps):
            W.device_fill_replica(r, w, covered, rank, s, j)
        sreps = [to_host(gather(r.view(torch.int16), idx_t)) for r in reps]
        dreps = [r.view(torch.int16) for r in reps]
        if s == 0:
            # whole-shard properties on the first step, before the state moves
            unfused_properties(Z, w, S, p0_head, dreps, idx, idx_t, sreps, sub_elems)
            del p0_head
        say(f"{name}: rank {rank} step {s}")
        step.step(dreps)
        flag, _ = tr.step(sreps)
        rec = step.state()
        st = step.last_stats()
        assert flag == 0 and st.overflow == 0 and rec.last_overflow == 0
        assert rec.t == tr.t == s + 1 and np.isfinite(st.sumsq) and st.sumsq > 0
        P, M, V = step.committed_at(idx_t)
        check_state(f"{name} rank {rank} step {s} (samples)", to_host(P), to_host(M), to_host(V),
                    to_host(gather(step.current_slot(), idx_t)), tr.p, tr.m, tr.v, tr.slot)
    del reps, dreps, step
    torch.cuda.empty_cache()


def unfused_properties(Z, w, S, p0_head, dreps, idx, idx_t, sreps, sub_elems):
    """On the first step's inputs: reduce_shard's g equals the oracle on the samples;
    its squared norm equals an fp64 sum of g^2; the fused kernel's own norm agrees;
    over the first `sub_elems` elements the unfused update equals the fused one
    bit for bit."""
    dev = torch.device("cuda")
    say(f"{w.name}: reduce_shard over the whole shard")
    G = torch.empty(S, dtype=torch.float32, device=dev)
    stats = torch.zeros(16, dtype=torch.uint8, device=dev)
    ws = torch.empty(Z.zero_workspace_bytes(S), dtype=torch.uint8, device=dev)
    Z.zero_reduce_shard(dreps, Z.ZERO_BF16, S, stats, ws, loss_scale=w.loss_scale, grad_out=G)
    torch.cuda.synchronize()
    st = Z.stats_from_tensor(stats)
    g_s, flag, _ = oracle.reduce(sreps, loss_scale=w.loss_scale, nthreads=NTHREADS)
    assert st.overflow == 0 and flag == 0
    gg = to_host(gather(G, idx_t))
    assert np.array_equal(gg.view(np.uint32), g_s.view(np.uint32)), "reduced g differs on samples"
    total = 0.0
    for c0 in range(0, S, 1 << 28):
        total += float(torch.sum(G[c0:c0 + (1 << 28)].double() ** 2).item())
    assert sumsq_close(st.sumsq, total, 1e-9), (st.sumsq, total)
    # unfused update over a sub-range equals the fused kernel on the same sub-range
    n = min(S, sub_elems)
    say(f"{w.name}: fused vs unfused over the first {n} elements")
    P0 = p0_head[:n]
    Zr = torch.zeros(n, dtype=torch.float32, device=dev)
    outs_u = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(3)]
    slot_u = torch.empty(n, dtype=torch.int16, device=dev)
    a = Z.make_adam_args(grad_f32=G[:n], p_in=P0, m_in=Zr, v_in=Zr, p_out=outs_u[0], m_out=outs_u[1],
                         v_out=outs_u[2], slot=slot_u, shard_S=n, lr=w.lr, beta1=w.beta1,
                         beta2=w.beta2, eps=w.eps, weight_decay=w.wd, step_t=1, stats=stats,
                         workspace=ws)
    Z.zero_adam_step(a)
    outs_f = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(3)]
    slot_f = torch.empty(n, dtype=torch.int16, device=dev)
    a = Z.make_adam_args(replicas=[r[:n] for r in dreps], grad_dtype=Z.ZERO_BF16, p_in=P0, m_in=Zr,
                         v_in=Zr, p_out=outs_f[0], m_out=outs_f[1], v_out=outs_f[2], slot=slot_f,
                         shard_S=n, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                         weight_decay=w.wd, loss_scale=w.loss_scale, step_t=1, stats=stats,
                         workspace=ws)
    Z.zero_adam_step(a)
    torch.cuda.synchronize()
    for x, y in zip(outs_u + [slot_u], outs_f + [slot_f]):
        assert torch.equal(x, y)
    del G, outs_u, outs_f, slot_u, slot_f, Zr
    torch.cuda.empty_cache()


@pytest.mark.parametrize("tiled", [True, False])
def test_llama7b_shard_full_size(Z, tiled):
    require_device_memory(60, "the Llama-7B shard")
    run_large(Z, "llama7b", steps=W.get("llama7b").steps, n_random=400_000, sub_elems=1 << 28,
              tiled=tiled)


@pytest.mark.parametrize("name,need", [("llama7b", 60), ("llama70b", 215)])
def test_large_shard_last_rank(Z, name, need):
    """Rank N - 1: its slot table in standard-ring order is the ascending walk."""
    w = W.get(name)
    require_device_memory(need, f"the {name} shard")
    run_large(Z, name, steps=w.steps, n_random=300_000, sub_elems=1 << 27, rank=w.N - 1)


class PinnedChunks:
    """Pinned host staging for chunk-wise device-to-host copies: ``get(k, t)``
    copies device tensor ``t`` (at most ``elems`` elements) into staging buffer
    k and returns a numpy view of it (valid until buffer k is reused)."""

    def __init__(self, n: int, elems: int, dtype):
        self.bufs = [torch.empty(elems, dtype=dtype, pin_memory=True) for _ in range(n)]

    def get(self, k: int, t) -> np.ndarray:
        b = self.bufs[k][: t.numel()]
        b.copy_(t)
        x = b.numpy()
        return x.view(np.uint16) if x.dtype == np.int16 else x


def tiled_chunk(set_buf, S: int, c0: int, c1: int, stage: PinnedChunks):
    """(p, m, v) of shard elements [c0, c1) of a tiled state set (c0 on a tile
    boundary), from one contiguous copy of the tiles that hold them."""
    T = ZERO_TILE
    t0, t1 = c0 // T, (c1 + T - 1) // T
    x = stage.get(0, set_buf[3 * T * t0: 3 * T * t1]).reshape(t1 - t0, 3, T)
    n = c1 - c0
    return tuple(np.ascontiguousarray(x[:, k, :].reshape(-1)[:n]) for k in range(3))


ZERO_TILE = 8192


def every_element(Z, name: str, chunk: int):
    """Every element of rank 0's shard of workload ``name`` through all its steps,
    in the bench's launch configuration, bit for bit against the oracle; the
    squared norm within 1e-9 relative (it is summed in another grouping)."""
    w = W.get(name)
    lay = oracle.Layout(w.numels, N=w.N, A=w.A, B=w.B)
    rank = 0
    S = lay.S
    assert chunk % ZERO_TILE == 0
    covered = [(int(s[2]), int(s[3])) for s in lay.segments(rank)]
    say(f"{name} every element: S={S} N={w.N}, allocating")
    p0, kw = new_step(Z, w, S, covered, rank)
    p = to_host(p0)
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    slot = oracle.f32_to_bf16(p)
    step = Z.DeviceShardStep(S, w.N, Z.ZERO_BF16, p0, **kw)
    del p0
    torch.cuda.empty_cache()
    reps = [torch.empty(S, dtype=torch.bfloat16, device="cuda") for _ in range(w.N)]
    rstage = PinnedChunks(w.N, chunk, torch.int16)
    sstage = PinnedChunks(1, 3 * (chunk + ZERO_TILE), torch.float32)
    slstage = PinnedChunks(1, chunk, torch.int16)
    for s in range(w.steps):
        say(f"{name} every element: generating step {s} replicas")
        for j, r in enumerate(reps):
            W.device_fill_replica(r, w, covered, rank, s, j)
        dreps = [r.view(torch.int16) for r in reps]
        say(f"{name} every element: step {s}")
        step.step(dreps)
        rec = step.state()
        assert rec.t == s + 1 and rec.last_overflow == 0
        cur = rec.cur & 1
        set_buf = step.sets[cur]
        cur_slot = step.slot_alt if cur else step.slot
        total = 0.0
        for c0 in range(0, S, chunk):
            c1 = min(S, c0 + chunk)
            hreps = [rstage.get(j, r[c0:c1]) for j, r in enumerate(dreps)]
            flag, sq = oracle.step(hreps, p[c0:c1], m[c0:c1], v[c0:c1], slot[c0:c1],
                                   loss_scale=w.loss_scale, t=s + 1, nthreads=NTHREADS,
                                   **w.hyper())
            assert flag == 0
            total += sq
            gp, gm, gv = tiled_chunk(set_buf, S, c0, c1, sstage)
            gs = slstage.get(0, cur_slot[c0:c1])
            # bit equality (which implies the 1e-6 / 1-ulp bar) over the chunk
            for what, g, want in (("p", gp, p), ("m", gm, m), ("v", gv, v), ("slot", gs, slot)):
                assert_bitexact(f"{name} step {s} {what} [{c0}, {c1})", g, want[c0:c1])
        assert sumsq_close(step.last_stats().sumsq, total, 1e-9), (step.last_stats().sumsq, total)
        say(f"{name} every element: step {s} matches on all {S} elements")
    del reps, dreps, step, rstage, sstage, slstage
    torch.cuda.empty_cache()


def test_llama7b_shard_every_element(Z):
    require_device_memory(60, "the Llama-7B shard")
    every_element(Z, "llama7b", 1 << 27)


def test_llama70b_shard_every_element(Z):
    require_device_memory(215, "the Llama-70B shard")
    every_element(Z, "llama70b", 1 << 26)
