"""zero_adam_step_noalloc -- the step with the library's own scratch, for callers
that cannot allocate -- against zero_adam_step with a caller workspace, on the
same inputs, through the C ABI: p, m, v and the slot bit for bit (outputs
filled with sentinels first; a bucket launch must leave those outside its
buckets), the overflow flag exactly, the squared norm within 1e-9 relative (its partials are grouped by
another grid). Three calls in a row on one stream, each on a smaller input than
the one before, so the second and third find the scratch holding what the call
before wrote:

1. a shard of 100,664,327 elements (N = 8): the scratch caps the grid at 49,153
   workgroups striding over 98,305 trips, one workgroup with a single trip also
   takes the quad after the last trip and the S % 4 tail;
2. the ragged workload's rank-0 shard (N = 64) over its 4,096-element bucket
   table, with one +inf injected (overflow on both sides);
3. 5,003 elements with 300 replicas: the pointer table beyond the kernel
   arguments lives in the scratch.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import say, sumsq_close

pytestmark = pytest.mark.gpu


def bf16_replicas(gen, S, N, scale):
    out = []
    for _ in range(N):
        x = torch.randn(S, generator=gen, device="cuda", dtype=torch.float32).mul_(scale)
        out.append(x.to(torch.bfloat16).view(torch.int16))
    return out


SENT32, SENT16 = 0x7FBADBAD, 0x5A5A


def run_pair(Z, name, reps, S, p, m, v, *, loss_scale, t, wd, buckets=None, n_buckets=0,
             inside=None):
    """One zero_adam_step (with a workspace) and one zero_adam_step_noalloc on the
    same inputs into separate outputs, both filled with the same sentinels first
    (a bucket launch writes only the elements inside its buckets); compare, and
    check that the elements outside the buckets (``inside``: a boolean device
    mask, or None for the whole shard) kept their sentinels."""
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd)
    outs = {}
    for mode in ("workspace", "noalloc"):
        P, M, V = (torch.full((S,), SENT32, dtype=torch.int32, device="cuda").view(torch.float32)
                   for _ in range(3))
        slot = torch.full((S,), SENT16, dtype=torch.int16, device="cuda")
        stats = torch.zeros(16, dtype=torch.uint8, device="cuda")
        ws = (torch.empty(Z.zero_workspace_bytes(S), dtype=torch.uint8, device="cuda")
              if mode == "workspace" else None)
        a = Z.make_adam_args(replicas=reps, grad_dtype=Z.ZERO_BF16, p_in=p, m_in=m, v_in=v,
                             p_out=P, m_out=M, v_out=V, slot=slot, shard_S=S, buckets=buckets,
                             n_buckets=n_buckets, loss_scale=loss_scale, step_t=t, stats=stats,
                             workspace=ws, **hy)
        say(f"no-alloc {name}: {mode} S={S} N={len(reps)} buckets={n_buckets}")
        (Z.zero_adam_step if mode == "workspace" else Z.zero_adam_step_noalloc)(a)
        torch.cuda.synchronize()
        outs[mode] = (P, M, V, slot, Z.stats_from_tensor(stats))
        del ws
    (P0, M0, V0, s0, st0), (P1, M1, V1, s1, st1) = outs["workspace"], outs["noalloc"]
    for what, x, y in (("p", P0, P1), ("m", M0, M1), ("v", V0, V1), ("slot", s0, s1)):
        xb = x.view(torch.int32) if x.dtype == torch.float32 else x
        yb = y.view(torch.int32) if y.dtype == torch.float32 else y
        assert torch.equal(xb, yb), f"{name}: {what} differs between the two entry points"
        if inside is not None:
            sent = SENT32 if x.dtype == torch.float32 else SENT16
            assert bool(torch.all(xb[~inside] == sent)), f"{name}: {what} written outside the buckets"
    assert st1.overflow == st0.overflow and st1.bad_buckets == st0.bad_buckets == 0
    assert sumsq_close(st1.sumsq, st0.sumsq, 1e-9), (st1.sumsq, st0.sumsq)
    return st0


def test_noalloc_equals_workspace_entry_point(Z):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2024)
    # 1: long shard, grid capped by the scratch
    S = 98_305 * 1024 + 7
    reps = bf16_replicas(gen, S, 8, 1e-3)
    p = torch.randn(S, generator=gen, device="cuda").mul_(0.02)
    m = torch.randn(S, generator=gen, device="cuda").mul_(1e-4)
    v = torch.randn(S, generator=gen, device="cuda").mul_(1e-4).square_()
    st = run_pair(Z, "long shard", reps, S, p, m, v, loss_scale=1.0, t=4, wd=0.01)
    assert st.overflow == 0
    del reps, p, m, v
    torch.cuda.empty_cache()
    # 2: ragged shard over its bucket table, one +inf injected
    w = W.get("ragged")
    lay = oracle.Layout(w.numels, N=w.N, A=w.A, B=w.B)
    S = lay.S
    covered = [(int(s[2]), int(s[3])) for s in lay.segments(0)]
    h = Z.zero_layout_build(list(w.numels), w.N, w.A, w.B)
    raw, nb = Z.zero_layout_buckets_raw(h, 0, 4096)
    Z.zero_layout_free(h)
    bt = torch.frombuffer(bytearray(bytes(raw)[: 16 * nb]), dtype=torch.uint8).to("cuda")
    reps = []
    for j in range(w.N):
        r = torch.empty(S, dtype=torch.bfloat16, device="cuda")
        W.device_fill_replica(r, w, covered, 0, 1, j)
        reps.append(r.view(torch.int16))
    off, ln = max(covered, key=lambda c: c[1])
    reps[5][off + ln // 2] = 0x7F80                         # +inf in bf16, inside a bucket
    p = torch.randn(S, generator=gen, device="cuda").mul_(0.02)
    z = torch.zeros(S, dtype=torch.float32, device="cuda")
    inside = torch.zeros(S, dtype=torch.bool)
    for o, ln in np.frombuffer(bytes(raw)[: 16 * nb], dtype=np.dtype(
            [("off", "<i8"), ("len", "<i4"), ("t", "<i4")]))[["off", "len"]].tolist():
        inside[o:o + ln] = True
    st = run_pair(Z, "ragged buckets", reps, S, p, z, z, loss_scale=65536.0, t=1, wd=0.0,
                  buckets=bt, n_buckets=nb, inside=inside.to("cuda"))
    assert st.overflow == 1
    # 3: 300 replicas, the pointer table in the scratch
    S = 5003
    reps = bf16_replicas(gen, S, 300, 1e-3)
    p = torch.randn(S, generator=gen, device="cuda").mul_(0.02)
    m = torch.randn(S, generator=gen, device="cuda").mul_(1e-4)
    v = torch.randn(S, generator=gen, device="cuda").mul_(1e-4).square_()
    st = run_pair(Z, "300 replicas", reps, S, p, m, v, loss_scale=65536.0, t=2, wd=0.01)
    assert st.overflow == 0


def test_noalloc_rejects_a_workspace(Z):
    S = 64
    x = torch.zeros(S, dtype=torch.float32, device="cuda")
    outs = [torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(3)]
    stats = torch.zeros(16, dtype=torch.uint8, device="cuda")
    ws = torch.empty(Z.zero_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    a = Z.make_adam_args(grad_f32=x, p_in=x, m_in=x, v_in=x, p_out=outs[0], m_out=outs[1],
                         v_out=outs[2], shard_S=S, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                         weight_decay=0.0, step_t=1, stats=stats, workspace=ws)
    with pytest.raises(Z.ZeroError) as ei:
        Z.zero_adam_step_noalloc(a)
    assert ei.value.status == -1 and "workspace" in str(ei.value)
