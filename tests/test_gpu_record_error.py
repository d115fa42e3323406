"""A device-committed record frozen by a bounded wait that ran out.

The host removes the pending step's tagged partials from the workspace (it
clears the workspace between two steps), so the next launch's workgroup 0 polls
for them until its 2 s bound and gives up; every kernel still exits normally.
That launch must freeze the record (error code, nothing else changed), later
steps and flushes must change nothing, the host must see the error, the state
set the frozen record's pending step names must still hold that step's result,
and a checkpoint taken earlier must resume the run exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import NTHREADS, check_state, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S,N", [(20_011, 4), ((1 << 22) + 517, 16)])
def test_collect_timeout_freezes_record(Z, S, N):
    rng = np.random.default_rng(7 + N)
    p0 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    reps = [[np.asarray(W._bf16_bits_from_f32(rng.standard_normal(S) * 1e-3)) for _ in range(N)]
            for _ in range(3)]
    hy = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    step = Z.DeviceShardStep(S, N, Z.ZERO_BF16, to_dev(p0), weight_decay=0.01, loss_scale=1.0,
                             double_slot=True, **hy)
    tr = oracle.Trainer(p0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32),
                        oracle.f32_to_bf16(p0), loss_scale=1.0, dynamic=False, wd=0.01,
                        nthreads=NTHREADS, **hy)
    d = [[to_dev(r) for r in rs] for rs in reps]
    say("record error: step 1, checkpoint")
    step.step(d[0])
    tr.step(reps[0])
    sd = step.state_dict()                     # flushed: record after step 1, nothing pending
    say("record error: step 2 (pending), then its partials cleared")
    step.step(d[1])
    tr.step(reps[1])
    step.ws.zero_()                            # the pending step's tagged partials are gone
    say("record error: step 3 (its fold waits 2 s and gives up)")
    step.step(d[2])
    torch.cuda.synchronize()
    snap = [x.clone() for x in (step.p[0], step.p[1], step.m[0], step.m[1], step.v[0], step.v[1],
                                step.slot, step.slot_alt, step.record, step.stats, step.ws)]
    say("record error: step 4 on the frozen record, flush")
    step.step(d[2])
    with pytest.raises(Z.ZeroRecordError) as ei:
        step.state()
    assert ei.value.code == Z.ZERO_RECORD_E_COLLECT
    after = (step.p[0], step.p[1], step.m[0], step.m[1], step.v[0], step.v[1], step.slot,
             step.slot_alt, step.record, step.stats, step.ws)
    for k, (x, y) in enumerate(zip(snap, after)):
        if k == 9:
            continue                           # stats: rewritten with the same error marker
        assert torch.equal(x, y), f"buffer {k} changed on a frozen record"
    rec = step.state(check=False)
    assert rec.error == Z.ZERO_RECORD_E_COLLECT
    assert rec.seq == 1 and rec.t == 1 and rec.n_skipped == 0 and rec.pending_n > 0
    st = Z.stats_from_tensor(step.stats)
    assert st.overflow == 1 and st.bad_buckets == 0xFFFFFFFF and np.isnan(st.sumsq)
    # the frozen record still names step 2's output: the pending step was clean, so
    # the set after the record's current one holds it, with its slot
    c = (rec.cur ^ 1) & 1
    P, M, V = step.set_state(c)
    slot = step.slot_alt if c else step.slot
    check_state("state named by the frozen record", to_host(P), to_host(M), to_host(V),
                to_host(slot), tr.p, tr.m, tr.v, tr.slot)
    # resuming from the checkpoint clears the error; steps 2 and 3 then match the oracle
    say("record error: resume from the checkpoint after step 1")
    step.load_state_dict(sd)
    step.step(d[1])
    step.step(d[2])
    tr.step(reps[2])
    rec = step.state()
    assert rec.error == 0 and rec.t == 3 and rec.seq == 2
    P, M, V = step.committed()
    check_state("resumed", to_host(P), to_host(M), to_host(V), to_host(step.current_slot()),
                tr.p, tr.m, tr.v, tr.slot)
