"""Host-side tests of libzero (no GPU needed): the library loads and exports every
function include/zero.h declares; its layout, segments, buckets and memory
accounting equal the oracle's exactly; argument checks reject bad calls before
touching the GPU; the host commit rule follows the skip rule."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def Z():
    import zero_partitioned_optimizer_amd as Z
    Z.lib()
    return Z


def declared_functions():
    src = open(os.path.join(ROOT, "include", "zero.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(zero_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(Z):
    names = declared_functions()
    assert len(names) >= 15
    L = ctypes.CDLL(os.path.join(ROOT, "zero_partitioned_optimizer_amd", "libzero.so"))
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert Z.zero_version().startswith("libzero")


def lib_layout(Z, numels, N, A, B):
    h = Z.zero_layout_build(list(numels), N, A, B)
    try:
        info = Z.zero_layout_info_get(h)
        offs = Z.zero_layout_offsets(h)
        return h, info, offs
    except Exception:
        Z.zero_layout_free(h)
        raise


@pytest.mark.parametrize("seed", range(30))
def test_layout_equals_oracle_random(Z, seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(0, 40))
    numels = [int(x) for x in rng.integers(0, 3000, size=T)]
    N = int(rng.integers(1, 17))
    A = int(rng.choice([1, 2, 8, 256]))
    B = int(rng.choice([1, 8, 16]))
    ref = oracle.Layout(numels, N=N, A=A, B=B)
    h, info, offs = lib_layout(Z, numels, N, A, B)
    try:
        assert offs == ref.offsets.tolist()
        assert (info.used_L, info.shard_S, info.padded_L) == (ref.L, ref.S, ref.L_pad)
        assert info.psi == sum(numels) and info.world_N == N and info.n_tensors == T
        for r in range(N):
            assert [list(s) for s in Z.zero_layout_segments(h, r)] == ref.segments(r).tolist()
            for be in (1, 7, 64, 1000):
                assert [list(b) for b in Z.zero_layout_buckets(h, r, be)] == ref.buckets(r, be).tolist()
        for stage in range(4):
            assert Z.zero_layout_mem_values(h, stage) == ref.mem_values(stage).tolist()
            assert Z.zero_layout_mem_bytes(h, stage) == ref.mem_bytes(stage).tolist()
    finally:
        Z.zero_layout_free(h)


@pytest.mark.parametrize("name", ["tiny", "gpt2s", "llama7b", "ragged", "llama70b"])
def test_layout_equals_oracle_workloads(Z, name):
    w = W.get(name)
    ref = oracle.Layout(w.numels, N=w.N, A=w.A, B=w.B)
    h, info, offs = lib_layout(Z, w.numels, w.N, w.A, w.B)
    try:
        assert offs == ref.offsets.tolist()
        assert (info.used_L, info.shard_S, info.padded_L) == (ref.L, ref.S, ref.L_pad)
        ranks = range(w.N) if name in ("tiny",) else (0, w.N // 2, w.N - 1)
        for r in ranks:
            assert [list(s) for s in Z.zero_layout_segments(h, r)] == ref.segments(r).tolist()
        if ref.S <= 2_000_000:
            for r in ranks:
                assert ([list(b) for b in Z.zero_layout_buckets(h, r, 4096)] ==
                        ref.buckets(r, 4096).tolist())
        for stage in range(4):
            assert Z.zero_layout_mem_values(h, stage) == ref.mem_values(stage).tolist()
    finally:
        Z.zero_layout_free(h)


def test_bucket_struct_is_16_bytes_and_matches(Z):
    h = Z.zero_layout_build([3, 200, 300], 4, 256, 8)
    try:
        raw, n = Z.zero_layout_buckets_raw(h, 1, 64)
        arr = np.frombuffer(bytes(raw)[: 16 * n], dtype=np.dtype([("off", "<i8"), ("len", "<i4"),
                                                                   ("t", "<i4")]))
        assert [tuple(int(v) for v in x) for x in arr] == [tuple(b) for b in Z.zero_layout_buckets(h, 1, 64)]
    finally:
        Z.zero_layout_free(h)


def test_layout_errors(Z):
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_layout_build([1, 2], 0)
    assert e.value.status == -1
    with pytest.raises(Z.ZeroError):
        Z.zero_layout_build([1, -2], 2)
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_layout_build([2 ** 62, 2 ** 62], 2)
    assert e.value.status == -3
    h = Z.zero_layout_build([10], 2)
    try:
        with pytest.raises(Z.ZeroError) as e:
            Z.zero_layout_segments(h, 2)
        assert e.value.status == -3
        with pytest.raises(Z.ZeroError):
            Z.zero_layout_buckets(h, 0, 0)
        with pytest.raises(Z.ZeroError):
            Z.zero_layout_mem_values(h, 4)
        # capacity protocol: too small a capacity reports the count and ZERO_E_RANGE
        n = ctypes.c_int64()
        out = (Z.zero_segment * 1)()
        h2 = Z.zero_layout_build([4, 4, 4], 1)
        rc = Z.lib().zero_layout_segments(h2, 0, out, 1, ctypes.byref(n))
        assert rc == -3 and n.value == 3
        Z.zero_layout_free(h2)
    finally:
        Z.zero_layout_free(h)


FAKE = 1 << 40          # a 16-byte aligned address; validation fails before any use


def base_args(Z, **kw):
    S = kw.pop("shard_S", 64)
    d = dict(p_in=FAKE, m_in=FAKE + 4096, v_in=FAKE + 8192, p_out=FAKE + 12288,
             m_out=FAKE + 16384, v_out=FAKE + 20480, slot=FAKE + 24576, shard_S=S,
             lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step_t=1,
             stats=FAKE + 28672, workspace=FAKE + 32768)
    d.update(kw)
    a = Z.make_adam_args(**d)
    a.ws_bytes = Z.zero_workspace_bytes(S)
    return a


@pytest.mark.parametrize("change,status", [
    (dict(), -1),                                             # neither replicas nor grad_f32
    (dict(grad_f32=FAKE + 40960, replicas=[FAKE + 45056]), -1),   # both
    (dict(grad_f32=FAKE + 40960, p_in=FAKE + 8), -2),          # misaligned
    (dict(grad_f32=FAKE + 40960, p_in=0), -1),                 # NULL
    (dict(grad_f32=FAKE + 40960, beta1=1.0), -1),
    (dict(grad_f32=FAKE + 40960, step_t=0), -1),
    (dict(grad_f32=FAKE + 40960, eps=float("nan")), -1),
    (dict(grad_f32=FAKE + 40960, shard_S=-1), -3),
    (dict(replicas=[FAKE + 45056] * 1025), -3),                 # too many replicas
    (dict(replicas=[FAKE + 45056], loss_scale=0.0), -1),
    (dict(replicas=[FAKE + 45056], p_out=FAKE), -1),            # fused must be out of place
    (dict(grad_f32=FAKE + 40960, p_out=FAKE + 100), -2),        # misaligned output
    (dict(grad_f32=FAKE + 40960, p_out=FAKE + 64), -1),         # partial overlap with p_in
    (dict(grad_f32=FAKE + 40960, slot=FAKE + 12288 + 16), -1),  # slot overlaps p_out
    (dict(replicas=[FAKE + 45056], m_out=FAKE + 45056), -1),    # output overlaps a replica
    (dict(grad_f32=FAKE + 40960, n_buckets=3), -1),             # bucket count without table
])
def test_adam_step_validation(Z, change, status):
    a = base_args(Z, **change)
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_adam_step(a, stream=0)
    assert e.value.status == status, str(e.value)
    assert Z.zero_last_error()


@pytest.mark.parametrize("change,status", [
    (dict(), -1), (dict(grad_f32=FAKE + 40960, p_in=FAKE + 8), -2),
    (dict(grad_f32=FAKE + 40960, step_t=0), -1), (dict(replicas=[FAKE + 45056] * 1025), -3),
    (dict(replicas=[FAKE + 45056], p_out=FAKE), -1), (dict(grad_f32=FAKE + 40960, stats=0), -1),
])
def test_adam_step_noalloc_validation(Z, change, status):
    """The allocation-free step checks its arguments like zero_adam_step, on the
    host, before it looks up its scratch or touches the GPU."""
    a = base_args(Z, **change)
    a.workspace_dev, a.ws_bytes = None, 0
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_adam_step_noalloc(a, stream=0)
    assert e.value.status == status, str(e.value)


def test_adam_step_noalloc_refuses_a_workspace(Z):
    a = base_args(Z, grad_f32=FAKE + 40960)
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_adam_step_noalloc(a, stream=0)
    assert e.value.status == -1 and "takes no workspace" in Z.zero_last_error()
    a.workspace_dev, a.ws_bytes = None, 64
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_adam_step_noalloc(a, stream=0)
    assert e.value.status == -1
    assert Z.ZERO_NOALLOC_SCRATCH_BYTES == 65536 * 24 + 8 * 1024 + 16


def test_adam_step_small_workspace_rejected(Z):
    a = base_args(Z, grad_f32=FAKE + 40960)
    a.ws_bytes = 8
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_adam_step(a, stream=0)
    assert e.value.status == -3


def test_workspace_holds_the_pointer_table(Z):
    # more than 256 replicas: the workspace must also hold their device pointer
    # table (8 bytes each, at its end); enough room for the partials alone is not
    S = 64                                 # one workgroup: 24 bytes of partials
    table = [FAKE + (1 << 20) + 256 * j for j in range(300)]
    for ws in (24, 24 + 8 * 300):          # partials only; no room for the alignment slack
        a = base_args(Z, replicas=table, loss_scale=1.0)
        a.ws_bytes = ws
        with pytest.raises(Z.ZeroError) as e:
            Z.zero_adam_step(a, stream=0)
        assert e.value.status == -3 and "workspace" in Z.zero_last_error()
    assert Z.zero_workspace_bytes(S) >= (4096 + 1) * 24 + 8 * 1024 + 16


def test_reduce_and_gather_validation(Z):
    L = Z.lib()
    tbl = (ctypes.c_void_p * 2)(FAKE, FAKE + 8)
    ws = Z.zero_workspace_bytes(64)
    assert L.zero_reduce_shard(tbl, 2, 1, 64, None, 0, 1.0, None, FAKE + 4096, FAKE + 8192, ws, None) == -2
    tbl = (ctypes.c_void_p * 2)(FAKE, FAKE + 256)
    assert L.zero_reduce_shard(tbl, 0, 1, 64, None, 0, 1.0, None, FAKE + 4096, FAKE + 8192, ws, None) == -3
    assert L.zero_reduce_shard(tbl, 2, 7, 64, None, 0, 1.0, None, FAKE + 4096, FAKE + 8192, ws, None) == -1
    assert L.zero_reduce_shard(tbl, 2, 1, 64, None, 0, -1.0, None, FAKE + 4096, FAKE + 8192, ws, None) == -1
    assert L.zero_reduce_shard(tbl, 2, 1, 64, None, 0, 1.0, FAKE + 64, FAKE + 4096, FAKE + 8192, ws, None) == -1
    assert L.zero_reduce_shard(tbl, 2, 1, 64, None, 0, 1.0, None, None, FAKE + 8192, ws, None) == -1
    # stats inside a replica, workspace over stats, workspace over the bucket table
    assert L.zero_reduce_shard(tbl, 2, 1, 64, None, 0, 1.0, None, FAKE + 16, FAKE + 8192, ws, None) == -1
    assert L.zero_reduce_shard(tbl, 2, 1, 64, None, 0, 1.0, None, FAKE + 8192, FAKE + 8192 - 16, ws,
                               None) == -1
    assert L.zero_reduce_shard(tbl, 2, 1, 64, FAKE + 8192 + 64, 2, 1.0, None, FAKE + 4096, FAKE + 8192,
                               ws, None) == -1
    assert L.zero_gather_slot(FAKE, 64, FAKE + 8, None) == -2
    assert L.zero_gather_slot(FAKE, 64, FAKE + 64, None) == -1
    assert L.zero_gather_slot(None, 64, FAKE, None) == -1
    assert L.zero_gather_slot(FAKE, -1, FAKE + 4096, None) == -3
    assert L.zero_gather_slot(FAKE, 0, FAKE + 4096, None) == 0     # empty: nothing to launch


def test_commit_rule_matches_oracle_trainer(Z):
    st = Z.zero_train_state(t=0, n_skipped=0, loss_scale=65536.0, min_loss_scale=1.0, dynamic=1)
    flags = [0, 1, 1, 0, 1]
    verdicts = []
    for f in flags:
        verdicts.append(Z.zero_commit_rule(st, Z.zero_stats(overflow=f, bad_buckets=0, sumsq=0.0)))
    assert verdicts == [1, 2, 2, 1, 2]
    assert st.t == 2 and st.n_skipped == 3 and st.loss_scale == 8192.0
    st = Z.zero_train_state(t=5, n_skipped=0, loss_scale=2.0, min_loss_scale=1.0, dynamic=1)
    for _ in range(3):
        Z.zero_commit_rule(st, Z.zero_stats(overflow=1))
    assert st.loss_scale == 1.0 and st.t == 5
    st = Z.zero_train_state(t=0, n_skipped=0, loss_scale=4.0, min_loss_scale=1.0, dynamic=0)
    Z.zero_commit_rule(st, Z.zero_stats(overflow=1))
    assert st.loss_scale == 4.0


def test_train_step_validation(Z):
    FAKEREC = FAKE + 65536
    base = dict(replicas=[FAKE + 45056], grad_dtype=1, p=(FAKE, FAKE + 4096), m=(FAKE + 8192, FAKE + 12288),
                v=(FAKE + 16384, FAKE + 20480), slot=FAKE + 24576, shard_S=64, lr=1e-3, eps=1e-8,
                weight_decay=0.0, state=FAKEREC, stats=FAKE + 28672, workspace=FAKE + 32768)
    def call(**kw):
        d = dict(base)
        d.update(kw)
        a = Z.make_train_args(**d)
        a.ws_bytes = 4096                   # enough for S = 64; ends below the replica
        with pytest.raises(Z.ZeroError) as e:
            Z.zero_train_step(a, stream=0)
        return e.value.status
    assert call(state=0) == -1
    assert call(state=FAKEREC + 8) == -2
    assert call(p=(FAKE, FAKE)) == -1                      # both sets alias
    assert call(m=(FAKE + 8192, FAKE + 8192 + 64)) == -1   # partial overlap
    assert call(slot=FAKE + 4096 + 32) == -1               # slot inside p[1]
    assert call(slot=(FAKE + 24576, FAKE + 24576 + 64)) == -1   # the two slots overlap
    assert call(slot=(0, FAKE + 24576)) == -1              # slot[1] without slot[0]
    assert call(replicas=[FAKE + 4096]) == -1              # replica overlaps p[1]
    assert call(lr=-1.0) == -1
    assert call(replicas=[]) == -3
    assert call(p=(FAKE + 4, FAKE + 4096)) == -2
    L = Z.lib()
    WS = FAKE + 32768
    assert L.zero_device_state_init(None, WS, 4096, 0.9, 0.999, 1.0, 1.0, 0, None) == -1
    assert L.zero_device_state_init(FAKEREC, None, 4096, 0.9, 0.999, 1.0, 1.0, 0, None) == -1
    assert L.zero_device_state_init(FAKEREC + 4, WS, 4096, 0.9, 0.999, 1.0, 1.0, 0, None) == -2
    assert L.zero_device_state_init(FAKEREC, WS, 4096, 0.9, 1.5, 1.0, 1.0, 0, None) == -1
    assert L.zero_device_state_init(FAKEREC, WS, 4096, 0.9, 0.999, float("inf"), 1.0, 0, None) == -1
    assert L.zero_device_state_init(FAKEREC, FAKEREC - 64, 4096, 0.9, 0.999, 1.0, 1.0, 0, None) == -1



def test_device_state_load_validation(Z):
    """Rejections happen on the host, before anything is enqueued."""
    L = Z.lib()
    REC, WS = FAKE + 65536, FAKE + 32768
    good = dict(beta1=0.9, beta2=0.999, beta1_pow=0.9 ** 3, beta2_pow=0.999 ** 3, loss_scale=1024.0,
                min_loss_scale=1.0, last_sumsq=0.5, t=3, n_skipped=1, cur=1, dynamic=1,
                last_overflow=0, seq=4)

    def status(state=REC, ws=WS, **kw):
        d = dict(good)
        d.update(kw)
        rec = Z.zero_device_state(**d)
        return L.zero_device_state_load(state, ws, 4096, ctypes.byref(rec), None)

    assert L.zero_device_state_load(REC, WS, 4096, None, None) == -1
    assert status(state=None) == -1
    assert status(state=REC + 8) == -2
    assert status(ws=REC - 64) == -1                   # workspace overlaps the record
    assert status(beta1=1.0) == -1
    assert status(loss_scale=0.5) == -1                # below min_loss_scale
    assert status(loss_scale=float("nan")) == -1
    assert status(t=-1) == -1
    assert status(n_skipped=-2) == -1
    assert status(cur=2) == -1
    assert status(last_overflow=3) == -1
    assert status(beta2_pow=1.5) == -1
    assert status(beta1_pow=float("nan")) == -1
    assert status(t=0) == -1                           # beta^0 must be 1
    assert status(pending_n=3) == -1                   # saved without a flush
    assert status(error=Z.ZERO_RECORD_E_COLLECT) == -1 # frozen by a wait that ran out
    assert status(error=Z.ZERO_RECORD_E_MARKS) == -1


def test_device_state_flush_validation(Z):
    """zero_device_state_flush checks its buffers on the host before enqueuing."""
    L = Z.lib()
    REC, STATS, WS = FAKE + 65536, FAKE + 69632, FAKE + (1 << 20)
    wsb = Z.zero_workspace_bytes(64)
    assert L.zero_device_state_flush(None, STATS, WS, wsb, None) == -1
    assert L.zero_device_state_flush(REC, None, WS, wsb, None) == -1
    assert L.zero_device_state_flush(REC, STATS, None, wsb, None) == -1
    assert L.zero_device_state_flush(REC + 8, STATS, WS, wsb, None) == -2
    assert L.zero_device_state_flush(REC, STATS + 4, WS, wsb, None) == -2
    assert L.zero_device_state_flush(REC, STATS, WS, 4096, None) == -3      # too small for any step
    assert L.zero_device_state_flush(REC, REC + 16, WS, wsb, None) == -1    # stats inside the record
    assert L.zero_device_state_flush(REC, WS + 64, WS, wsb, None) == -1     # stats inside the workspace


def test_workspace_layout_sizes(Z):
    """A device-committed record's workspace holds, per workgroup slot, the partials
    of two consecutive steps (2 x 24 bytes) and a start mark (8 bytes), then 64
    bytes of flag words and the replica pointer table."""
    for S in (1, 1024, 15_554_976, 842_301_952):
        slots = min((S + 1023) // 1024 + 4096, 4_194_304)
        assert Z.zero_workspace_bytes(S) == slots * 56 + 64 + 8 * 1024 + 16


def test_train_step_part_validation(Z):
    """Part tables are checked on the host before anything is enqueued."""
    FAKEREC = FAKE + 65536
    S = 64
    a = Z.make_train_args(replicas=[FAKE + 45056], grad_dtype=1, p=(FAKE, FAKE + 4096),
                          m=(FAKE + 8192, FAKE + 12288), v=(FAKE + 16384, FAKE + 20480),
                          slot=FAKE + 24576, shard_S=S, lr=1e-3, eps=1e-8, weight_decay=0.0,
                          state=FAKEREC, stats=FAKE + 28672, workspace=FAKE + 32768)
    a.ws_bytes = 4096

    def status(ends, part=0, n=None, args=a):
        tbl, cnt = Z.part_table(ends)
        with pytest.raises(Z.ZeroError) as e:
            Z.zero_train_step_part(args, tbl, cnt if n is None else n, part, stream=0)
        return e.value.status

    assert status([32, 60]) == -3            # last end is not shard_S
    assert status([12, 64]) == -3            # inner end not a multiple of 8
    assert status([40, 32, 64]) == -3        # decreasing
    assert status([-8, 64]) == -3
    assert status([32, 64], part=2) == -3    # part out of range
    assert status([32, 64], part=-1) == -3
    assert status([32, 64], n=0) == -3
    assert Z.lib().zero_train_step_part(ctypes.byref(a), None, 2, 0, None) == -1
    b = Z.make_train_args(replicas=[FAKE + 45056], grad_dtype=1, p=(FAKE, FAKE + 4096),
                          m=(FAKE + 8192, FAKE + 12288), v=(FAKE + 16384, FAKE + 20480),
                          slot=FAKE + 24576, shard_S=S, lr=1e-3, eps=1e-8, weight_decay=0.0,
                          state=FAKEREC, stats=FAKE + 28672, workspace=FAKE + 32768,
                          buckets=FAKE + 50000 - 50000 % 16, n_buckets=2)
    b.ws_bytes = 4096
    assert status([32, 64], args=b) == -6    # bucket tables are not split into parts
    a.lr = -1.0
    assert status([32, 64]) == -1            # the whole-step checks apply too


def test_gather_tensors_validation(Z):
    L = Z.lib()
    sh = (ctypes.c_void_p * 2)(FAKE, FAKE + 4096)
    offs = (ctypes.c_int64 * 2)(0, 10)
    nums = (ctypes.c_int64 * 2)(10, 20)
    outs = (ctypes.c_void_p * 2)(FAKE + 8192, FAKE + 12288)

    def call(shards=sh, n_shards=2, S=64, eb=2, o=offs, n=nums, out=outs, k=2):
        return L.zero_gather_tensors(shards, n_shards, S, eb, o, n, out, k, None)

    assert call(shards=None) == -1
    assert call(n_shards=0) == -3
    assert call(n_shards=300) == -3
    assert call(S=0) == -3
    assert call(eb=3) == -1
    assert call(k=-1) == -3
    assert call(o=None) == -1
    assert call(o=(ctypes.c_int64 * 2)(0, 120)) == -3           # 120 + 20 > 2 * 64
    assert call(n=(ctypes.c_int64 * 2)(10, -1)) == -3
    assert call(out=(ctypes.c_void_p * 2)(FAKE + 8192, FAKE + 12289)) == -2
    assert call(out=(ctypes.c_void_p * 2)(FAKE + 8192, FAKE + 8200)) == -1     # outs overlap
    assert call(out=(ctypes.c_void_p * 2)(FAKE + 8192, FAKE + 4100)) == -1     # out in a shard
    assert call(shards=(ctypes.c_void_p * 2)(FAKE, FAKE + 4097)) == -2
    assert call(k=0) == 0                                                      # nothing to do


def test_offload_step_validation(Z):
    """Checks that reject an offloaded step before any device work is enqueued."""
    L = Z.lib()
    st = Z.zero_train_state(t=0, n_skipped=0, loss_scale=1.0, min_loss_scale=1.0, dynamic=0)
    tbl = (ctypes.c_void_p * 1)(FAKE + 45056)

    def args(**kw):
        a = Z.zero_offload_args()
        a.replicas = ctypes.cast(tbl, ctypes.POINTER(ctypes.c_void_p))
        a.n_replicas, a.grad_dtype, a.shard_S = 1, 1, 64
        a.g_dev, a.g_host, a.p_host, a.m_host, a.v_host = FAKE, FAKE + 4096, FAKE + 8192, FAKE + 12288, FAKE + 16384
        a.slot_host, a.slot_dev = FAKE + 20480, FAKE + 24576
        a.lr, a.beta1, a.beta2, a.eps, a.weight_decay = 1e-3, 0.9, 0.999, 1e-8, 0.0
        a.state = ctypes.pointer(st)
        a.stats_dev, a.workspace_dev, a.ws_bytes = FAKE + 28672, FAKE + 32768, 4096
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    def status(**kw):
        return L.zero_offload_step(ctypes.byref(args(**kw)), None, None)

    assert L.zero_offload_step(None, None, None) == -1
    assert status(state=None) == -1
    assert status(stats_dev=None) == -1
    assert status(g_host=None) == -1
    assert status(slot_dev=None) == -1
    assert status(chunk_elems=-5) == -3
    assert status(beta1=1.5) == -1
    assert status(lr=float("nan")) == -1
    assert status(n_replicas=0) == -3          # from the reduce's own checks
    assert st.t == 0 and st.n_skipped == 0      # nothing was committed


def test_state_layout_sizes(Z):
    T = Z.ZERO_STATE_TILE
    assert T == 8192
    for S in (0, 1, 8191, 8192, 8193, 10**9 + 7):
        assert Z.zero_state_set_floats(S, Z.ZERO_STATE_SPLIT) == 3 * S
        assert Z.zero_state_set_floats(S, Z.ZERO_STATE_TILED) == 3 * ((S + T - 1) // T) * T
    assert Z.lib().zero_state_set_floats(-1, Z.ZERO_STATE_TILED) == -1
    assert Z.lib().zero_state_set_floats(10, 2) == -1


def test_state_layout_validation(Z):
    """Tiled-state arguments are checked on the host before anything is enqueued:
    the layout value, NULL m and v pointers, and overlaps over the whole set buffer
    (3 * ZERO_STATE_TILE floats for a 64-element shard, 96 KiB)."""
    big = 1 << 20                                # beyond one tiled set of S = 64
    tiled = dict(p_in=FAKE, m_in=0, v_in=0, p_out=FAKE + big, m_out=0, v_out=0,
                 slot=FAKE + 2 * big, stats=FAKE + 2 * big + 4096, workspace=FAKE + 2 * big + 8192,
                 state_layout=Z.ZERO_STATE_TILED)

    def adam(**kw):
        d = dict(tiled)
        d.update(kw)
        a = base_args(Z, **d)
        with pytest.raises(Z.ZeroError) as e:
            Z.zero_adam_step(a, stream=0)
        return e.value.status

    rep = [FAKE + 3 * big]
    assert adam(replicas=rep, state_layout=2) == -1                 # unknown layout
    assert adam(replicas=rep, m_in=FAKE + 4 * big) == -1            # m given with a tiled state
    assert adam(replicas=rep, v_out=FAKE + 4 * big) == -1
    assert adam(replicas=rep, p_out=FAKE + 4096) == -1              # p_out inside the p_in set
    assert adam(replicas=rep, slot=FAKE + big + 90000) == -1        # slot inside the p_out set
    assert adam(replicas=[FAKE + big + 50000 - 50000 % 16]) == -1   # replica inside the p_out set
    assert adam(grad_f32=FAKE + 3 * big, p_out=FAKE + 64) == -1     # partial in-place overlap
    assert adam(replicas=rep, p_in=FAKE + 8) == -2

    FAKEREC = FAKE + 5 * big
    tbase = dict(replicas=[FAKE + 3 * big], grad_dtype=1, p=(FAKE, FAKE + big), m=(0, 0), v=(0, 0),
                 slot=FAKE + 2 * big, shard_S=64, lr=1e-3, eps=1e-8, weight_decay=0.0,
                 state=FAKEREC, stats=FAKE + 2 * big + 4096, workspace=FAKE + 2 * big + 8192,
                 state_layout=Z.ZERO_STATE_TILED)

    def train(**kw):
        d = dict(tbase)
        d.update(kw)
        a = Z.make_train_args(**d)
        a.ws_bytes = 4096
        with pytest.raises(Z.ZeroError) as e:
            Z.zero_train_step(a, stream=0)
        return e.value.status

    assert train(p=(FAKE, FAKE + 4096)) == -1                        # the two sets overlap
    assert train(m=(FAKE + 4 * big, FAKE + 4 * big + 4096)) == -1    # m given with a tiled state
    assert train(state_layout=-1) == -1
    assert train(p=(FAKE, 0)) == -1
    # parts of a tiled step start on tiles
    a = Z.make_train_args(**dict(tbase, shard_S=20000, stats=FAKE + 2 * big + 65536,
                                 workspace=FAKE + 2 * big + 131072))
    a.ws_bytes = 1 << 16
    tbl, cnt = Z.part_table([8000, 20000])
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_train_step_part(a, tbl, cnt, 0, stream=0)
    assert e.value.status == -3 and "8192" in Z.zero_last_error()


def test_state_convert_validation(Z):
    L = Z.lib()
    S = 100
    SET, P, M, V = FAKE, FAKE + (1 << 20), FAKE + (1 << 20) + 4096, FAKE + (1 << 20) + 8192
    assert L.zero_state_pack(P, M, V, S, None, None) == -1
    assert L.zero_state_pack(P, None, V, S, SET, None) == -1          # pack needs all three
    assert L.zero_state_pack(P, M, V, S, SET + 4, None) == -2
    assert L.zero_state_pack(P, M, V, -1, SET, None) == -3
    assert L.zero_state_pack(SET + 4096, M, V, S, SET, None) == -1    # p inside the set
    assert L.zero_state_pack(P, P + 64, V, S, SET, None) == -1        # p and m overlap
    assert L.zero_state_unpack(SET, S, P, M, SET + 90000, None) == -1  # v inside the set
    assert L.zero_state_unpack(SET, S, P + 8, M, V, None) == -2
    assert L.zero_gather_slot_tiled(SET, S, SET + 90000, None) == -1  # slot inside the set
    assert L.zero_gather_slot_tiled(SET, -5, P, None) == -3
    assert L.zero_gather_slot_tiled(SET + 2, S, P, None) == -2
