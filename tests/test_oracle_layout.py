"""Pins of the oracle's flat layout, shard cut, segments and buckets.

The layout follows the partitioning the pages describe: one contiguous flat
buffer ("Why does not the stage 3 implementation use broadcast and
reduce-scatter?", replies on contiguous gradients), cut into N equal rank
partitions whose gradient slice matches the rank's optimizer-state and
parameter slice ("[REQUEST] Direct Correspondence between Gradient and
Optimizer States to Reduce Communication", section "Problem"), with small
tensors grouped into buckets ("ZeRO Optimizer", "Communication Optimization").

Pins: a hand-derived worked example, closed-form invariants, and a brute-force
element-by-element placement that shares no formula with the oracle.
"""
import numpy as np
import pytest


def brute_layout(numels, N, A, B):
    """Place tensors one element at a time; grow the shard until N shards cover L."""
    pos, offsets, owner = 0, [], []
    for i, n in enumerate(numels):
        if i > 0:
            while pos % A:
                owner.append(-1)
                pos += 1
        offsets.append(pos)
        owner.extend([i] * n)
        pos += n
    L = pos
    S = 0
    while N * S < L:
        S += B
    owner.extend([-1] * (N * S - L))
    return offsets, L, S, owner


def test_tiny_worked_example(orc):
    # Hand-derived: sizes [1000, 2048, 1000], A=1, B=8, N=2.
    # offsets 0, 1000, 3048; L = 4048; ceil(4048/2) = 2024 is a multiple of 8 -> S = 2024.
    lay = orc.Layout([1000, 2048, 1000], N=2, A=1, B=8)
    assert list(lay.offsets) == [0, 1000, 3048]
    assert (lay.L, lay.S, lay.L_pad) == (4048, 2024, 4048)
    # rank 0 window [0, 2024): all of tensor 0, the first 1024 of tensor 1
    assert lay.segments(0).tolist() == [[0, 0, 0, 1000], [1, 0, 1000, 1024]]
    # rank 1 window [2024, 4048): the last 1024 of tensor 1, all of tensor 2
    assert lay.segments(1).tolist() == [[1, 1024, 0, 1024], [2, 0, 1024, 1000]]
    # no padding: one bucket per rank without cuts
    assert lay.buckets(0, 0).tolist() == [[0, 2024, 0]]
    assert lay.buckets(1, 0).tolist() == [[0, 2024, 1]]
    # cut at multiples of 512 within the shard
    assert lay.buckets(1, 512).tolist() == [[0, 512, 1], [512, 512, 1], [1024, 512, 2],
                                            [1536, 488, 2]]


def test_tiny_three_ranks_has_tail_padding(orc):
    # ceil(4048/3) = 1350 -> S = 1352 (next multiple of 8), L_pad = 4056: 8 padding elements.
    lay = orc.Layout([1000, 2048, 1000], N=3, A=1, B=8)
    assert (lay.L, lay.S, lay.L_pad) == (4048, 1352, 4056)
    # rank 2 window [2704, 4056): tensor 1 from its element 2704 - 1000 = 1704 to 3048,
    # then all of tensor 2 ending at 4048, then 8 padding elements
    assert lay.segments(2).tolist() == [[1, 1704, 0, 344], [2, 0, 344, 1000]]
    assert lay.buckets(2, 0).tolist() == [[0, 1344, 1]]
    covered = sum(int(s[3]) for r in range(3) for s in lay.segments(r))
    assert covered == 4048 and lay.L_pad - covered == 8


def test_alignment_padding_between_tensors(orc):
    # A = 256: tensor starts at 0, 256 (after 3 elements), 512 (after 200 + 256 pad start)
    lay = orc.Layout([3, 200, 300], N=4, A=256, B=8)
    assert list(lay.offsets) == [0, 256, 512]
    assert lay.L == 812
    assert lay.S == 208 and lay.L_pad == 832          # ceil(812/4) = 203 -> 208
    segs = np.concatenate([lay.segments(r) for r in range(4)])
    assert segs[:, 3].sum() == 503


def test_empty_and_degenerate(orc):
    lay = orc.Layout([], N=4, A=1, B=8)
    assert (lay.L, lay.S, lay.L_pad) == (0, 0, 0)
    assert len(lay.segments(0)) == 0 and len(lay.buckets(0, 16)) == 0
    lay = orc.Layout([0, 0, 5], N=1, A=4, B=1)
    assert list(lay.offsets) == [0, 0, 0] and (lay.L, lay.S) == (5, 5)
    lay = orc.Layout([7], N=1, A=1, B=8)
    assert (lay.L, lay.S, lay.L_pad) == (7, 8, 8)
    with pytest.raises(ValueError):
        orc.Layout([1, 2], N=0)
    with pytest.raises(ValueError):
        orc.Layout([1, -2], N=2)


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_element_map(orc, seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(0, 12))
    numels = [int(x) for x in rng.integers(0, 60, size=T)]
    N = int(rng.integers(1, 9))
    A = int(rng.choice([1, 2, 3, 8, 16]))
    B = int(rng.choice([1, 4, 8]))
    offsets, L, S, owner = brute_layout(numels, N, A, B)
    lay = orc.Layout(numels, N=N, A=A, B=B)
    assert list(lay.offsets) == offsets
    assert (lay.L, lay.S, lay.L_pad) == (L, S, N * S)
    # segments reproduce the element -> tensor map exactly, each element once
    seen = np.full(N * S, -1)
    for r in range(N):
        for t, toff, soff, ln in lay.segments(r).tolist():
            assert ln > 0
            g0 = r * S + soff
            assert np.all(seen[g0:g0 + ln] == -1)
            seen[g0:g0 + ln] = t
            assert offsets[t] + toff == g0
    assert seen.tolist() == owner
    # buckets: cover exactly the non-padding elements, never cross a cut point
    for be in (0, 1, 5, 16):
        for r in range(N):
            bk = lay.buckets(r, be)
            mask = np.zeros(S, dtype=bool)
            prev_end = None
            for off, ln, t in bk.tolist():
                assert ln > 0
                assert not mask[off:off + ln].any()
                mask[off:off + ln] = True
                assert owner[r * S + off] == t
                if be > 0:
                    assert off // be == (off + ln - 1) // be
                if prev_end is not None and prev_end == off:
                    # adjacent buckets are only ever split at a cut point
                    assert be > 0 and off % be == 0
                prev_end = off + ln
            want = np.array(owner[r * S:(r + 1) * S]) >= 0
            assert (mask == want).all()


@pytest.mark.parametrize("N,A,B", [(2, 1, 8), (8, 1, 8), (64, 256, 8), (5, 3, 4)])
def test_closed_form_invariants(orc, N, A, B):
    rng = np.random.default_rng(N * 1000 + A)
    numels = [int(x) for x in rng.integers(1, 5000, size=50)]
    lay = orc.Layout(numels, N=N, A=A, B=B)
    assert all(o % A == 0 for o in lay.offsets)
    assert lay.S % B == 0
    assert lay.L_pad >= lay.L
    assert lay.S - (lay.L + N - 1) // N < B       # minimal multiple of B
    assert lay.L == lay.offsets[-1] + numels[-1]


def test_workload_tensor_lists_closed_forms():
    import workloads as W
    # GPT-2 small: V*d + ctx*d + L*(12 d^2 + 13 d) + 2 d
    d = 768
    assert W.get("gpt2s").psi == 50257 * d + 1024 * d + 12 * (12 * d * d + 13 * d) + 2 * d
    assert len(W.get("gpt2s").numels) == 148
    # Llama-7B: 2 V d + L (4 d^2 + 3 d f + 2 d) + d
    d, f = 4096, 11008
    assert W.get("llama7b").psi == 2 * 32000 * d + 32 * (4 * d * d + 3 * d * f + 2 * d) + d
    assert len(W.get("llama7b").numels) == 291
    # Llama-70B with kv dim 1024: 2 V d + L (2 d^2 + 2 d kv + 3 d f + 2 d) + d
    d, f, kv = 8192, 28672, 1024
    assert W.get("llama70b").psi == 2 * 32000 * d + 80 * (2 * d * d + 2 * d * kv + 3 * d * f + 2 * d) + d
    assert len(W.get("llama70b").numels) == 723
    rg = W.get("ragged")
    assert len(rg.numels) == 10_000 and min(rg.numels) >= 1 and max(rg.numels) <= 65536
    assert rg.psi % 64 != 0


def test_workload_shards(orc):
    import workloads as W
    want = {"tiny": 2024, "gpt2s": 15_554_976, "llama7b": 842_301_952, "llama70b": 2_155_520_256}
    for name, S in want.items():
        w = W.get(name)
        lay = orc.Layout(w.numels, N=w.N, A=w.A, B=w.B)
        assert lay.S == S
        assert lay.L_pad == lay.L       # these divide evenly: no padding
    w = W.get("ragged")
    lay = orc.Layout(w.numels, N=w.N, A=w.A, B=w.B)
    assert lay.L_pad > lay.L > w.psi
