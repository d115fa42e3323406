"""Pins of the stage-3 fetch (gather one tensor from the rank shards).

"ZeRO Optimizer", "ZeRO Stages" (stage 3 partitions the parameters too) and
"Communication Patterns" (parameters are all-gathered before each layer, only
the required subset): tensor t occupies [o_t, o_t + n_t) of the flat buffer, and
rank r holds [r*S, (r+1)*S) of it. Pinned against the ring all-gather simulator
(every rank ends with the whole buffer by message passing) and against a round
trip through the layout's segments (scatter each tensor's pieces into the
shards the segments name, gather back by flat offset).
"""
import numpy as np
import pytest


@pytest.mark.parametrize("N", [1, 2, 3, 8])
def test_gather_equals_ring_all_gather_slices(orc, N):
    rng = np.random.default_rng(40 + N)
    numels = rng.integers(1, 40, size=12)
    lay = orc.Layout(numels, N=N, A=1, B=8)
    chunks = rng.standard_normal((N, lay.S)).astype(np.float32)
    gathered, _, _ = orc.ring_all_gather(chunks)
    shards = [chunks[r].copy() for r in range(N)]
    for t, (o, n) in enumerate(zip(lay.offsets, numels)):
        got = orc.gather_tensor(shards, int(o), int(n))
        for k in range(N):                      # every rank's gathered copy agrees
            assert np.array_equal(got.view(np.uint32), gathered[k, o:o + n].view(np.uint32)), t


@pytest.mark.parametrize("seed,A", [(0, 1), (1, 1), (2, 256), (3, 8)])
def test_round_trip_through_segments(orc, seed, A):
    """Scatter each tensor into the shards via the segment lists, gather it back."""
    rng = np.random.default_rng(seed)
    numels = rng.integers(1, 3000, size=30)
    N = int(rng.integers(2, 9))
    lay = orc.Layout(numels, N=N, A=A, B=8)
    tensors = [rng.integers(0, 1 << 16, size=n, dtype=np.uint16) for n in numels]
    shards = [np.zeros(lay.S, np.uint16) for _ in range(N)]
    for r in range(N):
        for t, t_off, s_off, ln in lay.segments(r):
            shards[r][s_off:s_off + ln] = tensors[t][t_off:t_off + ln]
    for t, (o, n) in enumerate(zip(lay.offsets, numels)):
        assert np.array_equal(orc.gather_tensor(shards, int(o), int(n)), tensors[t]), t


def test_tensor_spanning_every_rank_and_edges(orc):
    N, S = 4, 16
    shards = [np.arange(S, dtype=np.uint16) + 100 * r for r in range(N)]
    full = np.concatenate(shards)
    got = orc.gather_tensor(shards, 5, N * S - 7)            # crosses all four shards
    assert got[0] == 5 and got[11] == 100 and got[-1] == 300 + 13
    assert np.array_equal(got, full[5:N * S - 2])
    assert orc.gather_tensor(shards, 16, 0).size == 0          # empty tensor
    assert np.array_equal(orc.gather_tensor(shards, 48, 16), shards[3])   # exactly one shard
    with pytest.raises(ValueError):
        orc.gather_tensor(shards, 60, 5)                        # runs past the padded buffer
