"""GPU parity of the stage-3 fetch (zero_gather_tensors) against the oracle.

Every tensor of a layout is copied out of the N rank shards into its own
temporary and compared bit for bit with the oracle's gather_tensor: the GPT-2
small tensor list (148 tensors, more than one launch), the ragged workload (256-
element alignment), unaligned layouts (alignment 1, odd sizes) where source and
destination differ in their 16-byte alignment, a tensor spanning every shard
with a tiny shard, fp32 elements, guard bands around the outputs, and a call
whose outputs exceed the Infinity Cache (stored past the caches).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import Guarded, assert_bitexact, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def check_layout(Z, numels, N, A, dtype=np.uint16, seed=0, tensors=None):
    lay = oracle.Layout(numels, N=N, A=A, B=8)
    rng = np.random.default_rng(seed)
    if dtype == np.uint16:
        shards_h = [rng.integers(0, 1 << 16, size=lay.S, dtype=np.uint16) for _ in range(N)]
    else:
        shards_h = [rng.standard_normal(lay.S).astype(np.float32) for _ in range(N)]
    shards = [to_dev(x) for x in shards_h]
    idx = range(len(numels)) if tensors is None else tensors
    offs = [int(lay.offsets[t]) for t in idx]
    nums = [int(numels[t]) for t in idx]
    outs = Z.zero_gather_tensors(shards, lay.S, offs, nums)
    torch.cuda.synchronize()
    for t, o, n, out in zip(idx, offs, nums, outs):
        want = oracle.gather_tensor(shards_h, o, n)
        assert_bitexact(f"tensor {t} (offset {o}, {n} elements)", to_host(out), want)
    return lay


def test_gpt2_small_every_tensor(Z):
    w = W.get("gpt2s")
    say("gather gpt2s, 148 tensors")
    check_layout(Z, w.numels, w.N, w.A, seed=1)


def test_ragged_every_tensor(Z):
    w = W.get("ragged")
    say("gather ragged, 10000 tensors")
    check_layout(Z, w.numels, w.N, w.A, seed=2, tensors=list(range(0, 10_000, 7)))


@pytest.mark.parametrize("seed", [3, 4, 5])
def test_unaligned_layouts(Z, seed):
    rng = np.random.default_rng(seed)
    numels = [int(x) for x in rng.integers(1, 70_000, size=40)]
    say(f"gather unaligned seed={seed}")
    check_layout(Z, numels, int(rng.integers(2, 12)), 1, seed=seed)


@pytest.mark.parametrize("N,count", [(8, 142), (8, 143), (8, 144), (8, 287), (64, 126), (64, 127),
                                     (64, 128), (200, 71), (200, 72), (200, 73), (200, 145)])
def test_tensor_counts_around_one_launch(Z, N, count):
    """Calls whose tensor counts sit just below, at and just above what one launch's
    argument block holds for their shard count (and twice that), so that the
    split into launches and the tensor lookup at the ends of a group are both
    exercised: every tensor bit-exact against the oracle."""
    rng = np.random.default_rng(1000 + N + count)
    numels = [int(x) for x in rng.integers(1, 3000, size=count)]
    numels[count // 2] = 40_000          # one tensor of several tasks
    say(f"gather N={N} count={count}")
    check_layout(Z, numels, N, 1, seed=N + count)


@pytest.mark.parametrize("dtype,N", [(np.uint16, 3), (np.float32, 16), (np.uint16, 100)])
def test_outputs_past_the_cache(Z, dtype, N):
    """A call whose outputs exceed the 256 MB Infinity Cache stores them with
    nontemporal stores: large tensors with odd sizes and offsets (pieces whose
    source and destination differ in their 16-byte alignment) among small ones,
    2- and 4-byte elements, 8-, 64- and 256-entry shard tables; every tensor
    bit-exact against the oracle."""
    numels = [3, 45_000_001, 7, 50_000_000, 1_001, 44_999_999, 2]
    say(f"gather past the cache: 140M elements over {N} shards ({np.dtype(dtype).name})")
    check_layout(Z, numels, N, 1, dtype=dtype, seed=12 + N)


def test_fp32_and_spanning_tensor(Z):
    say("gather fp32 + a tensor over every shard")
    check_layout(Z, [3, 5000, 1, 7], 64, 1, dtype=np.float32, seed=6)
    check_layout(Z, [0, 1, 100_000, 0, 2], 16, 1, seed=7)


def test_guard_bands_and_empty(Z):
    numels = [1001, 33, 4096, 7]
    lay = oracle.Layout(numels, N=3, A=1, B=8)
    rng = np.random.default_rng(8)
    shards_h = [rng.integers(0, 1 << 16, size=lay.S, dtype=np.uint16) for _ in range(3)]
    shards = [to_dev(x) for x in shards_h]
    gs = [Guarded(2 * n, torch.int16) for n in numels]
    Z.zero_gather_tensors(shards, lay.S, lay.offsets, numels, outs=[g.t for g in gs])
    torch.cuda.synchronize()
    for t, g in enumerate(gs):
        assert g.intact(), t
        assert_bitexact(f"guarded {t}", to_host(g.t), oracle.gather_tensor(shards_h, int(lay.offsets[t]), numels[t]))
    assert Z.zero_gather_tensors(shards, lay.S, [], []) == []


@pytest.mark.slow
def test_tensor_beyond_one_launch(Z):
    """One bf16 tensor of 2^33 + 12,345 elements (17 GB) over two shards: its
    8192-element tasks outnumber one launch's 2^20 workgroups, so the copy takes
    two launches over consecutive task ranges. The output must equal the two
    shard slices, compared on the device (the oracle's gather is that same
    concatenation; at this size it is checked as a property)."""
    n = (1 << 33) + 12_345
    S = (n + 1) // 2 + 8
    say(f"gather one tensor of {n} elements over 2 shards of {S}")
    g = torch.Generator(device="cuda").manual_seed(11)
    shards = [torch.randint(-32768, 32767, (S,), dtype=torch.int16, device="cuda", generator=g)
              for _ in range(2)]
    out = Z.zero_gather_tensors(shards, S, [5], [n])[0]
    torch.cuda.synchronize()
    assert torch.equal(out[: S - 5], shards[0][5:])
    assert torch.equal(out[S - 5:], shards[1][: n - (S - 5)])
    del out, shards
    torch.cuda.empty_cache()
