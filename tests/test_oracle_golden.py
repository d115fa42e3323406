"""The oracle against the figures the pages print (fixtures in tests/golden/).

memory_per_device.json holds the "ZeRO Optimizer" page's per-device memory
coefficients (in P and P/N) and its stated stage-1/2 reductions;
ring_volumes_8_ranks.json holds the 8-rank communication fractions and the walk
of the first chunk from the reduce-scatter discussion. Each fixture names its
page and sections. The oracle computes these from its own layout and its
message-passing ring simulator.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def frac(pair):
    return Fraction(pair[0], pair[1])


@pytest.mark.parametrize("N", [2, 8, 64])
def test_memory_per_device_matches_page(orc, N):
    g = load("memory_per_device.json")
    Pn = 1000
    lay = orc.Layout([N * Pn], N=N, A=1, B=1)
    P = lay.L_pad
    for stage, key in enumerate(("data_parallel", "stage1", "stage2", "stage3")):
        vals = lay.mem_values(stage)
        cp, cn = g[key]["total"]
        assert vals[3] == cp * P + cn * Pn, key
        comps = g[key]["components"]
        want = [comps[c][0] * P + comps[c][1] * Pn
                for c in ("parameters", "gradients", "optimizer_states")]
        assert vals[:3].tolist() == want, key


def test_stated_reductions_are_byte_model_limits(orc):
    g = load("memory_per_device.json")["stated_reduction"]
    N = 1 << 20
    lay = orc.Layout([N * 100], N=N, A=1, B=1)
    b = [int(lay.mem_bytes(s)[3]) for s in range(4)]
    assert abs(Fraction(b[0], b[1]) - g["stage1"]) < Fraction(1, 1000)
    assert abs(Fraction(b[0], b[2]) - g["stage2"]) < Fraction(1, 1000)
    assert Fraction(b[0], b[3]) == N


def test_ring_fractions_for_eight_ranks(orc):
    g = load("ring_volumes_8_ranks.json")
    N = g["ranks"]
    S = 24
    psi = N * S
    _, sent, recv, order = orc.ring_reduce_scatter(np.ones((N, psi), np.float32))
    steps = N - 1
    for k in range(N):
        assert Fraction(int(sent[k]), steps * psi) == frac(g["guanhuawang_ring"]["sent_per_step"])
        assert Fraction(int(recv[k]), steps * psi) == frac(g["guanhuawang_ring"]["received_per_step"])
        # the naive count (all other ranks' data in, all own data out) equals the ring's totals
        assert Fraction(int(recv[k]), psi) == frac(g["civat_naive_count_per_rank"]["received"])
        assert Fraction(int(sent[k]), psi) == frac(g["civat_naive_count_per_rank"]["sent"])
        assert Fraction(int(sent[k] + recv[k]), psi) == frac(g["civat_naive_count_per_rank"]["total"])
    # one chunk costs each rank a send and a receive of one chunk
    assert Fraction(int(sent[0] + recv[0]), steps * psi) == frac(g["civat_per_chunk"]["sent_and_received_per_chunk"])
    # the walk of the first chunk as the reply tells it: GPU0, GPU1, ..., GPU7, back to GPU0
    _, wsent, wrecv, worder = orc.ring_reduce_scatter(np.ones((N, psi), np.float32), walk=True)
    assert worder[0].tolist() + [0] == g["guanhuawang_ring"]["first_chunk_walk"]
    _, ag_sent, ag_recv = orc.ring_all_gather(np.ones((N, S), np.float32))
    assert Fraction(int(ag_recv[0]), psi) == frac(g["civat_all_gather_per_rank"]["received"])
    assert Fraction(int(ag_sent[0]) // steps, psi) == frac(g["civat_all_gather_per_rank"]["sent"])
    # the ZeRO passage counts one direction, asymptotically: (N-1)/N Psi -> Psi
    z = g["zero_paper"]
    assert Fraction(int(sent[0]), psi) == Fraction(N - 1, N) * frac(z["reduce_scatter_total"])
    assert Fraction(int(ag_sent[0]), psi) == Fraction(N - 1, N) * frac(z["all_gather_total"])
    assert Fraction(int(sent[0] + ag_sent[0]), psi) == Fraction(N - 1, N) * frac(z["data_parallel_all_reduce_total"])
