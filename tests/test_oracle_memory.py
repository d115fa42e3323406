"""Pins of the oracle's memory accounting against the page formulas.

"ZeRO Optimizer" wiki page: "Memory Components" (P parameters, P gradients, 2P
Adam moments per GPU under plain data parallelism) and "Theoretical Reductions"
(per-device memory 2P + 2P/N for stage 1, P + 3P/N for stage 2, 4P/N for
stage 3). The oracle sums the three components; these tests check the page's
collapsed closed forms. The "4x" and "8x" reductions ("ZeRO Stages") are the
N -> infinity limits of the byte model (2-byte parameters and gradients, 12
bytes of fp32 master + m + v), not of the value model (which gives 2x and 4x).
"""
from fractions import Fraction

import pytest


@pytest.mark.parametrize("name", ["tiny", "gpt2s", "llama7b", "ragged", "llama70b"])
def test_page_formulas(orc, name):
    import workloads as W
    w = W.get(name)
    lay = orc.Layout(w.numels, N=w.N, A=w.A, B=w.B)
    P, Pn = lay.L_pad, lay.S
    assert P == w.N * Pn
    assert lay.mem_values(0)[3] == 4 * P
    assert lay.mem_values(1)[3] == 2 * P + 2 * Pn
    assert lay.mem_values(2)[3] == P + 3 * Pn
    assert lay.mem_values(3)[3] == 4 * Pn
    # per-component form, as the page writes it before collapsing
    assert lay.mem_values(1)[:3].tolist() == [P, P, 2 * Pn]
    assert lay.mem_values(2)[:3].tolist() == [P, Pn, 2 * Pn]
    assert lay.mem_values(3)[:3].tolist() == [Pn, Pn, 2 * Pn]
    with pytest.raises(ValueError):
        lay.mem_values(4)


def test_value_model_limits(orc):
    # value model: 4P / (2P + 2P/N) -> 2, 4P / (P + 3P/N) -> 4
    N = 1 << 20
    lay = orc.Layout([N * 1000], N=N, A=1, B=1)
    r1 = Fraction(int(lay.mem_values(0)[3]), int(lay.mem_values(1)[3]))
    r2 = Fraction(int(lay.mem_values(0)[3]), int(lay.mem_values(2)[3]))
    assert abs(r1 - 2) < Fraction(1, 1000) and abs(r2 - 4) < Fraction(1, 1000)


def test_byte_model_gives_page_4x_8x(orc):
    # byte model: 16P / (4P + 12P/N) -> 4 ("4x"), 16P / (2P + 14P/N) -> 8 ("8x")
    N = 1 << 20
    lay = orc.Layout([N * 1000], N=N, A=1, B=1)
    b0, b1, b2, b3 = (int(lay.mem_bytes(s)[3]) for s in range(4))
    P, Pn = lay.L_pad, lay.S
    assert b0 == 16 * P and b1 == 4 * P + 12 * Pn and b2 == 2 * P + 14 * Pn and b3 == 16 * Pn
    assert abs(Fraction(b0, b1) - 4) < Fraction(1, 1000)
    assert abs(Fraction(b0, b2) - 8) < Fraction(1, 1000)
    assert Fraction(b0, b3) == N                       # stage 3: linear in N


def test_small_n_exact(orc):
    # N = 8 ranks, Psi = 8000: stage 1 = 16000 + 2000, stage 2 = 8000 + 3000, stage 3 = 4000
    lay = orc.Layout([8000], N=8, A=1, B=1)
    assert [int(lay.mem_values(s)[3]) for s in range(4)] == [32000, 18000, 11000, 4000]
