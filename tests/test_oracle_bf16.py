"""Pins of the oracle's fp32 -> bf16 rounding (the updated parameters written into
the rank's slot of the gathered buffer, "[REQUEST] Direct Correspondence between
Gradient and Optimizer States to Reduce Communication", "Problem").

Library routine: torch's CPU float32 -> bfloat16 cast (round to nearest even).
"""
import numpy as np
import torch


def torch_bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_random_bit_patterns(orc):
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    got = orc.f32_to_bf16(x)
    want = torch_bf16(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all(got[nan] == 0x7FC0)


def test_ties_and_edges(orc):
    pats = []
    for hi in (0x0000, 0x0001, 0x3F80, 0x3F81, 0x7F7E, 0x7F7F, 0x8000, 0xBF80, 0xFF7F, 0x0080):
        for lo in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
            pats.append((hi << 16) | lo)
    pats += [0x7F800000, 0xFF800000, 0x7F7FFFFF, 0x00000001, 0x807FFFFF]
    x = np.array(pats, dtype=np.uint32).view(np.float32)
    got = orc.f32_to_bf16(x)
    want = torch_bf16(x)
    assert np.array_equal(got, want)
    # ties: 1 + half a bf16 ulp rounds to 1 (even), 1 + 3 halves rounds up to 1 + 2 ulp
    assert orc.f32_to_bf16(np.array([1.0 + 2.0 ** -8], np.float32))[0] == 0x3F80
    assert orc.f32_to_bf16(np.array([1.0 + 3 * 2.0 ** -8], np.float32))[0] == 0x3F82
    # largest finite fp32 rounds up to infinity
    assert orc.f32_to_bf16(np.array([np.finfo(np.float32).max], np.float32))[0] == 0x7F80


def test_widening_is_exact(orc):
    h = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    x = orc.bf16_to_f32(h)
    fin = ~np.isnan(x)
    assert np.array_equal(orc.f32_to_bf16(x)[fin], h[fin])
    tw = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(x[fin].view(np.uint32), tw[fin].view(np.uint32))
