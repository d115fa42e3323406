"""Helpers for the GPU parity tests: device buffers, guard bands, oracle runs.

Nothing here computes the method: inputs come from ``workloads``, expected values
from ``oracle``, results from libzero through its C ABI.
"""
from __future__ import annotations

import os
import sys

import numpy as np

NTHREADS = max(1, min(16, os.cpu_count() or 1))
GUARD = 4096                         # bytes of sentinel before and after a guarded buffer
SENTINEL = 0xA5


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def dev():
    import torch
    return torch.device("cuda", torch.cuda.current_device())


class Guarded:
    """A device buffer with sentinel bytes on both sides (16-byte aligned body)."""

    def __init__(self, nbytes: int, dtype, fill=None):
        import torch
        self.nbytes = int(nbytes)
        self.raw = torch.full((GUARD + self.nbytes + GUARD,), SENTINEL, dtype=torch.uint8, device=dev())
        body = self.raw[GUARD:GUARD + self.nbytes]
        self.t = body.view(dtype)
        if fill is not None:
            self.t.copy_(fill)

    def intact(self) -> bool:
        import torch
        head = self.raw[:GUARD]
        tail = self.raw[GUARD + self.nbytes:]
        return bool(torch.all(head == SENTINEL).item()) and bool(torch.all(tail == SENTINEL).item())


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(dev())
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_host(t) -> np.ndarray:
    import torch
    x = t.detach().to("cpu")
    if x.dtype in (torch.int16, torch.bfloat16):
        return x.view(torch.int16).numpy().view(np.uint16).copy()
    return x.numpy().copy()


def bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32) if a.dtype == np.float32 else a


def assert_bitexact(name: str, got: np.ndarray, want: np.ndarray):
    assert got.shape == want.shape, (name, got.shape, want.shape)
    gb, wb = bits(got), bits(want)
    if not np.array_equal(gb, wb):
        bad = np.nonzero(gb != wb)[0]
        i = int(bad[0])
        raise AssertionError(f"{name}: {bad.size} of {got.size} differ; first at {i}: "
                             f"got {got[i]!r} want {want[i]!r}")


def max_rel(got: np.ndarray, want: np.ndarray) -> float:
    g, w = got.astype(np.float64), want.astype(np.float64)
    den = np.maximum(np.abs(w), 1e-30)
    return float(np.max(np.abs(g - w) / den)) if g.size else 0.0


def check_state(prefix, got_p, got_m, got_v, got_slot, p, m, v, slot):
    """Acceptance: p, m, v within 1e-6 relative, slot within 1 bf16 ulp.
    The implementation is expected bit-exact, so report that too."""
    for name, g, w in (("p", got_p, p), ("m", got_m, m), ("v", got_v, v)):
        r = max_rel(g, w)
        assert r <= 1e-6, f"{prefix} {name}: max relative error {r:.3e} > 1e-6"
        assert_bitexact(f"{prefix} {name}", g, w)
    if slot is not None:
        du = np.abs(got_slot.astype(np.int32) - slot.astype(np.int32))
        assert int(du.max(initial=0)) <= 1, f"{prefix} slot: {int(du.max())} bf16 ulp"
        assert_bitexact(f"{prefix} slot", got_slot, slot)


def sumsq_close(got: float, want: float, rel: float = 1e-9) -> bool:
    if not np.isfinite(want):
        return not np.isfinite(got)
    return abs(got - want) <= rel * max(abs(want), 1e-300)
