"""Seeded synthetic workloads for the per-rank ZeRO shard step.

This module holds inputs only: tensor-size lists, hyperparameters, seeds and the
random generators that fill gradient replicas and optimizer state. It holds none
of the method's arithmetic (no layout, no reduction, no update), so that the CPU
oracle and the GPU path can both be fed from it without sharing any code.

Workloads (tensor shapes only; no trained weights exist or are needed):

* ``tiny``     3 tensors [1000, 2048, 1000], N=2, fp32 grads ~N(0, 0.01^2), Adam.
* ``gpt2s``    GPT-2 small (12 layers, d=768, vocab 50257, ctx 1024, tied head),
               148 tensors, 124,439,808 params, N=8, bf16 grads ~N(0, 1e-3^2), AdamW.
* ``llama7b``  Llama-7B shape (32 layers, d=4096, ffn 11008, vocab 32000, untied head),
               291 tensors, 6,738,415,616 params, N=8, bf16(65536 x), x~N(0,1e-4^2).
* ``ragged``   10,000 tensors with log-uniform sizes in [1, 65536], 256-element
               alignment, N=64, dynamic loss scale from 65536, one +inf injected.
* ``llama70b`` Llama-70B shape (80 layers, d=8192, 64 q heads x 128, 8 kv heads,
               ffn 28672, vocab 32000), 723 tensors, 68,976,648,192 params, N=32.

"~N(0, s^2)" means standard deviation s. A replica under loss scale K stores the
value a loss-scaled backward would write: dtype(K * x) with x ~ N(0, s^2).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

# ---------------------------------------------------------------------------
# tensor lists
# ---------------------------------------------------------------------------


def gpt2_small_numels() -> List[int]:
    d, L, V, ctx = 768, 12, 50257, 1024
    out = [V * d, ctx * d]                       # token + position embedding (head tied)
    for _ in range(L):
        out += [d, d,                            # ln_1 w, b
                d * 3 * d, 3 * d,                # attention qkv w, b
                d * d, d,                        # attention out-proj w, b
                d, d,                            # ln_2 w, b
                d * 4 * d, 4 * d,                # mlp fc w, b
                4 * d * d, d]                    # mlp proj w, b
    out += [d, d]                                # final ln w, b
    return out


def llama_numels(layers: int, d: int, ffn: int, vocab: int, kv_dim: Optional[int] = None) -> List[int]:
    kv = d if kv_dim is None else kv_dim
    out = [vocab * d]                            # embedding
    for _ in range(layers):
        out += [d,                               # attention norm
                d * d, d * kv, d * kv, d * d,    # q, k, v, o
                d,                               # mlp norm
                d * ffn, d * ffn, ffn * d]       # gate, up, down
    out += [d, vocab * d]                        # final norm, untied LM head
    return out


def layer_tensor_count(name: str) -> int:
    """Tensors per transformer layer in the lists above (1 for the other lists)."""
    return {"gpt2s": 12, "llama7b": 9, "llama70b": 9}.get(name, 1)


def first_layer_tensor(name: str) -> int:
    """Index of the first tensor of layer 0 (after the embeddings)."""
    return {"gpt2s": 2, "llama7b": 1, "llama70b": 1}.get(name, 0)


def ragged_numels(seed: int = 1234, count: int = 10_000, hi: int = 65536, N: int = 64) -> List[int]:
    """Log-uniform sizes in [1, hi]; the raw total is kept non-divisible by N."""
    rng = np.random.default_rng(seed)
    n = np.clip(np.rint(np.exp(rng.uniform(0.0, math.log(hi), size=count))), 1, hi).astype(np.int64)
    if int(n.sum()) % N == 0:
        n[-1] += 1 if n[-1] < hi else -1
    return [int(x) for x in n]


# ---------------------------------------------------------------------------
# workload presets
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    numels: tuple
    N: int                    # simulated data-parallel ranks = gradient replicas
    A: int                    # tensor start alignment (elements)
    B: int                    # shard granularity (elements)
    grad_dtype: str           # "bf16" or "f32"
    grad_sigma: float
    param_sigma: float
    loss_scale: float
    dynamic_loss_scale: bool
    lr: float
    beta1: float
    beta2: float
    eps: float
    wd: float
    steps: int
    seed: int                 # base seed; replicas and params derive from it
    inject_inf: bool = False

    @property
    def psi(self) -> int:
        return int(sum(self.numels))

    @property
    def grad_bytes(self) -> int:
        return 2 if self.grad_dtype == "bf16" else 4

    def hyper(self) -> dict:
        return dict(lr=self.lr, beta1=self.beta1, beta2=self.beta2, eps=self.eps, wd=self.wd)


_ADAM = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)

WORKLOADS = {
    "tiny": Workload("tiny", (1000, 2048, 1000), N=2, A=1, B=8, grad_dtype="f32", grad_sigma=1e-2,
                     param_sigma=0.02, loss_scale=1.0, dynamic_loss_scale=False, wd=0.0, steps=3,
                     seed=1001, **_ADAM),
    "gpt2s": Workload("gpt2s", tuple(gpt2_small_numels()), N=8, A=1, B=8, grad_dtype="bf16",
                      grad_sigma=1e-3, param_sigma=0.02, loss_scale=1.0, dynamic_loss_scale=False,
                      wd=0.01, steps=10, seed=1002, **_ADAM),
    "llama7b": Workload("llama7b", tuple(llama_numels(32, 4096, 11008, 32000)), N=8, A=1, B=8,
                        grad_dtype="bf16", grad_sigma=1e-4, param_sigma=0.02, loss_scale=65536.0,
                        dynamic_loss_scale=False, wd=0.0, steps=5, seed=1003, **_ADAM),
    "ragged": Workload("ragged", tuple(ragged_numels()), N=64, A=256, B=8, grad_dtype="bf16",
                       grad_sigma=1e-4, param_sigma=0.02, loss_scale=65536.0,
                       dynamic_loss_scale=True, wd=0.0, steps=5, seed=1004, inject_inf=True, **_ADAM),
    "llama70b": Workload("llama70b", tuple(llama_numels(80, 8192, 28672, 32000, kv_dim=1024)), N=32,
                         A=1, B=8, grad_dtype="bf16", grad_sigma=1e-4, param_sigma=0.02,
                         loss_scale=1.0, dynamic_loss_scale=False, wd=0.01, steps=3, seed=1005,
                         **_ADAM),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


# ---------------------------------------------------------------------------
# seeds
# ---------------------------------------------------------------------------

_REPLICA, _PARAM, _INJECT = 1, 2, 3


def seed_for(*key: int) -> int:
    """A 63-bit seed derived from a key tuple (numpy SeedSequence)."""
    return int(np.random.SeedSequence([int(k) for k in key]).generate_state(2, np.uint64)[0] >> 1)


def replica_seed(w: Workload, rank: int, step: int, slot: int) -> int:
    return seed_for(w.seed, _REPLICA, rank, step, slot)


def param_seed(w: Workload, rank: int) -> int:
    return seed_for(w.seed, _PARAM, rank)


# ---------------------------------------------------------------------------
# host generators (numpy); covered = list of (shard_off, len) runs holding data
# ---------------------------------------------------------------------------


def _bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Storage conversion of a generated fp32 sample to bf16 via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def mask_from_runs(S: int, covered: Sequence) -> np.ndarray:
    m = np.zeros(S, dtype=bool)
    for off, ln in covered:
        m[int(off):int(off) + int(ln)] = True
    return m


def host_replica(w: Workload, S: int, covered, rank: int, step: int, slot: int) -> np.ndarray:
    """One gradient replica of rank ``rank``'s shard: uint16 bf16 patterns or float32."""
    rng = np.random.default_rng(replica_seed(w, rank, step, slot))
    x = (rng.standard_normal(S, dtype=np.float32) * np.float32(w.grad_sigma)).astype(np.float32)
    x = (x * np.float32(w.loss_scale)).astype(np.float32)
    x[~mask_from_runs(S, covered)] = 0.0
    if w.grad_dtype == "bf16":
        return _bf16_bits_from_f32(x)
    return x


def host_replicas(w: Workload, S: int, covered, rank: int, step: int) -> List[np.ndarray]:
    reps = [host_replica(w, S, covered, rank, step, j) for j in range(w.N)]
    inj = injection(w, S, covered, rank)
    if inj is not None and inj[0] == step:
        _, j, i = inj
        if w.grad_dtype == "bf16":
            reps[j][i] = 0x7F80                     # +inf
        else:
            reps[j][i] = np.float32(np.inf)
    return reps


def host_params(w: Workload, S: int, covered, rank: int) -> np.ndarray:
    rng = np.random.default_rng(param_seed(w, rank))
    p = (rng.standard_normal(S, dtype=np.float32) * np.float32(w.param_sigma)).astype(np.float32)
    p[~mask_from_runs(S, covered)] = 0.0
    return p


def injection(w: Workload, S: int, covered, rank: int):
    """(step index, slot, shard element) of the injected +inf, or None.
    The step is one of 1, 2, 3 (0-based), i.e. never the first step."""
    if not w.inject_inf:
        return None
    rng = np.random.default_rng(seed_for(w.seed, _INJECT, rank))
    step = int(rng.integers(1, min(4, w.steps)))
    slot = int(rng.integers(0, w.N))
    runs = [(int(o), int(n)) for o, n in covered if int(n) > 0]
    total = sum(n for _, n in runs)
    k = int(rng.integers(0, total))
    for o, n in runs:
        if k < n:
            return step, slot, o + k
        k -= n
    raise AssertionError("unreachable")


# ---------------------------------------------------------------------------
# device generators (torch RNG on the GPU) for the large shards
# ---------------------------------------------------------------------------

_CHUNK = 1 << 27


def device_fill_replica(buf, w: Workload, covered, rank: int, step: int, slot: int) -> None:
    """Fill ``buf`` (torch bf16 or float32 tensor of S elements on the GPU) with
    dtype(K * sigma * randn), chunk by chunk from a seeded device generator, and
    zero every position outside ``covered``."""
    import torch
    S = buf.numel()
    base = replica_seed(w, rank, step, slot)
    gen = torch.Generator(device=buf.device)
    scale = float(w.grad_sigma) * float(w.loss_scale)
    for c0 in range(0, S, _CHUNK):
        c1 = min(S, c0 + _CHUNK)
        gen.manual_seed(seed_for(base, c0 // _CHUNK))
        x = torch.randn(c1 - c0, generator=gen, device=buf.device, dtype=torch.float32)
        x.mul_(scale)
        buf[c0:c1].copy_(x)
        del x
    _zero_outside(buf, covered)


def device_prefix(fill, S: int, n: int, dtype, device, *args):
    """The first n elements of what ``fill`` (device_fill_replica or
    device_fill_params, with ``args`` after the buffer) writes into a buffer of
    S elements, without allocating S: the fills draw chunk by chunk, so the first
    min(S, 2^27) elements come from the first chunk's draw alone."""
    import torch
    L = min(S, _CHUNK)
    if not 0 < n <= L:
        raise ValueError(f"a prefix of {n} elements of a {S}-element fill (at most {L})")
    buf = torch.empty(L, dtype=dtype, device=device)
    fill(buf, *args)
    out = buf[:n].clone()
    del buf
    return out


def device_fill_params(buf, w: Workload, covered, rank: int) -> None:
    import torch
    S = buf.numel()
    base = param_seed(w, rank)
    gen = torch.Generator(device=buf.device)
    for c0 in range(0, S, _CHUNK):
        c1 = min(S, c0 + _CHUNK)
        gen.manual_seed(seed_for(base, c0 // _CHUNK))
        x = torch.randn(c1 - c0, generator=gen, device=buf.device, dtype=torch.float32)
        x.mul_(float(w.param_sigma))
        buf[c0:c1].copy_(x)
        del x
    _zero_outside(buf, covered)


_MASKS: dict = {}


def _zero_outside(buf, covered) -> None:
    """Write +0 at every position of ``buf`` outside the ``covered`` runs. Few
    gaps: one fill per gap. Many gaps (the ragged workload's padding between
    aligned tensors): one masked fill with a device mask built once per layout,
    instead of a launch per gap."""
    import torch
    S = buf.numel()
    gaps = []
    pos = 0
    for off, ln in sorted((int(o), int(n)) for o, n in covered):
        if off > pos:
            gaps.append((pos, off))
        pos = max(pos, off + ln)
    if pos < S:
        gaps.append((pos, S))
    if len(gaps) <= 64 or S > (1 << 26):
        for a, b in gaps:
            buf[a:b].zero_()
        return
    key = (S, str(buf.device), tuple(gaps))
    mask = _MASKS.get(key)
    if mask is None:
        host = np.zeros(S, dtype=bool)
        for a, b in gaps:
            host[a:b] = True
        mask = torch.from_numpy(host).to(buf.device)
        _MASKS.clear()
        _MASKS[key] = mask
    buf.masked_fill_(mask, 0)
