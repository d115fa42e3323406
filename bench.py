#!/usr/bin/env python3
"""Benchmark of the per-rank ZeRO stage-1/2 fused shard step on one MI355X.

A step is one pass of the whole path over one rank's shard: fold the N resident
gradient replicas in ring (slot) order, average and unscale, flag overflow and
form the squared norm, Adam/AdamW on fp32 master / m / v, bf16 write into this
rank's slot of the gathered parameter buffer, then the 16-byte stats read-back
and the commit rule. The default workload is the Llama-70B-shaped shard, the
largest configuration one GPU holds (rank 0 of N=32, 2,155,520,256 elements,
32 bf16 replicas, AdamW; about 200 GB of HBM); inputs are synthetic, seeded,
and resident in HBM before the timed region starts. The GPT-2-small, Llama-7B,
ragged and tiny shards run with --config (GPT-2 and ragged with --flush-mall,
since their working sets fit or partly fit the 256 MB Infinity Cache).

Prints one JSON line. ``roofline`` is for the dominant kernel (the fused step
kernel): algorithmic bytes per launch, S * (N * 2 + 26), over its mean duration
measured with HIP events that the kernel's own launch carries on its stream
(hipExtLaunchKernel: they take the kernel's start and end), on every timed step
by default. ``wall_gbps`` and ``wall_frac`` give the same bytes over the wall
time per step (``ms_per_step``). ``cpu_baseline`` is the CPU oracle timed on
this host on a sample of the same shard.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "fused shard step: elements/s and achieved HBM GB/s (% of MI355X peak)"
CPU_SAMPLE_ELEMS = 64 << 20
KERNEL_SOURCES = [os.path.join(ROOT, "zero_partitioned_optimizer_amd", "csrc", f)
                  for f in ("step_kernels.hip", "zero_internal.h")] + [
                      os.path.join(ROOT, "include", "zero.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """sha256[:16] of the step kernel's code: step_kernels.hip, zero_internal.h
    and include/zero.h (whose structs the kernel reads and writes) with comments
    and whitespace removed, so that a comment edit does not count as a kernel
    change."""
    import re
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, state: str):
    """HBM bytes per launch of the step kernel from the committed rocprofv3 counter
    runs, or None if there are none for this workload and state layout or the
    kernel changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_sha") != kernel_source_hash():
        return None
    if rec.get("state", "split") != state:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, host_reps, p0_host, S, seconds: float, wire: bool = False):
    """The oracle, as it stands, on this host: repeated steps over the shard."""
    import numpy as np

    import oracle
    nthreads = max(1, min(16, os.cpu_count() or 1))
    p = p0_host.copy()
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    slot = np.zeros(S, np.uint16)
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.step(host_reps, p, m, v, slot, loss_scale=w.loss_scale, t=n + 1, nthreads=nthreads,
                    wire=wire, **w.hyper())
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    # the same oracle on one thread, for a quarter of the time
    n1 = 0
    t1 = time.perf_counter()
    while True:
        oracle.step(host_reps, p, m, v, slot, loss_scale=w.loss_scale, t=n + n1 + 1, nthreads=1,
                    wire=wire, **w.hyper())
        n1 += 1
        el1 = time.perf_counter() - t1
        if el1 >= seconds / 4:
            break
    return {"value": n * S / el, "unit": "elements/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{w.name} rank-0 shard, {S} elements, N={w.N} replicas, {n} oracle "
                      f"steps in {el:.1f} s, OpenMP threads={nthreads}",
            "cpu_model": cpu_model(),
            "single_thread": {"value": n1 * S / el1, "unit": "elements/s",
                              "sample": f"{n1} oracle steps in {el1:.1f} s, 1 thread"}}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def overlap_bench(args, Z, w, S, pool, p0, kw, gdt) -> int:
    """A stand-in backward pass writes the gradient replicas part by part (for
    each part: one bf16 GEMM of compute, then the part's N replica ranges copied
    in from a resident pool), then the step runs. Serial: the whole step after the
    last part is written. Overlapped: the step as K parts on its own stream, part
    k starting when part k of the gradients has landed. Both orders compute the
    same committed state; the line reports the time per iteration of each."""
    import torch
    dev = torch.device("cuda:0")
    K = args.overlap
    ends = [min(S, (S * (k + 1) // K) // 8 * 8) for k in range(K - 1)] + [S]
    bufs = [torch.empty_like(r) for r in pool]
    M = args.gemm
    A = torch.randn(M, M, device=dev, dtype=torch.bfloat16)
    Bm = torch.randn(M, M, device=dev, dtype=torch.bfloat16)
    C = torch.empty(M, M, device=dev, dtype=torch.bfloat16)
    producer, stepper = torch.cuda.Stream(), torch.cuda.Stream()
    step = Z.DeviceShardStep(S, w.N, gdt, p0, double_slot=True, **kw)

    def produce(mode):
        producer.wait_stream(stepper)           # the previous step has read the buffers
        ready = []
        lo = 0
        with torch.cuda.stream(producer):
            for hi in ends:
                if mode != "step_only":
                    torch.matmul(A, Bm, out=C)
                    for j in range(w.N):
                        bufs[j][lo:hi].copy_(pool[j][lo:hi])
                ev = torch.cuda.Event()
                ev.record(producer)
                ready.append(ev)
                lo = hi
        return ready

    def iteration(mode):
        ready = produce(mode)
        if mode == "producer_only":
            return
        if mode == "overlap":
            step.step_parts(bufs, ends, ready=ready, stream=stepper)
        else:
            stepper.wait_event(ready[-1])
            step.step(bufs, stream=stepper)

    def timed(mode, n):
        for _ in range(args.warmup):
            iteration(mode)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            iteration(mode)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n * 1e3

    n = args.steps
    res = {m: timed(m, n) for m in ("serial", "overlap", "producer_only", "step_only")}
    log("overlap: " + ", ".join(f"{m} {v:.3f} ms" for m, v in res.items()))
    out = {
        "metric": "stand-in backward + fused step, ms per iteration (overlapped parts)",
        "value": res["overlap"], "unit": "ms", "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "ms_per_step": res["overlap"], "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name} shard, rank {args.rank} of N={w.N}", "shard_elems": S,
                   "n_replicas": w.N, "parts": K, "part_ends": ends, "gemm": [M, M, M],
                   "commit": "device", "slot": "double"},
        "serial_ms": res["serial"], "overlap_ms": res["overlap"],
        "producer_only_ms": res["producer_only"], "step_only_ms": res["step_only"],
        "overlap_gain": res["serial"] / res["overlap"],
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def offload_bench(args, Z, w, S, reps, p0, gdt) -> int:
    """The offloaded step: GPU fold and check, the fp32 gradient to the host in
    chunks, host Adam on each chunk as it lands, bf16 back into the slot. Beside
    it, the parts on their own: the gradient's device-to-host copy, the slot's
    host-to-device copy (both pinned, one transfer each) and the host Adam over
    the whole shard with the same threads."""
    import numpy as np
    import torch
    nthreads = len(os.sched_getaffinity(0))
    step = Z.OffloadShardStep(S, w.N, gdt, p0.cpu(), lr=w.lr, beta1=w.beta1, beta2=w.beta2,
                              eps=w.eps, weight_decay=w.wd, loss_scale=w.loss_scale,
                              dynamic=w.dynamic_loss_scale, chunk_elems=args.chunk_elems,
                              nthreads=nthreads)
    for _ in range(args.warmup):
        step.step(reps)
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    skipped = 0
    for _ in range(K):
        st, verdict = step.step(reps)
        skipped += verdict == Z.ZERO_SKIP
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    def best_of(fn, n=5):
        ts = []
        for _ in range(n):
            torch.cuda.synchronize()
            a = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - a)
        return min(ts)
    t_d2h = best_of(lambda: step.g_host.copy_(step.g_dev, non_blocking=True))
    t_h2d = best_of(lambda: step.slot.copy_(step.slot_host, non_blocking=True))
    g = np.ones(S, np.float32) * 1e-3
    pp, mm, vv = (np.zeros(S, np.float32) for _ in range(3))
    sl = np.zeros(S, np.uint16)
    t_adam = best_of(lambda: Z.zero_host_adam(g, pp, mm, vv, S, lr=w.lr, beta1=w.beta1,
                                              beta2=w.beta2, eps=w.eps, weight_decay=w.wd,
                                              step_t=1, slot=sl, nthreads=nthreads), 3)
    ms = elapsed / K * 1e3
    log(f"offload: {ms:.3f} ms/step; D2H {S * 4 / t_d2h / 1e9:.1f} GB/s, H2D "
        f"{S * 2 / t_h2d / 1e9:.1f} GB/s, host Adam {S / t_adam / 1e9:.2f} G elem/s "
        f"({nthreads} threads)")
    out = {
        "metric": "offloaded shard step: elements/s (state in host memory)",
        "value": S * K / elapsed, "unit": "elements/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name} shard, rank {args.rank} of N={w.N}", "shard_elems": S,
                   "n_replicas": w.N, "grad_dtype": w.grad_dtype, "state": "host",
                   "chunk_elems": args.chunk_elems or 1 << 20, "host_threads": nthreads},
        "parts_alone_ms": {"d2h_gradient": t_d2h * 1e3, "h2d_slot": t_h2d * 1e3,
                           "host_adam": t_adam * 1e3},
        "pcie_gbs": {"d2h": S * 4 / t_d2h / 1e9, "h2d": S * 2 / t_h2d / 1e9},
        "host_adam_elems_per_s": S / t_adam,
        "skipped_steps": skipped, "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def gather_bench(args, Z, W, w, S) -> int:
    """Stage-3 fetch: the model's tensors copied out of the N bf16 rank shards
    (the gathered parameter buffer's slots) into temporaries, one layer at a time
    and all at once. Algorithmic bytes: 2 bytes read + 2 written per element."""
    import torch
    dev = torch.device("cuda:0")
    h = Z.zero_layout_build(list(w.numels), w.N, w.A, w.B)
    try:
        offsets = Z.zero_layout_offsets(h)
    finally:
        Z.zero_layout_free(h)
    shards = [torch.randint(-32768, 32767, (S,), dtype=torch.int16, device=dev) for _ in range(w.N)]
    numels = list(w.numels)
    per_layer = W.layer_tensor_count(w.name)
    first = W.first_layer_tensor(w.name)
    layer = list(range(first, first + per_layer))
    outs_all = [torch.empty(n, dtype=torch.int16, device=dev) for n in numels]

    def plan_of(idx):
        return Z.GatherPlan(shards, S, [offsets[t] for t in idx], [numels[t] for t in idx],
                            [outs_all[t] for t in idx])

    def timed(plans, reps):
        for _ in range(args.warmup):
            for plan in plans:
                plan()
        # back to back, one event pair around all calls: the host's call overhead
        # overlaps the copies of the calls before it
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            for plan in plans:
                plan()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / (reps * len(plans))

    def graphed(plans, reps):
        # the same calls captured once in a HIP graph and replayed: the GPU's time
        # per call with no host work per launch
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            for plan in plans:
                plan()
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=cap):
                for plan in plans:
                    plan()
        torch.cuda.synchronize()
        for _ in range(2):
            graph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / (reps * len(plans))

    n_layer = sum(numels[t] for t in layer)
    t_layer = timed([plan_of(layer)], args.steps)
    # every layer in turn: no layer's tensors are still cached when it comes round
    n_layers = (len(numels) - first) // per_layer
    layers = [list(range(first + k * per_layer, first + (k + 1) * per_layer)) for k in range(n_layers)]
    turn_plans = [plan_of(ix) for ix in layers]
    n_turn = sum(numels[t] for ix in layers for t in ix) / n_layers
    t_turn = timed(turn_plans, max(1, args.steps // n_layers))
    t_turn_g = graphed(turn_plans, max(2, args.steps // n_layers))
    n_all = sum(numels)
    t_all = timed([plan_of(list(range(len(numels))))], max(5, args.steps // 10))
    gbs_all = 4 * n_all / t_all / 1e9
    log(f"gather: layer ({per_layer} tensors, {n_layer} elements) {t_layer * 1e6:.1f} us "
        f"= {4 * n_layer / t_layer / 1e9:.0f} GB/s; the {n_layers} layers in turn "
        f"{t_turn * 1e6:.1f} us = {4 * n_turn / t_turn / 1e9:.0f} GB/s per layer "
        f"({t_turn_g * 1e6:.1f} us = {4 * n_turn / t_turn_g / 1e9:.0f} GB/s replayed from a graph); "
        f"model ({len(numels)} tensors) {t_all * 1e3:.3f} ms = {gbs_all:.0f} GB/s")
    out = {
        "metric": "stage-3 fetch: achieved HBM GB/s (bf16 tensors out of the rank shards)",
        "value": gbs_all, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": t_all * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (bit copy)", "data": "synthetic",
        "config": {"workload": f"{w.name} parameters, N={w.N} shards of S={S}",
                   "n_tensors": len(numels), "elements": n_all},
        "layer": {"tensors": per_layer, "elements": n_layer, "us": t_layer * 1e6,
                  "gbs": 4 * n_layer / t_layer / 1e9, "repeated": "the same layer back to back"},
        "layers_in_turn": {"layers": n_layers, "elements_per_layer": n_turn, "us": t_turn * 1e6,
                           "gbs": 4 * n_turn / t_turn / 1e9, "graph_us": t_turn_g * 1e6,
                           "graph_gbs": 4 * n_turn / t_turn_g / 1e9},
        "roofline": {"bound": "hbm", "achieved": gbs_all, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs_all / HBM_PEAK_GBS, "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def graph_bench(args, w, S, step, reps) -> int:
    """G device-commit steps captured in one HIP graph, replayed back to back: the
    step rate with no host work per step. Every step reads the committed-state
    record, so a replayed step is the next step. HIP events on the replay stream
    bracket every replay."""
    import torch
    G = args.graph
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        step._args_for(reps)               # the argument block exists before the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            for _ in range(G):
                step.step(reps)
    torch.cuda.synchronize()
    t_before = int(step.state().t)
    for _ in range(2):
        graph.replay()
    R = max(1, args.steps // G)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(R)]
    for e0, e1 in ev:
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record()
        graph.replay()
        e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    st = step.state()
    steps_run = int(st.t) + int(st.n_skipped) - t_before
    K = R * G
    assert steps_run == K + 2 * G, (steps_run, K)
    per_step = [a.elapsed_time(b) / 1e3 / G for a, b in ev]
    kernel_s = statistics.mean(per_step)
    bpe = w.N * w.grad_bytes + 26
    achieved = S * bpe / kernel_s / 1e9
    log(f"graph of {G} steps, {R} replays: {elapsed / K * 1e6:.2f} us per step (wall), "
        f"{kernel_s * 1e6:.2f} us per step (replay events)")
    out = {
        "metric": METRIC, "value": S * K / elapsed, "unit": "elements/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": elapsed / K * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name} shard, rank {args.rank} of N={w.N}", "shard_elems": S,
                   "n_replicas": w.N, "grad_dtype": w.grad_dtype, "bytes_per_elem": bpe,
                   "commit": "device", "graph_steps": G},
        "step_us_replay_events": kernel_s * 1e6,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "note": "per step of a replayed graph (kernels plus the gaps between them)"},
        "cpu_baseline": None,
        "skipped_steps": int(st.n_skipped),
    }
    print(json.dumps(out), flush=True)
    return 0


def unfused_bench(args, Z, w, S, reps, p0, gdt) -> int:
    """The unfused step: the reduce kernel writes the fp32 gradient (fold, average,
    unscale, flag, norm), the host reads the 16-byte stats and applies the commit
    rule, and on a clean step the Adam kernel updates p, m, v in place from that
    gradient and writes the slot. 8 more bytes per element than the fused step
    (the gradient written and read back) and a host round trip inside every
    step. HIP events bracket each of the two kernels' calls on the stream."""
    import torch
    dev = p0.device
    g = torch.empty(S, dtype=torch.float32, device=dev)
    stats = torch.zeros(16, dtype=torch.uint8, device=dev)
    stats_host = torch.zeros(16, dtype=torch.uint8, pin_memory=True)
    ws = torch.empty(Z.zero_workspace_bytes(S), dtype=torch.uint8, device=dev)
    p = p0.clone()
    m = torch.zeros_like(p0)
    v = torch.zeros_like(p0)
    slot = torch.empty(S, dtype=torch.int16, device=dev)
    state = Z.zero_train_state(t=0, n_skipped=0, loss_scale=w.loss_scale, min_loss_scale=1.0,
                               dynamic=int(w.dynamic_loss_scale))
    hy = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.wd)
    stream = torch.cuda.current_stream()

    def one(evs=None):
        if evs:
            evs[0].record()
        Z.zero_reduce_shard(reps, gdt, S, stats, ws, loss_scale=state.loss_scale, grad_out=g)
        if evs:
            evs[1].record()
        stats_host.copy_(stats, non_blocking=True)
        stream.synchronize()
        st = Z.zero_stats.from_buffer_copy(stats_host.numpy().tobytes())
        if Z.zero_commit_rule(state, st) != Z.ZERO_COMMIT:
            return 1
        a = Z.make_adam_args(grad_f32=g, p_in=p, m_in=m, v_in=v, p_out=p, m_out=m, v_out=v,
                             slot=slot, shard_S=S, step_t=int(state.t), stats=stats, workspace=ws,
                             event_begin=evs[2] if evs else None, event_end=evs[3] if evs else None,
                             **hy)
        Z.zero_adam_step(a)
        return 0

    for _ in range(args.warmup):
        one()
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for e in evs:
        for x in e:
            x.record()
    torch.cuda.synchronize()
    skips = []
    t0 = time.perf_counter()
    for k in range(K):
        skips.append(one(evs[k]))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    skipped = sum(skips)
    clean = [e for e, sk in zip(evs, skips) if not sk]
    assert clean, "every timed step overflowed"
    t_red = statistics.mean(e[0].elapsed_time(e[1]) for e in evs) / 1e3
    t_adam = statistics.mean(e[2].elapsed_time(e[3]) for e in clean) / 1e3
    red_b = S * (w.N * w.grad_bytes + 4)
    adam_b = S * 30
    bpe = w.N * w.grad_bytes + 34
    achieved = S * bpe / (t_red + t_adam) / 1e9
    log(f"unfused: reduce {t_red * 1e6:.1f} us ({red_b / t_red / 1e9:.0f} GB/s), adam "
        f"{t_adam * 1e6:.1f} us ({adam_b / t_adam / 1e9:.0f} GB/s), {elapsed / K * 1e6:.1f} us "
        f"per step (wall)")
    out = {
        "metric": METRIC, "value": S * K / elapsed, "unit": "elements/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": elapsed / K * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name} shard, rank {args.rank} of N={w.N}", "shard_elems": S,
                   "n_replicas": w.N, "grad_dtype": w.grad_dtype, "bytes_per_elem": bpe,
                   "commit": "host", "path": "unfused"},
        "reduce_kernel": {"us": t_red * 1e6, "bytes": red_b, "gbps": red_b / t_red / 1e9},
        "adam_kernel": {"us": t_adam * 1e6, "bytes": adam_b, "gbps": adam_b / t_adam / 1e9},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "note": "S * (2N + 34) bytes over the two kernels' times"},
        "cpu_baseline": None,
        "skipped_steps": skipped,
    }
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="llama70b",
                    choices=["tiny", "gpt2s", "llama7b", "ragged", "llama70b"])
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--seed", type=int, default=None,
                    help="base seed of the synthetic replicas and parameters (default: the "
                         "workload's own)")
    ap.add_argument("--bucket-elems", type=int, default=0,
                    help="launch over the layout's bucket table cut at this size (0: whole shard)")
    ap.add_argument("--commit", default="device", choices=["device", "host"],
                    help="device: commit kernel, no host round trip per step; host: read the "
                         "stats back and apply the commit rule on the host every step")
    ap.add_argument("--state", default="tiled", choices=["tiled", "split"],
                    help="fp32 state layout of the device-commit step: one tiled buffer per "
                         "state set (p, m, v in tiles of 8192 elements) or three arrays "
                         "(the host commit always uses three arrays)")
    ap.add_argument("--single-slot", action="store_true",
                    help="device commit with one slot buffer (restore kernel after an overflow) "
                         "instead of a double-buffered slot")
    ap.add_argument("--event-every", type=int, default=1,
                    help="time the step kernel of every k-th timed step with HIP events its "
                         "launch carries (a timed launch costs the stream a few us, which "
                         "shows on shards whose step takes ~100 us)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run a plain device copy of 1 GiB three times "
                         "(the known-size reference for HBM byte counters under rocprofv3)")
    ap.add_argument("--fold", default="f32", choices=["f32", "bf16-wire"],
                    help="f32: the fold keeps its running sum in fp32; bf16-wire: rounded to "
                         "bf16 after every add, as a ring with bf16 buffers (bf16 replicas only)")
    ap.add_argument("--overlap", type=int, default=0, metavar="K",
                    help="instead of the default line: time a stand-in backward (per part, a "
                         "bf16 GEMM and the write of that part's gradient replicas) followed by "
                         "the step, serially and with the step split into K parts that start as "
                         "their gradients land (device commit)")
    ap.add_argument("--gemm", type=int, default=4096,
                    help="--overlap: the stand-in backward's GEMM is (M x M) @ (M x M) per part")
    ap.add_argument("--offload", action="store_true",
                    help="instead of the default line: time the offloaded step (fp32 master, m, "
                         "v in host memory; host Adam on chunks as they cross)")
    ap.add_argument("--chunk-elems", type=int, default=0,
                    help="--offload: elements per host chunk (0: the library's default)")
    ap.add_argument("--gather", action="store_true",
                    help="instead of the default line: time the stage-3 fetch (whole tensors out "
                         "of the N bf16 rank shards) for one transformer layer and for the model")
    ap.add_argument("--flush-mall", action="store_true",
                    help="write a 1 GiB buffer before every timed step so no step finds its data "
                         "in the 256 MB Infinity Cache; `value` then comes from the step kernels' "
                         "own event times (every step timed), not the wall clock")
    ap.add_argument("--unfused", action="store_true",
                    help="instead of the default line: time the unfused step (reduce kernel to "
                         "an fp32 gradient, host commit rule, Adam kernel from the gradient)")
    ap.add_argument("--graph", type=int, default=0, metavar="G",
                    help="device commit: capture G consecutive steps in one HIP graph and time "
                         "its replays (no host work per step; for launch-bound shards)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.graph and (args.commit != "device" or args.flush_mall or args.overlap or args.offload
                       or args.gather):
        print("--graph times device-commit steps alone", file=sys.stderr)
        return 2

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU's share of the step; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported: run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import workloads as W
    import zero_partitioned_optimizer_amd as Z

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    w = W.get(args.config)
    if args.seed is not None:
        import dataclasses
        w = dataclasses.replace(w, seed=int(args.seed))
    gdt = Z.ZERO_BF16 if w.grad_dtype == "bf16" else Z.ZERO_F32
    wire = args.fold == "bf16-wire"
    if wire:
        if w.grad_dtype != "bf16":
            print("--fold bf16-wire needs bf16 replicas", file=sys.stderr)
            return 2
        gdt = Z.ZERO_BF16_WIRE
    h = Z.zero_layout_build(list(w.numels), w.N, w.A, w.B)
    try:
        S = Z.zero_layout_info_get(h).shard_S
        covered = [(s[2], s[3]) for s in Z.zero_layout_segments(h, args.rank)]
        buckets_t, nb = None, 0
        if args.bucket_elems:
            raw, nb = Z.zero_layout_buckets_raw(h, args.rank, args.bucket_elems)
            buckets_t = torch.frombuffer(bytearray(bytes(raw)[: 16 * nb]), dtype=torch.uint8).to(dev)
    finally:
        Z.zero_layout_free(h)
    log(f"workload {w.name}: S={S} N={w.N} grad={w.grad_dtype} buckets={nb}")
    if args.gather:
        return gather_bench(args, Z, W, w, S)

    tdt = torch.int16 if w.grad_dtype == "bf16" else torch.float32
    fdt = torch.bfloat16 if w.grad_dtype == "bf16" else torch.float32
    cpu = None
    if not (args.no_cpu_baseline or args.overlap or args.offload or args.unfused or args.graph):
        # The oracle's timing runs first, on the first CPU_SAMPLE_ELEMS elements of
        # the same inputs (drawn alone, without the whole shard; elements/s does
        # not depend on the shard length), and only then is the shard allocated.
        # A process that allocates the Llama-70B shard's ~200 GB within a few
        # seconds of another process freeing as much streams it about 5% slower
        # (33.0 against 31.6 ms per step); ten seconds between the two are enough,
        # and the oracle's timing takes longer than that.
        n_cpu = min(S, CPU_SAMPLE_ELEMS)
        log(f"cpu baseline (oracle) on {n_cpu} of {S} elements ...")
        host_reps = []
        for j in range(w.N):
            x = W.device_prefix(W.device_fill_replica, S, n_cpu, fdt, dev, w, covered, args.rank, 0, j)
            x = x.view(tdt).cpu().numpy()
            host_reps.append(x.view(np.uint16) if w.grad_dtype == "bf16" else x)
        p_host = W.device_prefix(W.device_fill_params, S, n_cpu, torch.float32, dev, w, covered,
                                 args.rank).cpu().numpy()
        torch.cuda.empty_cache()
        cpu = cpu_baseline(w, host_reps, p_host, n_cpu, args.cpu_seconds, wire)
        if n_cpu < S:
            cpu["sample"] += f" (the first {n_cpu} of the shard's {S} elements)"
        del host_reps, p_host
    reps = []
    for j in range(w.N):
        buf = torch.empty(S, dtype=fdt, device=dev)
        W.device_fill_replica(buf, w, covered, args.rank, 0, j)
        reps.append(buf.view(tdt))
    p0 = torch.empty(S, dtype=torch.float32, device=dev)
    W.device_fill_params(p0, w, covered, args.rank)
    kw = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.wd,
              loss_scale=w.loss_scale, dynamic=w.dynamic_loss_scale, buckets=buckets_t,
              n_buckets=nb)
    state = args.state if args.commit == "device" else "split"
    if args.commit == "device":
        step = Z.DeviceShardStep(S, w.N, gdt, p0, double_slot=not args.single_slot,
                                 state_layout=Z.ZERO_STATE_TILED if state == "tiled"
                                 else Z.ZERO_STATE_SPLIT, **kw)
    else:
        step = Z.ShardStep(S, w.N, gdt, p0, **kw)
    torch.cuda.synchronize()
    # Python's generation-2 garbage collection walks every object torch and numpy
    # created (tens of milliseconds) and fires after a count of allocations, so
    # sooner or later inside the step loop; collect once now and move what exists
    # out of its reach
    gc.collect()
    gc.freeze()
    if args.overlap:
        return overlap_bench(args, Z, w, S, reps, p0, kw, gdt)
    if args.offload:
        return offload_bench(args, Z, w, S, reps, p0, gdt)
    if args.unfused:
        if nb:
            print("--unfused runs the whole shard (no bucket table)", file=sys.stderr)
            return 2
        return unfused_bench(args, Z, w, S, reps, p0, gdt)
    log("inputs resident; warmup", args.warmup)

    for _ in range(args.warmup):
        step.step(reps)
    if args.graph:
        return graph_bench(args, w, S, step, reps)
    K = args.steps
    every = 1 if args.flush_mall else max(1, args.event_every)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev) if args.flush_mall else None
    ev = {k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for k in range(0, K, every)}
    # record every event once before the timed region: the HIP runtime grows its
    # event pool on first use, a one-time stall of tens of milliseconds
    for e0, e1 in ev.values():
        e0.record()
        e1.record()
    skipped = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if args.commit == "device":
        for k in range(K):
            if flush is not None:
                flush.fill_(float(k))
            step.step(reps, events=ev.get(k))
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        skipped = int(step.state().n_skipped)
    else:
        for k in range(K):
            if flush is not None:
                flush.fill_(float(k))
            st, verdict = step.step(reps, events=ev.get(k))
            skipped += verdict == Z.ZERO_SKIP
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    kms = [a.elapsed_time(b) for a, b in ev.values()]
    if flush is not None:                  # the flushes are not part of the step
        elapsed = sum(kms) / 1e3
    log(f"timed {K} steps in {elapsed:.4f} s; kernel mean {statistics.mean(kms) * 1e3:.1f} us, "
        f"median {statistics.median(kms) * 1e3:.1f} us, skipped {skipped}")

    bpe = w.N * w.grad_bytes + 26
    kernel_s = statistics.mean(kms) / 1e3
    achieved = S * bpe / kernel_s / 1e9
    wall_gbps = S * bpe / (elapsed / K) / 1e9
    # a working set that fits the 256 MB Infinity Cache (plus the replicas reused
    # step after step) is partly served from it: FETCH_SIZE then counts L2 fills,
    # not HBM reads
    fits_mall = S * bpe < 256e6
    # the committed counter runs cover the default launch of each workload: device
    # commit, whole shard, fp32 fold; other launches report no traffic
    default_launch = not wire and args.commit == "device" and not args.bucket_elems
    traffic = measured_traffic(w.name, state) if default_launch else None
    out = {
        "metric": METRIC,
        "value": S * K / elapsed,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": elapsed / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name} shard, rank {args.rank} of N={w.N}", "shard_elems": S,
                   "n_replicas": w.N, "grad_dtype": w.grad_dtype, "state_dtype": "f32",
                   "bytes_per_elem": bpe, "bucket_elems": args.bucket_elems,
                   "commit": args.commit, "state": state, "fold": args.fold,
                   "mall_flushed": bool(args.flush_mall),
                   "slot": "single" if (args.single_slot or args.commit == "host") else "double",
                   "seed": w.seed},
        "step_gbps": wall_gbps,
        "wall_gbps": wall_gbps,
        "wall_frac": wall_gbps / HBM_PEAK_GBS,
        # measured bytes (the committed counter runs) over the same mean kernel time
        "physical_gbps": traffic / kernel_s / 1e9 if traffic else None,
        "kernel_us_mean": kernel_s * 1e6,
        "kernel_us_median": statistics.median(kms) * 1e3,
        "kernel_us_min": min(kms) * 1e3,
        "kernel_samples": len(kms),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_kind": ("L2 fill bytes (FETCH_SIZE, MALL hits included) + written bytes"
                                      if fits_mall else "HBM bytes read + written")},
        "cpu_baseline": cpu,
        "skipped_steps": skipped,
    }
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["calibration_copy_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4,
                                         "launches": 3}
        del src, dst
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
