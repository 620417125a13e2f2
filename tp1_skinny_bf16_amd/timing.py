"""Timing of projection calls on the GPU with HIP events (via torch events on
the stream the calls are enqueued on).

Weights are rotated over distinct copies so that consecutive calls never
find their weight in the 256 MB Infinity Cache (MALL) or the L2: every call
then streams its weight from HBM, which is what a decode step over many
layers does.
"""
from __future__ import annotations

import statistics
import time

import torch

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 MFMA peak, TFLOP/s


def rotation_copies(W0: torch.Tensor, min_total_bytes: float = 1.0e9,
                    max_copies: int = 64, seed: int = 1000):
    """[W0] plus distinct copies, drawn on the device, until the copies hold
    at least `min_total_bytes` (values: same distribution, N(0, 0.02)).  A
    small weight (a tensor-parallel shard of 13-100 MB) takes up to 64 copies,
    so that even then the set is four times the 256 MB MALL."""
    copies = [W0]
    nbytes = W0.numel() * W0.element_size()
    g = torch.Generator(device=W0.device)
    g.manual_seed(seed)
    while len(copies) * nbytes < min_total_bytes and len(copies) < max_copies:
        t = torch.randn(W0.shape, generator=g, device=W0.device, dtype=torch.float32)
        copies.append(t.mul_(0.02).to(torch.bfloat16))
        del t
    return copies


def time_calls(calls, warmup: int = 5, reps: int = 50, warm_seconds: float = 0.25):
    """Time a list of zero-argument callables, run round-robin.

    Returns per-call durations in microseconds (GPU event time of each call,
    each bracketed by its own pair of events) and, from a second pass of the
    same calls enqueued back to back between one pair of events, the mean
    time per call without per-call markers.
    """
    stream = torch.cuda.current_stream()
    n = len(calls)
    for i in range(warmup * n):
        calls[i % n]()
    # keep the GPU busy for a moment first: after host-side work the clocks
    # have dropped, and the first timings would run slow
    t_end = time.perf_counter() + warm_seconds
    while time.perf_counter() < t_end:
        for c in calls:
            c()
        torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for i in range(reps):
        starts[i].record(stream)
        calls[i % n]()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(reps):
        calls[i % n]()
    t1.record(stream)
    torch.cuda.synchronize()
    per = [s.elapsed_time(e) * 1e3 for s, e in zip(starts, ends)]
    total = t0.elapsed_time(t1) * 1e3
    return {
        "us_median": statistics.median(per),
        "us_p10": sorted(per)[max(0, int(0.1 * reps) - 1)],
        "us_p90": sorted(per)[min(reps - 1, int(0.9 * reps))],
        "us_mean_b2b": total / reps,
        "reps": reps,
    }


def time_graph(calls, replays: int = 5):
    """Mean GPU time per call of `calls` (zero-argument callables that launch
    on torch's current stream) captured in order into one graph and
    replayed: the host's launch submission, ~6-10 us per call through the
    binding, is then off the critical path, which matters for kernels of
    about that length.  Returns microseconds per call."""
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        for c in calls:
            c()
    cur.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for c in calls:
            c()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(cur)
    for _ in range(replays):
        graph.replay()
    t1.record(cur)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / (replays * len(calls))
    del graph
    return us


def gbs(nbytes: float, us: float) -> float:
    return nbytes / (us * 1e-6) / 1e9
