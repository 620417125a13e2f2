"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import os
import re

import numpy as np
import torch

import oracle
import parity
import tp1_skinny_bf16_amd as tp
import workloads as wl

DEV = torch.device("cuda:0")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def say(*a):
    print(*a, flush=True)


def gpu_run(plan, x_cpu, W_dev, B=None, ldx_pad=0):
    """y bits [B, N] of the HIP path; x optionally read with a row stride."""
    B = x_cpu.shape[0] if B is None else B
    K = x_cpu.shape[1]
    if ldx_pad:
        big = torch.zeros((B, K + ldx_pad), dtype=torch.bfloat16)
        big[:, :K] = x_cpu[:B]
        xd = big.to(DEV)[:, :K]
    else:
        xd = x_cpu[:B].contiguous().to(DEV)
    y = torch.empty((B, plan.N), dtype=torch.bfloat16, device=DEV)
    plan.run(xd, W_dev, y)
    torch.cuda.synchronize()
    return wl.bits(y.cpu())


def check_random(label, y_bits, x_cpu, W_cpu, threads=None):
    """G1/G2/D1 gates of y_bits against the oracle, over every output."""
    xb = wl.bits(x_cpu)
    wb = wl.bits(W_cpu)
    y_orc, S = oracle.proj(xb, wb, want_sum=True, threads=threads)
    wmax = float(np.abs(parity.bf16_to_f64(wb)).max())
    rep = parity.gate(y_bits, y_orc, S, xb, wmax, label=label)
    say(f"[{label}] elements={rep['elements']} g1_fail={rep['g1_fail']} "
        f"g2={rep['g2_max_beyond_rounding']:.3g}/{rep['g2_limit']:.3g} "
        f"diff_frac={rep['d1_diff_frac']:.2e} max_ulp={rep['max_ulp']}")
    assert rep["ok"], rep
    return rep


def check_exact(label, y_bits, x_cpu, W_cpu):
    """Bitwise equality with the oracle over every output (exact-sum or
    closed-form inputs)."""
    xb = wl.bits(x_cpu)
    wb = wl.bits(W_cpu)
    want = oracle.proj(xb, wb)
    bad = np.argwhere(y_bits != want)
    say(f"[{label}] exact: {y_bits.size} elements, {len(bad)} mismatches")
    assert bad.size == 0, f"{label}: first mismatch at {bad[0]}: " \
        f"{y_bits[tuple(bad[0])]:#06x} vs {want[tuple(bad[0])]:#06x}"


def tactic_label(plan, B):
    t, b = plan.tactic(B)
    return f"{t.kernel_name} bcap={t.bcap} S={t.split} rows={t.rows} waves={t.waves} wpc={t.wpc} bin={b}"


def pipe_instances():
    """The compiled pipelined-kernel instances, read from the library's
    instance list (plan.hpp), so every compiled instance is tested."""
    src = open(os.path.join(ROOT, "tp1_skinny_bf16_amd", "csrc", "plan.hpp")).read()
    blk = src[src.index("TP1_PIPE_INSTANCES(X)"):]
    blk = blk[:blk.index("\n\n")]
    pat = r"X\((\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)\)"
    return [tuple(map(int, m)) for m in re.findall(pat, blk)]


def candidate_tactics(N: int, K: int, bin_: int):
    """A spread of valid tactics for a bin (every family and split path)."""
    out = []
    if bin_ <= 8:
        for bc in (1, 2, 4, 8):
            if bc < bin_:
                continue
            for rows in (1, 2, 4):
                for split in (1, 3):
                    for waves, wpc in ((4, 8), (2, 4), (8, 16), (1, 1), (3, 5)):
                        out.append(tp.Tactic(tp.KERNEL_STREAM, bc, split, rows, waves, wpc))
                    out.append(tp.Tactic(tp.KERNEL_STREAM_DOT2, bc, split, rows, 4, 8))
    for bc, shapes in ((16, ((4, 1, 128, 1), (4, 1, 256, 2), (4, 1, 512, 1), (8, 1, 128, 2),
                             (16, 1, 128, 1))),
                       (32, ((4, 1, 128, 2), (4, 2, 128, 1), (8, 2, 256, 1))),
                       (64, ((4, 1, 128, 1), (4, 2, 128, 2), (4, 4, 128, 1), (8, 2, 256, 1))),
                       (128, ((4, 2, 128, 1), (4, 4, 128, 1))),
                       (256, ((4, 4, 128, 1), (2, 4, 128, 1)))):
        if bc < bin_:
            continue
        for (rows, waves, kc, depth) in shapes:
            for split in (1, 3):
                for wpc in (1, 2):
                    out.append(tp.Tactic(tp.KERNEL_MFMA_XS, bc, split, rows, waves, wpc, kc, depth))
                    if wpc == 1:  # the same with a staggered chunk order
                        out.append(tp.Tactic(tp.KERNEL_MFMA_XS, bc, split, rows, waves, wpc, kc,
                                             depth, stagger=1))
    # every compiled pipelined instance: X(bcap, rows, waves, kw, kc, depth, nw)
    pipe = {}
    for (bc, rows, waves, kw, kc, depth, nw) in pipe_instances():
        pipe.setdefault(bc, []).append((rows, waves, kw, kc, depth, nw))
    for bc, shapes in pipe.items():
        # each instance at the bins it would serve: capacity / 2 < bin <= capacity
        if bc < bin_ or (bc > 16 and 2 * bin_ <= bc):
            continue
        for (rows, waves, kw, kc, depth, nw) in shapes:
            for split in (1, 3):
                for wpc in ((1, 2) if nw == 4 else (1,)):
                    out.append(tp.Tactic(tp.KERNEL_MFMA_PIPE, bc, split, rows, waves, wpc, kc,
                                         depth, kw, nw))
                    if wpc == 1:  # the same with a staggered chunk order
                        out.append(tp.Tactic(tp.KERNEL_MFMA_PIPE, bc, split, rows, waves, wpc,
                                             kc, depth, kw, nw, stagger=1))
    return out
