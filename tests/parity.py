"""Parity gates between a GPU result and the CPU oracle (test infrastructure).

The dep page (vllm.models.kimi_k3.nvidia.specialized_decode.runtime.dep,
opening text) lets a kernel choose its FP32 summation order, so several BF16
results are correct wherever the FP32 sum lands near a rounding midpoint.
The gates therefore allow one-step differences from the oracle:

G1 (per element): BF16 ulp distance <= 2, or
    |y - y_oracle| <= 1e-3 * ||x_b||_2 * max|W|.
G2 (aggregate, error beyond the output's own rounding):
    max_e max(0, |y - S| - ulp(y)/2) <= 0.005 * RMS(y_oracle),
    S being the oracle's unrounded double sum.
D1 (diagnostic, gated loosely): at most 1e-3 * n + 3 of the n elements
    differ from the oracle at all (an FP32 kernel differs only at near-ties,
    ~1e-5..1e-4 of them; a truncating epilogue would differ at ~50%; the
    constant 3 keeps a single legitimate flip in a few hundred elements from
    failing a fraction test).
Exact-sum workloads are compared bit for bit instead.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(
        np.float32).astype(np.float64)


def ordered(bits):
    """Map BF16 patterns to integers whose order is the numeric order (+-0 equal)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_distance(a_bits, b_bits):
    return np.abs(ordered(a_bits) - ordered(b_bits))


def bf16_spacing(bits):
    """Spacing of BF16 values in the binade of each value (2^-133 at zero)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int32)
    exp = (b >> 7) & 0xFF
    e = np.maximum(exp, 1) - 127 - 7
    return np.exp2(e.astype(np.float64))


def gate(y_bits, y_orc_bits, S, x_bits, w_absmax: float, *, label: str = "",
         rows=None):
    """Evaluate G1/G2/D1; returns a report dict with 'ok' and details.

    y_bits, y_orc_bits, S: [B', N'] (possibly a sample of rows/columns)
    x_bits: the [B', K] rows the outputs belong to (for ||x_b||_2)
    w_absmax: max |W| over the whole weight of the call
    """
    y = np.asarray(y_bits, dtype=np.uint16)
    yo = np.asarray(y_orc_bits, dtype=np.uint16)
    assert y.shape == yo.shape == np.shape(S), (y.shape, yo.shape, np.shape(S))
    yv = bf16_to_f64(y)
    yov = bf16_to_f64(yo)
    S = np.asarray(S, dtype=np.float64)
    xn = np.sqrt(np.sum(bf16_to_f64(x_bits) ** 2, axis=1))[:, None]
    ulp = ulp_distance(y, yo)
    absdiff = np.abs(yv - yov)
    with np.errstate(invalid="ignore"):
        g1_elem = (ulp <= 2) | (absdiff <= 1e-3 * xn * w_absmax)
    g1_elem &= np.isfinite(yv)
    rms = float(np.sqrt(np.mean(yov ** 2))) if yov.size else 0.0
    beyond = np.maximum(0.0, np.abs(yv - S) - 0.5 * bf16_spacing(y))
    g2 = float(beyond.max()) if beyond.size else 0.0
    ndiff = int(np.count_nonzero(ulp))
    frac = ndiff / max(1, y.size)
    rep = {
        "label": label,
        "elements": int(y.size),
        "g1_fail": int(np.count_nonzero(~g1_elem)),
        "g2_max_beyond_rounding": g2,
        "g2_limit": 0.005 * rms,
        "rms": rms,
        "d1_literal_maxabs_over_rms": float(absdiff.max() / rms) if rms > 0 else 0.0,
        "d1_diff_1ulp": int(np.count_nonzero(ulp == 1)),
        "d1_diff_2ulp": int(np.count_nonzero(ulp == 2)),
        "d1_diff_frac": frac,
        "max_ulp": int(ulp.max()) if ulp.size else 0,
    }
    if rep["g1_fail"]:
        idx = np.argwhere(~g1_elem)[0]
        rep["worst"] = {"index": [int(i) for i in idx],
                        "gpu": float(yv[tuple(idx)]), "oracle": float(yov[tuple(idx)])}
    rep["d1_limit"] = 1e-3 * y.size + 3
    rep["ok"] = (rep["g1_fail"] == 0 and g2 <= rep["g2_limit"] and ndiff <= rep["d1_limit"])
    return rep


def assert_gate(*args, **kw):
    rep = gate(*args, **kw)
    assert rep["ok"], f"parity gate failed: {rep}"
    return rep
