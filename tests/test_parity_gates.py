"""Unit tests of the parity gates on hand-made BF16 pairs (CPU only)."""
import numpy as np

import parity


def test_ulp_distance_orders_signs_and_zero():
    a = np.array([0x3F80, 0x3F80, 0x0000, 0x8000, 0x0001, 0xBF80], dtype=np.uint16)
    b = np.array([0x3F81, 0x3F7F, 0x8000, 0x0001, 0x8001, 0x3F80], dtype=np.uint16)
    d = parity.ulp_distance(a, b)
    assert list(d[:5]) == [1, 1, 0, 1, 2]
    assert d[5] == 2 * 0x3F80


def test_spacing():
    s = parity.bf16_spacing(np.array([0x3F80, 0x4000, 0x0000, 0x0080], dtype=np.uint16))
    assert list(s) == [2.0 ** -7, 2.0 ** -6, 2.0 ** -133, 2.0 ** -133]


def _case(y, yo, S, xrow=(1.0,)):
    xb = (np.array([xrow], dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return parity.gate(np.array([y], dtype=np.uint16), np.array([yo], dtype=np.uint16),
                       np.array([S], dtype=np.float64), xb, 0.02)


def test_one_step_flip_at_a_tie_passes():
    # S just above the 1 / 1+2^-7 midpoint; GPU took the lower neighbour.
    S = [1 + 2 ** -8 + 1e-9]
    rep = _case([0x3F80], [0x3F81], S)
    assert rep["g1_fail"] == 0 and rep["g2_max_beyond_rounding"] < 1e-8


def test_large_error_fails_both_gates():
    rep = _case([0x3F90], [0x3F80], [1.0])      # 16 ulps off
    assert rep["g1_fail"] == 1 and not rep["ok"]
    assert rep["g2_max_beyond_rounding"] > rep["g2_limit"]


def test_many_flips_fail_d1():
    n = 2000
    y = np.full((1, n), 0x3F80, dtype=np.uint16)
    yo = y.copy()
    yo[0, :10] = 0x3F81                         # 10 > 0.001 * 2000 + 3 differ
    S = np.full((1, n), 1.0)
    xb = np.full((1, 4), 0x3F80, dtype=np.uint16)
    rep = parity.gate(y, yo, S, xb, 0.02)
    assert rep["g1_fail"] == 0 and not rep["ok"] and rep["d1_diff_frac"] == 0.005


def test_nonfinite_gpu_output_fails():
    rep = _case([0x7FC0], [0x3F80], [1.0])
    assert rep["g1_fail"] == 1


def test_single_flip_in_a_small_sample_passes():
    y = np.full((1, 231), 0x3F80, dtype=np.uint16)
    yo = y.copy()
    yo[0, 5] = 0x3F81
    S = np.full((1, 231), 1.0 + 2 ** -8)
    rep = parity.gate(y, yo, S, np.full((1, 4), 0x3F80, dtype=np.uint16), 0.02)
    assert rep["ok"], rep
