"""The CPU oracle against its pins, and the pins against planted mistakes."""
import numpy as np
import pytest

import oracle
from oracle import build as oracle_build
import pins


def _proj(mutant=0):
    return lambda x, w: oracle.proj(x, w, mutant=mutant)


def _proj_sum(mutant=0):
    return lambda x, w: oracle.proj(x, w, want_sum=True, mutant=mutant)


def _round(mutant=0):
    return lambda v: oracle.round_bf16(v, mutant=mutant)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    if pin in (pins.invariants, pins.unrounded_sum):
        pin(_proj(), _round(), proj_sum=_proj_sum())
    else:
        pin(_proj(), _round())


def test_thread_count_does_not_change_result():
    rng = np.random.default_rng(3)
    xb = (rng.standard_normal((3, 777)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wb = ((rng.standard_normal((101, 777)) * 0.02).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y1, s1 = oracle.proj(xb, wb, threads=1, want_sum=True)
    y7, s7 = oracle.proj(xb, wb, threads=7, want_sum=True)
    assert np.array_equal(y1, y7) and np.array_equal(s1, s7)


def test_strided_rows_and_empty_shapes():
    rng = np.random.default_rng(4)
    big = (rng.standard_normal((4, 300)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wb = ((rng.standard_normal((9, 256)) * 0.02).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    view = big[:, :256]                      # row stride 300, like a column gather
    assert np.array_equal(oracle.proj(view, wb), oracle.proj(np.ascontiguousarray(view), wb))
    assert oracle.proj(big[:0, :256], wb).shape == (0, 9)
    assert oracle.proj(big[:, :256], wb[:0]).shape == (4, 0)


# A planted mistake in the oracle (compiled in with -DORACLE_MUTANT=n) must
# fail at least one pin: dropped term, wrong weight index, truncation, ties
# away from zero, float accumulator, wrong x row, double rounding via float,
# unrounded sums stored transposed (only the S output is wrong there).
@pytest.mark.parametrize("mutant", [1, 2, 3, 4, 5, 6, 7, 8])
def test_pins_catch_planted_mistake(mutant):
    oracle_build.build(mutant)
    failures = []
    for pin in pins.ALL_PINS:
        try:
            if pin in (pins.invariants, pins.unrounded_sum):
                pin(_proj(mutant), _round(mutant), proj_sum=_proj_sum(mutant))
            elif pin is pins.one_hot:
                pin(_proj(mutant), _round(mutant), shapes=((640, 256), (256, 384)))
            else:
                pin(_proj(mutant), _round(mutant))
        except AssertionError:
            failures.append(pin.__name__)
    assert failures, f"mutant {mutant} passed every pin"
    if mutant == 8:
        # the rounded outputs are untouched; only the sum pin can see it
        assert "unrounded_sum" in failures, failures
