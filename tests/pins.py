"""Pins of the CPU oracle: checks against facts other than the oracle itself.

Each pin takes the oracle's two entry points (the projection and the rounding
step) as callables, so the same pins run against the real oracle and against
builds with a planted mistake (tests/test_oracle.py shows every planted
mistake fails at least one pin).  A pin raises AssertionError on failure.

What pins what:
  exact_bruteforce  exact rationals on tiny shapes: summation, indexing, rounding
  golden_ties       hand-derived ties (tests/golden/rne_ties.txt): ties-to-even
  closed_forms      constant inputs with known integer results at full K
  one_hot           identity / one-hot weights at full shapes: row/column indexing
  invariants        power-of-two scaling, negation, permutations, linearity
  numpy_f64         numpy float64 products + an independent bit-level rounder
  rounding          the rounding step alone against exact rational rounding,
                    plus the non-finite cases against binary32's encodings
  unrounded_sum     the unrounded double sums S (the reference value of the
                    GPU tests' aggregate gate) against exact rational sums,
                    within the error bound of K-term double accumulation, and
                    against numpy float64 products
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

from oracle import exact

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _f32_to_bf16_bits_trunc_exact(v: np.ndarray) -> np.ndarray:
    """BF16 bits of float32 values that are already exactly BF16."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value is not exactly a BF16"
    return (u >> 16).astype(np.uint16)


def _bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(
        np.float32).astype(np.float64)


def _random_bf16(rng, shape, std):
    """Random finite BF16 bit patterns ~ N(0, std) (rounded by bit arithmetic:
    these only need to be valid BF16 values, any rounding will do)."""
    v = (rng.standard_normal(shape) * std).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def _wide_bf16(rng, shape):
    """BF16 values with random signs, mantissas and exponents in [-20, 20]."""
    sign = rng.integers(0, 2, shape).astype(np.uint16) << 15
    exp = (rng.integers(-20, 21, shape) + 127).astype(np.uint16) << 7
    man = rng.integers(0, 128, shape).astype(np.uint16)
    return sign | exp | man


def _hex_row(s):
    return [int(t, 16) for t in s.split(",")]


def load_golden_ties():
    cases = []
    with open(os.path.join(GOLDEN, "rne_ties.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            xs, ws, ys = (p.strip() for p in line.split("|"))
            cases.append((_hex_row(xs), _hex_row(ws), int(ys, 16)))
    return cases


# --------------------------------------------------------------------------
def exact_bruteforce(proj, rounder=None):
    rng = _rng(1234)
    cases = []
    for (B, N, K, std_x, std_w) in [(1, 1, 1, 1.0, 0.02), (2, 3, 17, 1.0, 0.02),
                                    (3, 8, 64, 1.0, 0.02), (1, 5, 40, 1.0, 1.0)]:
        cases.append((_random_bf16(rng, (B, K), std_x),
                      _random_bf16(rng, (N, K), std_w)))
    cases.append((_wide_bf16(rng, (3, 33)), _wide_bf16(rng, (7, 33))))
    # near-ties: 1 + 2^-8 is a tie in [1,2); a term far below float32's
    # precision (but inside double's) decides the direction.
    one, h8, t30, mt30 = 0x3F80, 0x3B80, 0x3080, 0xB080  # 1, 2^-8, +-2^-30
    cases.append((np.array([[one, h8, t30], [one, h8, mt30], [0x3F81, h8, t30]],
                           dtype=np.uint16),
                  np.array([[one, one, one], [one, one, 0]], dtype=np.uint16)))
    for xb, wb in cases:
        got = np.asarray(proj(xb, wb))
        want = np.array(exact.proj_exact(xb, wb), dtype=np.uint16)
        assert got.shape == want.shape, (got.shape, want.shape)
        bad = np.argwhere(got != want)
        assert bad.size == 0, (
            f"exact brute force: {len(bad)} mismatches, first at {bad[0]}: "
            f"{got[tuple(bad[0])]:#06x} vs {want[tuple(bad[0])]:#06x}")


def golden_ties(proj, rounder=None):
    for xs, ws, want in load_golden_ties():
        xb = np.array([xs], dtype=np.uint16)
        wb = np.array([ws], dtype=np.uint16)
        got = int(np.asarray(proj(xb, wb))[0, 0])
        assert got == want, f"golden tie {xs}.{ws}: {got:#06x} != {want:#06x}"


def closed_forms(proj, rounder=None):
    # x == 1, W == 2^-10 over K = 7168 sums to exactly 7; W == 2^-12 over
    # K = 12288 sums to exactly 3.  2^-10 = 0x3A80, 2^-12 = 0x3980.
    for K, wbits, want in [(7168, 0x3A80, 0x40E0), (12288, 0x3980, 0x4040)]:
        xb = np.full((2, K), 0x3F80, dtype=np.uint16)
        xb[1] = 0xBF80                                    # second row: -1
        wb = np.full((3, K), wbits, dtype=np.uint16)
        got = np.asarray(proj(xb, wb))
        assert np.all(got[0] == want), f"closed form K={K}: {got[0]}"
        assert np.all(got[1] == (want | 0x8000)), f"closed form K={K}: {got[1]}"


def one_hot(proj, rounder=None, shapes=((14560, 7168), (7168, 12288),
                                        (49376, 7168)), B=2):
    rng = _rng(77)
    for (N, K) in shapes:
        xb = _random_bf16(rng, (B, K), 1.0)
        for scale_bits, scale in [(0x3F80, 1.0), (0x3E00, 0.125)]:
            wb = np.zeros((N, K), dtype=np.uint16)
            n = np.arange(N)
            wb[n, n % K] = scale_bits
            got = np.asarray(proj(xb, wb))
            want_vals = _bf16_to_f64(xb)[:, n % K] * scale
            want = _f32_to_bf16_bits_trunc_exact(want_vals.astype(np.float32))
            bad = np.argwhere(got != want)
            assert bad.size == 0, (
                f"one-hot N={N} K={K} scale={scale}: {len(bad)} mismatches, "
                f"first {bad[0]}")


def invariants(proj, rounder=None, proj_sum=None):
    rng = _rng(99)
    B, N, K = 4, 48, 384
    xb = _random_bf16(rng, (B, K), 1.0)
    wb = _random_bf16(rng, (N, K), 0.02)
    y = np.asarray(proj(xb, wb))
    # power-of-two scaling of x: exponent field shifts, no overflow here
    for j in (-3, 5):
        xs = xb.copy()
        nz = (xs & 0x7FFF) != 0
        xs[nz] = (xs[nz].astype(np.int32) + (j << 7)).astype(np.uint16)
        ys = np.asarray(proj(xs, wb))
        yz = (y & 0x7FFF) != 0
        want = y.copy()
        want[yz] = (want[yz].astype(np.int32) + (j << 7)).astype(np.uint16)
        assert np.array_equal(ys, want), f"scaling by 2^{j} not exact"
    # negation
    assert np.array_equal(np.asarray(proj(xb ^ 0x8000, wb)) & 0x7FFF, y & 0x7FFF)
    nz = (y & 0x7FFF) != 0
    assert np.array_equal((np.asarray(proj(xb ^ 0x8000, wb)) ^ 0x8000)[nz], y[nz])
    # row permutation of x permutes rows of y; of W permutes columns
    p = rng.permutation(B)
    assert np.array_equal(np.asarray(proj(xb[p], wb)), y[p])
    q = rng.permutation(N)
    assert np.array_equal(np.asarray(proj(xb, wb[q])), y[:, q])
    if proj_sum is None:
        return
    # permuting k consistently leaves the double sum unchanged to ~1e-15
    _, S = proj_sum(xb, wb)
    r = rng.permutation(K)
    _, Sp = proj_sum(xb[:, r], wb[:, r])
    scale = np.abs(_bf16_to_f64(xb)) @ np.abs(_bf16_to_f64(wb)).T
    assert np.all(np.abs(S - Sp) <= 1e-14 * scale), "k permutation changed S"
    # linearity with disjoint supports: S(x1) + S(x2) == S(x1 + x2)
    mask = rng.integers(0, 2, (B, K)).astype(bool)
    x1 = np.where(mask, xb, np.uint16(0))
    x2 = np.where(mask, np.uint16(0), xb)
    _, S1 = proj_sum(x1, wb)
    _, S2 = proj_sum(x2, wb)
    assert np.all(np.abs(S1 + S2 - S) <= 1e-14 * scale), "linearity"


def bits_round_f64_to_bf16(v: np.ndarray) -> np.ndarray:
    """Independent RNE of normal-range float64 to BF16 by integer bit
    arithmetic on the binary64 encoding (drop 45 mantissa bits, ties to
    even, rebias the exponent 1023 -> 127)."""
    u = np.asarray(v, dtype=np.float64).view(np.uint64)
    sign = (u >> np.uint64(63)).astype(np.uint16) << 15
    mag = u & np.uint64(0x7FFFFFFFFFFFFFFF)
    lsb = (mag >> np.uint64(45)) & np.uint64(1)
    r = (mag + np.uint64((1 << 44) - 1) + lsb) >> np.uint64(45)
    # r = (exp64 << 7) | man7, with the rounding carry already propagated
    exp64 = (r >> np.uint64(7)).astype(np.int64)
    man = (r & np.uint64(0x7F)).astype(np.uint16)
    exp32 = exp64 - 1023 + 127
    assert np.all((exp32 >= 1) & (exp32 <= 254)), "outside BF16 normal range"
    return sign | (exp32.astype(np.uint16) << 7) | man


def numpy_f64(proj, rounder=None):
    rng = _rng(5)
    B, N, K = 4, 512, 1024
    xb = _random_bf16(rng, (B, K), 1.0)
    wb = _random_bf16(rng, (N, K), 0.02)
    S = _bf16_to_f64(xb) @ _bf16_to_f64(wb).T     # numpy / BLAS float64
    want = bits_round_f64_to_bf16(S)
    got = np.asarray(proj(xb, wb))
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    # both are double sums in different orders: only a near-tie may differ
    assert diff.max() <= 1, "numpy float64 product disagrees by > 1 ulp"
    assert np.count_nonzero(diff) <= 1, "too many near-tie disagreements"


def rounding(proj, rounder):
    rng = _rng(11)
    vals = list(rng.standard_normal(4000) * np.exp2(rng.integers(-30, 30, 4000)))
    # exact ties and their neighbours at several binades
    for e in (-20, -1, 0, 1, 7, 100):
        for m in (0, 1, 2, 127):
            base = (1 + m / 128.0) * 2.0 ** e
            half = 2.0 ** (e - 8)
            vals += [base + half, base - half, base + half * (1 + 2 ** -30),
                     -(base + half)]
    # subnormal BF16 range, the normal/subnormal boundary and overflow
    vals += [2.0 ** -127, 3 * 2.0 ** -134, 2.0 ** -134, 2.0 ** -133 * 1.5,
             2.0 ** -126 - 2.0 ** -134, (2 - 2 ** -8) * 2.0 ** 127,
             (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** 128, 0.0, -0.0]
    v = np.array(vals, dtype=np.float64)
    got = np.asarray(rounder(v))
    for val, g in zip(v, got):
        want = exact.round_fraction_to_bf16(Fraction(float(val)))
        if val == 0 and np.signbit(val):
            want = 0x8000                      # a zero keeps its sign
        assert int(g) == want, f"rounding {val!r}: {int(g):#06x} != {want:#06x}"
    # Non-finite sums have no exact value: any NaN maps to the canonical
    # quiet NaN (sign dropped) and an infinity keeps its sign.  The expected
    # patterns are the upper halves of binary32's own encodings of NaN and of
    # +-inf (BF16 is the top half of binary32).
    special = np.array([np.nan, -np.nan, np.inf, -np.inf], dtype=np.float64)
    f32 = special.astype(np.float32).view(np.uint32) >> np.uint32(16)
    want = [int(f32[0]) & 0x7FFF, int(f32[1]) & 0x7FFF, int(f32[2]), int(f32[3])]
    got = [int(g) for g in np.asarray(rounder(special))]
    assert want[0] == 0x7FC0 and want[2] == 0x7F80 and want[3] == 0xFF80, want
    assert got == want, f"non-finite rounding: {[hex(g) for g in got]}"


def _sum_bound(xb, wb):
    """Error bound of a K-term double sum, as exact rationals per (b, n):
    gamma_(K-1) * sum_k |x[b,k] W[n,k]|, gamma_m = m u / (1 - m u), u = 2^-53
    (each BF16 x BF16 product is exact in double; only the K-1 additions
    round)."""
    K = xb.shape[1]
    u = Fraction(1, 2 ** 53)
    m = max(K - 1, 0)
    gamma = m * u / (1 - m * u)
    xs = [[abs(exact.bf16_to_fraction(int(v))) for v in row] for row in xb]
    ws = [[abs(exact.bf16_to_fraction(int(v))) for v in row] for row in wb]
    return [[gamma * sum((a * b for a, b in zip(xr, wr)), Fraction(0)) for wr in ws]
            for xr in xs]


def unrounded_sum(proj, rounder=None, proj_sum=None):
    assert proj_sum is not None, "this pin needs the oracle's sum output"
    rng = _rng(4321)
    # B != N everywhere, so a transposed or mis-strided store cannot land on
    # the right element by symmetry.
    cases = [(_random_bf16(rng, (2, 17), 1.0), _random_bf16(rng, (3, 17), 0.02)),
             (_random_bf16(rng, (3, 64), 1.0), _random_bf16(rng, (8, 64), 0.02)),
             (_random_bf16(rng, (1, 40), 1.0), _random_bf16(rng, (5, 40), 1.0)),
             (_wide_bf16(rng, (4, 33)), _wide_bf16(rng, (7, 33)))]
    for xb, wb in cases:
        _, S = proj_sum(xb, wb)
        S = np.asarray(S)
        assert S.shape == (xb.shape[0], wb.shape[0]), S.shape
        E = exact.exact_sums(xb, wb)
        bound = _sum_bound(xb, wb)
        for b in range(S.shape[0]):
            for n in range(S.shape[1]):
                err = abs(Fraction(float(S[b, n])) - E[b][n])
                assert err <= bound[b][n], (
                    f"S[{b},{n}] = {S[b, n]!r} is {float(err):.3g} from the exact sum "
                    f"{float(E[b][n])!r} (bound {float(bound[b][n]):.3g})")
    # A second, independent float64 sum: numpy's matrix product.  Both are
    # double sums of the same exact products, each within gamma_(K-1) of the
    # exact value, so they agree to 2 gamma_(K-1) |x| |W|^T < 1e-12 of it.
    rng = _rng(6)
    B, N, K = 4, 512, 1024
    xb = _random_bf16(rng, (B, K), 1.0)
    wb = _random_bf16(rng, (N, K), 0.02)
    xd, wd = _bf16_to_f64(xb), _bf16_to_f64(wb)
    S_np = xd @ wd.T
    scale = np.abs(xd) @ np.abs(wd).T
    _, S = proj_sum(xb, wb)
    S = np.asarray(S)
    assert S.shape == (B, N)
    bad = np.argwhere(np.abs(S - S_np) > 1e-12 * scale)
    assert bad.size == 0, f"S differs from numpy float64 at {len(bad)} elements, first {bad[0]}"


ALL_PINS = (exact_bruteforce, golden_ties, closed_forms, one_hot, invariants,
            numpy_f64, rounding, unrounded_sum)
