"""Exact-rational brute force of the TP1 projection for tiny shapes.

TEST INFRASTRUCTURE ONLY (a pin for the C oracle; never used by the product).

The result definition is the one of the vLLM API page "vllm.models.kimi_k3.
nvidia.specialized_decode.runtime.dep" (section "DepProjection": the GEMM of x
with the transposed N x K weight; opening text: BF16 in and out).  Here every
BF16 is decoded to an exact Fraction, the dot product is summed exactly, and
the exact sum is rounded to BF16 by integer arithmetic with ties to even.
Nothing here uses floating point, so it cannot share a rounding mistake with
oracle.c, which sums in double and rounds with frexp/rint.
"""
from fractions import Fraction


def bf16_to_fraction(h: int) -> Fraction:
    """Exact value of a finite BF16 bit pattern (1 sign, 8 exponent, 7 mantissa)."""
    h &= 0xFFFF
    sign = -1 if h & 0x8000 else 1
    exp = (h >> 7) & 0xFF
    man = h & 0x7F
    if exp == 0xFF:
        raise ValueError("non-finite BF16 has no exact value")
    if exp == 0:                       # subnormal: man * 2^-133
        return sign * Fraction(man, 1 << 133)
    e = exp - 127 - 7                  # (128 + man) * 2^(exp-127-7)
    v = Fraction(128 + man)
    v = v * (1 << e) if e >= 0 else v / (1 << -e)
    return sign * v


def _floor_log2(a: Fraction) -> int:
    """floor(log2 a) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # now 2^(e-1) < a < 2^(e+1); settle which side of 2^e a lies on
    p = Fraction(2) ** e
    return e if a >= p else e - 1


def _encode(v: Fraction, negative: bool) -> int:
    """Bit pattern of an exactly representable BF16 magnitude v >= 0."""
    sign = 0x8000 if negative else 0
    if v == 0:
        return sign
    if v >= Fraction(2) ** 128:
        return sign | 0x7F80
    E = _floor_log2(v)
    if E < -126:
        m = v * (Fraction(2) ** 133)
        assert m.denominator == 1 and m.numerator < 128
        return sign | m.numerator
    m = v / (Fraction(2) ** (E - 7))
    assert m.denominator == 1 and 128 <= m.numerator < 256
    return sign | ((E + 127) << 7) | (m.numerator - 128)


def round_fraction_to_bf16(s: Fraction) -> int:
    """Nearest BF16 to the exact rational s, ties to the even mantissa."""
    negative = s < 0
    a = -s if negative else s
    if a == 0:
        return 0x8000 if negative else 0
    e = max(_floor_log2(a), -126)
    q = Fraction(2) ** (e - 7)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return _encode(fl * q, negative)


def proj_exact(x_bits, w_bits):
    """y[b][n] = round_bf16(exact sum_k x[b][k] * W[n][k]); lists of ints."""
    xs = [[bf16_to_fraction(int(v)) for v in row] for row in x_bits]
    ws = [[bf16_to_fraction(int(v)) for v in row] for row in w_bits]
    out = []
    for xr in xs:
        row = []
        for wr in ws:
            if len(wr) != len(xr):
                raise ValueError("K mismatch")
            s = sum((a * b for a, b in zip(xr, wr)), Fraction(0))
            row.append(round_fraction_to_bf16(s))
        out.append(row)
    return out


def exact_sums(x_bits, w_bits):
    """The exact rational sums themselves, for tolerance checks."""
    xs = [[bf16_to_fraction(int(v)) for v in row] for row in x_bits]
    ws = [[bf16_to_fraction(int(v)) for v in row] for row in w_bits]
    return [[sum((a * b for a, b in zip(xr, wr)), Fraction(0)) for wr in ws]
            for xr in xs]
