"""Exact-arithmetic evaluation of the boundary for tiny inputs (a pin of the oracle).

Sums, squares and means are exact ``Fraction`` arithmetic; the square root is a
60-digit ``Decimal``; rounding to bf16 and to e4m3 is decided by exact
comparison with the neighbouring representable values. This is a second,
independent evaluation of the same definition the oracle implements (the plain
add, then RMSNorm with eps inside the square root), used only to pin the
oracle on inputs small enough for pure-Python loops.
"""
from __future__ import annotations

from decimal import Decimal, getcontext
from fractions import Fraction

getcontext().prec = 60

# ---------------------------------------------------------------- formats


def bf16_value(bits: int) -> Fraction:
    bits = int(bits)
    s = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    assert e != 0xFF, "inf/nan not used"
    if e == 0:
        return s * Fraction(m, 1 << 7) * Fraction(1, 1 << 126)
    return s * (1 + Fraction(m, 128)) * (Fraction(2) ** (e - 127))


def f32_value(x: float) -> Fraction:
    return Fraction(x)  # float -> exact rational


def _binade(a: Fraction) -> int:
    """e with 2^e <= a < 2^(e+1), a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _round_grid(a: Fraction, step: Fraction) -> tuple[Fraction, Fraction]:
    """Round a >= 0 to the grid step*Z, ties to even multiple; return (value, distance to tie)."""
    n = a / step
    lo = n.numerator // n.denominator
    frac = n - lo
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return lo * step, abs(frac - Fraction(1, 2)) * step


def bf16_round(v: Fraction) -> tuple[int, Fraction]:
    """(bits, distance of |v| from the nearest rounding tie)."""
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    if a == 0:
        return sign, Fraction(1)
    e = max(_binade(a), -126)
    step = Fraction(2) ** (e - 7)
    r, tie_dist = _round_grid(a, step)
    if r == 0:
        return sign, tie_dist
    e_r = _binade(r)
    if e_r < -126:  # subnormal
        m = int(r / (Fraction(2) ** -133))
        return sign | m, tie_dist
    m = int((r / (Fraction(2) ** e_r) - 1) * 128)
    return sign | ((e_r + 127) << 7) | m, tie_dist


def e4m3_value(code: int) -> Fraction:
    code = int(code)
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    assert not (e == 0xF and m == 0x7)
    if e == 0:
        return s * Fraction(m, 512)
    return s * (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))


def e4m3_round(v: Fraction) -> tuple[int, Fraction]:
    """RNE to E4M3FN for |v| <= 448; returns (code, distance from the nearest tie)."""
    sign = 0x80 if v < 0 else 0
    a = abs(v)
    assert a <= 448
    if a == 0:
        return sign, Fraction(1)
    e = max(_binade(a), -6)
    step = Fraction(2) ** (e - 3)
    r, tie_dist = _round_grid(a, step)
    if r == 0:
        return sign, tie_dist
    e_r = _binade(r)
    if e_r < -6:
        return sign | int(r * 512), tie_dist
    m = int((r / (Fraction(2) ** e_r) - 1) * 8)
    return sign | ((e_r + 7) << 3) | m, tie_dist


# ---------------------------------------------------------------- the read


def rms_inverse(x: list[Fraction], eps: float) -> Fraction:
    ms = sum((v * v for v in x), Fraction(0)) / len(x) + Fraction(eps)
    d = Decimal(ms.numerator) / Decimal(ms.denominator)
    return Fraction(Decimal(1) / d.sqrt())


def boundary_row(r_bits, contrib: list[Fraction], w: list[float], eps: float):
    """x = r + s, inv, y (all exact or 60-digit); r_bits None means r = 0."""
    H = len(contrib)
    x = [(bf16_value(r_bits[h]) if r_bits is not None else Fraction(0)) + contrib[h]
         for h in range(H)]
    inv = rms_inverse(x, eps)
    y = [x[h] * inv * f32_value(float(w[h])) for h in range(H)]
    return x, inv, y


def f32_round(v: Fraction) -> tuple[Fraction, Fraction]:
    """Round to the nearest fp32 (ties to even, normal and subnormal range), decided exactly;
    returns (value, distance from the nearest rounding tie in units of the fp32 step)."""
    a = abs(v)
    if a == 0:
        return Fraction(0), Fraction(1)
    e = max(_binade(a), -126)
    step = Fraction(2) ** (e - 23)
    r, tie_dist = _round_grid(a, step)
    return (r if v > 0 else -r), tie_dist / step


def fp8_row(y: list[Fraction]):
    """The per-token fp8 read decided in fp32: y32 = fp32(y), scale = fp32(max|y32| / 448),
    q = e4m3(clamp(fp32(y32 / scale))). The two fp32 divisions are IEEE single-precision
    divisions (numpy float32); every rounding to fp32 or e4m3 is decided exactly. Returns
    (scale, codes, the smallest distance of a y from an fp32 rounding tie, in fp32 steps)."""
    import numpy as np

    y32, tie = [], Fraction(10**9)
    for v in y:
        r, d = f32_round(v)
        y32.append(r)
        tie = min(tie, d)
    amax = max(abs(v) for v in y32)
    scale = float(np.float32(float(amax)) / np.float32(448.0))
    if scale == 0.0:
        return 0.0, [0] * len(y), tie
    codes = []
    for v in y32:
        t = Fraction(float(np.float32(float(v)) / np.float32(scale)))
        t = min(max(t, Fraction(-448)), Fraction(448))
        codes.append(e4m3_round(t)[0])
    return scale, codes, tie
