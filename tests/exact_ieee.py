"""An exact, pure-Python model of the IEEE-754 operations the reduction uses.

Independent of the oracle (it shares no code with ``oracle/``): values are
exact rationals (``fractions.Fraction``), binary32 addition is "the exact sum,
correctly rounded to binary32" as IEEE 754 defines it, and the bf16 rounding
is "the nearest bf16 value, ties to the even significand".  Slow; meant for
brute force on tiny inputs.

A value is a tuple ``(kind, sign, mag)``: kind in {"num", "inf", "nan"},
sign in {0, 1}, mag a non-negative Fraction (zero keeps its sign).
"""
from __future__ import annotations

from fractions import Fraction

BF16_P, F32_P = 8, 24          # significand bits including the hidden bit
EMIN, EMAX = -126, 127          # shared by binary32 and bf16
QNAN_BF16 = 0x7FC0


def decode_bf16(bits: int):
    bits &= 0xFFFF
    sign = bits >> 15
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        return ("nan", 0, Fraction(0)) if f else ("inf", sign, Fraction(0))
    if e == 0:
        return ("num", sign, Fraction(f, 1) * Fraction(2) ** (EMIN - (BF16_P - 1)))
    return ("num", sign, Fraction(128 + f) * Fraction(2) ** (e - 127 - (BF16_P - 1)))


def _floor_log2(m: Fraction) -> int:
    e = m.numerator.bit_length() - m.denominator.bit_length()
    if Fraction(2) ** e > m:
        e -= 1
    while Fraction(2) ** (e + 1) <= m:
        e += 1
    return e


def round_to(v, p: int):
    """Round a value to a binary format with p significand bits and the
    binary32 exponent range, to nearest with ties to even; overflow -> inf."""
    kind, sign, m = v
    if kind != "num" or m == 0:
        return v
    e = max(_floor_log2(m), EMIN)
    quantum = Fraction(2) ** (e - (p - 1))
    k = m / quantum
    ki = k.numerator // k.denominator
    rem = k - ki
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and ki % 2 == 1):
        ki += 1
    r = ki * quantum
    # IEEE: round-to-nearest overflows when the exact value reaches
    # 2^EMAX * (2 - 2^-p), i.e. when the rounded result leaves the format.
    if r >= Fraction(2) ** (EMAX + 1):
        return ("inf", sign, Fraction(0))
    return ("num", sign, r)


def add32(a, b):
    """binary32 addition: exact sum, rounded to nearest even."""
    if a[0] == "nan" or b[0] == "nan":
        return ("nan", 0, Fraction(0))
    if a[0] == "inf" and b[0] == "inf":
        return a if a[1] == b[1] else ("nan", 0, Fraction(0))
    if a[0] == "inf":
        return a
    if b[0] == "inf":
        return b
    s = (-a[2] if a[1] else a[2]) + (-b[2] if b[1] else b[2])
    if s == 0:
        # exact zero sum: -0 only when both operands are -0 (round to nearest)
        return ("num", 1 if (a[1] and b[1] and a[2] == 0 and b[2] == 0) else 0, Fraction(0))
    return round_to(("num", 1 if s < 0 else 0, abs(s)), F32_P)


def to_bf16(v):
    """Round a binary32 value to bf16 and encode the bits (NaN -> 0x7FC0)."""
    v = round_to(v, BF16_P)
    kind, sign, m = v
    if kind == "nan":
        return QNAN_BF16
    if kind == "inf":
        return (sign << 15) | 0x7F80
    if m == 0:
        return sign << 15
    e = _floor_log2(m)
    if e < EMIN:
        f = m / Fraction(2) ** (EMIN - (BF16_P - 1))
        assert f.denominator == 1 and f < 128
        return (sign << 15) | int(f)
    f = m / Fraction(2) ** (e - (BF16_P - 1)) - 128
    assert f.denominator == 1 and 0 <= f < 128
    return (sign << 15) | ((e + 127) << 7) | int(f)


def value_of(v) -> Fraction:
    assert v[0] == "num"
    return -v[2] if v[1] else v[2]


def seq_sum(bits_per_rank):
    """rn(((x0 + x1) + x2) + ...) with binary32 partials."""
    acc = decode_bf16(bits_per_rank[0])
    for b in bits_per_rank[1:]:
        acc = add32(acc, decode_bf16(b))
    return to_bf16(acc)


def tree_sum(bits_per_rank, round_each_node: bool):
    """Balanced binary tree over the rank index range: ranks [lo, hi) split at
    the midpoint; with round_each_node every internal node is rounded to bf16
    (the exchanged partial is bf16), otherwise partials stay binary32."""
    def rec(lo, hi):
        if hi - lo == 1:
            return decode_bf16(bits_per_rank[lo])
        mid = (lo + hi) // 2
        s = add32(rec(lo, mid), rec(mid, hi))
        return decode_bf16(to_bf16(s)) if round_each_node else s
    return to_bf16(rec(0, len(bits_per_rank)))


def exact_sum(bits_per_rank) -> Fraction:
    return sum((value_of(decode_bf16(b)) for b in bits_per_rank), Fraction(0))
