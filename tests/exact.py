"""Exact-rational model of the GLU projection's roundings, for pinning the oracle.

Independent of the oracle's C source: every value is a ``fractions.Fraction``,
every rounding is done by :func:`round_to_format` below from the definition of
a binary floating-point format (p significand bits, minimum normal exponent
emin, maximum exponent emax, round to nearest with ties to even), and exp is
evaluated by Python's ``decimal`` module at 60 significant digits, so the
rounded fp32 exp is the correctly rounded one unless the true value lies within
about 1e-60 (relative) of an fp32 rounding boundary.

Only small inputs go through it: it is slow by design.
"""
from __future__ import annotations

import decimal
import math
import struct
from fractions import Fraction
from typing import Optional, Sequence, Union

Num = Union[Fraction, float]  # float only for +-inf and nan

BF16 = (8, -126, 127)    # (significand bits incl. the implicit one, emin, emax)
FP32 = (24, -126, 127)

_DEC = decimal.Context(prec=60, rounding=decimal.ROUND_HALF_EVEN,
                       Emin=-999999, Emax=999999, traps=[])


def bf16_bits_to_value(bits: int) -> Num:
    """Exact value of a bf16 bit pattern (Fraction; float for inf/nan)."""
    f = struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
    if math.isnan(f) or math.isinf(f):
        return f
    return Fraction(f)


def round_to_format(q: Fraction, fmt=BF16) -> Num:
    """Round an exact rational to the nearest value of a binary format, ties to even.

    Returns a Fraction, or +-inf when the magnitude rounds past the largest
    finite value.  The sign of a zero result is lost (callers track it).
    """
    p, emin, emax = fmt
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum_exp = max(e, emin) - (p - 1)
    quantum = Fraction(2) ** quantum_exp
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    max_finite = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if r > max_finite:
        return sign * math.inf
    return sign * r


def value_to_bf16_bits(v: Num, negative_zero: bool = False) -> int:
    """Bit pattern of a value already representable in bf16."""
    if isinstance(v, float):
        if math.isnan(v):
            return 0x7FC0
        if math.isinf(v):
            return 0xFF80 if v < 0 else 0x7F80
        v = Fraction(v)
    if v == 0:
        return 0x8000 if negative_zero else 0
    f = float(v)  # exact: bf16 values are doubles
    bits = struct.unpack("<I", struct.pack("<f", f))[0]
    assert bits & 0xFFFF == 0, "value is not a bf16 value"
    return bits >> 16


def exp_fp32(x: Fraction) -> Num:
    """exp(x) correctly rounded to fp32 (60-digit decimal evaluation, then exact rounding)."""
    # exp(89) > 2^128 rounds past the largest fp32; exp(-104) < 2^-150 (half the
    # smallest subnormal) rounds to zero.  Skipping the evaluation there keeps
    # the rationals small.
    if x >= 89:
        return math.inf
    if x <= -104:
        return Fraction(0)
    xf = float(x)
    if Fraction(xf) == x:
        xd = decimal.Decimal(xf)  # exact conversion
    else:
        xd = _DEC.divide(decimal.Decimal(x.numerator), decimal.Decimal(x.denominator))
    d = _DEC.exp(xd)
    if d.is_infinite():
        return math.inf
    return round_to_format(Fraction(d), FP32)


def silu_fp32(g: Num) -> Num:
    """fp32 evaluation of g / (1 + exp(-g)) with each operation rounded to fp32."""
    if isinstance(g, float):  # inf or nan
        if math.isnan(g):
            return math.nan
        return g if g > 0 else math.nan  # -inf / (1 + inf) is nan
    e = exp_fp32(-g)
    if isinstance(e, float):  # exp overflowed: g / inf
        return Fraction(0)   # a negative zero; the sign is restored by the caller
    d = round_to_format(1 + e, FP32)
    if isinstance(d, float):
        return Fraction(0)
    return round_to_format(g / d, FP32)


def glu_out_bits(h_row: Sequence[int], wg_row: Sequence[int], wu_row: Sequence[int]) -> dict:
    """Exact evaluation of one output from bf16 bit sequences (finite inputs only).

    Returns the exact dots, the rounded gate/up/act bits and the output bits.
    """
    hv = [bf16_bits_to_value(b) for b in h_row]
    G = sum((a * bf16_bits_to_value(b) for a, b in zip(hv, wg_row)), Fraction(0))
    U = sum((a * bf16_bits_to_value(b) for a, b in zip(hv, wu_row)), Fraction(0))
    g = round_to_format(G, BF16)
    u = round_to_format(U, BF16)
    res = epilogue_bits(value_to_bf16_bits(g, negative_zero=_neg_zero_of_sum(G, g)),
                        value_to_bf16_bits(u, negative_zero=_neg_zero_of_sum(U, u)))
    res.update(G=G, U=U)
    return res


def _neg_zero_of_sum(exact: Fraction, rounded: Num) -> bool:
    # A non-zero negative sum that rounds to zero keeps its sign; an exact zero
    # sum of products is +0 under round-to-nearest unless every term is -0.
    return rounded == 0 and exact < 0


def epilogue_bits(g_bits: int, u_bits: int) -> dict:
    """Exact evaluation of act = bf16(silu(g)) and out = bf16(fl32(act*u))."""
    g = bf16_bits_to_value(g_bits)
    u = bf16_bits_to_value(u_bits)
    g_neg = bool(g_bits & 0x8000)
    s32 = silu_fp32(g)
    if isinstance(s32, float):
        s = s32
        s_bits = value_to_bf16_bits(s)
    else:
        s = round_to_format(s32, BF16)
        # a zero act keeps the sign of g (g / positive denominator)
        s_bits = value_to_bf16_bits(s, negative_zero=(s == 0 and g_neg))
    s_neg = bool(s_bits & 0x8000)
    sv = bf16_bits_to_value(s_bits)
    if isinstance(sv, float) or isinstance(u, float):
        p = float(sv) * float(u)
        out_bits = value_to_bf16_bits(p) if not math.isnan(p) else 0x7FC0
    else:
        p = round_to_format(sv * u, FP32)
        if isinstance(p, float):
            out_bits = value_to_bf16_bits(p)
        else:
            o = round_to_format(p, BF16)
            neg = (sv * u < 0) or (sv * u == 0 and (s_neg != bool(u_bits & 0x8000)))
            out_bits = value_to_bf16_bits(o, negative_zero=(o == 0 and neg))
    return {"g_bits": g_bits, "u_bits": u_bits, "s_bits": s_bits, "out_bits": out_bits}


def is_nan_bits(bits: int) -> bool:
    return (bits & 0x7F80) == 0x7F80 and (bits & 0x7F) != 0


def bits_equal(a: int, b: int) -> bool:
    """Bitwise equality with every NaN equal to every NaN."""
    if is_nan_bits(a) or is_nan_bits(b):
        return is_nan_bits(a) and is_nan_bits(b)
    return a == b


def exact_fraction_of_float(x: float) -> Optional[Fraction]:
    return None if (math.isnan(x) or math.isinf(x)) else Fraction(x)
