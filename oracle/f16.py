"""Binary16 / binary32 rounding written out from the IEEE-754 definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The pages decode every weight "in float, then convert to half" (minfer 05 · 8p,
§3.2 second and third sites: products in f32, ``__float2half`` per element;
§3.3 third pitfall: the fused path must follow the same rounding).  That
conversion is round-to-nearest, ties-to-even, with subnormals kept.  These
helpers implement it on Python floats (IEEE binary64), which hold every f16
and f32 value and every product in the three decoders exactly, so the only
roundings are the ones written here.
"""

from __future__ import annotations

import math

# (fraction bits, minimum normal exponent, maximum exponent) per format.
_F16 = (10, -14, 15)
_F32 = (23, -126, 127)


def _round_to_format(x: float, fmt: tuple[int, int, int]) -> float:
    """Nearest value of the binary format to ``x``; ties go to the even significand.

    Works on the exact binary64 value ``x``.  Below the minimum normal
    exponent the quantum stays at 2^(emin - p) (gradual underflow).  Overflow
    returns an infinity of the right sign.
    """
    p, emin, emax = fmt
    if x == 0.0 or math.isnan(x) or math.isinf(x):
        return x
    ax = abs(x)
    _, e2 = math.frexp(ax)          # ax = f * 2**e2 with 0.5 <= f < 1
    e = e2 - 1                      # floor(log2(ax))
    q = math.ldexp(1.0, max(e, emin) - p)   # spacing of representable values here
    n = ax / q                      # exact: q is a power of two
    r = round(n)                    # Python rounds float halves to even
    v = r * q
    if v > _max_finite(fmt):       # rounded past the largest finite value
        v = math.inf
    return math.copysign(v, x)


def _max_finite(fmt: tuple[int, int, int]) -> float:
    p, _, emax = fmt
    return math.ldexp(2.0 - math.ldexp(1.0, -p), emax)


def f64_to_f32(x: float) -> float:
    """Round an exact binary64 value to the nearest binary32 value (RNE)."""
    return _round_to_format(x, _F32)


def f16_bits_to_float(bits: int) -> float:
    """Exact value of an IEEE binary16 bit pattern."""
    bits = int(bits) & 0xFFFF
    sign = -1.0 if bits >> 15 else 1.0
    exp = (bits >> 10) & 0x1F
    man = bits & 0x3FF
    if exp == 0:
        return sign * math.ldexp(man, -24)
    if exp == 0x1F:
        return sign * math.inf if man == 0 else math.nan
    return sign * math.ldexp(1024 + man, exp - 25)


def f32_to_f16_bits(x: float) -> int:
    """Bit pattern of the binary16 nearest to ``x`` (RNE, subnormals kept, sign of zero kept).

    ``x`` is expected to be a binary32 value already (the pages convert f32
    results); any binary64 input is rounded to f16 directly.
    """
    if math.isnan(x):
        return 0x7E00
    v = _round_to_format(x, _F16)
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    av = abs(v)
    if av == 0.0:
        return sign
    if math.isinf(av):
        return sign | 0x7C00
    _, e2 = math.frexp(av)
    e = e2 - 1
    if e < -14:                       # subnormal: value = man * 2^-24
        man = int(av / math.ldexp(1.0, -24))
        return sign | man
    man = int(av / math.ldexp(1.0, e - 10)) - 1024
    return sign | ((e + 15) << 10) | man
