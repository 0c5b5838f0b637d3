"""Pins of the oracle's hand-written f16/f32 rounding against the IEEE definition.

The pages convert every decoded weight from float to half (minfer "05 · 8p",
§3.2 and §3.3); these tests fix that conversion independently of the oracle:
exhaustive decode of all 65,536 patterns, printed closed-form values, and
round-to-nearest-even at every f16 midpoint and one f32 ulp around it.
"""

import math

import numpy as np
import pytest

from conftest import read_golden
from oracle.f16 import f16_bits_to_float, f32_to_f16_bits, f64_to_f32

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_decode_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    mine = np.array([f16_bits_to_float(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    # signs of zero
    assert math.copysign(1.0, f16_bits_to_float(0x8000)) == -1.0
    assert math.copysign(1.0, f16_bits_to_float(0x0000)) == 1.0


def test_golden_values():
    rows = read_golden("f16_values.txt")["_rows"]
    assert len(rows) >= 10
    for row in rows:
        b, v = row.split()
        b = int(b, 16)
        val = float(v)
        got = f16_bits_to_float(b)
        assert got == val and math.copysign(1.0, got) == math.copysign(1.0, val), row
        assert f32_to_f16_bits(val) == b, row


def test_encode_roundtrip_every_finite_value():
    for b in range(65536):
        if (b & 0x7C00) == 0x7C00:
            continue
        assert f32_to_f16_bits(f16_bits_to_float(b)) == b


def _finite_positive_f16():
    return [b for b in range(0x7C00)]


def test_midpoints_round_to_even_and_neighbours():
    """At every midpoint between adjacent positive f16 values the even one wins;
    one f32 ulp either side decides the direction.  numpy's float32→float16 cast
    must agree on all of them."""
    pos = _finite_positive_f16()
    mids, below, above, expect_mid, lo_bits, hi_bits = [], [], [], [], [], []
    for a in pos[:-1]:
        b = a + 1
        va, vb = f16_bits_to_float(a), f16_bits_to_float(b)
        mid = (va + vb) / 2.0                       # exact: needs 12 significant bits
        even = a if a % 2 == 0 else b
        m32 = np.float32(mid)
        assert float(m32) == mid
        mids.append(mid)
        below.append(float(np.nextafter(m32, np.float32(0))))
        above.append(float(np.nextafter(m32, np.float32(np.inf))))
        expect_mid.append(even)
        lo_bits.append(a)
        hi_bits.append(b)
    for mid, bl, ab, ev, a, b in zip(mids, below, above, expect_mid, lo_bits, hi_bits):
        assert f32_to_f16_bits(mid) == ev
        assert f32_to_f16_bits(bl) == a
        assert f32_to_f16_bits(ab) == b
        assert f32_to_f16_bits(-mid) == ev | 0x8000
    for arr, exp in ((mids, expect_mid), (below, lo_bits), (above, hi_bits)):
        got = np.array(arr, dtype=np.float32).astype(np.float16).view(np.uint16)
        assert np.array_equal(got, np.array(exp, dtype=np.uint16))


def test_overflow_and_tiny():
    assert f32_to_f16_bits(65504.0) == 0x7BFF
    assert f32_to_f16_bits(65519.99) == 0x7BFF          # below the overflow midpoint
    assert f32_to_f16_bits(65520.0) == 0x7C00           # midpoint to 2^16 rounds to even -> inf
    assert f32_to_f16_bits(2.0 ** -25) == 0x0000        # half the smallest subnormal: tie to even 0
    assert f32_to_f16_bits(2.0 ** -25 * 1.5) == 0x0001
    assert f32_to_f16_bits(-(2.0 ** -26)) == 0x8000     # underflow keeps the sign


def test_f64_to_f32_matches_numpy_and_ties():
    g = np.random.default_rng(1)
    xs = g.standard_normal(20000) * np.exp2(g.integers(-30, 30, 20000))
    for x in xs:
        assert f64_to_f32(float(x)) == float(np.float32(x))
    one = 1.0
    ulp = 2.0 ** -23
    assert f64_to_f32(one + ulp / 2) == one                 # tie -> even (1.0)
    assert f64_to_f32(one + 3 * ulp / 2) == one + 2 * ulp   # tie -> even (1 + 2 ulp)
    assert f64_to_f32(one + ulp / 2 + 2.0 ** -40) == one + ulp
