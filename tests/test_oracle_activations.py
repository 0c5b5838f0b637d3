"""Pins of the oracle's f32 → f16 activation rounding (``activations_to_f16``),
which defines the f32-activation GEMM as the f16 GEMM on the rounded
activations (Fucina "Eager GPU Offload Without A Compute Graph", quantized
linears: f32 activations converted to half in the operand tile):

* hand-derived IEEE-754 cases (ties to even at normal and subnormal scale,
  the overflow midpoint, signed zeros) in tests/golden/f32_to_f16_rounding.txt;
* the vectorized cast against the scalar IEEE converter of ``oracle.f16`` on
  random f32 bit patterns over every exponent;
* closed forms: f16 values round-trip unchanged, and a value strictly
  between two f16 neighbours lands on one of them, the nearer one."""

import numpy as np

import oracle
from conftest import read_golden


def _golden():
    rows = []
    for row in read_golden("f32_to_f16_rounding.txt")["value"]:
        f32, f16, _ = (t.strip() for t in row.split("|"))
        rows.append((int(f32, 16), int(f16, 16)))
    return rows


def test_hand_derived_cases():
    rows = _golden()
    x = np.array([r[0] for r in rows], np.uint32).view(np.float32)
    exp = np.array([r[1] for r in rows], np.uint16)
    got = oracle.activations_to_f16(x)
    bad = [(hex(a), hex(b), hex(c)) for (a, b), c in zip(rows, got) if b != c]
    assert not bad, bad
    assert np.array_equal(oracle.activations_to_f16_scalar(x), exp)


def test_vectorized_equals_scalar_on_random_bit_patterns():
    g = np.random.default_rng(71)
    bits = g.integers(0, 2 ** 32, 60000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    assert np.array_equal(oracle.activations_to_f16(x), oracle.activations_to_f16_scalar(x))
    # the range the GEMM tests draw from: N(0, 1) and small integers
    y = np.concatenate([g.standard_normal(20000).astype(np.float32),
                        g.integers(-3, 4, 2000).astype(np.float32)])
    assert np.array_equal(oracle.activations_to_f16(y), oracle.activations_to_f16_scalar(y))


def test_f16_values_round_trip_and_nearest():
    all16 = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    finite = all16[np.isfinite(all16.view(np.float16))]
    vals = finite.view(np.float16).astype(np.float32)
    assert np.array_equal(oracle.activations_to_f16(vals), finite)
    # midpoints +/- a tiny nudge go to the nearer neighbour
    pos = np.sort(finite.view(np.float16)[finite.view(np.float16) > 0].astype(np.float64))
    lo, hi = pos[:-1], pos[1:]
    mid = (lo + hi) / 2
    below = np.nextafter(mid.astype(np.float32), np.float32(0))
    above = np.nextafter(mid.astype(np.float32), np.float32(np.inf))
    ok_b = mid.astype(np.float32) == mid        # midpoint exact in f32
    got_b = oracle.activations_to_f16(below[ok_b]).view(np.float16).astype(np.float64)
    got_a = oracle.activations_to_f16(above[ok_b]).view(np.float16).astype(np.float64)
    assert np.array_equal(got_b, lo[ok_b])
    assert np.array_equal(got_a, hi[ok_b])
