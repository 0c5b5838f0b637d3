"""Pins of the MMQ oracle (``oracle.mmq``): Q8_1-style activation
quantization, the weight decomposition w = α·c − β, and the block product.

* hand-derived activation blocks (tests/golden/q81_worked.txt): ties away
  from zero, zero blocks, a negative maximum, an inexact d = fl32(1/127);
* blocks whose scale is a power of two, where every code is fixed by exact
  rational rounding;
* the vectorized and the scalar quantizer agree; |x − d·q| ≤ d/2;
* fl32(α·c − β) rounded to f16 is the pinned decode, bit for bit, for every
  format (so a wrong factor, code offset or element order fails);
* the product against an exact rational brute force over blocks and groups;
* closed form: integer activations with 127 in every block (d = 1, q = x,
  s = Σx) and integer weights give exactly the plain matmul X·W."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden
from oracle import mmq

ALL = [synth.Q4_0, synth.Q5_0, synth.Q5_1, synth.Q8_0, synth.Q4_K, synth.Q5_K, synth.Q6_K]
ELEMS = {2: 32, 6: 32, 7: 32, 8: 32, 12: 256, 13: 256, 14: 256}


def _f32(bits):
    return np.array([int(b, 16) for b in bits], np.uint32).view(np.float32)


def test_hand_derived_blocks():
    for row in read_golden("q81_worked.txt")["block"]:
        xs, dbits, sbits, codes = (t.split() for t in row.split("|"))
        x = np.zeros((1, 32), np.float32)
        x[0, :len(xs)] = _f32(xs)
        exp_q = [int(c) for c in codes]
        for impl in (mmq.quantize_q8_1, mmq.quantize_q8_1_scalar):
            q, d, s = impl(x)
            assert [int(v) for v in q[0, :len(exp_q)]] == exp_q, (impl.__name__, row)
            assert np.all(q[0, len(exp_q):] == 0)
            assert d.view(np.uint32)[0, 0] == int(dbits[0], 16), (impl.__name__, hex(d.view(np.uint32)[0, 0]))
            assert s.view(np.uint32)[0, 0] == int(sbits[0], 16), (impl.__name__, hex(s.view(np.uint32)[0, 0]))


def _round_half_away(fr: Fraction) -> int:
    n = abs(fr)
    f = int(n)
    if n - f >= Fraction(1, 2):
        f += 1
    return f if fr >= 0 else -f


def test_power_of_two_scale_is_exact_rounding():
    """a = 127·2^e makes d = 2^e exact, so x/d is exact and each code is the
    rational x·2^-e rounded half away from zero."""
    g = np.random.default_rng(90)
    for e in (-9, -3, 0, 2, 7):
        x = (g.integers(-254 * 4, 254 * 4 + 1, (6, 32)) / 8.0).astype(np.float64) * 2.0 ** e
        x = np.clip(x, -127 * 2.0 ** e, 127 * 2.0 ** e)
        x[:, 5] = 127 * 2.0 ** e * np.where(g.integers(0, 2, 6) == 1, 1, -1)
        x = x.astype(np.float32)
        for impl in (mmq.quantize_q8_1, mmq.quantize_q8_1_scalar):
            q, d, _ = impl(x)
            assert np.all(d == np.float32(2.0 ** e))
            exp = [[_round_half_away(Fraction(float(v)) / Fraction(2) ** e) for v in r] for r in x]
            assert np.array_equal(q.astype(np.int64), np.array(exp)), (impl.__name__, e)


def test_vectorized_equals_scalar_and_error_bound():
    g = np.random.default_rng(91)
    x = g.standard_normal((40, 256)).astype(np.float32)
    x[0, :32] = 0.0                                    # a zero block
    x[1, :32] *= np.float32(1e-30)                     # tiny scale
    x[2, 32:64] *= np.float32(1e30)                    # huge scale
    x[3, 64:96] = np.float32(-7.25)                    # constant block
    q1, d1, s1 = mmq.quantize_q8_1(x)
    q2, d2, s2 = mmq.quantize_q8_1_scalar(x)
    assert np.array_equal(q1, q2) and np.array_equal(d1.view(np.uint32), d2.view(np.uint32))
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    dd = np.repeat(d1.astype(np.float64), 32, axis=1)
    err = np.abs(x.astype(np.float64) - dd * q1)
    assert np.all(err <= dd / 2 * (1 + 2.0 ** -20))
    amax = np.abs(x.reshape(40, 8, 32)).max(axis=-1)
    qmax = np.abs(q1.reshape(40, 8, 32).astype(np.int32)).max(axis=-1)
    assert np.all(qmax[amax > 0] == 127)


@pytest.mark.parametrize("mode", ["random", "integer"])
@pytest.mark.parametrize("fmt", ALL)
def test_decomposition_reproduces_the_decode(fmt, mode):
    N, K = 12, 2 * ELEMS[fmt] if ELEMS[fmt] == 256 else 256
    wq = synth.weights(fmt, synth.rng(92, 0, fmt, 0), N, K, mode=mode)
    w32 = mmq.weights_f32(fmt, wq, N, K)
    assert np.array_equal(w32.astype(np.float16).view(np.uint16), oracle.dequant_ref(fmt, wq, N, K))
    c, alpha, beta, gsz = mmq.decompose(fmt, wq, N, K)
    lo, hi = {2: (-8, 7), 6: (-16, 15), 7: (0, 31), 8: (-127, 127), 12: (0, 15),
              13: (0, 31), 14: (-32, 31)}[fmt]
    assert c.min() >= lo and c.max() <= hi
    assert gsz == (16 if fmt == synth.Q6_K else 32)
    assert alpha.shape == (N, K // gsz) and beta.shape == (N, K // 32)


@pytest.mark.parametrize("fmt", ALL)
def test_product_equals_exact_bruteforce(fmt):
    M, N, K = 2, 3, ELEMS[fmt] if ELEMS[fmt] == 256 else 64
    wq = synth.weights(fmt, synth.rng(93, 0, fmt, 0), N, K)
    x = np.random.default_rng(93).standard_normal((M, K)).astype(np.float32)
    xq, xd, xs = mmq.quantize_q8_1(x)
    Y, S = mmq.mmq_ref(xq, xd, xs, fmt, wq, N, K)
    Yb = mmq.mmq_bruteforce(xq, xd, xs, fmt, wq, N, K)
    assert np.all(np.abs(Y - Yb) <= 1e-12 * S + 1e-300)


@pytest.mark.parametrize("fmt", ALL)
def test_integer_closed_form_is_the_plain_matmul(fmt):
    M, N, K = 5, 7, 512
    wq = synth.weights(fmt, synth.rng(94, 0, fmt, 0), N, K, mode="integer")
    g = np.random.default_rng(94)
    x = g.integers(-3, 4, (M, K)).astype(np.float32)
    x[:, ::32] = 127 * np.where(g.integers(0, 2, (M, K // 32)) == 1, 1, -1)
    xq, xd, xs = mmq.quantize_q8_1(x)
    assert np.all(xd == 1) and np.array_equal(xq.astype(np.float32), x)
    Y, _ = mmq.mmq_ref(xq, xd, xs, fmt, wq, N, K)
    Yp, _ = oracle.gemm_ref(x.astype(np.float16).view(np.uint16), oracle.dequant_ref(fmt, wq, N, K))
    assert np.array_equal(Y, Yp)


@pytest.mark.parametrize("fmt", [synth.Q4_K, synth.Q5_1, synth.Q6_K])
def test_product_approximates_the_matmul(fmt):
    """|Y_mmq − X·W| is bounded by the activation rounding Σ|w|·|x − d q| plus
    the rounding of the sums s (planting a wrong sign on β breaks it)."""
    M, N, K = 6, 9, 512
    wq = synth.weights(fmt, synth.rng(95, 0, fmt, 0), N, K)
    x = np.random.default_rng(95).standard_normal((M, K)).astype(np.float32)
    xq, xd, xs = mmq.quantize_q8_1(x)
    Y, S = mmq.mmq_ref(xq, xd, xs, fmt, wq, N, K)
    W = mmq.weights_f32(fmt, wq, N, K).astype(np.float64)
    exact = x.astype(np.float64) @ W.T
    xt = xq.astype(np.float64) * np.repeat(xd.astype(np.float64), 32, axis=1)
    act = np.abs(x.astype(np.float64) - xt) @ np.abs(W).T
    _, _, beta, _ = mmq.decompose(fmt, wq, N, K)
    ds = np.abs(xs.astype(np.float64) - xd.astype(np.float64) *
                xq.reshape(M, K // 32, 32).astype(np.int64).sum(-1))
    sums = ds @ np.abs(beta.astype(np.float64)).T
    bound = act + sums + 1e-9 * S
    assert np.all(np.abs(Y - exact) <= bound)
    assert np.abs(Y - exact).max() > 0      # the approximation is not the identity
