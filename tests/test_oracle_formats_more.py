"""Pins of the oracle's decoders of Q4_0, Q5_0, Q5_1 and Q5_K.

What fixes them, independently of the decoders' own code:
* hand-built blocks under tests/golden/ written as raw bytes (so the encoder is
  pinned too), each expected f16 pattern worked by hand in the fixture;
* the field-wise encoders (oracle/encode.py): packing random quants with unit
  scales must decode to q − 8, q − 16, q + m, sc·q − m;
* exact rational arithmetic for the f32-then-f16 rounding of every element;
* the per-element and vectorized decoders agreeing on generated data;
* closed-form means of the synthetic distributions;
* a planted layout mistake (transposed Q5_K qh) failing the worked block.
"""

from fractions import Fraction

import numpy as np
import pytest

import synth
from conftest import read_golden
from oracle import Q4_0, Q5_0, Q5_1, Q5_K, dequant_ref, dequant_scalar, f16_bits_to_float, row_bytes
from oracle.encode import concat_blocks, pack_q40, pack_q50, pack_q51, pack_q5k

from test_oracle_formats import _rne  # exact round-to-nearest-even of a rational

BB = {Q4_0: 18, Q5_0: 22, Q5_1: 24, Q5_K: 176}
BE = {Q4_0: 32, Q5_0: 32, Q5_1: 32, Q5_K: 256}
FIXTURE = {Q4_0: "q40_worked.txt", Q5_0: "q50_worked.txt", Q5_1: "q51_worked.txt",
           Q5_K: "q5k_worked.txt"}


def _both(fmt, q, N, K):
    a = dequant_ref(fmt, q, N, K)
    b = dequant_scalar(fmt, q, N, K)
    assert np.array_equal(a, b)
    return a


@pytest.mark.parametrize("fmt", [Q4_0, Q5_0, Q5_1, Q5_K])
def test_hand_built_blocks(fmt):
    rows = read_golden(FIXTURE[fmt])["block"]
    assert rows
    for row in rows:
        hexs, exp = row.split("|")
        blk = np.array([int(t, 16) for t in hexs.split()], np.uint8)
        assert blk.size == BB[fmt]
        w = _both(fmt, blk, 1, BE[fmt])[0]
        for tok in exp.split():
            e, v = tok.split(":")
            assert int(w[int(e)]) == int(v, 16), (fmt, row[:20], tok)


def test_unit_scale_round_trips():
    g = np.random.default_rng(40)
    q4 = g.integers(0, 16, (24, 32))
    w = _both(Q4_0, concat_blocks([pack_q40(0x3C00, q) for q in q4]), 3, 8 * 32)
    assert np.array_equal(w.reshape(-1, 32).view(np.float16).astype(np.int64), q4 - 8)
    q5 = g.integers(0, 32, (24, 32))
    w = _both(Q5_0, concat_blocks([pack_q50(0x3C00, q) for q in q5]), 3, 8 * 32)
    assert np.array_equal(w.reshape(-1, 32).view(np.float16).astype(np.int64), q5 - 16)
    # m = -3: value q - 3
    w = _both(Q5_1, concat_blocks([pack_q51(0x3C00, 0xC200, q) for q in q5]), 3, 8 * 32)
    assert np.array_equal(w.reshape(-1, 32).view(np.float16).astype(np.int64), q5 - 3)
    sc = g.integers(0, 64, (4, 8))
    mn = g.integers(0, 64, (4, 8))
    qk = g.integers(0, 32, (4, 256))
    w = _both(Q5_K, concat_blocks([pack_q5k(0x3C00, 0x3C00, sc[i], mn[i], qk[i]) for i in range(4)]),
              2, 512)
    exp = np.repeat(sc, 32, axis=1) * qk - np.repeat(mn, 32, axis=1)
    assert np.array_equal(w.reshape(4, 256).view(np.float16).astype(np.int64), exp)


def _frac16(lo, hi):
    return Fraction(f16_bits_to_float(lo | hi << 8))


@pytest.mark.parametrize("fmt", [Q4_0, Q5_0, Q5_1, Q5_K])
def test_random_blocks_match_exact_rational_decode(fmt):
    """Every element of generated blocks equals its exact rational value rounded
    to f32 and then to f16, with the fields read by hand from the bytes."""
    K = 512
    q = synth.weights(fmt, synth.rng(910, 0, fmt, 0), 4, K)
    w = _both(fmt, q, 4, K)
    raw = q.reshape(-1)
    nbr = K // BE[fmt]
    for bi in range(raw.size // BB[fmt]):
        b = raw[bi * BB[fmt]:(bi + 1) * BB[fmt]].tolist()
        n, kb = divmod(bi, nbr)
        for e in range(0, BE[fmt], 3):
            if fmt == Q5_K:
                d, dmin = _frac16(b[0], b[1]), _frac16(b[2], b[3])
                s = b[4:16]
                j = e // 32
                if j < 4:
                    sc, m = s[j] & 63, s[j + 4] & 63
                else:
                    sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4)
                    m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4)
                c, r = divmod(e, 64)
                byte = b[48 + 32 * c + r % 32]
                qq = (byte & 15 if r < 32 else byte >> 4) + 16 * ((b[16 + r % 32] >> j) & 1)
                exact = d * sc * qq - dmin * m
            else:
                qs_off = {Q4_0: 2, Q5_0: 6, Q5_1: 8}[fmt]
                byte = b[qs_off + e % 16]
                nib = byte & 15 if e < 16 else byte >> 4
                d = _frac16(b[0], b[1])
                if fmt == Q4_0:
                    exact = d * (nib - 8)
                else:
                    qh_off = 2 if fmt == Q5_0 else 4
                    qh = b[qh_off] | b[qh_off + 1] << 8 | b[qh_off + 2] << 16 | b[qh_off + 3] << 24
                    qq = nib + 16 * ((qh >> e) & 1)
                    exact = d * (qq - 16) if fmt == Q5_0 else d * qq + _frac16(b[2], b[3])
            v16 = _rne(_rne(exact, 23, -126), 10, -14)
            got = Fraction(f16_bits_to_float(int(w[n, kb * BE[fmt] + e])))
            assert got == v16, (fmt, bi, e)


@pytest.mark.parametrize("fmt,N,K", [(Q4_0, 64, 320), (Q5_0, 48, 352), (Q5_1, 40, 96),
                                     (Q5_K, 24, 768)])
def test_two_decoders_agree_on_synthetic(fmt, N, K):
    _both(fmt, synth.weights(fmt, synth.rng(911, 0, fmt, 0), N, K), N, K)


def test_distribution_closed_forms():
    """Means fixed by the generator's distributions (E|N(0,1)| = sqrt(2/pi))."""
    e_abs = np.sqrt(2 / np.pi)
    for fmt, mean in ((Q4_0, e_abs * 2 ** -7 * (7.5 - 8)), (Q5_0, e_abs * 2 ** -7 * (15.5 - 16)),
                      (Q5_1, e_abs * 2 ** -7 * 15.5 - e_abs * 2 ** -3),
                      (Q5_K, e_abs * 2 ** -7 * (31.5 * 15.5 - 31.5))):
        K = 2048
        w = dequant_ref(fmt, synth.weights(fmt, synth.rng(912, 0, fmt, 0), 1024, K), 1024, K)
        got = w.view(np.float16).astype(np.float64).mean()
        assert abs(got - mean) < 0.03 * max(1.0, abs(mean)), (fmt, got, mean)


def test_row_bytes():
    assert row_bytes(Q4_0, 4096) == 128 * 18
    assert row_bytes(Q5_0, 4096) == 128 * 22
    assert row_bytes(Q5_1, 4096) == 128 * 24
    assert row_bytes(Q5_K, 3584) == 14 * 176


def test_planted_transposed_qh_is_caught():
    """A Q5_K decoder that reads the 16s bit as bit l of qh[s] (not bit s of qh[l])
    must disagree with the worked block."""
    row = read_golden("q5k_worked.txt")["block"][0]
    hexs, exp = row.split("|")
    b = np.array([int(t, 16) for t in hexs.split()], np.uint8)
    qh = b[16:48]
    # transposed reading planted in a copy of the block: move bit s of qh[l] to bit l of qh[s]
    bits = np.zeros((32, 8), np.uint8)
    for l in range(32):
        for s in range(8):
            bits[l, s] = (qh[l] >> s) & 1
    planted = np.zeros(32, np.uint8)
    for l in range(8):
        for s in range(32):
            if s < 8 and bits[s, l] and l < 8:
                planted[l] |= 1 << s
    b2 = b.copy()
    b2[16:48] = planted
    w = dequant_ref(Q5_K, b2, 1, 256)[0]
    mism = [tok for tok in exp.split() if int(w[int(tok.split(":")[0])]) != int(tok.split(":")[1], 16)]
    assert mism
