"""Pins of the oracle's block decoders (Q4_K, Q6_K, Q8_0) and the cache layout.

What fixes them, independently of the decoders' own code:
* hand-derived worked blocks under tests/golden/ (each with its derivation);
* a field-wise encoder written separately (oracle/encode.py): packing random
  fields with unit scales and decoding must give back sc·q − m, s·(q − 32), q;
* exact rational arithmetic (fractions) for the f32-then-f16 rounding;
* two decoders (per-element Python floats vs vectorized numpy f32) agreeing;
* closed-form moments of the synthetic distributions;
* the cache stride rule of llama.cpp PR #57 (Summary, second bullet).
"""

from fractions import Fraction

import numpy as np
import pytest

import synth
from conftest import read_golden
from oracle import (
    Q4_K,
    Q6_K,
    Q8_0,
    cache_ld,
    cache_ref,
    dequant_ref,
    dequant_scalar,
    f16_bits_to_float,
    row_bytes,
)
from oracle.encode import concat_blocks, pack_q4k, pack_q6k, pack_q80


def _nums(s):
    return [int(t, 0) for t in s.split()]


def _expect_pairs(s):
    out = {}
    for tok in s.split():
        k, v = tok.split(":")
        out[int(k)] = v
    return out


def _both(fmt, q, N, K):
    a = dequant_ref(fmt, q, N, K)
    b = dequant_scalar(fmt, q, N, K)
    assert np.array_equal(a, b)
    return a


# --------------------------------------------------------------------------- worked vectors

def test_q4k_worked_block():
    g = read_golden("q4k_worked.txt")
    sc, mn = _nums(g["scales"][0]), _nums(g["mins"][0])
    qs = [(i % 16) | ((15 - i % 16) << 4) for i in range(128)]
    q = []
    for e in range(256):
        c, r = divmod(e, 64)
        byte = qs[32 * c + r % 32]
        q.append(byte & 15 if r < 32 else byte >> 4)
    blk = pack_q4k(int(g["d_bits"][0], 16), int(g["dmin_bits"][0], 16), sc, mn, q)
    assert blk[4:16].hex(" ") == g["packed_scale_bytes"][0].lower()
    assert list(blk[16:]) == qs
    w = _both(Q4_K, np.frombuffer(blk, np.uint8), 1, 256)[0]
    vals = w.view(np.float16).astype(np.float64)
    for e, v in _expect_pairs(g["expect"][0]).items():
        assert vals[e] == float(v), (e, vals[e], v)


def test_q6k_worked_block():
    g = read_golden("q6k_worked.txt")
    ql = [(7 * i) & 255 for i in range(128)]
    qh = [(37 * i + 5) & 255 for i in range(64)]
    sc = [(j - 8) & 255 for j in range(16)]
    d = int(g["d_bits"][0], 16)
    blk = np.array(ql + qh + sc + [d & 255, d >> 8], dtype=np.uint8)
    w = _both(Q6_K, blk, 1, 256)[0]
    for e, v in _expect_pairs(g["expect_bits"][0]).items():
        assert int(w[e]) == int(v, 16), (e, hex(w[e]), v)


def test_q80_hand_blocks():
    rows = read_golden("q80_worked.txt")["block"]
    assert len(rows) == 4
    for row in rows:
        d_s, q_s, e_s = row.split("|")
        d = int(d_s, 16)
        qv = [int(t) for t in q_s.split()]
        exp = [int(t, 16) for t in e_s.split()]
        blk = np.frombuffer(pack_q80(d, qv + [0] * (32 - len(qv))), np.uint8)
        w = _both(Q8_0, blk, 1, 32)[0]
        assert [int(x) for x in w[: len(exp)]] == exp, row


def test_q4k_double_rounding_pin():
    g = read_golden("q4k_double_rounding.txt")
    q = [0] * 256
    q[0] = int(g["q0"][0])
    blk = pack_q4k(int(g["d_bits"][0], 16), int(g["dmin_bits"][0], 16),
                   _nums(g["scales"][0]), _nums(g["mins"][0]), q)
    w = _both(Q4_K, np.frombuffer(blk, np.uint8), 1, 256)[0]
    for e, v in _expect_pairs(g["expect_bits"][0]).items():
        assert int(w[e]) == int(v, 16)


# --------------------------------------------------------------------------- layout round trips

def test_q4k_roundtrip_unit_scales():
    g = np.random.default_rng(11)
    blocks, expect = [], []
    for _ in range(64):
        sc = g.integers(0, 64, 8)
        mn = g.integers(0, 64, 8)
        q = g.integers(0, 16, 256)
        blocks.append(pack_q4k(0x3C00, 0x3C00, sc, mn, q))
        expect.append([sc[e // 32] * q[e] - mn[e // 32] for e in range(256)])
    buf = concat_blocks(blocks)
    w = _both(Q4_K, buf, 4, 16 * 256).reshape(-1, 256).view(np.float16).astype(np.float64)
    assert np.array_equal(w, np.array(expect, dtype=np.float64))


def test_q6k_roundtrip_unit_scale():
    g = np.random.default_rng(12)
    blocks, expect = [], []
    for _ in range(64):
        s = g.integers(-32, 32, 16)          # |s*(q-32)| <= 1024: exact in f16
        q = g.integers(0, 64, 256)
        blocks.append(pack_q6k(0x3C00, s, q))
        expect.append([s[e // 16] * (q[e] - 32) for e in range(256)])
    buf = concat_blocks(blocks)
    w = _both(Q6_K, buf, 2, 32 * 256).reshape(-1, 256).view(np.float16).astype(np.float64)
    ref = np.array(expect, dtype=np.float64)
    assert np.array_equal(w, ref)


def test_q80_roundtrip_unit_scale():
    g = np.random.default_rng(13)
    qs = g.integers(-128, 128, (48, 32))
    buf = concat_blocks([pack_q80(0x3C00, q) for q in qs])
    w = _both(Q8_0, buf, 3, 16 * 32).reshape(-1, 32).view(np.float16).astype(np.float64)
    assert np.array_equal(w, qs.astype(np.float64))


# --------------------------------------------------------------------------- exact arithmetic

def _rne(fr: Fraction, p: int, emin: int) -> Fraction:
    """Round an exact rational to p fraction bits, gradual underflow below emin (RNE)."""
    if fr == 0:
        return fr
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = Fraction(2) ** (max(e, emin) - p)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * q


def _frac_f16(bits: int) -> Fraction:
    return Fraction(f16_bits_to_float(bits))


@pytest.mark.parametrize("fmt", [Q4_K, Q6_K, Q8_0])
def test_random_blocks_match_exact_rational_decode(fmt):
    """Decode of synthetic blocks equals the exact rational value rounded to f32
    and then to f16, computed with fractions only (no float arithmetic)."""
    g = synth.rng(900, 0, fmt, 0)
    K = 256 if fmt != Q8_0 else 64
    q = synth.weights(fmt, g, 6, K)
    w = _both(fmt, q, 6, K)
    raw = q.reshape(-1)
    bb = {Q4_K: 144, Q6_K: 210, Q8_0: 34}[fmt]
    for blk_i in range(raw.size // bb):
        b = raw[blk_i * bb:(blk_i + 1) * bb].tolist()
        n = blk_i // (K // (256 if fmt != Q8_0 else 32))
        kb = blk_i % (K // (256 if fmt != Q8_0 else 32))
        for e in range(0, 256 if fmt != Q8_0 else 32, 7):
            if fmt == Q4_K:
                d, dmin = _frac_f16(b[0] | b[1] << 8), _frac_f16(b[2] | b[3] << 8)
                s = b[4:16]
                j = e // 32
                if j < 4:
                    sc, m = s[j] & 63, s[j + 4] & 63
                else:
                    sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4)
                    m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4)
                c, r = divmod(e, 64)
                byte = b[16 + 32 * c + r % 32]
                qq = byte & 15 if r < 32 else byte >> 4
                exact = d * sc * qq - dmin * m
                col = kb * 256 + e
            elif fmt == Q6_K:
                d = _frac_f16(b[208] | b[209] << 8)
                h, r = divmod(e, 128)
                gg, l = divmod(r, 32)
                lo = b[64 * h + l + 32 * (gg & 1)]
                lo = lo & 15 if gg < 2 else lo >> 4
                hi = (b[128 + 32 * h + l] >> (2 * gg)) & 3
                s = b[192 + e // 16]
                s = s - 256 if s >= 128 else s
                exact = d * s * ((lo | hi << 4) - 32)
                col = kb * 256 + e
            else:
                d = _frac_f16(b[0] | b[1] << 8)
                qq = b[2 + e]
                qq = qq - 256 if qq >= 128 else qq
                exact = d * qq
                col = kb * 32 + e
            v16 = _rne(_rne(exact, 23, -126), 10, -14)
            got = Fraction(f16_bits_to_float(int(w[n, col])))
            assert got == v16, (fmt, blk_i, e)


# --------------------------------------------------------------------------- generated data

@pytest.mark.parametrize("fmt,N,K", [(Q4_K, 96, 512), (Q6_K, 40, 768), (Q8_0, 64, 320)])
def test_two_decoders_agree_on_synthetic(fmt, N, K):
    q = synth.weights(fmt, synth.rng(901, 0, fmt, 0), N, K)
    _both(fmt, q, N, K)


def test_distribution_closed_forms():
    """Means fixed by the generator's distributions catch gross layout/scale errors."""
    w4 = dequant_ref(Q4_K, synth.weights(Q4_K, synth.rng(902, 0, 0, 0), 1024, 2048), 1024, 2048)
    m4 = w4.view(np.float16).astype(np.float64).mean()
    # E|N(0,1)| * 2^-7 * (E sc * E q - E m) with sc, m uniform 0..63 and q uniform 0..15
    assert abs(m4 - np.sqrt(2 / np.pi) * 2 ** -7 * (31.5 * 7.5 - 31.5)) < 0.03
    w6 = dequant_ref(Q6_K, synth.weights(Q6_K, synth.rng(902, 0, 1, 0), 1024, 2048), 1024, 2048)
    v6 = w6.view(np.float16).astype(np.float64)
    # E[d^2] E[s^2] E[(q-32)^2] = 2^-18 * 341.5^2 (s and q-32 uniform on -32..31)
    assert abs((v6 ** 2).mean() - 2 ** -18 * 341.5 ** 2) < 0.02
    assert abs(v6.mean()) < 0.01
    # share of -0: (s = 0, q < 32) or (s < 0, q = 32) -> 1/64*1/2 + 1/2*1/64
    assert abs(np.mean(w6 == 0x8000) - (1 / 128 + 1 / 128)) < 0.002
    w8 = dequant_ref(Q8_0, synth.weights(Q8_0, synth.rng(902, 0, 2, 0), 1024, 2048), 1024, 2048)
    v8 = w8.view(np.float16).astype(np.float64)
    assert abs(v8.mean()) < 0.01
    # E[d^2] E[q^2] = 2^-14 * (127*128/3) for q uniform on -127..127
    assert abs((v8 ** 2).mean() - 2 ** -14 * 127 * 128 / 3) < 0.01


def test_integer_mode_values_are_integers():
    q = synth.weights(Q4_K, synth.rng(903), 8, 512, mode="integer")
    v = dequant_ref(Q4_K, q, 8, 512).view(np.float16).astype(np.float64)
    assert np.array_equal(v, np.round(v)) and np.abs(v).max() <= 63 * 15


# --------------------------------------------------------------------------- cache layout

@pytest.mark.parametrize("K,ld", [(256, 256), (512, 512), (1024, 1088), (3584, 3584),
                                  (4096, 4160), (14336, 14400), (18944, 18944), (2048, 2112)])
def test_cache_ld_rule(K, ld):
    assert cache_ld(K) == ld


def test_cache_ref_pad_is_zero_and_body_is_decode():
    q = synth.weights(Q4_K, synth.rng(904), 16, 1024)
    c = cache_ref(Q4_K, q, 16, 1024)
    assert c.shape == (16, 1088)
    assert np.all(c[:, 1024:] == 0)
    assert np.array_equal(c[:, :1024], dequant_ref(Q4_K, q, 16, 1024))


def test_row_bytes():
    assert row_bytes(Q4_K, 3584) == 2016
    assert row_bytes(Q6_K, 18944) == 15540
    assert row_bytes(Q8_0, 4096) == 4352
    with pytest.raises(ValueError):
        row_bytes(Q4_K, 100)


def test_planted_layout_mistake_is_caught():
    """A decoder that swaps the nibble halves of a Q4_K chunk must fail the worked vector."""
    g = read_golden("q4k_worked.txt")
    qs = [(i % 16) | ((15 - i % 16) << 4) for i in range(128)]
    sc, mn = _nums(g["scales"][0]), _nums(g["mins"][0])
    q = []
    for e in range(256):
        c, r = divmod(e, 64)
        byte = qs[32 * c + r % 32]
        q.append(byte & 15 if r < 32 else byte >> 4)
    blk = bytearray(pack_q4k(0x3C00, 0x3800, sc, mn, q))
    blk[16:] = bytes(((b >> 4) | ((b & 15) << 4)) for b in blk[16:])     # planted swap
    w = dequant_ref(Q4_K, np.frombuffer(bytes(blk), np.uint8), 1, 256)[0]
    vals = w.view(np.float16).astype(np.float64)
    exp = _expect_pairs(g["expect"][0])
    assert any(vals[e] != float(v) for e, v in exp.items())
