"""Field-wise encoders of the block formats (inverse of the decoders).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Written from the field lists independently of ``oracle.formats``: they pack
named fields (scales, mins, quants, f16 scale bits) into block bytes so that
tests can build blocks with known contents and check that decoding the packed
bytes returns the fields (round trip), and can build the hand-derived worked
vectors.  Layouts as documented in ``oracle.formats``.
"""

from __future__ import annotations

import numpy as np


def pack_q4k(d_bits: int, dmin_bits: int, sc, mn, q) -> bytes:
    """One Q4_K block from f16 bits of d and dmin, 8 six-bit scales, 8 six-bit mins,
    and 256 four-bit quants in element order."""
    sc = [int(v) for v in sc]
    mn = [int(v) for v in mn]
    q = [int(v) for v in q]
    assert len(sc) == 8 and len(mn) == 8 and len(q) == 256
    assert all(0 <= v < 64 for v in sc + mn) and all(0 <= v < 16 for v in q)
    s = [0] * 12
    for j in range(4):
        # low 6 bits: scale/min of sub-blocks 0..3; top 2 bits: high bits of 4..7
        s[j] = sc[j] | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = mn[j] | ((mn[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4)
    qs = [0] * 128
    for c in range(4):               # 64-element chunk: low nibbles then high nibbles
        for p in range(32):
            qs[32 * c + p] = q[64 * c + p] | (q[64 * c + 32 + p] << 4)
    out = [d_bits & 255, d_bits >> 8, dmin_bits & 255, dmin_bits >> 8] + s + qs
    return bytes(out)


def pack_q6k(d_bits: int, scales, q) -> bytes:
    """One Q6_K block from f16 bits of d, 16 int8 scales and 256 six-bit quants (0..63)."""
    scales = [int(v) for v in scales]
    q = [int(v) for v in q]
    assert len(scales) == 16 and len(q) == 256
    assert all(-128 <= v < 128 for v in scales) and all(0 <= v < 64 for v in q)
    ql = [0] * 128
    qh = [0] * 64
    for e in range(256):
        h, r = divmod(e, 128)
        g, l = divmod(r, 32)
        lo, hi = q[e] & 15, q[e] >> 4
        idx = 64 * h + l + 32 * (g & 1)
        ql[idx] |= lo if g < 2 else lo << 4
        qh[32 * h + l] |= hi << (2 * g)
    sc_bytes = [v & 255 for v in scales]
    return bytes(ql + qh + sc_bytes + [d_bits & 255, d_bits >> 8])


def pack_q80(d_bits: int, q) -> bytes:
    """One Q8_0 block from f16 bits of d and 32 int8 quants."""
    q = [int(v) for v in q]
    assert len(q) == 32 and all(-128 <= v < 128 for v in q)
    return bytes([d_bits & 255, d_bits >> 8] + [v & 255 for v in q])


def _nibble_bytes32(q) -> list[int]:
    """16 bytes holding 32 four-bit values: element j < 16 in the low nibble of
    byte j, element j + 16 in its high nibble."""
    return [(q[j] & 15) | ((q[j + 16] & 15) << 4) for j in range(16)]


def _u32_le(v: int) -> list[int]:
    return [(v >> (8 * i)) & 255 for i in range(4)]


def pack_q40(d_bits: int, q) -> bytes:
    """One Q4_0 block from f16 bits of d and 32 four-bit quants (0..15)."""
    q = [int(v) for v in q]
    assert len(q) == 32 and all(0 <= v < 16 for v in q)
    return bytes([d_bits & 255, d_bits >> 8] + _nibble_bytes32(q))


def pack_q50(d_bits: int, q) -> bytes:
    """One Q5_0 block from f16 bits of d and 32 five-bit quants (0..31)."""
    q = [int(v) for v in q]
    assert len(q) == 32 and all(0 <= v < 32 for v in q)
    qh = sum(((v >> 4) & 1) << j for j, v in enumerate(q))
    return bytes([d_bits & 255, d_bits >> 8] + _u32_le(qh) + _nibble_bytes32(q))


def pack_q51(d_bits: int, m_bits: int, q) -> bytes:
    """One Q5_1 block from f16 bits of d and m and 32 five-bit quants (0..31)."""
    q = [int(v) for v in q]
    assert len(q) == 32 and all(0 <= v < 32 for v in q)
    qh = sum(((v >> 4) & 1) << j for j, v in enumerate(q))
    return bytes([d_bits & 255, d_bits >> 8, m_bits & 255, m_bits >> 8] + _u32_le(qh)
                 + _nibble_bytes32(q))


def pack_q5k(d_bits: int, dmin_bits: int, sc, mn, q) -> bytes:
    """One Q5_K block from f16 bits of d and dmin, 8 six-bit scales, 8 six-bit
    mins and 256 five-bit quants (0..31) in element order."""
    q = [int(v) for v in q]
    assert len(q) == 256 and all(0 <= v < 32 for v in q)
    # the scale bytes, the low nibbles and the layout of d / dmin are Q4_K's
    q4 = pack_q4k(d_bits, dmin_bits, sc, mn, [v & 15 for v in q])
    qh = [0] * 32
    for e in range(256):
        qh[e % 32] |= ((q[e] >> 4) & 1) << (e // 32)
    return bytes(q4[:16]) + bytes(qh) + bytes(q4[16:144])


def concat_blocks(blocks) -> np.ndarray:
    return np.frombuffer(b"".join(blocks), dtype=np.uint8).copy()
