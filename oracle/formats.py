"""Decoders of the three GGUF block formats the prefill matmul reads.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources.
* The method: minfer "05 · 8p — Persistent f16 weight cache + fused
  dequant-in-GEMM" §2 (the cache holds an f16 copy of each quantized weight,
  decoded once) and §3.2 (decode in float, one ``__float2half`` per element;
  nibble j / j+16 convention of the printed Q5_0 kernels).
* The cache row stride: llama.cpp PR #57 "GEMM weight row padding + one-time
  K-padded f16 dequant for prefill", Summary: pad by one 128-byte line only
  when the f16 row size is a multiple of 2048 bytes.
* Field lists: Q4_K = f16 d, f16 dmin, 12 bytes of eight 6-bit scales and
  eight 6-bit mins, 128 bytes of 4-bit quants, value d·sc·q − dmin·m per
  32-element sub-block; Q6_K = 128 B low nibbles, 64 B high 2-bit pairs, 16
  int8 scales, f16 d, value d·s·(q − 32); Q8_0 = f16 d + 32 int8, value d·q.
  The pages print no bit positions for these three formats; the positions
  below are the GGUF ones (the pages' Q5_0 kernels follow the same
  conventions: little-endian fields, low nibble first).

Rounding (the pages: float math, then one conversion to half):
* Q4_K: A = d·sc, B = A·q, C = dmin·m are exact in f32; V = fl32(B − C);
  the element is f16_rne(V).  This is a double rounding (to f32, then to
  f16), which differs from one rounding of the exact value in rare cases.
* Q6_K: (d·s)·(q − 32) evaluated left to right; exact in f32, so the only
  rounding is to f16.  IEEE signed zeros are kept: s = 0 with q < 32 gives −0.
* Q8_0: d·q, exact in f32, one rounding to f16.

Four more formats of the same family (the pages' coverage list: minfer "79 ·
Phase-8 coverage & first-measurement batch" §3.4 and §3.6, and "05 · 8p"
§2–§3.2 for Q5_0):
* Q4_0 (18 B): f16 d, 16 bytes of nibbles; element j < 16 is the low nibble
  of byte j, element j + 16 its high nibble; value d·(q − 8).  Exact in f32.
* Q5_0 (22 B, page "05 · 8p" §2 / §3.2): f16 d, a 32-bit qh plane, 16 bytes
  of nibbles; the nibble as Q4_0, plus bit j (element j) of qh as its 16s
  bit; value d·(q − 16).  Exact in f32.
* Q5_1 (24 B; qh at byte 4, "05 · 8p" §2): f16 d, f16 m, qh, nibbles as Q5_0;
  value d·q + m: the product is exact, the sum is the one f32 rounding.
* Q5_K (176 B, "79" §3.4: transposed qh, deinterleaved qs chunks): f16 d, f16
  dmin, the 12 scale/min bytes of Q4_K, 32 bytes of qh, 128 bytes of nibbles
  laid out as Q4_K's; element l of sub-block s takes bit s of qh[l] as its
  16s bit; value fl32(d·sc·q − dmin·m) as for Q4_K (A·q still exact).
The pages give no bit positions for Q4_0, Q5_1 and Q5_K; the ones used are
the GGUF ones, consistent with the pages' Q5_0 layout and Q5_K description.

Two independent decoders live here: ``dequant_scalar`` walks one element at a
time in Python floats with the hand-written converters of ``oracle.f16``;
``dequant_ref`` is a vectorized numpy decode in float32 with numpy's f16 cast.
Tests require them to agree bit for bit.
"""

from __future__ import annotations

import numpy as np

from .f16 import f16_bits_to_float, f32_to_f16_bits, f64_to_f32

# GGUF type numbers; minfer's type_id 6 for Q5_0 (page "79 · Phase-8 coverage
# batch", §3.6) follows the same numbering.
Q4_0 = 2
Q5_0 = 6
Q5_1 = 7
Q8_0 = 8
Q4_K = 12
Q5_K = 13
Q6_K = 14

BLOCK_ELEMS = {Q4_0: 32, Q5_0: 32, Q5_1: 32, Q8_0: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256}
BLOCK_BYTES = {Q4_0: 18, Q5_0: 22, Q5_1: 24, Q8_0: 34, Q4_K: 144, Q5_K: 176, Q6_K: 210}


def row_bytes(fmt: int, K: int) -> int:
    """Bytes of one quantized weight row of K elements (rows are contiguous)."""
    if K % BLOCK_ELEMS[fmt]:
        raise ValueError(f"K={K} is not a multiple of the block size {BLOCK_ELEMS[fmt]}")
    return K // BLOCK_ELEMS[fmt] * BLOCK_BYTES[fmt]


def cache_ld(K: int) -> int:
    """Row stride (elements) of the f16 cache: K, plus 64 halves (one 128-B line)
    when the f16 row size 2K bytes is a multiple of 2048 (llama.cpp PR #57, Summary)."""
    return K + 64 if (2 * K) % 2048 == 0 else K


def q4k_scale_min(j: int, s) -> tuple[int, int]:
    """6-bit (scale, min) of Q4_K sub-block j from the 12 packed bytes s.

    Sub-blocks 0..3 keep their scale in the low 6 bits of s[j] and their min
    in the low 6 bits of s[j+4].  Sub-blocks 4..7 take their low 4 bits from
    the nibbles of s[j+4] (scale: low nibble, min: high nibble) and their top
    2 bits from the top 2 bits of s[j-4] (scale) and s[j] (min).
    """
    if j < 4:
        return s[j] & 63, s[j + 4] & 63
    sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4)
    m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4)
    return sc, m


# ---------------------------------------------------------------------------
# Scalar decoder: one element at a time, Python floats, hand-written rounding.
# ---------------------------------------------------------------------------

def _u16(b, off: int) -> int:
    return b[off] | (b[off + 1] << 8)


def _i8(v: int) -> int:
    return v - 256 if v >= 128 else v


def _q4k_block_scalar(b) -> list[int]:
    d = f16_bits_to_float(_u16(b, 0))
    dmin = f16_bits_to_float(_u16(b, 2))
    s = [b[4 + i] for i in range(12)]
    out = []
    for e in range(256):
        j = e // 32                      # 32-element sub-block
        sc, m = q4k_scale_min(j, s)
        c, r = divmod(e, 64)             # 64 elements share 32 quant bytes
        byte = b[16 + 32 * c + r % 32]
        q = byte & 15 if r < 32 else byte >> 4
        # d*sc*q and dmin*m are exact; their difference is exact in binary64.
        v = f64_to_f32(d * sc * q - dmin * m)
        out.append(f32_to_f16_bits(v))
    return out


def _q6k_block_scalar(b) -> list[int]:
    d = f16_bits_to_float(_u16(b, 208))
    out = []
    for e in range(256):
        h, r = divmod(e, 128)            # two halves of 128 elements
        g, l = divmod(r, 32)             # four groups of 32 within a half
        lo_byte = b[64 * h + l + 32 * (g & 1)]
        low4 = lo_byte & 15 if g < 2 else lo_byte >> 4
        high2 = (b[128 + 32 * h + l] >> (2 * g)) & 3
        q = low4 | (high2 << 4)
        s = _i8(b[192 + e // 16])
        v = f64_to_f32((d * float(s)) * float(q - 32))
        out.append(f32_to_f16_bits(v))
    return out


def _q80_block_scalar(b) -> list[int]:
    d = f16_bits_to_float(_u16(b, 0))
    return [f32_to_f16_bits(f64_to_f32(d * float(_i8(b[2 + j])))) for j in range(32)]


def _u32(b, off: int) -> int:
    return _u16(b, off) | (_u16(b, off + 2) << 16)


def _nibble32(b, qs_off: int, j: int) -> int:
    """4-bit quant of element j (0..31) of a 32-element block: low nibble of
    byte j for j < 16, high nibble of byte j - 16 otherwise."""
    byte = b[qs_off + (j % 16)]
    return byte & 15 if j < 16 else byte >> 4


def _q40_block_scalar(b) -> list[int]:
    d = f16_bits_to_float(_u16(b, 0))
    return [f32_to_f16_bits(f64_to_f32(d * float(_nibble32(b, 2, j) - 8))) for j in range(32)]


def _q50_block_scalar(b) -> list[int]:
    d = f16_bits_to_float(_u16(b, 0))
    qh = _u32(b, 2)
    out = []
    for j in range(32):
        q = _nibble32(b, 6, j) + 16 * ((qh >> j) & 1)
        out.append(f32_to_f16_bits(f64_to_f32(d * float(q - 16))))
    return out


def _q51_block_scalar(b) -> list[int]:
    d = f16_bits_to_float(_u16(b, 0))
    m = f16_bits_to_float(_u16(b, 2))
    qh = _u32(b, 4)
    out = []
    for j in range(32):
        q = _nibble32(b, 8, j) + 16 * ((qh >> j) & 1)
        # d*q is exact; d*q + m is exact in binary64 and rounds once to f32
        out.append(f32_to_f16_bits(f64_to_f32(d * q + m)))
    return out


def _q5k_block_scalar(b) -> list[int]:
    d = f16_bits_to_float(_u16(b, 0))
    dmin = f16_bits_to_float(_u16(b, 2))
    s = [b[4 + i] for i in range(12)]
    out = []
    for e in range(256):
        j = e // 32
        sc, m = q4k_scale_min(j, s)
        c, r = divmod(e, 64)
        l = r % 32
        byte = b[48 + 32 * c + l]
        low4 = byte & 15 if r < 32 else byte >> 4
        q = low4 + 16 * ((b[16 + l] >> j) & 1)
        out.append(f32_to_f16_bits(f64_to_f32(d * sc * q - dmin * m)))
    return out


_SCALAR = {Q4_K: _q4k_block_scalar, Q6_K: _q6k_block_scalar, Q8_0: _q80_block_scalar,
           Q4_0: _q40_block_scalar, Q5_0: _q50_block_scalar, Q5_1: _q51_block_scalar,
           Q5_K: _q5k_block_scalar}


def dequant_scalar(fmt: int, qbytes, N: int, K: int) -> np.ndarray:
    """Per-element decode (slow; for small inputs).  Returns uint16 f16 bits [N, K]."""
    q = np.frombuffer(bytes(np.asarray(qbytes, dtype=np.uint8).tobytes()), dtype=np.uint8)
    rb = row_bytes(fmt, K)
    if q.size != N * rb:
        raise ValueError(f"expected {N * rb} bytes, got {q.size}")
    bb, be = BLOCK_BYTES[fmt], BLOCK_ELEMS[fmt]
    out = np.empty((N, K), dtype=np.uint16)
    for n in range(N):
        for blk in range(K // be):
            off = n * rb + blk * bb
            out[n, blk * be:(blk + 1) * be] = _SCALAR[fmt](q[off:off + bb].tolist())
    return out


# ---------------------------------------------------------------------------
# Vectorized decoder: numpy float32 arithmetic, numpy's f16 cast.
# ---------------------------------------------------------------------------

def _f16_field(blk: np.ndarray, off: int) -> np.ndarray:
    """f16 field at byte ``off`` of every block, widened (exactly) to float32."""
    raw = blk[..., off].astype(np.uint16) | (blk[..., off + 1].astype(np.uint16) << 8)
    return raw.view(np.float16).astype(np.float32)


def _q4k_vec(blk: np.ndarray) -> np.ndarray:
    N, nb, _ = blk.shape
    d = _f16_field(blk, 0)
    dmin = _f16_field(blk, 2)
    s = blk[..., 4:16].astype(np.int32)
    sc = np.empty((N, nb, 8), np.int32)
    mn = np.empty((N, nb, 8), np.int32)
    sc[..., :4] = s[..., 0:4] & 63
    mn[..., :4] = s[..., 4:8] & 63
    sc[..., 4:] = (s[..., 8:12] & 15) | ((s[..., 0:4] >> 6) << 4)
    mn[..., 4:] = (s[..., 8:12] >> 4) | ((s[..., 4:8] >> 6) << 4)
    qs = blk[..., 16:144].reshape(N, nb, 4, 32)
    # sub-block 2c = low nibbles of chunk c, sub-block 2c+1 = high nibbles
    q = np.stack([qs & 15, qs >> 4], axis=3).reshape(N, nb, 8, 32).astype(np.float32)
    A = d[..., None] * sc.astype(np.float32)          # exact
    C = dmin[..., None] * mn.astype(np.float32)       # exact
    B = A[..., None] * q                              # exact
    V = B - C[..., None]                              # the one f32 rounding
    return V.astype(np.float16).view(np.uint16).reshape(N, nb * 256)


def _q6k_vec(blk: np.ndarray) -> np.ndarray:
    N, nb, _ = blk.shape
    ql = blk[..., 0:128].reshape(N, nb, 2, 2, 32)     # [half][g & 1][l]
    qh = blk[..., 128:192].reshape(N, nb, 2, 32)      # [half][l]
    sc = blk[..., 192:208].view(np.int8).astype(np.float32)
    d = _f16_field(blk, 208)
    low = np.empty((N, nb, 2, 4, 32), np.uint8)
    low[..., 0, :] = ql[..., 0, :] & 15
    low[..., 1, :] = ql[..., 1, :] & 15
    low[..., 2, :] = ql[..., 0, :] >> 4
    low[..., 3, :] = ql[..., 1, :] >> 4
    high = np.stack([(qh >> (2 * g)) & 3 for g in range(4)], axis=3)   # [N, nb, 2, 4, 32]
    q = (low | (high << 4)).astype(np.int32).reshape(N, nb, 16, 16)    # element 16*i + t
    ds = d[..., None] * sc                                             # [N, nb, 16], exact
    V = ds[..., None] * (q - 32).astype(np.float32)                    # exact, IEEE zero signs
    return V.astype(np.float16).view(np.uint16).reshape(N, nb * 256)


def _q80_vec(blk: np.ndarray) -> np.ndarray:
    N, nb, _ = blk.shape
    d = _f16_field(blk, 0)
    qv = np.ascontiguousarray(blk[..., 2:34]).view(np.int8).astype(np.float32)
    V = d[..., None] * qv
    return V.astype(np.float16).view(np.uint16).reshape(N, nb * 32)


def _nibbles32(qs: np.ndarray) -> np.ndarray:
    """[..., 16] bytes -> [..., 32] quants: elements 0..15 low nibbles, 16..31 high."""
    return np.concatenate([qs & 15, qs >> 4], axis=-1)


def _qh_bits32(blk: np.ndarray, off: int) -> np.ndarray:
    """Bit j of the little-endian u32 at byte ``off``, for j = 0..31."""
    b = blk[..., off:off + 4]
    bits = np.unpackbits(b, axis=-1, bitorder="little")      # byte 0 bits 0..7, byte 1 ...
    return bits


def _q40_vec(blk: np.ndarray) -> np.ndarray:
    N, nb, _ = blk.shape
    d = _f16_field(blk, 0)
    q = _nibbles32(blk[..., 2:18]).astype(np.float32) - 8.0
    V = d[..., None] * q
    return V.astype(np.float16).view(np.uint16).reshape(N, nb * 32)


def _q50_vec(blk: np.ndarray) -> np.ndarray:
    N, nb, _ = blk.shape
    d = _f16_field(blk, 0)
    q = _nibbles32(blk[..., 6:22]).astype(np.int32) + 16 * _qh_bits32(blk, 2).astype(np.int32)
    V = d[..., None] * (q - 16).astype(np.float32)
    return V.astype(np.float16).view(np.uint16).reshape(N, nb * 32)


def _q51_vec(blk: np.ndarray) -> np.ndarray:
    N, nb, _ = blk.shape
    d = _f16_field(blk, 0)
    m = _f16_field(blk, 2)
    q = _nibbles32(blk[..., 8:24]).astype(np.int32) + 16 * _qh_bits32(blk, 4).astype(np.int32)
    P = d[..., None] * q.astype(np.float32)          # exact
    V = P + m[..., None]                             # the one f32 rounding
    return V.astype(np.float16).view(np.uint16).reshape(N, nb * 32)


def _q5k_vec(blk: np.ndarray) -> np.ndarray:
    N, nb, _ = blk.shape
    d = _f16_field(blk, 0)
    dmin = _f16_field(blk, 2)
    s = blk[..., 4:16].astype(np.int32)
    sc = np.empty((N, nb, 8), np.int32)
    mn = np.empty((N, nb, 8), np.int32)
    sc[..., :4] = s[..., 0:4] & 63
    mn[..., :4] = s[..., 4:8] & 63
    sc[..., 4:] = (s[..., 8:12] & 15) | ((s[..., 0:4] >> 6) << 4)
    mn[..., 4:] = (s[..., 8:12] >> 4) | ((s[..., 4:8] >> 6) << 4)
    qh = blk[..., 16:48]                                              # [N, nb, 32] byte l
    hi = np.stack([(qh >> j) & 1 for j in range(8)], axis=2)          # [N, nb, 8, 32]
    qs = blk[..., 48:176].reshape(N, nb, 4, 32)
    low = np.stack([qs & 15, qs >> 4], axis=3).reshape(N, nb, 8, 32)
    q = (low.astype(np.int32) + 16 * hi.astype(np.int32)).astype(np.float32)
    A = d[..., None] * sc.astype(np.float32)
    C = dmin[..., None] * mn.astype(np.float32)
    V = A[..., None] * q - C[..., None]
    return V.astype(np.float16).view(np.uint16).reshape(N, nb * 256)


_VEC = {Q4_K: _q4k_vec, Q6_K: _q6k_vec, Q8_0: _q80_vec, Q4_0: _q40_vec, Q5_0: _q50_vec,
        Q5_1: _q51_vec, Q5_K: _q5k_vec}


def dequant_ref(fmt: int, qbytes: np.ndarray, N: int, K: int) -> np.ndarray:
    """Decode an N×K quantized weight (rows contiguous) to f16 bits, uint16 [N, K]."""
    q = np.ascontiguousarray(qbytes, dtype=np.uint8).reshape(-1)
    rb = row_bytes(fmt, K)
    if q.size != N * rb:
        raise ValueError(f"expected {N * rb} bytes, got {q.size}")
    blk = q.reshape(N, K // BLOCK_ELEMS[fmt], BLOCK_BYTES[fmt])
    out = np.empty((N, K), dtype=np.uint16)
    # row chunks keep the float32 temporaries small for the 18944-row matrices
    step = max(1, (1 << 22) // K)
    for n0 in range(0, N, step):
        out[n0:n0 + step] = _VEC[fmt](blk[n0:n0 + step])
    # the pages' "benign d" rule: inputs are built so no decode is NaN/Inf
    if np.any((out & 0x7C00) == 0x7C00):
        raise ValueError("decode produced Inf/NaN: the block scale fields are not benign")
    return out


def cache_ref(fmt: int, qbytes: np.ndarray, N: int, K: int, pad: bool = True) -> np.ndarray:
    """The persistent f16 cache: decode in columns [0, K), +0 (0x0000) in pad columns."""
    ld = cache_ld(K) if pad else K
    out = np.zeros((N, ld), dtype=np.uint16)
    out[:, :K] = dequant_ref(fmt, qbytes, N, K)
    return out
