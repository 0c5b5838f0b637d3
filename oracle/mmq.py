"""Reference for the int8 "MMQ" prefill product — TEST INFRASTRUCTURE ONLY
(see ``oracle/__init__``).

Source: Fucina "Eager GPU Offload Without A Compute Graph", the section on
what the ik_llama.cpp audit contributed.  Read there: the int8 backend turns
the f32 activations into int8 blocks carrying a scale and a code sum (the
Q8_1 arrangement), turns the quantized weights into signed int8 codes, runs
the contraction on the integer matrix units, and therefore computes with
other activation values than the f16 paths — so it gets a parity gate of its
own instead of the f16 tolerance.  minfer "05 · 8p" (§1, §6) and
"79" (§1, §5) name the int8 MMQ prefill GEMM that streams raw quantized
bytes.

The pages give no formulas; the readings used here:

* **Activation blocks.**  Each row of X (f32) is cut into blocks of 32
  consecutive elements.  Per block: a = max |x|; d = fl32(a / 127); each code
  q = the integer nearest to fl32(x / d), halves away from zero (q = 0 for
  every element when d = 0); s = fl32(d · Σq).  Codes are int8 (|q| ≤ 127);
  d and s are kept in f32.
* **Weights.**  Every format splits into an integer code c (int8 range) and
  per-group f32 factors with w = α·c − β, all exact in f32:
    Q8_0  α = d,       c = q,       β = 0
    Q4_0  α = d,       c = q − 8,   β = 0
    Q5_0  α = d,       c = q − 16,  β = 0
    Q5_1  α = d,       c = q,       β = −m
    Q4_K  α = d·sc,    c = q,       β = dmin·m   (per 32-element sub-block)
    Q5_K  α = d·sc,    c = q,       β = dmin·m   (per 32-element sub-block)
    Q6_K  α = d·s,     c = q − 32,  β = 0        (per 16-element group)
  fl32(α·c − β) is then exactly the f32 value the f16 decode rounds.
* **Product.**  For activation block b of row m and weight row n:
  Σ_{i∈b} (α c_i − β)·d q_i = d·Σ_G α_G·I_G − β·s with I_G = Σ_{i∈G} c_i q_i an
  exact integer over each weight group G inside b (one group of 32, or two of
  16 for Q6_K), and s standing for d·Σq.  Y[m, n] is the sum of that over b.

``mmq_ref`` evaluates the product in binary64 from the exact integers and f32
factors; the tolerance scale S bounds the magnitudes of the summed terms.
"""

from __future__ import annotations

import math

import numpy as np

from .f16 import f64_to_f32
from .formats import (BLOCK_BYTES, BLOCK_ELEMS, Q4_0, Q4_K, Q5_0, Q5_1, Q5_K, Q6_K, Q8_0,
                      _f16_field, _nibbles32, _qh_bits32, row_bytes)

QBLOCK = 32   # activation block


# ---------------------------------------------------------------------------
# Activation quantization
# ---------------------------------------------------------------------------

def quantize_q8_1(x: np.ndarray):
    """(q int8 [M, K], d float32 [M, K/32], s float32 [M, K/32]) for finite f32 X."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    if K % QBLOCK:
        raise ValueError("K must be a multiple of 32")
    xb = x.reshape(M, K // QBLOCK, QBLOCK)
    a = np.max(np.abs(xb), axis=-1)
    d = (a / np.float32(127)).astype(np.float32)
    live = d > 0
    safe = np.where(live, d, np.float32(1))
    t = (xb / safe[..., None]).astype(np.float32)                 # one f32 division
    tt = t.astype(np.float64)
    q = np.sign(tt) * np.floor(np.abs(tt) + 0.5)                  # exact in f64
    q = np.where(live[..., None], q, 0).astype(np.int64)
    s = (d * q.sum(axis=-1).astype(np.float32)).astype(np.float32)
    return q.reshape(M, K).astype(np.int8), d, s


def quantize_q8_1_scalar(x: np.ndarray):
    """The same, element by element in Python floats with explicit f32
    roundings (small inputs only).  Division and products are done in
    binary64 and rounded once to binary32, which equals the correctly rounded
    binary32 operation (53 ≥ 2·24 + 2)."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    nb = K // QBLOCK
    q = np.zeros((M, K), np.int8)
    d = np.zeros((M, nb), np.float32)
    s = np.zeros((M, nb), np.float32)
    for m in range(M):
        for b in range(nb):
            vals = [float(v) for v in x[m, b * QBLOCK:(b + 1) * QBLOCK]]
            a = max(abs(v) for v in vals)
            db = f64_to_f32(a / 127.0)
            codes = []
            for v in vals:
                if db == 0.0:
                    codes.append(0)
                    continue
                t = f64_to_f32(v / db)
                codes.append(int(math.copysign(math.floor(abs(t) + 0.5), t)))
            q[m, b * QBLOCK:(b + 1) * QBLOCK] = codes
            d[m, b] = db
            s[m, b] = f64_to_f32(db * sum(codes))
    return q, d, s


# ---------------------------------------------------------------------------
# Weight decomposition w = α·c − β
# ---------------------------------------------------------------------------

def _blocks(fmt: int, wq, N: int, K: int) -> np.ndarray:
    q = np.frombuffer(np.asarray(wq, dtype=np.uint8).tobytes(), dtype=np.uint8)
    if q.size != N * row_bytes(fmt, K):
        raise ValueError("quantized size does not match N, K")
    return q.reshape(N, K // BLOCK_ELEMS[fmt], BLOCK_BYTES[fmt])


def _ksub_scales(blk: np.ndarray):
    """Q4_K / Q5_K: (sc, m) [N, nb, 8] of the eight 32-element sub-blocks."""
    N, nb, _ = blk.shape
    s = blk[..., 4:16].astype(np.int32)
    sc = np.empty((N, nb, 8), np.int32)
    mn = np.empty((N, nb, 8), np.int32)
    sc[..., :4] = s[..., 0:4] & 63
    mn[..., :4] = s[..., 4:8] & 63
    sc[..., 4:] = (s[..., 8:12] & 15) | ((s[..., 0:4] >> 6) << 4)
    mn[..., 4:] = (s[..., 8:12] >> 4) | ((s[..., 4:8] >> 6) << 4)
    return sc, mn


def decompose(fmt: int, wq, N: int, K: int):
    """(c int8 [N, K], alpha float32 [N, K/g], beta float32 [N, K/32], g)."""
    blk = _blocks(fmt, wq, N, K)
    nb = blk.shape[1]
    zero_beta = np.zeros((N, K // QBLOCK), np.float32)
    if fmt == Q8_0:
        c = np.ascontiguousarray(blk[..., 2:34]).view(np.int8).astype(np.int32)
        return c.reshape(N, K).astype(np.int8), _f16_field(blk, 0), zero_beta, 32
    if fmt == Q4_0:
        c = _nibbles32(blk[..., 2:18]).astype(np.int32) - 8
        return c.reshape(N, K).astype(np.int8), _f16_field(blk, 0), zero_beta, 32
    if fmt in (Q5_0, Q5_1):
        qs, qh = (6, 2) if fmt == Q5_0 else (8, 4)
        q = _nibbles32(blk[..., qs:qs + 16]).astype(np.int32) + \
            16 * _qh_bits32(blk, qh).astype(np.int32)
        if fmt == Q5_0:
            return (q - 16).reshape(N, K).astype(np.int8), _f16_field(blk, 0), zero_beta, 32
        beta = (-_f16_field(blk, 2)).astype(np.float32)
        return q.reshape(N, K).astype(np.int8), _f16_field(blk, 0), beta, 32
    if fmt in (Q4_K, Q5_K):
        d = _f16_field(blk, 0)
        dmin = _f16_field(blk, 2)
        sc, mn = _ksub_scales(blk)
        if fmt == Q4_K:
            qs = blk[..., 16:144].reshape(N, nb, 4, 32)
            q = np.stack([qs & 15, qs >> 4], axis=3).reshape(N, nb, 8, 32).astype(np.int32)
        else:
            qh = blk[..., 16:48]
            hi = np.stack([(qh >> j) & 1 for j in range(8)], axis=2).astype(np.int32)
            qs = blk[..., 48:176].reshape(N, nb, 4, 32)
            q = np.stack([qs & 15, qs >> 4], axis=3).reshape(N, nb, 8, 32).astype(np.int32) + 16 * hi
        alpha = (d[..., None] * sc.astype(np.float32)).astype(np.float32).reshape(N, nb * 8)
        beta = (dmin[..., None] * mn.astype(np.float32)).astype(np.float32).reshape(N, nb * 8)
        return q.reshape(N, K).astype(np.int8), alpha, beta, 32
    if fmt == Q6_K:
        ql = blk[..., 0:128].reshape(N, nb, 2, 2, 32)
        qh = blk[..., 128:192].reshape(N, nb, 2, 32)
        low = np.empty((N, nb, 2, 4, 32), np.int32)
        low[..., 0, :] = ql[..., 0, :] & 15
        low[..., 1, :] = ql[..., 1, :] & 15
        low[..., 2, :] = ql[..., 0, :] >> 4
        low[..., 3, :] = ql[..., 1, :] >> 4
        high = np.stack([(qh >> (2 * g)) & 3 for g in range(4)], axis=3).astype(np.int32)
        q = (low | (high << 4)).reshape(N, K)
        sc = blk[..., 192:208].view(np.int8).astype(np.float32)
        alpha = (_f16_field(blk, 208)[..., None] * sc).astype(np.float32).reshape(N, nb * 16)
        return (q - 32).astype(np.int8), alpha, zero_beta, 16
    raise ValueError(f"unknown format {fmt}")


def weights_f32(fmt: int, wq, N: int, K: int) -> np.ndarray:
    """fl32(α·c − β) per element: the f32 value each format's decode rounds to f16."""
    c, alpha, beta, g = decompose(fmt, wq, N, K)
    a = np.repeat(alpha, g, axis=1)
    b = np.repeat(beta, QBLOCK, axis=1)
    return (a * c.astype(np.float32) - b).astype(np.float32)


# ---------------------------------------------------------------------------
# The product
# ---------------------------------------------------------------------------

def mmq_ref(xq: np.ndarray, xd: np.ndarray, xs: np.ndarray, fmt: int, wq, N: int, K: int):
    """(Y, S) in float64 [M, N]: Y = Σ_b (d_b·Σ_G α_G·I_G − β_b·s_b), S the sum of
    the magnitudes |d q|·|α c| over elements plus |β|·|s| over blocks."""
    c, alpha, beta, g = decompose(fmt, wq, N, K)
    Qt = xq.astype(np.float64) * np.repeat(xd.astype(np.float64), QBLOCK, axis=1)  # exact
    Wt = c.astype(np.float64) * np.repeat(alpha.astype(np.float64), g, axis=1)     # exact
    sx = xs.astype(np.float64)
    bw = beta.astype(np.float64)
    Y = Qt @ Wt.T - sx @ bw.T
    S = np.abs(Qt) @ np.abs(Wt).T + np.abs(sx) @ np.abs(bw).T
    return Y, S


def mmq_bruteforce(xq, xd, xs, fmt: int, wq, N: int, K: int) -> np.ndarray:
    """Exact rational Y by explicit loops over activation blocks, weight groups
    and elements (tiny inputs only); returned as float64."""
    from fractions import Fraction

    c, alpha, beta, g = decompose(fmt, wq, N, K)
    M = xq.shape[0]
    Y = np.empty((M, N), np.float64)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for b in range(K // QBLOCK):
                inner = Fraction(0)
                for G in range(QBLOCK // g):
                    k0 = b * QBLOCK + G * g
                    I = sum(int(c[n, k]) * int(xq[m, k]) for k in range(k0, k0 + g))
                    inner += Fraction(float(alpha[n, k0 // g])) * I
                tot += Fraction(float(xd[m, b])) * inner - Fraction(float(beta[n, b])) * Fraction(float(xs[m, b]))
            Y[m, n] = float(tot)
    return Y
