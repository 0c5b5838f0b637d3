"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module only draws random numbers and places them into the block byte
layouts; it decodes nothing and holds none of the matmul's arithmetic.  The
quantized weights stand in for the real GGUF models the pages measure (7B
q4_k_m, Llama-3.1 8B Q4_K_M), which are not available here.

Distributions (per matrix, drawn in this order, arrays shaped [N, nb, ...]):

* Q4_K: d = f16(|N(0,1)|·2⁻⁷); dmin the same; 12 uniform bytes of packed
  scales/mins (uniform 6-bit scales and mins, since the packing is a
  bijection on the 96 bits); 128 uniform bytes of quants (uniform 0..15).
* Q6_K: 128 uniform bytes of low nibbles; 64 uniform bytes of 2-bit pairs
  (so q is uniform 0..63); 16 int8 scales uniform −32..31; d = f16(|N|·2⁻⁹).
* Q8_0: d = f16(|N(0,1)|·2⁻⁷); 32 int8 uniform −127..127.
* X: f16(N(0,1)), [M, K].

``mode="integer"`` sets every f16 scale field to 1.0 (d = dmin = 1), so that
decoded weights are small integers; with integer X every partial sum of the
matmul is an exact integer in f32 whatever the summation order.
"""

from __future__ import annotations

import numpy as np

SEED_BASE = 20260831

# format ids (GGUF type numbers)
Q8_0 = 8
Q4_K = 12
Q6_K = 14
_ELEMS = {Q8_0: 32, Q4_K: 256, Q6_K: 256}
_BYTES = {Q8_0: 34, Q4_K: 144, Q6_K: 210}
_ONE_F16 = 0x3C00


def rng(cfg: int, layer: int = 0, mat: int = 0, role: int = 0) -> np.random.Generator:
    """Generator for one (config, layer, matrix, role) tuple; role 0 = W, 1 = X."""
    return np.random.default_rng(np.random.SeedSequence([SEED_BASE, cfg, layer, mat, role]))


def _f16_abs_normal(g: np.random.Generator, shape, scale: float) -> np.ndarray:
    return (np.abs(g.standard_normal(shape)) * scale).astype(np.float16).view(np.uint16)


def _put_u16(blk: np.ndarray, off: int, v: np.ndarray) -> None:
    v = np.asarray(v, dtype=np.uint16)
    blk[..., off] = (v & 0xFF).astype(np.uint8)
    blk[..., off + 1] = (v >> 8).astype(np.uint8)


def weights(fmt: int, g: np.random.Generator, N: int, K: int, mode: str = "random") -> np.ndarray:
    """Quantized N×K weight as uint8 [N, row_bytes] (rows contiguous)."""
    if K % _ELEMS[fmt]:
        raise ValueError(f"K={K} not a multiple of {_ELEMS[fmt]}")
    nb = K // _ELEMS[fmt]
    blk = np.empty((N, nb, _BYTES[fmt]), dtype=np.uint8)
    if fmt == Q4_K:
        d = _f16_abs_normal(g, (N, nb), 2.0 ** -7)
        dmin = _f16_abs_normal(g, (N, nb), 2.0 ** -7)
        if mode == "integer":
            d[:] = _ONE_F16
            dmin[:] = _ONE_F16
        _put_u16(blk, 0, d)
        _put_u16(blk, 2, dmin)
        blk[..., 4:16] = g.integers(0, 256, (N, nb, 12), dtype=np.uint8)
        blk[..., 16:144] = g.integers(0, 256, (N, nb, 128), dtype=np.uint8)
    elif fmt == Q6_K:
        blk[..., 0:128] = g.integers(0, 256, (N, nb, 128), dtype=np.uint8)
        blk[..., 128:192] = g.integers(0, 256, (N, nb, 64), dtype=np.uint8)
        blk[..., 192:208] = g.integers(-32, 32, (N, nb, 16), dtype=np.int8).view(np.uint8)
        d = _f16_abs_normal(g, (N, nb), 2.0 ** -9)
        if mode == "integer":
            d[:] = _ONE_F16
        _put_u16(blk, 208, d)
    elif fmt == Q8_0:
        d = _f16_abs_normal(g, (N, nb), 2.0 ** -7)
        if mode == "integer":
            d[:] = _ONE_F16
        _put_u16(blk, 0, d)
        blk[..., 2:34] = g.integers(-127, 128, (N, nb, 32), dtype=np.int8).view(np.uint8)
    else:
        raise ValueError(f"unknown format {fmt}")
    return blk.reshape(N, nb * _BYTES[fmt])


def activations(g: np.random.Generator, M: int, K: int, mode: str = "random") -> np.ndarray:
    """f16 activations as uint16 bit patterns [M, K]."""
    if mode == "integer":
        return g.integers(-2, 3, (M, K)).astype(np.float16).view(np.uint16)
    if mode == "onehot":
        if M != K:
            raise ValueError("one-hot activations need M == K")
        return np.eye(M, dtype=np.float16).view(np.uint16)
    return g.standard_normal((M, K), dtype=np.float32).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------------------
# Workload shapes (matrix name, format, N, K)
# ---------------------------------------------------------------------------

#: one 7B layer: attention projections (GQA, 4 KV heads × 128) and the FFN
LAYER_7B = (
    ("q", Q4_K, 3584, 3584),
    ("k", Q4_K, 512, 3584),
    ("v", Q4_K, 512, 3584),
    ("o", Q4_K, 3584, 3584),
    ("gate", Q4_K, 18944, 3584),
    ("up", Q4_K, 18944, 3584),
    ("down", Q6_K, 3584, 18944),
)
N_LAYERS_7B = 28

#: Llama-3.1-8B-like sweep shapes
SWEEP_8B = (
    ("q4k_4096x4096", Q4_K, 4096, 4096),
    ("q4k_14336x4096", Q4_K, 14336, 4096),
    ("q4k_4096x14336", Q4_K, 4096, 14336),
    ("q80_4096x4096", Q8_0, 4096, 4096),
)
SWEEP_M = (128, 512, 1024, 2048)
