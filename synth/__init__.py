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
* Q4_0: d = f16(|N(0,1)|·2⁻⁷); 16 uniform bytes of nibbles.
* Q5_0: d = f16(|N(0,1)|·2⁻⁷); 4 uniform bytes of qh; 16 uniform bytes.
* Q5_1: d = f16(|N(0,1)|·2⁻⁷); m = f16(−|N(0,1)|·2⁻³); 4 + 16 uniform bytes.
* Q5_K: as Q4_K, with 32 uniform bytes of qh between the scales and quants.
* X: f16(N(0,1)), [M, K].

``mode="integer"`` sets every f16 scale field to 1.0 (d = dmin = m = 1), so that
decoded weights are small integers; with integer X every partial sum of the
matmul is an exact integer in f32 whatever the summation order.
"""

from __future__ import annotations

import numpy as np

SEED_BASE = 20260831

# format ids (GGUF type numbers)
Q4_0 = 2
Q5_0 = 6
Q5_1 = 7
Q8_0 = 8
Q4_K = 12
Q5_K = 13
Q6_K = 14
_ELEMS = {Q4_0: 32, Q5_0: 32, Q5_1: 32, Q8_0: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256}
_BYTES = {Q4_0: 18, Q5_0: 22, Q5_1: 24, Q8_0: 34, Q4_K: 144, Q5_K: 176, Q6_K: 210}
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
    elif fmt in (Q4_0, Q5_0):
        d = _f16_abs_normal(g, (N, nb), 2.0 ** -7)
        if mode == "integer":
            d[:] = _ONE_F16
        _put_u16(blk, 0, d)
        blk[..., 2:] = g.integers(0, 256, (N, nb, _BYTES[fmt] - 2), dtype=np.uint8)
    elif fmt == Q5_1:
        d = _f16_abs_normal(g, (N, nb), 2.0 ** -7)
        m = _f16_abs_normal(g, (N, nb), 2.0 ** -3) | np.uint16(0x8000)
        if mode == "integer":
            d[:] = _ONE_F16
            m[:] = _ONE_F16
        _put_u16(blk, 0, d)
        _put_u16(blk, 2, m)
        blk[..., 4:24] = g.integers(0, 256, (N, nb, 20), dtype=np.uint8)
    elif fmt == Q5_K:
        d = _f16_abs_normal(g, (N, nb), 2.0 ** -7)
        dmin = _f16_abs_normal(g, (N, nb), 2.0 ** -7)
        if mode == "integer":
            d[:] = _ONE_F16
            dmin[:] = _ONE_F16
        _put_u16(blk, 0, d)
        _put_u16(blk, 2, dmin)
        blk[..., 4:176] = g.integers(0, 256, (N, nb, 172), dtype=np.uint8)
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
# extra M points measured when the crossover falls between two sweep points
SWEEP_REFINE = (256, 384, 768)


# ---------------------------------------------------------------------------
# Device-side drawing of the same distributions (torch's seeded generator),
# used where gigabytes of weights are needed quickly (the 28-layer benchmark
# set).  Same fields and distributions as ``weights``; a different random
# stream, so values differ from the numpy generator for the same seed.
# ---------------------------------------------------------------------------

def weights_device(fmt: int, seed: int, N: int, K: int, device, mode: str = "random"):
    """Quantized N×K weight as a contiguous uint8 device tensor [N, row_bytes]."""
    import torch

    if K % _ELEMS[fmt]:
        raise ValueError(f"K={K} not a multiple of {_ELEMS[fmt]}")
    nb = K // _ELEMS[fmt]
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([SEED_BASE, seed]).generate_state(1)[0]))

    def f16_abs_normal(scale):
        z = torch.randn((N, nb), generator=g, device=device, dtype=torch.float32)
        return (z.abs() * scale).to(torch.float16).view(torch.uint8).view(N, nb, 2)

    one = torch.tensor([0x00, 0x3C], dtype=torch.uint8, device=device)
    blk = torch.randint(0, 256, (N, nb, _BYTES[fmt]), generator=g, device=device,
                        dtype=torch.uint8)
    if fmt == Q4_K:
        blk[..., 0:2] = one if mode == "integer" else f16_abs_normal(2.0 ** -7)
        blk[..., 2:4] = one if mode == "integer" else f16_abs_normal(2.0 ** -7)
    elif fmt == Q6_K:
        sc = torch.randint(-32, 32, (N, nb, 16), generator=g, device=device, dtype=torch.int8)
        blk[..., 192:208] = sc.view(torch.uint8)
        blk[..., 208:210] = one if mode == "integer" else f16_abs_normal(2.0 ** -9)
    elif fmt == Q8_0:
        q = torch.randint(-127, 128, (N, nb, 32), generator=g, device=device, dtype=torch.int8)
        blk[..., 2:34] = q.view(torch.uint8)
        blk[..., 0:2] = one if mode == "integer" else f16_abs_normal(2.0 ** -7)
    elif fmt in (Q4_0, Q5_0):
        blk[..., 0:2] = one if mode == "integer" else f16_abs_normal(2.0 ** -7)
    elif fmt == Q5_1:
        blk[..., 0:2] = one if mode == "integer" else f16_abs_normal(2.0 ** -7)
        if mode == "integer":
            blk[..., 2:4] = one
        else:
            m = f16_abs_normal(2.0 ** -3).clone()
            m[..., 1] |= 0x80                       # sign bit of the f16 min
            blk[..., 2:4] = m
    elif fmt == Q5_K:
        blk[..., 0:2] = one if mode == "integer" else f16_abs_normal(2.0 ** -7)
        blk[..., 2:4] = one if mode == "integer" else f16_abs_normal(2.0 ** -7)
    else:
        raise ValueError(f"unknown format {fmt}")
    return blk.view(N, nb * _BYTES[fmt])


def activations_device(seed: int, M: int, K: int, device):
    """f16 N(0,1) activations [M, K] drawn on the device."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([SEED_BASE, seed, 1]).generate_state(1)[0]))
    return torch.randn((M, K), generator=g, device=device, dtype=torch.float32).to(torch.float16)
