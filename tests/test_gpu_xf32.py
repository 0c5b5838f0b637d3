"""Parity of the f32-activation entry points with the oracle: the standalone
convert (bit for bit against ``oracle.activations_to_f16``) and both GEMM
shapes with f32 X, whose defined result is the f16 GEMM on f16_rne(X):

* both ways the library runs them: M <= 64 rounds X inside the A-tile load
  (its own tiles), M > 64 converts X into the workspace first (padded row
  stride when 2K bytes is a multiple of 2048) and runs the f16 kernel;
* without a K split, bit-identical to the f16-activation entry point fed the
  oracle's rounding of X (so a conversion that rounds differently anywhere, or
  a wrong stride, fails), at ragged shapes and padded f32 rows;
* integer-valued X and W exact, with automatic and forced K splits;
* one-hot X reproduces the expanded weights for every format;
* random inputs within the tolerance of the f64 oracle."""

import numpy as np
import pytest

import oracle
import synth
from gpu_common import (announce, assert_bits_equal, check_gemm, dev, f16_bits, needs_gpu,
                        to_dev_f16, to_dev_u8, to_host)

pytestmark = [pytest.mark.gpu, needs_gpu]

import torch  # noqa: E402

import quantized_weight_prefill_q4_amd as mq  # noqa: E402

NAME = {0: "f16", 2: "Q4_0", 6: "Q5_0", 7: "Q5_1", 8: "Q8_0", 12: "Q4_K", 13: "Q5_K", 14: "Q6_K"}
ALL = [2, 6, 7, 8, 12, 13, 14]


def _x32(seed, M, K, mode="random"):
    g = np.random.default_rng(seed)
    if mode == "integer":
        return g.integers(-2, 3, (M, K)).astype(np.float32)
    if mode == "onehot":
        return np.eye(M, K, dtype=np.float32)
    return g.standard_normal((M, K), dtype=np.float32)


def _dev_x32(x, pad=0):
    """Device f32 copy with row stride K + pad (pad a multiple of 4)."""
    M, K = x.shape
    buf = torch.full((M, K + pad), float("nan"), dtype=torch.float32, device=dev())
    buf[:, :K] = torch.from_numpy(x).to(dev())
    return buf[:, :K]


def _cache(fmt, N, K, seed, mode="random"):
    q = synth.weights(fmt, synth.rng(seed, 0, fmt, N), N, K, mode=mode)
    return q, oracle.cache_ref(fmt, q, N, K, pad=True)


def test_convert_hand_derived_and_random_bits():
    from conftest import read_golden
    rows = [r.split("|") for r in read_golden("f32_to_f16_rounding.txt")["value"]]
    special = np.array([int(r[0], 16) for r in rows], np.uint32).view(np.float32)
    g = np.random.default_rng(72)
    bits = g.integers(0, 2 ** 32, 37 * 520, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32).copy()
    x[np.isnan(x)] = 1.5
    x[: special.size] = special
    x = x.reshape(37, 520)
    out = torch.full((37, 528), float("nan"), dtype=torch.float16, device=dev())
    announce("convert_f32_to_f16", "M=37 K=520 ldx=524 ld16=528")
    mq.convert_f32_to_f16(_dev_x32(x, pad=4), out=out[:, :520])
    got = f16_bits(out)
    assert_bits_equal(got[:, :520], oracle.activations_to_f16(x), "convert")
    assert np.all(got[:, 520:] == 0x7E00), "columns past K were written"


def test_convert_beyond_one_grid():
    """65537 × 32768 elements = 2^28 + 4096 chunks of 8: more than the capped
    grid covers in one pass, so the last row is converted on the second pass
    of the grid-stride loop (8.6 GB in, 4.3 GB out)."""
    M, K = 65537, 32768
    announce("convert_f32_to_f16", f"M={M} K={K}")
    gen = torch.Generator(device=dev())
    gen.manual_seed(73)
    x = torch.randn((M, K), generator=gen, device=dev(), dtype=torch.float32)
    y = mq.convert_f32_to_f16(x)
    for r in (0, 1, 32767, M - 2, M - 1):
        xr = x[r].cpu().numpy()
        assert_bits_equal(f16_bits(y[r]), oracle.activations_to_f16(xr), f"row {r}")
    del x, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M,N,K,pad", [(1, 1, 8, 0), (7, 33, 56, 4), (64, 200, 264, 4),
                                       (65, 130, 72, 0), (64, 300, 4096, 0),
                                       (100, 300, 4096, 4), (129, 257, 520, 8),
                                       (300, 1000, 1024, 4), (2048, 8448, 2048, 0)])
def test_cache_xf32_equals_f16_path_at_split1(M, N, K, pad):
    x = _x32(80 + M, M, K)
    w = oracle.activations_to_f16(_x32(81 + N, N, K))      # any f16 weights
    wd = to_dev_f16(w)
    announce("gemm_f16cache_xf32", f"M={M} N={N} K={K} pad={pad}", "split=1")
    y32 = to_host(mq.gemm_f16cache(_dev_x32(x, pad), wd, K, split_k=1))
    announce("gemm_f16cache", f"M={M} N={N} K={K}", "split=1")
    y16 = to_host(mq.gemm_f16cache(to_dev_f16(oracle.activations_to_f16(x)), wd, K, split_k=1))
    assert np.array_equal(y32, y16)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(M).choice(M, min(M, 8))]))
    check_gemm(y32[rows], oracle.activations_to_f16(x), w, K, f"xf32 cache {M}x{N}x{K}",
               rows=rows)


@pytest.mark.parametrize("M", [37, 129])
@pytest.mark.parametrize("fmt", ALL)
def test_fused_xf32_random_tolerance_and_identity(fmt, M):
    N, K = 300, 1024 if fmt not in (12, 13, 14) else 1280
    q = synth.weights(fmt, synth.rng(82, 0, fmt, 0), N, K)
    x = _x32(83, M, K)
    xd = _dev_x32(x, pad=4)
    announce("gemm_fused_xf32", NAME[fmt], f"M={M} N={N} K={K}")
    y = to_host(mq.gemm_fused(xd, to_dev_u8(q), fmt, N, K))
    xb = oracle.activations_to_f16(x)
    check_gemm(y, xb, oracle.dequant_ref(fmt, q, N, K), K, f"fused xf32 {NAME[fmt]}")
    announce("gemm_fused_xf32 vs gemm_fused", NAME[fmt], "split=1")
    y1 = to_host(mq.gemm_fused(xd, to_dev_u8(q), fmt, N, K, split_k=1))
    y16 = to_host(mq.gemm_fused(to_dev_f16(xb), to_dev_u8(q), fmt, N, K, split_k=1))
    assert np.array_equal(y1, y16)


@pytest.mark.parametrize("fmt", ALL)
def test_fused_xf32_onehot_expansion(fmt):
    N, K = 130, 256
    q = synth.weights(fmt, synth.rng(84, 0, fmt, 0), N, K)
    exp = oracle.dequant_ref(fmt, q, N, K).view(np.float16).astype(np.float32).T
    announce("gemm_fused_xf32", NAME[fmt], f"onehot K={K} N={N}")
    y = to_host(mq.gemm_fused(_dev_x32(_x32(0, K, K, "onehot")), to_dev_u8(q), fmt, N, K))
    assert np.array_equal(y, exp)
    # in-tile conversion: the first 64 rows of the identity give elements 0..63
    announce("gemm_fused_xf32", NAME[fmt], f"onehot rows 0..63 K={K} N={N}")
    y = to_host(mq.gemm_fused(_dev_x32(_x32(0, 64, K, "onehot")), to_dev_u8(q), fmt, N, K))
    assert np.array_equal(y, exp[:64])


@pytest.mark.parametrize("fmt,M,N,K", [(12, 2048, 512, 3584), (14, 70, 130, 2048),
                                       (14, 50, 130, 2048), (8, 33, 257, 1056),
                                       (0, 100, 300, 1024), (13, 64, 300, 2048),
                                       (13, 2048, 8448, 2048), (0, 2048, 8448, 2048)])
@pytest.mark.parametrize("split", [0, 3])
def test_xf32_integer_exact(fmt, M, N, K, split):
    """Integer X and W: every partial sum exact, whatever the split; the
    2048 × 512 × 3584 case takes the automatic tail split."""
    mode = "integer"
    x = _x32(85, M, K, mode)
    if fmt == 0:
        w = _x32(86, N, K, mode)
        wb = oracle.activations_to_f16(w)
        announce("gemm_f16cache_xf32", f"M={M} N={N} K={K} split={split}")
        y = to_host(mq.gemm_f16cache(_dev_x32(x), to_dev_f16(wb), K, split_k=split))
    else:
        q = synth.weights(fmt, synth.rng(86, 0, fmt, 0), N, K, mode=mode)
        wb = oracle.dequant_ref(fmt, q, N, K)
        announce("gemm_fused_xf32", NAME[fmt], f"M={M} N={N} K={K} split={split}")
        y = to_host(mq.gemm_fused(_dev_x32(x), to_dev_u8(q), fmt, N, K, split_k=split))
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(86).choice(M, min(M, 24))]))
    yref, _ = oracle.gemm_ref(oracle.activations_to_f16(x[rows]), wb)
    assert np.array_equal(y[rows].astype(np.float64), yref)


def test_xf32_workspace_query_matches_binding():
    assert mq.workspace_bytes(12, 2048, 18944, 3584, 0, x_f32=True) == \
        2048 * 3584 * 2 + mq.workspace_bytes(12, 2048, 18944, 3584, 0)
    assert mq.workspace_bytes(14, 64, 4096, 4096, 1, x_f32=True) == 0
