"""Parity of the four further block formats (Q4_0, Q5_0, Q5_1, Q5_K) on both
shapes of the method, against the oracle:

* the hand-built blocks of tests/golden/ (bit patterns derived by hand from the
  formats' definitions) through the decode and, with one-hot activations,
  through the fused kernel's expansion;
* every 2-byte residue of an 18- or 22-byte block start inside a row;
* small, ragged and padded shapes and a full 4096 × 4096 compare of the decode;
* a batched decode mixing all seven formats;
* the fused GEMM: one-hot expansion, integer-exact at several K splits and on
  the 256 × 256 tile grid, random inputs within tolerance, and bit identity with
  the cache path at split 1."""

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden
from gpu_common import (announce, assert_bits_equal, check_gemm, f16_bits, needs_gpu,
                        to_dev_f16, to_dev_u8, to_host)

pytestmark = [pytest.mark.gpu, needs_gpu]

import quantized_weight_prefill_q4_amd as mq  # noqa: E402

NEW = [synth.Q4_0, synth.Q5_0, synth.Q5_1, synth.Q5_K]
NAME = {2: "Q4_0", 6: "Q5_0", 7: "Q5_1", 8: "Q8_0", 12: "Q4_K", 13: "Q5_K", 14: "Q6_K"}
GOLDEN = {2: "q40_worked.txt", 6: "q50_worked.txt", 7: "q51_worked.txt", 13: "q5k_worked.txt"}
ELEMS = {2: 32, 6: 32, 7: 32, 13: 256}


def _golden(fmt):
    """(blocks as one uint8 array of N rows, list of {element: f16 bits} per row)."""
    blocks, expect = [], []
    for row in read_golden(GOLDEN[fmt])["block"]:
        b, e = row.split("|")
        blocks.append(bytes(int(t, 16) for t in b.split()))
        expect.append({int(k): int(v, 16) for k, v in (t.split(":") for t in e.split())})
    return np.frombuffer(b"".join(blocks), np.uint8).copy(), expect


def _dequant(fmt, q, N, K, pad):
    announce("dequant", NAME[fmt], f"N={N}", f"K={K}", f"pad={pad}")
    return f16_bits(mq.dequant_to_f16(to_dev_u8(q), fmt, N, K, pad=pad))


def _fused(fmt, x_bits, q, N, K, split_k=0):
    announce("gemm_fused", NAME[fmt], f"M={x_bits.shape[0]}", f"N={N}", f"K={K}",
             f"split={split_k}")
    return to_host(mq.gemm_fused(to_dev_f16(x_bits), to_dev_u8(q), fmt, N, K, split_k=split_k))


@pytest.mark.parametrize("fmt", NEW)
def test_golden_blocks_decode(fmt):
    q, expect = _golden(fmt)
    K = ELEMS[fmt]
    w = _dequant(fmt, q, len(expect), K, False)
    for r, exp in enumerate(expect):
        for e, bits in exp.items():
            assert int(w[r, e]) == bits, f"row {r} element {e}: {w[r, e]:#06x} != {bits:#06x}"


@pytest.mark.parametrize("fmt", NEW)
def test_golden_blocks_fused(fmt):
    """One-hot X makes Y[e, r] the expanded weight (e, r); compared by value."""
    q, expect = _golden(fmt)
    K = ELEMS[fmt]
    Y = _fused(fmt, synth.activations(None, K, K, mode="onehot"), q, len(expect), K)
    for r, exp in enumerate(expect):
        for e, bits in exp.items():
            want = float(np.uint16(bits).view(np.float16))
            assert Y[e, r] == want, f"row {r} element {e}: {Y[e, r]} != {want}"


@pytest.mark.parametrize("fmt,K", [(2, 32), (2, 96), (6, 32), (6, 160), (7, 32), (7, 64)])
def test_block_start_residues(fmt, K):
    """Rows of 1, 3 or 5 small blocks: with 18- and 22-byte blocks every even
    residue mod 16 occurs as a block start, in both paths."""
    N = 24
    q = synth.weights(fmt, synth.rng(50, 0, fmt, K), N, K)
    exp = oracle.dequant_ref(fmt, q, N, K)
    assert_bits_equal(_dequant(fmt, q, N, K, False), exp, f"{NAME[fmt]} {N}x{K}")
    Y = _fused(fmt, synth.activations(None, K, K, mode="onehot"), q, N, K)
    assert np.array_equal(Y, exp.view(np.float16).astype(np.float32).T)


@pytest.mark.parametrize("fmt,N,K", [
    (2, 1, 32), (2, 37, 1024), (2, 64, 4096 + 32), (6, 5, 96), (6, 33, 2048),
    (7, 1, 32), (7, 65, 1056), (13, 1, 256), (13, 37, 512), (13, 7, 18944),
])
@pytest.mark.parametrize("pad", [True, False])
def test_small_and_ragged(fmt, N, K, pad):
    q = synth.weights(fmt, synth.rng(51, 0, fmt, N), N, K)
    got = _dequant(fmt, q, N, K, pad)
    exp = oracle.cache_ref(fmt, q, N, K, pad=pad)
    assert got.shape == exp.shape
    assert_bits_equal(got, exp, f"{NAME[fmt]} {N}x{K} pad={pad}")


@pytest.mark.parametrize("fmt", NEW)
def test_full_4096_square(fmt):
    q = synth.weights(fmt, synth.rng(52, 0, fmt, 0), 4096, 4096)
    assert_bits_equal(_dequant(fmt, q, 4096, 4096, True),
                      oracle.cache_ref(fmt, q, 4096, 4096, pad=True), f"{NAME[fmt]} 4096^2")


def test_batch_of_all_formats():
    """One batched call over 18 jobs of all seven formats (two launches: 16 + 2),
    each cache equal to the oracle's."""
    shapes = [(2, 33, 96), (6, 7, 2048), (7, 130, 32), (13, 3, 768), (12, 5, 256),
              (14, 9, 512), (8, 65, 64), (13, 64, 4096), (2, 1, 4096)]
    jobs, exp = [], []
    for i in range(18):
        fmt, N, K = shapes[i % len(shapes)]
        q = synth.weights(fmt, synth.rng(53, 0, fmt, i), N, K)
        jobs.append((to_dev_u8(q), fmt, N, K))
        exp.append((fmt, N, K, oracle.cache_ref(fmt, q, N, K, pad=True)))
    announce("dequant_batch", f"{len(jobs)} jobs, seven formats")
    for (fmt, N, K, e), o in zip(exp, mq.dequant_to_f16_batch(jobs, pad=True)):
        assert_bits_equal(f16_bits(o), e, f"batch {NAME[fmt]} {N}x{K}")


@pytest.mark.parametrize("fmt,N,K", [(2, 300, 256), (6, 130, 512), (7, 257, 96),
                                     (13, 200, 256), (13, 64, 512)])
def test_onehot_expansion_is_the_decode(fmt, N, K):
    q = synth.weights(fmt, synth.rng(54, 0, fmt, N), N, K)
    Y = _fused(fmt, synth.activations(None, K, K, mode="onehot"), q, N, K)
    exp = oracle.dequant_ref(fmt, q, N, K).view(np.float16).astype(np.float32).T
    assert np.array_equal(Y, exp)


@pytest.mark.parametrize("fmt,M,N,K", [(2, 100, 300, 1024), (6, 33, 257, 1056),
                                       (7, 70, 130, 2048), (13, 65, 200, 1280)])
@pytest.mark.parametrize("split", [0, 1, 3])
def test_integer_exact(fmt, M, N, K, split):
    q = synth.weights(fmt, synth.rng(55, 0, fmt, 0), N, K, mode="integer")
    x = synth.activations(synth.rng(55, role=1), M, K, mode="integer")
    Y = _fused(fmt, x, q, N, K, split_k=split)
    Yref, _ = oracle.gemm_ref(x, oracle.dequant_ref(fmt, q, N, K))
    assert np.array_equal(Y.astype(np.float64), Yref)


@pytest.mark.parametrize("fmt", NEW)
def test_large_tile_mixed_grid_integer_exact(fmt):
    """M = 2048, N = 8448: 264 tiles of 256 × 256, one round over all of K plus
    8 K-split tail tiles; integer inputs keep every partial sum exact (the
    largest Q5_K weight is 63·31, so |Y| < 2·1953·2048 < 2^24)."""
    M, N, K = 2048, 8448, 2048
    q = synth.weights(fmt, synth.rng(56, 0, fmt, 0), N, K, mode="integer")
    x = synth.activations(synth.rng(56, role=1), M, K, mode="integer")
    Y = _fused(fmt, x, q, N, K)
    rows = np.unique(np.concatenate([[0, 255, 1023, 1024, 2047],
                                     np.random.default_rng(56).choice(M, 16)]))
    Yref, _ = oracle.gemm_ref(x[rows], oracle.dequant_ref(fmt, q, N, K))
    assert np.array_equal(Y[rows].astype(np.float64), Yref)


@pytest.mark.parametrize("fmt,M,N,K", [(2, 129, 200, 1280), (6, 64, 512, 512),
                                       (7, 257, 96, 768), (13, 65, 333, 2304),
                                       (7, 1, 1, 32), (13, 1, 3, 256)])
def test_random_tolerance_and_cache_identity(fmt, M, N, K):
    q = synth.weights(fmt, synth.rng(57, 0, fmt, M), N, K)
    x = synth.activations(synth.rng(57, role=1), M, K)
    check_gemm(_fused(fmt, x, q, N, K), x, oracle.dequant_ref(fmt, q, N, K), K,
               f"fused {NAME[fmt]} {M}x{N}x{K}")
    Yf1 = _fused(fmt, x, q, N, K, split_k=1)
    announce("dequant+gemm_f16cache", NAME[fmt], f"M={M} N={N} K={K}", "split=1")
    cache = mq.dequant_to_f16(to_dev_u8(q), fmt, N, K)
    Yc1 = to_host(mq.gemm_f16cache(to_dev_f16(x), cache, K, split_k=1))
    assert np.array_equal(Yf1, Yc1), f"fused and cache paths differ: max {np.abs(Yf1 - Yc1).max()}"


@pytest.mark.parametrize("fmt", NEW)
def test_4096_square_m2048_sampled(fmt):
    """The Llama-3.1-8B q/o shape at M = 2048: sampled rows within tolerance,
    and the whole output equal to the cache path's at split 1."""
    M, N, K = 2048, 4096, 4096
    q = synth.weights(fmt, synth.rng(58, 0, fmt, 0), N, K)
    x = synth.activations(synth.rng(58, role=1), M, K)
    Yf = _fused(fmt, x, q, N, K)
    Yf1 = _fused(fmt, x, q, N, K, split_k=1)
    announce("dequant+gemm_f16cache", NAME[fmt], f"M={M} N={N} K={K}", "split=1")
    cache = mq.dequant_to_f16(to_dev_u8(q), fmt, N, K)
    Yc1 = to_host(mq.gemm_f16cache(to_dev_f16(x), cache, K, split_k=1))
    assert np.array_equal(Yf1, Yc1)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(58).choice(M, 12)]))
    check_gemm(Yf[rows], x, oracle.dequant_ref(fmt, q, N, K), K, f"{NAME[fmt]} 4096^2",
               rows=rows)
