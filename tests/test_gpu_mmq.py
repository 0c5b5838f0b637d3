"""Parity of the int8 product (mq_quantize_q8_1 + mq_gemm_mmq) with the MMQ
oracle (``oracle.mmq``), which defines its numerics:

* the activation codes and the (d, s) factors bit for bit, on hand-derived
  blocks, random bit-level edge cases, padded strides and more chunks than one
  grid covers;
* integer activations with 127 in every block (d = 1) and integer weights:
  the product is the plain matmul, exact, for every format and K split;
* random inputs within 1e-3·S + 1e-5 of the exact evaluation of the same
  integers and factors, at ragged shapes, forced and automatic K splits, and
  on sampled rows of the 7B gate (Q4_K) and down (Q6_K) shapes."""

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden
from gpu_common import announce, dev, needs_gpu, to_dev_u8, to_host
from oracle import mmq as omq

pytestmark = [pytest.mark.gpu, needs_gpu]

import torch  # noqa: E402

import quantized_weight_prefill_q4_amd as mq  # noqa: E402

NAME = {2: "Q4_0", 6: "Q5_0", 7: "Q5_1", 8: "Q8_0", 12: "Q4_K", 13: "Q5_K", 14: "Q6_K"}
ALL = [2, 6, 7, 8, 12, 13, 14]
ELEMS = {2: 32, 6: 32, 7: 32, 8: 32, 12: 256, 13: 256, 14: 256}


def _dev_x32(x, pad=0):
    M, K = x.shape
    buf = torch.full((M, K + pad), float("nan"), dtype=torch.float32, device=dev())
    buf[:, :K] = torch.from_numpy(x).to(dev())
    return buf[:, :K]


def _quantize(x, pad=0, ldq=None):
    M, K = x.shape
    ldq = ldq or (K + 15) // 16 * 16
    xq = torch.full((M, ldq), 0x55, dtype=torch.int8, device=dev())
    announce("quantize_q8_1", f"M={M} K={K} ldq={ldq}")
    q, ds = mq.quantize_q8_1(_dev_x32(x, pad), K, xq=xq)
    torch.cuda.synchronize()
    return q, ds


def _check_codes(x, q, ds):
    M, K = x.shape
    eq, ed, es = omq.quantize_q8_1(x)
    gq = q.cpu().numpy()
    gds = ds.cpu().numpy().reshape(M, K // 32, 2)
    assert np.array_equal(gq[:, :K], eq), f"codes differ at {np.argwhere(gq[:, :K] != eq)[:4]}"
    assert np.array_equal(gds[..., 0].view(np.uint32), ed.view(np.uint32)), "d differs"
    assert np.array_equal(gds[..., 1].view(np.uint32), es.view(np.uint32)), "s differs"
    return gq


def test_quantize_hand_blocks_and_edges():
    rows = read_golden("q81_worked.txt")["block"]
    g = np.random.default_rng(100)
    x = g.standard_normal((37, 288)).astype(np.float32)
    for i, row in enumerate(rows):                     # golden blocks in row i, block 0
        xs = row.split("|")[0].split()
        x[i, :32] = 0
        x[i, :len(xs)] = np.array([int(t, 16) for t in xs], np.uint32).view(np.float32)
    x[6, 32:64] = np.float32(1e-30) * x[6, 32:64]
    x[7, 64:96] = np.float32(3e36) * np.sign(x[7, 64:96])
    x[8, 96:128] = np.float32(-2.5)
    x[9, 128:160] = 0.0
    bits = g.integers(0, 2 ** 32, 32 * 8, dtype=np.uint64).astype(np.uint32)
    r = bits.view(np.float32).copy()
    r[~np.isfinite(r)] = 1.0
    x[10:18, 160:192] = r.reshape(8, 32)
    q, ds = _quantize(x, pad=4, ldq=304)
    gq = _check_codes(x, q, ds)
    assert np.all(gq[:, 288:] == 0x55), "codes past K were written"


def test_quantize_beyond_one_grid():
    """65537 × 32768: 2^28 + 4096 chunks of 8, more than the capped grid
    covers in one pass; rows at both ends and the last row (second pass)."""
    M, K = 65537, 32768
    gen = torch.Generator(device=dev())
    gen.manual_seed(101)
    x = torch.randn((M, K), generator=gen, device=dev(), dtype=torch.float32)
    announce("quantize_q8_1", f"M={M} K={K}")
    q, ds = mq.quantize_q8_1(x)
    for r in (0, 1, 40000, M - 2, M - 1):
        xr = x[r:r + 1].cpu().numpy()
        _check_codes(xr, q[r:r + 1], ds[r:r + 1])
    del x, q, ds
    torch.cuda.empty_cache()


def _int_x(seed, M, K):
    g = np.random.default_rng(seed)
    x = g.integers(-2, 3, (M, K)).astype(np.float32)
    x[:, ::32] = 127 * np.where(g.integers(0, 2, (M, K // 32)) == 1, 1, -1)
    return x


def _mmq(fmt, q, ds, wq, N, K, split=0):
    announce("gemm_mmq", NAME[fmt], f"M={q.shape[0]} N={N} K={K} split={split}")
    return to_host(mq.gemm_mmq(q, ds, to_dev_u8(wq), fmt, N, K, split_k=split))


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("split", [0, 1, 3])
def test_integer_closed_form_exact(fmt, split):
    M, N, K = 70, 130, 1024
    wq = synth.weights(fmt, synth.rng(102, 0, fmt, 0), N, K, mode="integer")
    x = _int_x(102, M, K)
    q, ds = _quantize(x)
    Y = _mmq(fmt, q, ds, wq, N, K, split)
    Yp, _ = oracle.gemm_ref(x.astype(np.float16).view(np.uint16), oracle.dequant_ref(fmt, wq, N, K))
    assert np.array_equal(Y.astype(np.float64), Yp)


def _check_tol(fmt, x, Y, wq, N, K, rows=None, what=""):
    xs = x if rows is None else x[rows]
    eq, ed, es = omq.quantize_q8_1(xs)
    Yr, S = omq.mmq_ref(eq, ed, es, fmt, wq, N, K)
    Yg = Y if rows is None else Y[rows]
    err = np.abs(Yg.astype(np.float64) - Yr)
    assert np.all(err <= 1e-3 * S + 1e-5), f"{what}: worst {(err / (1e-3 * S + 1e-5)).max():.3g}"
    rel = (err / np.maximum(S, 1e-30)).max()
    assert rel < 1e-4, f"{what}: max |dY|/S = {rel:.3g}"


@pytest.mark.parametrize("fmt,M,N,K", [(8, 1, 1, 32), (8, 37, 130, 96), (2, 129, 257, 160),
                                       (6, 200, 70, 1056), (7, 65, 300, 544), (12, 33, 129, 768),
                                       (13, 128, 128, 1280), (14, 257, 200, 512), (14, 5, 3, 256)])
def test_random_within_tolerance(fmt, M, N, K):
    wq = synth.weights(fmt, synth.rng(103, 0, fmt, M), N, K)
    x = np.random.default_rng(103 + M).standard_normal((M, K)).astype(np.float32)
    q, ds = _quantize(x)
    Y = _mmq(fmt, q, ds, wq, N, K)
    _check_tol(fmt, x, Y, wq, N, K, what=f"{NAME[fmt]} {M}x{N}x{K}")


@pytest.mark.parametrize("fmt", [8, 12, 14])
@pytest.mark.parametrize("split", [2, 5, 16])
def test_forced_splits(fmt, split):
    M, N, K = 150, 260, 2048
    wq = synth.weights(fmt, synth.rng(104, 0, fmt, 0), N, K)
    x = np.random.default_rng(104).standard_normal((M, K)).astype(np.float32)
    q, ds = _quantize(x)
    Y = _mmq(fmt, q, ds, wq, N, K, split)
    _check_tol(fmt, x, Y, wq, N, K, what=f"{NAME[fmt]} split {split}")


@pytest.mark.parametrize("fmt", [12, 7])
def test_automatic_tail_split_integer_exact(fmt):
    """2048 × 4224: 528 tiles = two whole rounds + 16 tiles split 16 ways."""
    M, N, K = 2048, 4224, 1024
    wq = synth.weights(fmt, synth.rng(105, 0, fmt, 0), N, K, mode="integer")
    x = _int_x(105, M, K)
    q, ds = _quantize(x)
    Y = _mmq(fmt, q, ds, wq, N, K)
    rows = np.unique(np.concatenate([[0, 127, 128, 1919, 1920, 2047],
                                     np.random.default_rng(105).choice(M, 12)]))
    Yp, _ = oracle.gemm_ref(x[rows].astype(np.float16).view(np.uint16),
                            oracle.dequant_ref(fmt, wq, N, K))
    assert np.array_equal(Y[rows].astype(np.float64), Yp)


@pytest.mark.parametrize("name,fmt,N,K", [("7B gate", 12, 18944, 3584), ("7B down", 14, 3584, 18944)])
def test_7b_shapes_sampled_rows(name, fmt, N, K):
    M = 2048
    wq = synth.weights(fmt, synth.rng(106, 0, fmt, 0), N, K)
    x = np.random.default_rng(106).standard_normal((M, K)).astype(np.float32)
    q, ds = _quantize(x)
    Y = _mmq(fmt, q, ds, wq, N, K)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(107).choice(M, 6)]))
    _check_tol(fmt, x, Y, wq, N, K, rows=rows, what=name)
