"""Parity of mq_gemm_f16cache (Y = X·W16ᵀ on the f16 cache) with the oracle.

Exact checks: integer operands (every partial sum is an integer below 2²⁴, so
any summation order is exact) and one-hot activations (Y = W16ᵀ).  Tolerance
checks: |Y − Yref| ≤ 1e-3·S + 1e-5 with Yref, S from the f64 oracle, on ragged
and tiny shapes, forced K splits, padded strides (pad filled with NaN, so any
read past K shows), and the 7B shapes at M = 2048 on sampled rows."""

import numpy as np
import pytest

import oracle
import synth
from gpu_common import (announce, check_gemm, dev, f16_bits, needs_gpu, to_dev_f16, to_dev_u8,
                        to_host)

pytestmark = [pytest.mark.gpu, needs_gpu]

import torch  # noqa: E402

import quantized_weight_prefill_q4_amd as mq  # noqa: E402

NAN16 = 0x7E00


def _padded(bits: np.ndarray, ld: int, fill=NAN16) -> np.ndarray:
    out = np.full((bits.shape[0], ld), fill, dtype=np.uint16)
    out[:, : bits.shape[1]] = bits
    return out


def _cache(fmt, N, K, seed, mode="random"):
    q = synth.weights(fmt, synth.rng(seed, 0, fmt, 0), N, K, mode=mode)
    w16 = oracle.dequant_ref(fmt, q, N, K)
    return q, w16


def _gemm(x_bits, w_bits, K, split_k=0, ldy=None):
    M, N = x_bits.shape[0], w_bits.shape[0]
    announce("gemm_f16cache", f"M={M}", f"N={N}", f"K={K}", f"ldx={x_bits.shape[1]}",
             f"ldw={w_bits.shape[1]}", f"split={split_k}")
    X = to_dev_f16(x_bits)
    W = to_dev_f16(w_bits)
    out = None
    if ldy is not None:
        out = torch.full((M, ldy), -7.0, dtype=torch.float32, device="cuda:0")[:, :N]
    Y = mq.gemm_f16cache(X, W, K, split_k=split_k, out=out)
    return to_host(Y), (None if ldy is None else to_host(out.as_strided((M, ldy), (ldy, 1))))


def test_tiny_config_q4k_512():
    """Q4_K W 512×512 (2 super-blocks per row), X 64×512."""
    _, w16 = _cache(12, 512, 512, 10)
    x = synth.activations(synth.rng(10, role=1), 64, 512)
    Y, _ = _gemm(x, w16, 512)
    check_gemm(Y, x, w16, 512, "tiny")


@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (7, 33, 56), (65, 130, 72), (129, 257, 520),
                                   (300, 128, 64), (64, 300, 1000), (256, 128, 256),
                                   (257, 129, 136), (513, 1000, 384)])
def test_ragged_with_nan_padding(M, N, K):
    g = np.random.default_rng(M * 7 + N)
    x = g.standard_normal((M, K)).astype(np.float16).view(np.uint16)
    w = (g.standard_normal((N, K)) * 0.1).astype(np.float16).view(np.uint16)
    xp, wp = _padded(x, K + 24), _padded(w, K + 40)
    Y, _ = _gemm(xp, wp, K)
    check_gemm(Y, x, w, K, f"{M}x{N}x{K}")


def test_integer_exact():
    _, w16 = _cache(12, 300, 1024, 11, mode="integer")
    x = synth.activations(synth.rng(11, role=1), 100, 1024, mode="integer")
    Y, _ = _gemm(x, w16, 1024)
    Yref, _ = oracle.gemm_ref(x, w16)
    assert np.array_equal(Y.astype(np.float64), Yref)


@pytest.mark.parametrize("split", [1, 2, 3, 5, 16])
def test_forced_split_integer_exact(split):
    _, w16 = _cache(12, 200, 2048, 12, mode="integer")
    x = synth.activations(synth.rng(12, role=1), 70, 2048, mode="integer")
    Y, _ = _gemm(x, w16, 2048, split_k=split)
    Yref, _ = oracle.gemm_ref(x, w16)
    assert np.array_equal(Y.astype(np.float64), Yref)


def test_mixed_grid_tail_split_integer_exact():
    """One launch with both kinds of workgroup: M = 2048, N = 8448 gives 8 x 33 =
    264 tiles of 256 x 256, i.e. one whole round of 256 tiles over all of K and 8
    tail tiles split along K (their partials summed by the reduce kernel).  With
    integer inputs every partial sum is exact, so Y must equal the oracle on
    rows that cross both the whole tiles and the tail tiles."""
    M, N, K = 2048, 8448, 2048
    ws = mq.workspace_bytes(0, M, N, K)
    assert ws > 0 and ws % (256 * 256 * 4 * 8) == 0   # split * 8 tail tiles
    x = synth.activations(synth.rng(24, role=1), M, K, mode="integer")
    _, w16 = _cache(12, N, K, 24, mode="integer")
    Y, _ = _gemm(x, w16, K)
    rows = np.unique(np.concatenate([[0, 255, 1023, 1024, 2047],
                                     np.random.default_rng(24).choice(M, 40)]))
    Yref, _ = oracle.gemm_ref(x[rows], w16, K)
    assert np.array_equal(Y[rows].astype(np.float64), Yref)


def test_onehot_reproduces_cache():
    _, w16 = _cache(14, 384, 512, 13)
    x = synth.activations(None, 512, 512, mode="onehot")
    Y, _ = _gemm(x, w16, 512)
    exp = w16.view(np.float16).astype(np.float32).T
    assert np.array_equal(Y, exp)   # by value: -0 == +0


def test_output_stride_untouched_columns():
    _, w16 = _cache(12, 100, 256, 14)
    x = synth.activations(synth.rng(14, role=1), 50, 256)
    Y, full = _gemm(x, w16, 256, ldy=112)
    check_gemm(Y, x, w16, 256, "ldy=112")
    assert np.all(full[:, 100:] == -7.0)


def test_padded_cache_from_device_dequant():
    """The path as used: device dequant into a padded cache, then the GEMM on it."""
    q = synth.weights(12, synth.rng(15), 1024, 4096)
    announce("dequant+gemm", "Q4_K", "N=1024 K=4096 ld=4160 M=256")
    w16 = mq.dequant_to_f16(to_dev_u8(q), 12, 1024, 4096)
    assert w16.shape == (1024, 4160)
    x = synth.activations(synth.rng(15, role=1), 256, 4096)
    Y = to_host(mq.gemm_f16cache(to_dev_f16(x), w16, 4096))
    check_gemm(Y, x, oracle.dequant_ref(12, q, 1024, 4096), 4096, "padded cache")


SHAPES_7B = [("q/o", 12, 3584, 3584), ("k/v", 12, 512, 3584), ("gate/up", 12, 18944, 3584),
             ("down", 14, 3584, 18944)]


@pytest.mark.parametrize("name,fmt,N,K", SHAPES_7B)
def test_7b_shapes_m2048_sampled_rows(name, fmt, N, K):
    q = synth.weights(fmt, synth.rng(20, 0, fmt, N % 1000), N, K)
    announce("dequant", name, f"N={N} K={K}")
    w16_dev = mq.dequant_to_f16(to_dev_u8(q), fmt, N, K)
    w16 = f16_bits(w16_dev)[:, :K]
    assert np.array_equal(w16, oracle.dequant_ref(fmt, q, N, K))
    x = synth.activations(synth.rng(20, role=1), 2048, K)
    announce("gemm_f16cache", name, f"M=2048 N={N} K={K}")
    Y = to_host(mq.gemm_f16cache(to_dev_f16(x), w16_dev, K))
    rows = np.sort(np.random.default_rng(N).choice(2048, 24, replace=False))
    rows = np.concatenate([[0, 255, 256, 2047], rows])
    check_gemm(Y[rows], x, w16, K, f"7B {name}", rows=rows)
    assert np.all(np.isfinite(Y))


@pytest.mark.parametrize("split", [0, 1])
def test_large_k_padded_strides_exact(split):
    """K = 65536 with padded strides (ldx = K + 8, ldw = K + 64): 1024 k-steps
    in one tile (split 1) or 16 K ranges (auto).  Small-integer operands keep
    every partial sum below 2^24, so the result is exact and any lost, repeated
    or misaddressed k-step shows."""
    M, N, K = 64, 300, 65536
    g = np.random.default_rng(25)
    x = g.integers(-2, 3, (M, K)).astype(np.float16).view(np.uint16)
    w = g.integers(-2, 3, (N, K)).astype(np.float16).view(np.uint16)
    Y, _ = _gemm(_padded(x, K + 8), _padded(w, K + 64), K, split_k=split)
    Yref, _ = oracle.gemm_ref(x, w)
    assert np.array_equal(Y.astype(np.float64), Yref)


def test_grouped_shared_input_gemm_exact():
    """Shared-input weights grouped into one cache (q|k|v-like: 300 + 64 + 64 rows),
    each decoded by one batched call into its row slice, then one GEMM: Y of the
    group equals the separate GEMMs column block by column block, and the oracle,
    exactly (integer mode)."""
    K, M = 1024, 130
    parts = [(12, 300), (12, 64), (14, 64)]
    qs = [synth.weights(f, synth.rng(26, 0, i, 0), n, K, mode="integer") for i, (f, n) in enumerate(parts)]
    rows = sum(n for _, n in parts)
    dev_q = [to_dev_u8(q) for q in qs]
    group = torch.empty((rows, mq.cache_ld(K)), dtype=torch.float16, device=dev())
    jobs, r0 = [], 0
    for (f, n), dq in zip(parts, dev_q):
        jobs.append((dq, f, n, K, group[r0:r0 + n]))
        r0 += n
    announce("dequant_batch", "group of 3 into row slices")
    mq.dequant_to_f16_batch(jobs)
    x = synth.activations(synth.rng(26, role=1), M, K, mode="integer")
    announce("gemm_f16cache", "grouped", f"M={M} N={rows} K={K}")
    Yg = to_host(mq.gemm_f16cache(to_dev_f16(x), group, K))
    w16 = np.concatenate([oracle.dequant_ref(f, q, n, K) for (f, n), q in zip(parts, qs)])
    Yref, _ = oracle.gemm_ref(x, w16)
    assert np.array_equal(Yg.astype(np.float64), Yref)
    r0 = 0
    for (f, n), dq in zip(parts, dev_q):
        c = mq.dequant_to_f16(dq, f, n, K)
        Ys = to_host(mq.gemm_f16cache(to_dev_f16(x), c, K))
        assert np.array_equal(Ys, Yg[:, r0:r0 + n])
        r0 += n


def test_split_256_tiles_for_sub_round_grids_exact():
    """M = 2048, N = 3584, K = 8192: the 256 × 128 grid (224 tiles) is less than
    one round, so the plan takes 112 tiles of 256 × 256 split twice along K
    (4096 k per range; the 7B down shape's plan).  Small-integer operands keep
    every partial sum exact, so sampled rows across all tiles equal the oracle,
    and the workspace is the two partial planes of every tile."""
    M, N, K = 2048, 3584, 8192
    assert mq.workspace_bytes(0, M, N, K) == 2 * 112 * 256 * 256 * 4
    g = np.random.default_rng(27)
    x = g.integers(-2, 3, (M, K)).astype(np.float16).view(np.uint16)
    w = g.integers(-3, 4, (N, K)).astype(np.float16).view(np.uint16)
    Y, _ = _gemm(x, w, K)
    rows = np.unique(np.concatenate([[0, 255, 256, 1791, 2047], g.choice(M, 11)]))
    Yref, _ = oracle.gemm_ref(x[rows], w)
    assert np.array_equal(Y[rows].astype(np.float64), Yref)


def test_three_quarter_round_256_tiles_exact():
    """M = 1000, N = 14336: 4 × 56 = 224 tiles of 256 × 256 (more than 3/4 of a
    round), which the plan takes unsplit instead of 448 tiles of 256 × 128; the
    last M-tile holds 232 rows.  Cache and fused Q4_K paths, integer operands:
    sampled rows exact, the two paths identical."""
    M, N, K = 1000, 14336, 768
    assert mq.workspace_bytes(0, M, N, K) == 0 and mq.workspace_bytes(12, M, N, K) == 0
    g = np.random.default_rng(29)
    x = g.integers(-2, 3, (M, K)).astype(np.float16).view(np.uint16)
    q = synth.weights(synth.Q4_K, synth.rng(29, 0, 12, 0), N, K, mode="integer")
    w = oracle.dequant_ref(synth.Q4_K, q, N, K)
    Yc, _ = _gemm(x, w, K)
    announce("gemm_fused", "Q4_K", f"M={M} N={N} K={K}")
    Yf = to_host(mq.gemm_fused(to_dev_f16(x), to_dev_u8(q), synth.Q4_K, N, K))
    assert np.array_equal(Yc, Yf)
    rows = np.unique(np.concatenate([[0, 255, 767, 768, 999], g.choice(M, 11)]))
    Yref, _ = oracle.gemm_ref(x[rows], w)
    assert np.array_equal(Yc[rows].astype(np.float64), Yref)


def test_narrow_output_64_row_tiles_exact():
    """M = 2048, N = 512, K = 1024 (a k/v-like narrow output, short K): 64-row
    tiles, 128 tiles split twice along K.  Integer operands: exact."""
    M, N, K = 2048, 512, 1024
    assert mq.workspace_bytes(0, M, N, K) == 2 * 128 * 64 * 128 * 4
    g = np.random.default_rng(28)
    x = g.integers(-2, 3, (M, K)).astype(np.float16).view(np.uint16)
    w = g.integers(-3, 4, (N, K)).astype(np.float16).view(np.uint16)
    Y, _ = _gemm(x, w, K)
    Yref, _ = oracle.gemm_ref(x, w)
    assert np.array_equal(Y.astype(np.float64), Yref)


def test_grouped_fused_equals_per_matrix():
    """The shared-input batch on the fused path: the quantized q, k, v rows of
    a 7B layer (all Q4_K over K = 3584) placed one after another form one
    4608-row weight, and gate and up one 37888-row weight.  One fused GEMM on
    each group equals the per-matrix fused GEMMs column for column, bit for
    bit at split 1 (each output sums the same products in the same order), and
    sampled outputs are within the oracle's tolerance."""
    M, K = 256, 3584
    x = synth.activations(synth.rng(33, role=1), M, K)
    xd = to_dev_f16(x)
    for members in (("q", 3584), ("k", 512), ("v", 512)), (("gate", 18944), ("up", 18944)):
        qs = [synth.weights(synth.Q4_K, synth.rng(33, 0, i, n), n, K) for i, (_, n) in enumerate(members)]
        grouped = np.concatenate([q.reshape(n, -1) for q, (_, n) in zip(qs, members)])
        n_tot = grouped.shape[0]
        announce("gemm_fused grouped", "+".join(m for m, _ in members), f"M={M} N={n_tot} K={K}")
        yg = to_host(mq.gemm_fused(xd, to_dev_u8(grouped), synth.Q4_K, n_tot, K, split_k=1))
        c0 = 0
        for q, (name, n) in zip(qs, members):
            y = to_host(mq.gemm_fused(xd, to_dev_u8(q), synth.Q4_K, n, K, split_k=1))
            assert np.array_equal(yg[:, c0:c0 + n], y), f"{name}: grouped != per-matrix"
            c0 += n
        rows = np.array([0, 77, 255])
        cols = np.unique(np.concatenate([[0, n_tot - 1], np.random.default_rng(n_tot).choice(n_tot, 62)]))
        w = oracle.dequant_ref(synth.Q4_K, grouped[cols].reshape(-1), len(cols), K)
        check_gemm(yg[rows][:, cols], x, w, K, "grouped fused", rows=rows)
