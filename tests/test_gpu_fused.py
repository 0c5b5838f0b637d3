"""Parity of mq_gemm_fused (dequant inside the GEMM) with the oracle and with
the cache path.

* one-hot activations: Y = dequant(W)ᵀ exactly, so the in-kernel expansion is
  checked bit for bit against the oracle's decode (by value; ±0 compare equal);
* integer-mode weights and activations: exact;
* random inputs: within tolerance of the f64 oracle, and — both run without a
  K split, so every output sums the same products in the same k order —
  bit-identical to the f16-cache GEMM on the device-built cache (the invariant
  that the two shapes of the method agree; their automatic splits may differ,
  since the two kernels use different tiles);
* the Llama-3.1-8B-like sweep shapes at M = 128 and 2048 on sampled rows."""

import numpy as np
import pytest

import oracle
import synth
from gpu_common import announce, check_gemm, needs_gpu, to_dev_f16, to_dev_u8, to_host

pytestmark = [pytest.mark.gpu, needs_gpu]

import quantized_weight_prefill_q4_amd as mq  # noqa: E402

FMT_NAME = {12: "Q4_K", 14: "Q6_K", 8: "Q8_0", 2: "Q4_0", 6: "Q5_0", 7: "Q5_1", 13: "Q5_K"}


def _fused(fmt, x_bits, q, N, K, split_k=0):
    announce("gemm_fused", FMT_NAME[fmt], f"M={x_bits.shape[0]}", f"N={N}", f"K={K}",
             f"split={split_k}")
    return mq.gemm_fused(to_dev_f16(x_bits), to_dev_u8(q), fmt, N, K, split_k=split_k)


@pytest.mark.parametrize("fmt,N,K", [(12, 300, 256), (12, 128, 512), (14, 200, 256),
                                     (14, 130, 512), (8, 257, 96), (8, 64, 512), (8, 100, 32)])
def test_onehot_expansion_is_the_decode(fmt, N, K):
    q = synth.weights(fmt, synth.rng(30, 0, fmt, N), N, K)
    x = synth.activations(None, K, K, mode="onehot")
    Y = to_host(_fused(fmt, x, q, N, K))
    exp = oracle.dequant_ref(fmt, q, N, K).view(np.float16).astype(np.float32).T
    assert np.array_equal(Y, exp)


@pytest.mark.parametrize("fmt,M,N,K", [(12, 100, 300, 1024), (14, 70, 130, 2048),
                                       (8, 33, 257, 1056)])
@pytest.mark.parametrize("split", [0, 1, 3])
def test_integer_exact(fmt, M, N, K, split):
    q = synth.weights(fmt, synth.rng(31, 0, fmt, 0), N, K, mode="integer")
    x = synth.activations(synth.rng(31, role=1), M, K, mode="integer")
    Y = to_host(_fused(fmt, x, q, N, K, split_k=split))
    Yref, _ = oracle.gemm_ref(x, oracle.dequant_ref(fmt, q, N, K))
    assert np.array_equal(Y.astype(np.float64), Yref)


@pytest.mark.parametrize("fmt", [2, 6, 7, 8, 12, 13, 14])
@pytest.mark.parametrize("M,N,K,split", [(700, 2900, 1536, 0), (700, 2900, 1536, 1),
                                         (97, 390, 1024, 0), (97, 390, 1024, 3)])
def test_eight_wave_tiles_integer_exact(fmt, M, N, K, split):
    """Tiles of 128 columns with 256 rows (M = 700: 69 tiles, split 3 ways
    along K by the plan, or whole) and with 128 rows (M = 97) run on 8 waves,
    waves 0-3 decoding the weights: every format, ragged in M and N, exact
    with integer inputs on sampled rows."""
    q = synth.weights(fmt, synth.rng(38, 0, fmt, M), N, K, mode="integer")
    x = synth.activations(synth.rng(38, role=1), M, K, mode="integer")
    Y = to_host(_fused(fmt, x, q, N, K, split_k=split))
    edges = np.array([0, 63, 64, 127, 128, 255, 256, 511, 512, M - 1])
    rows = np.unique(np.concatenate([edges[edges < M], np.random.default_rng(M).choice(M, 12)]))
    Yref, _ = oracle.gemm_ref(x[rows], oracle.dequant_ref(fmt, q, N, K))
    assert np.array_equal(Y[rows].astype(np.float64), Yref)


@pytest.mark.parametrize("fmt", [8, 12, 14])
@pytest.mark.parametrize("M,N,K", [(2048, 512, 3584), (2011, 900, 2048), (1024, 512, 3584)])
def test_narrow_output_tiles_integer_exact(fmt, M, N, K):
    """Narrow outputs take 128-row tiles in the fused GEMM while 64 or more of
    them exist (k/v at M = 2048: 64 tiles split 4 ways; M = 2011, N = 900:
    ragged, 16 x 8 tiles split 2 ways), else 64-row tiles as the cache GEMM
    does (M = 1024).  Integer inputs: every sampled element exact."""
    q = synth.weights(fmt, synth.rng(40, 0, fmt, N), N, K, mode="integer")
    x = synth.activations(synth.rng(40, role=1), M, K, mode="integer")
    Y = to_host(_fused(fmt, x, q, N, K))
    edges = np.array([0, 63, 64, 127, 128, 255, 256, M - 1])
    rows = np.unique(np.concatenate([edges[edges < M], np.random.default_rng(40).choice(M, 12)]))
    Yref, _ = oracle.gemm_ref(x[rows], oracle.dequant_ref(fmt, q, N, K))
    assert np.array_equal(Y[rows].astype(np.float64), Yref)


@pytest.mark.parametrize("fmt", [12, 8])
def test_large_tile_mixed_grid_integer_exact(fmt):
    """Q4_K and Q8_0 take the 256 x 256 tile once a full round of such tiles
    exists: M = 2048, N = 8448 gives 264 tiles, one round over all of K plus 8
    K-split tail tiles.  Integer weights and activations keep every partial sum
    exact, so sampled rows across both kinds of tile must equal the oracle."""
    M, N, K = 2048, 8448, 2048
    q = synth.weights(fmt, synth.rng(34, 0, fmt, 0), N, K, mode="integer")
    x = synth.activations(synth.rng(34, role=1), M, K, mode="integer")
    Y = to_host(_fused(fmt, x, q, N, K))
    rows = np.unique(np.concatenate([[0, 255, 1023, 1024, 2047],
                                     np.random.default_rng(34).choice(M, 24)]))
    Yref, _ = oracle.gemm_ref(x[rows], oracle.dequant_ref(fmt, q, N, K))
    assert np.array_equal(Y[rows].astype(np.float64), Yref)


@pytest.mark.parametrize("fmt", [12, 13])
@pytest.mark.parametrize("M,N,K,split", [(2011, 8348, 2048, 0), (2011, 8348, 2048, 3),
                                         (2048, 18944, 3584, 0), (300, 32768, 1280, 3)])
def test_q4k_large_tile_k_ranges_exact(fmt, M, N, K, split):
    """The Q4_K 256 x 256 kernel stages whole super-blocks, so its K ranges are
    rounded to multiples of 4 k-steps: a forced 3-way split of 32 steps runs
    ranges of 12, 12 and 8; the 7B gate shape's automatic tail (3 ways over 56
    steps) runs 20, 20, 16; 300 rows over N = 32768 (256 tiles, the second
    M-tile 44 rows deep) split 3 ways over 20 steps runs 8, 8, 4.  Ragged M
    and N (rows of the last tiles past the matrix read as zero weights) and
    integer inputs: every sampled element exact.  Q5_K (176-byte super-blocks,
    11 chunks per row) takes the same kernel."""
    q = synth.weights(fmt, synth.rng(35, 0, fmt, N), N, K, mode="integer")
    x = synth.activations(synth.rng(35, role=1), M, K, mode="integer")
    Y = to_host(_fused(fmt, x, q, N, K, split_k=split))
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(35).choice(M, 12)]))
    Yref, _ = oracle.gemm_ref(x[rows], oracle.dequant_ref(fmt, q, N, K))
    assert np.array_equal(Y[rows].astype(np.float64), Yref)


@pytest.mark.parametrize("M,N,K,split", [(2011, 8348, 2048, 0), (2011, 8348, 2048, 3),
                                         (2048, 3584, 8192, 0), (1000, 14336, 768, 0),
                                         (300, 32768, 768, 5)])
def test_q6k_large_tile_k_ranges_exact(M, N, K, split):
    """The Q6_K 256 x 256 kernel stages half super-blocks (2 k-steps) whose
    bytes it re-aligns from 2-byte-aligned blocks: ragged M and N, a forced
    3-way split of 32 steps (ranges 12, 12, 8), the down-like split of 128
    steps in 2 ranges of 64, and with K = 768 (630-byte rows, so row starts
    fall on every even residue mod 16) a 3/4 round unsplit and a 5-way split
    of 12 steps (ranges of 4, 4, 4) with the second M-tile 44 rows deep.  Integer inputs: every sampled
    element exact, and equal to the cache path at split 1."""
    q = synth.weights(14, synth.rng(36, 0, 14, N), N, K, mode="integer")
    x = synth.activations(synth.rng(36, role=1), M, K, mode="integer")
    Y = to_host(_fused(14, x, q, N, K, split_k=split))
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(36).choice(M, 12)]))
    w16 = oracle.dequant_ref(14, q, N, K)
    Yref, _ = oracle.gemm_ref(x[rows], w16)
    assert np.array_equal(Y[rows].astype(np.float64), Yref)
    if split == 0:
        Yf1 = to_host(_fused(14, x, q, N, K, split_k=1))
        announce("gemm_f16cache", "Q6_K cache", f"M={M} N={N} K={K}", "split=1")
        Yc1 = to_host(mq.gemm_f16cache(to_dev_f16(x), to_dev_f16(w16), K, split_k=1))
        assert np.array_equal(Yf1, Yc1)


@pytest.mark.parametrize("fmt", [8, 2, 6, 7])
@pytest.mark.parametrize("M,N,K,split", [(2011, 8348, 2048, 0), (2011, 8348, 2048, 3),
                                         (300, 32768, 1280, 7), (1000, 14336, 768, 0),
                                         (2011, 8348, 1056, 0), (2011, 8348, 1056, 3)])
def test_b32_large_tile_k_ranges_exact(fmt, M, N, K, split):
    """The 256 x 256 kernel of the 32-element block formats (K a multiple of
    256) stages half runs of 4 blocks (2 k-steps): ragged M and N, the plan's
    tail, a forced 3-way split of 32 steps (ranges 12, 12, 8), a forced 7-way
    split of 20 steps (5 ranges of 4), a 3/4 round unsplit with K = 768; with
    K = 1056 (not a multiple of 256) the 2 x 2 kernel takes the same tiles.
    Integer inputs: every sampled element exact, and equal to the cache path
    at split 1."""
    q = synth.weights(fmt, synth.rng(39, 0, fmt, N), N, K, mode="integer")
    x = synth.activations(synth.rng(39, role=1), M, K, mode="integer")
    Y = to_host(_fused(fmt, x, q, N, K, split_k=split))
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(39).choice(M, 12)]))
    w16 = oracle.dequant_ref(fmt, q, N, K)
    Yref, _ = oracle.gemm_ref(x[rows], w16)
    assert np.array_equal(Y[rows].astype(np.float64), Yref)
    if split == 0:
        Yf1 = to_host(_fused(fmt, x, q, N, K, split_k=1))
        announce("gemm_f16cache", f"{FMT_NAME[fmt]} cache", f"M={M} N={N} K={K}", "split=1")
        Yc1 = to_host(mq.gemm_f16cache(to_dev_f16(x), to_dev_f16(w16), K, split_k=1))
        assert np.array_equal(Yf1, Yc1)


def _large_tile_cases(seed, n):
    """Seeded shapes that take the 256 x 256 register-expansion kernels: more
    than 3/4 of a round of tiles (so N >= 48 · 256 / ceil(M / 256)), ragged M
    and N, K a multiple of 256, and a random forced split (0 = the plan's)."""
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        tm = int(g.integers(1, 9))
        M = 256 * tm - int(g.integers(0, 200)) if tm > 1 else int(g.integers(129, 257))
        tn = -(-193 // tm) + int(g.integers(0, 8))
        N = 256 * tn - int(g.integers(0, 256))
        K = 256 * int(g.integers(1, 7))
        out.append((M, N, K, int(g.choice([0, 0, 2, 3, 5]))))
    return out


@pytest.mark.parametrize("fmt", [2, 6, 7, 8, 12, 13, 14])
@pytest.mark.parametrize("M,N,K,split", _large_tile_cases(37, 4))
def test_register_expansion_kernels_random_shapes_exact(fmt, M, N, K, split):
    q = synth.weights(fmt, synth.rng(37, 0, fmt, N + K), N, K, mode="integer")
    x = synth.activations(synth.rng(37, role=1), M, K, mode="integer")
    Y = to_host(_fused(fmt, x, q, N, K, split_k=split))
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(M).choice(M, 8)]))
    Yref, _ = oracle.gemm_ref(x[rows], oracle.dequant_ref(fmt, q, N, K))
    assert np.array_equal(Y[rows].astype(np.float64), Yref)


@pytest.mark.parametrize("fmt,M,N,K", [(12, 64, 512, 512), (12, 129, 200, 1280),
                                       (14, 257, 96, 768), (8, 65, 333, 4128),
                                       (8, 1, 1, 32), (14, 1, 3, 256)])
def test_random_tolerance_and_cache_identity(fmt, M, N, K):
    q = synth.weights(fmt, synth.rng(32, 0, fmt, M), N, K)
    x = synth.activations(synth.rng(32, role=1), M, K)
    Yf = to_host(_fused(fmt, x, q, N, K))
    w16 = oracle.dequant_ref(fmt, q, N, K)
    check_gemm(Yf, x, w16, K, f"fused {FMT_NAME[fmt]} {M}x{N}x{K}")
    Yf1 = to_host(_fused(fmt, x, q, N, K, split_k=1))
    announce("dequant+gemm_f16cache", FMT_NAME[fmt], f"M={M} N={N} K={K}", "split=1")
    cache = mq.dequant_to_f16(to_dev_u8(q), fmt, N, K)
    Yc1 = to_host(mq.gemm_f16cache(to_dev_f16(x), cache, K, split_k=1))
    assert np.array_equal(Yf1, Yc1), f"fused and cache paths differ: max {np.abs(Yf1 - Yc1).max()}"


@pytest.mark.parametrize("fmt", [0, 12, 14])
def test_large_m_exact(fmt):
    """M = 16400 tokens (65 M-tiles, the last 16 rows deep): 1040 tiles of
    256 × 256 over N = 4096, four whole rounds and a K-split tail of 16 tiles;
    cache GEMM (fmt 0, on the decoded weight) and both register-expansion
    fused kernels.  Integer inputs: sampled rows exact, including the last."""
    M, N, K = 16400, 4096, 512
    wf = 12 if fmt == 0 else fmt
    q = synth.weights(wf, synth.rng(39, 0, wf, 0), N, K, mode="integer")
    x = synth.activations(synth.rng(39, role=1), M, K, mode="integer")
    w16 = oracle.dequant_ref(wf, q, N, K)
    if fmt == 0:
        announce("gemm_f16cache", f"M={M} N={N} K={K}")
        Y = to_host(mq.gemm_f16cache(to_dev_f16(x), to_dev_f16(w16), K))
    else:
        Y = to_host(_fused(fmt, x, q, N, K))
    rows = np.unique(np.concatenate([[0, 255, 16383, 16384, M - 1],
                                     np.random.default_rng(39).choice(M, 11)]))
    Yref, _ = oracle.gemm_ref(x[rows], w16)
    assert np.array_equal(Y[rows].astype(np.float64), Yref)


SHAPES_7B = [("q/o", 12, 3584, 3584), ("k/v", 12, 512, 3584), ("gate/up", 12, 18944, 3584),
             ("down", 14, 3584, 18944)]


@pytest.mark.parametrize("name,fmt,N,K", SHAPES_7B)
def test_7b_shapes_m2048_random(name, fmt, N, K):
    """The fused forward's products at full size, random data: sampled rows
    within tolerance under the plan the bench times, and the whole output
    equal to the cache GEMM's when neither splits K."""
    M = 2048
    q = synth.weights(fmt, synth.rng(38, 0, fmt, N % 1000), N, K)
    x = synth.activations(synth.rng(38, role=1), M, K)
    Y = to_host(_fused(fmt, x, q, N, K))
    w16 = oracle.dequant_ref(fmt, q, N, K)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(N).choice(M, 12)]))
    check_gemm(Y[rows], x, w16, K, f"fused 7B {name}", rows=rows)
    assert np.all(np.isfinite(Y))
    Yf1 = to_host(_fused(fmt, x, q, N, K, split_k=1))
    announce("gemm_f16cache", name, f"M={M} N={N} K={K}", "split=1")
    Yc1 = to_host(mq.gemm_f16cache(to_dev_f16(x), to_dev_f16(w16), K, split_k=1))
    assert np.array_equal(Yf1, Yc1)


SWEEP = [("Q4_K 4096^2", 12, 4096, 4096), ("Q4_K 14336x4096", 12, 14336, 4096),
         ("Q4_K 4096x14336", 12, 4096, 14336), ("Q8_0 4096^2", 8, 4096, 4096),
         ("Q6_K 3584x18944", 14, 3584, 18944)]


@pytest.mark.parametrize("M", [128, 2048])
@pytest.mark.parametrize("name,fmt,N,K", SWEEP)
def test_sweep_shapes(name, fmt, N, K, M):
    q = synth.weights(fmt, synth.rng(33, 0, fmt, N % 1000), N, K)
    x = synth.activations(synth.rng(33, role=1), M, K)
    Yf = to_host(_fused(fmt, x, q, N, K))
    Yf1 = to_host(_fused(fmt, x, q, N, K, split_k=1))
    announce("dequant+gemm_f16cache", name, f"M={M}", "split=1")
    cache = mq.dequant_to_f16(to_dev_u8(q), fmt, N, K)
    Yc1 = to_host(mq.gemm_f16cache(to_dev_f16(x), cache, K, split_k=1))
    assert np.array_equal(Yf1, Yc1)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(M).choice(M, 16)]))
    check_gemm(Yf[rows], x, oracle.dequant_ref(fmt, q, N, K), K, name, rows=rows)


def test_fused_expands_golden_blocks():
    """The hand-derived Q4_K blocks (worked vector, f32-then-f16 double rounding)
    expanded inside the GEMM: one-hot X makes Y the expanded weights."""
    from conftest import read_golden
    from oracle.encode import pack_q4k

    g = read_golden("q4k_worked.txt")
    qs = [(i % 16) | ((15 - i % 16) << 4) for i in range(128)]
    q = []
    for e in range(256):
        c, r = divmod(e, 64)
        b = qs[32 * c + r % 32]
        q.append(b & 15 if r < 32 else b >> 4)
    row0 = pack_q4k(0x3C00, 0x3800, [int(t) for t in g["scales"][0].split()],
                    [int(t) for t in g["mins"][0].split()], q)
    gd = read_golden("q4k_double_rounding.txt")
    qd = [0] * 256
    qd[0] = int(gd["q0"][0])
    row1 = pack_q4k(int(gd["d_bits"][0], 16), int(gd["dmin_bits"][0], 16),
                    [int(t) for t in gd["scales"][0].split()],
                    [int(t) for t in gd["mins"][0].split()], qd)
    wq = np.frombuffer(row0 + row1, np.uint8).copy()
    x = synth.activations(None, 256, 256, mode="onehot")
    Y = to_host(_fused(12, x, wq, 2, 256))
    for tok in g["expect"][0].split():
        e, v = tok.split(":")
        assert Y[int(e), 0] == float(v), tok
    assert np.float16(Y[0, 1]).view(np.uint16) == 0x3C02


def test_large_k_q80_exact():
    """Fused Q8_0 at K = 32768 (1024 blocks per row, 512 k-steps): integer
    weights (d = 1, q in -127..127) and activations in -2..2 keep |Y| < 2^24."""
    M, N, K = 70, 257, 32768
    q = synth.weights(8, synth.rng(35, 0, 8, 0), N, K, mode="integer")
    x = synth.activations(synth.rng(35, role=1), M, K, mode="integer")
    Y = to_host(_fused(8, x, q, N, K))
    Yref, _ = oracle.gemm_ref(x, oracle.dequant_ref(8, q, N, K))
    assert np.array_equal(Y.astype(np.float64), Yref)
