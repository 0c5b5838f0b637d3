"""Pins of the GEMM oracle Y = X·Wᵀ (f16 operands, exact f64 evaluation).

Fixed by: a brute-force triple loop with correctly rounded sums (math.fsum);
integer inputs (exact results); one-hot activations (Y = Wᵀ exactly);
non-square shapes that catch a transposed operand; and the tolerance check
catching a planted error.
"""

import numpy as np
import pytest

import synth
from oracle import Q4_K, dequant_ref, gemm_bruteforce, gemm_ref, within_tolerance


def test_matches_bruteforce_nonsquare():
    g = np.random.default_rng(5)
    X = g.standard_normal((7, 40)).astype(np.float16).view(np.uint16)
    W = (g.standard_normal((11, 40)) * 3).astype(np.float16).view(np.uint16)
    Y, S = gemm_ref(X, W)
    Yb = gemm_bruteforce(X, W)
    assert Y.shape == (7, 11)
    assert np.all(np.abs(Y - Yb) <= 40 * 2.0 ** -52 * S + 1e-300)


def test_entrywise_definition_small():
    """Y[m, n] = sum_k X[m, k] * W[n, k] for a hand-made 2x3 by 3x3 case."""
    X = np.array([[1, 2, 0], [0, -1, 3]], dtype=np.float16).view(np.uint16)
    W = np.array([[1, 0, 0], [0, 1, 1], [2, 0, -1]], dtype=np.float16).view(np.uint16)
    Y, S = gemm_ref(X, W)
    assert np.array_equal(Y, np.array([[1, 2, 2], [0, 2, -3]], dtype=np.float64))
    assert np.array_equal(S, np.array([[1, 2, 2], [0, 4, 3]], dtype=np.float64))


def test_integer_inputs_exact():
    q = synth.weights(Q4_K, synth.rng(910), 24, 512, mode="integer")
    W = dequant_ref(Q4_K, q, 24, 512)
    X = synth.activations(synth.rng(910, role=1), 9, 512, mode="integer")
    Y, _ = gemm_ref(X, W)
    Yb = gemm_bruteforce(X, W)
    assert np.array_equal(Y, Yb)
    assert np.array_equal(Y, np.round(Y))


def test_onehot_gives_transposed_weights():
    q = synth.weights(Q4_K, synth.rng(911), 16, 256)
    W = dequant_ref(Q4_K, q, 16, 256)
    X = synth.activations(None, 256, 256, mode="onehot")
    Y, _ = gemm_ref(X, W)
    assert np.array_equal(Y, W.view(np.float16).astype(np.float64).T)


def test_padded_cache_columns_ignored():
    g = np.random.default_rng(6)
    X = g.standard_normal((4, 64)).astype(np.float16).view(np.uint16)
    W = g.standard_normal((5, 64)).astype(np.float16).view(np.uint16)
    Wp = np.concatenate([W, np.full((5, 64), 0x3C00, np.uint16)], axis=1)
    assert np.array_equal(gemm_ref(X, Wp, K=64)[0], gemm_ref(X, W)[0])


def test_tolerance_catches_planted_error():
    g = np.random.default_rng(7)
    X = g.standard_normal((8, 128)).astype(np.float16).view(np.uint16)
    W = g.standard_normal((8, 128)).astype(np.float16).view(np.uint16)
    Yref, S = gemm_ref(X, W)
    ok, worst, _, _ = within_tolerance(Yref.astype(np.float32), Yref, S)
    assert ok and worst < 0.01
    bad = Yref.copy()
    bad[3, 5] += 2e-3 * S[3, 5]
    assert not within_tolerance(bad, Yref, S)[0]
    near = Yref.copy()
    near[3, 5] += 0.5e-3 * S[3, 5]
    assert within_tolerance(near, Yref, S)[0]
    nan = Yref.copy()
    nan[0, 0] = np.nan
    assert not within_tolerance(nan, Yref, S)[0]


@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (3, 2, 256)])
def test_degenerate_shapes(M, N, K):
    g = np.random.default_rng(8)
    X = g.standard_normal((M, K)).astype(np.float16).view(np.uint16)
    W = g.standard_normal((N, K)).astype(np.float16).view(np.uint16)
    Y, S = gemm_ref(X, W)
    assert np.allclose(Y, gemm_bruteforce(X, W), rtol=0, atol=1e-12)
