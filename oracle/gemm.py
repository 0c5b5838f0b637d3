"""Reference for the prefill matmul Y = X·Wᵀ over f16 operands.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The pages' problem: an "NT" GEMM with nt tokens (M), od output rows (N) and
id inner size (K) — minfer 05 · 8p §3.2 third site (``gemm_qb_nt_kernel``
arguments) — with f16 inputs and f32 output (Fucina "Eager GPU Offload
Without A Compute Graph", F16 NT GEMM paragraph: f16 inputs, f32 C).  Both
of the method's shapes (f16 cache, fused dequant) feed the same f16-rounded
weights to the contraction (minfer 05 · 8p §3.3: same rounding path), so the
exact result they approximate is the product of the f16 values.

``gemm_ref`` evaluates it in binary64: each f16×f16 product is exact there,
and the only error is the f64 summation, at most K·2⁻⁵³·S per element, far
inside the acceptance bound |Y − Yref| ≤ 1e-3·S + 1e-5 with S = |X|·|W|ᵀ.
"""

from __future__ import annotations

import math

import numpy as np


def activations_to_f16(x: np.ndarray) -> np.ndarray:
    """f16 bit patterns of f32 activations, each rounded once to the nearest
    binary16 (ties to even, subnormals kept, overflow to ±inf).

    The pages' callers hold f32 activations; the f16 GEMM consumes them
    converted to half (Fucina "Eager GPU Offload Without A Compute Graph",
    quantized linears: f32 activation loads converted with half2 conversions
    into the half operand tile; llama.cpp PR #57, batch-size dependence: the
    activation convert ahead of the f16 GEMM).  The f32-activation GEMM is
    therefore ``gemm_ref(activations_to_f16(x), w)``.  numpy's float32 →
    float16 cast is that single rounding.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):        # overflow to ±inf is the defined result
        return x.astype(np.float16).view(np.uint16)


def activations_to_f16_scalar(x: np.ndarray) -> np.ndarray:
    """The same rounding element by element with the IEEE converter of
    ``oracle.f16`` (small inputs only); a second, independent implementation."""
    from .f16 import f32_to_f16_bits

    x = np.asarray(x, dtype=np.float32)
    flat = [f32_to_f16_bits(float(v)) for v in x.reshape(-1)]
    return np.array(flat, dtype=np.uint16).reshape(x.shape)


def _as_f64(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def gemm_ref(x_bits: np.ndarray, w_bits: np.ndarray, K: int | None = None):
    """(Yref, S) in float64 for X [M, K] and W [N, >=K] given as f16 bit patterns.

    Only the first K columns of W are used, so a padded cache row can be
    passed directly.
    """
    X = _as_f64(x_bits)
    W = _as_f64(w_bits)
    if K is None:
        K = X.shape[1]
    X = X[:, :K]
    W = W[:, :K]
    Y = X @ W.T
    S = np.abs(X) @ np.abs(W).T
    return Y, S


def gemm_bruteforce(x_bits: np.ndarray, w_bits: np.ndarray, K: int | None = None) -> np.ndarray:
    """Correctly rounded binary64 Y by a triple loop with math.fsum (small inputs only)."""
    X = _as_f64(x_bits)
    W = _as_f64(w_bits)
    if K is None:
        K = X.shape[1]
    M, N = X.shape[0], W.shape[0]
    Y = np.empty((M, N), dtype=np.float64)
    for m in range(M):
        xr = X[m, :K].tolist()
        for n in range(N):
            wr = W[n, :K].tolist()
            Y[m, n] = math.fsum(a * b for a, b in zip(xr, wr))
    return Y


def within_tolerance(Y: np.ndarray, Yref: np.ndarray, S: np.ndarray,
                     rel: float = 1e-3, abs_: float = 1e-5):
    """Per-element acceptance |Y − Yref| ≤ rel·S + abs_.

    Returns (all_ok, worst_ratio, max_abs_err, max_rel_to_S) where worst_ratio is
    max |Y − Yref| / (rel·S + abs_) (≤ 1 passes).
    """
    Y = np.asarray(Y, dtype=np.float64)
    err = np.abs(Y - Yref)
    bound = rel * S + abs_
    ratio = err / bound
    worst = float(ratio.max()) if ratio.size else 0.0
    max_abs = float(err.max()) if err.size else 0.0
    max_rel = float((err / (S + 1e-30)).max()) if err.size else 0.0
    ok = bool(np.all(np.isfinite(Y))) and worst <= 1.0
    return ok, worst, max_abs, max_rel
