"""Helpers of the GPU parity tests: device transfer, announcements, oracle checks."""

import sys

import numpy as np
import pytest

import oracle

try:
    import torch
    HAVE_GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    torch = None
    HAVE_GPU = False

needs_gpu = pytest.mark.skipif(not HAVE_GPU, reason="no GPU")


def announce(*parts):
    """Name the case on stdout (flushed) before a GPU step, so a crash is attributable."""
    sys.stdout.write("\n[case] " + " ".join(str(p) for p in parts) + "\n")
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev_u8(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).to(dev())


def to_dev_f16(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16)).to(dev())


def f16_bits(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def to_host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def assert_bits_equal(got: np.ndarray, exp: np.ndarray, what: str):
    """Bit-exact comparison; on failure report how many differ only in the sign of zero."""
    if np.array_equal(got, exp):
        return
    diff = got != exp
    n = int(diff.sum())
    zero_sign = int((diff & ((got & 0x7FFF) == 0) & ((exp & 0x7FFF) == 0)).sum())
    idx = np.argwhere(diff)[:5].tolist()
    raise AssertionError(f"{what}: {n} elements differ ({zero_sign} only in the sign of zero); "
                         f"first at {idx}: got {[hex(got[tuple(i)]) for i in idx]} "
                         f"expected {[hex(exp[tuple(i)]) for i in idx]}")


def check_gemm(Y: np.ndarray, x_bits: np.ndarray, w_bits: np.ndarray, K: int, what: str,
               rows=None):
    """Y (float32 [M, N], or the selected rows) against the f64 oracle within
    |Y − Yref| ≤ 1e-3·S + 1e-5.  Returns (worst ratio, max |Δ|/S)."""
    xs = x_bits if rows is None else x_bits[rows]
    Yref, S = oracle.gemm_ref(xs, w_bits, K)
    ok, worst, max_abs, max_rel = oracle.within_tolerance(Y, Yref, S)
    assert ok, f"{what}: worst ratio {worst:.3g}, max abs {max_abs:.3g}"
    # f32 accumulation of exact products: errors far below the bound
    assert max_rel < 1e-5, f"{what}: max |dY|/S = {max_rel:.3g} is suspiciously large"
    return worst, max_rel
