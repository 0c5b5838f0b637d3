"""Seeded random shapes through both GEMM entry points, integer inputs (exact).

Each case draws a format, M, N, K (a multiple of the format's block), a K
split (automatic, none, or forced 2..16), the activation kind (f16, or f32
rounded to f16 inside the call) and row strides of X and Y wider than the
matrices: X and Y are views into wider buffers, X's extra columns hold NaN and
Y's a sentinel.  The weights and activations take small integer values, so
every partial sum is exact in f32 whatever the tile, split or k order; the
sampled rows of Y must equal the oracle exactly for the cache GEMM (on the
device-built, row-padded cache) and for the fused GEMM, and the columns of Y
past N must keep the sentinel."""

import numpy as np
import pytest

import oracle
import synth
from gpu_common import announce, dev, needs_gpu, to_dev_u8, to_host

pytestmark = [pytest.mark.gpu, needs_gpu]

import torch  # noqa: E402

import quantized_weight_prefill_q4_amd as mq  # noqa: E402

NAME = {2: "Q4_0", 6: "Q5_0", 7: "Q5_1", 8: "Q8_0", 12: "Q4_K", 13: "Q5_K", 14: "Q6_K"}
FMTS = (12, 14, 8, 13, 2, 6, 7)
SENTINEL = -12345.0


def _case(i):
    g = np.random.default_rng(9100 + i)
    fmt = FMTS[i % len(FMTS)]
    be = mq.block_elems(fmt)
    M = (1, 7, 63, 64, 65, 100, 128, 129, 300, 700, 1100)[i % 11]
    N = int(g.integers(1, 2600))
    K = be * int(g.integers(1, 4096 // be + 1))
    split = int(g.choice([0, 0, 1, 2, 3, 5, 16]))
    x_f32 = i % 3 == 2
    padx = int(g.choice([0, 8, 64]))
    pady = int(g.choice([0, 4, 37]))
    return fmt, M, N, K, split, x_f32, padx, pady


@pytest.mark.parametrize("i", range(28))
def test_random_shape_integer_exact(i):
    fmt, M, N, K, split, x_f32, padx, pady = _case(i)
    g = np.random.default_rng(9200 + i)
    q = synth.weights(fmt, synth.rng(92, i, fmt, N), N, K, mode="integer")
    x_bits = synth.activations(synth.rng(92, i, role=1), M, K, mode="integer")
    xv = x_bits.view(np.float16).astype(np.float32)      # integers, exact in f16 and f32
    tdt = torch.float32 if x_f32 else torch.float16
    xbuf = torch.full((M, K + padx), float("nan"), dtype=tdt, device=dev())
    xbuf[:, :K] = torch.from_numpy(xv).to(dev()).to(tdt)
    x = xbuf[:, :K]
    qd = to_dev_u8(q)
    rows = np.unique(np.concatenate([[0, M - 1], g.integers(0, M, 6)]))
    Yref, _ = oracle.gemm_ref(x_bits[rows], oracle.dequant_ref(fmt, q, N, K))
    tag = (NAME[fmt], f"M={M}", f"N={N}", f"K={K}", f"split={split}",
           "x=f32" if x_f32 else "x=f16", f"ldx=K+{padx}", f"ldy=N+{pady}")

    cache = mq.dequant_to_f16(qd, fmt, N, K)              # row-padded when 2K % 2048 == 0
    for path in ("cache", "fused"):
        ybuf = torch.full((M, N + pady), SENTINEL, dtype=torch.float32, device=dev())
        y = ybuf[:, :N]
        announce("random shape", path, *tag)
        if path == "cache":
            mq.gemm_f16cache(x, cache, K, split_k=split, out=y)
        else:
            mq.gemm_fused(x, qd, fmt, N, K, split_k=split, out=y)
        yb = to_host(ybuf)
        assert np.array_equal(yb[rows, :N].astype(np.float64), Yref), f"{path} {tag}"
        assert (yb[:, N:] == SENTINEL).all(), f"{path} {tag}: columns past N written"
