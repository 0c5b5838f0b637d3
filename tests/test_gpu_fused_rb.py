"""The fused 256 × 256 register-expansion kernels (gemm_q4k_rb_kernel for
Q4_K and Q5_K, gemm_q6k_rb_kernel, gemm_b32_rb_kernel for Q8_0, Q4_0, Q5_0
and Q5_1) on random weights, at shapes whose plan takes them.

* One-hot activations (M = K, X = I): Y[m, n] = W16[n, m] with one nonzero
  product per output, so every expanded element is compared with the oracle's
  decode bit for bit.  An exact zero may come back as +0 where the decode
  gives −0 (the MFMA sum starts at +0); those are counted apart and allowed,
  every other element must be bit-identical.  Run whole and with a forced K
  split (the partial tiles then hold the value or +0).
* Random activations: fused and cache GEMMs, both unsplit, are bit-identical
  (same operands, same k order), and sampled rows are within the oracle's
  tolerance (minfer "05 · 8p" §3.3: the two shapes must agree)."""

import numpy as np
import pytest

import oracle
import synth
from gpu_common import announce, check_gemm, needs_gpu, to_dev_f16, to_dev_u8, to_host

pytestmark = [pytest.mark.gpu, needs_gpu]

import quantized_weight_prefill_q4_amd as mq  # noqa: E402
import torch  # noqa: E402

FMT_NAME = {12: "Q4_K", 14: "Q6_K", 8: "Q8_0", 2: "Q4_0", 6: "Q5_0", 7: "Q5_1", 13: "Q5_K"}
FMTS = (12, 13, 14, 8, 2, 6, 7)
# 8 x 25 tiles of 256 x 256 (more than 3/4 of a round: unsplit 256 x 256)
M = K = 2048
N = 6400


def _plan_is_rb(fmt, split_k):
    p = mq.gemm_plan(fmt, M, N, K, split_k)
    assert (p["bm"], p["bn"]) == (256, 256), p
    return p


@pytest.mark.parametrize("split", [0, 3])
@pytest.mark.parametrize("fmt", FMTS)
def test_rb_onehot_bits(fmt, split):
    p = _plan_is_rb(fmt, split)
    q = synth.weights(fmt, synth.rng(60, 0, fmt, N), N, K)
    x = synth.activations(None, K, K, mode="onehot")
    announce("gemm_fused one-hot", FMT_NAME[fmt], f"M={M}", f"N={N}", f"K={K}",
             f"split={split}", f"plan split={p['split']}")
    Y = to_host(mq.gemm_fused(to_dev_f16(x), to_dev_u8(q), fmt, N, K, split_k=split))
    exp = oracle.dequant_ref(fmt, q, N, K).view(np.float16).astype(np.float32).T
    got_b, exp_b = Y.view(np.uint32), np.ascontiguousarray(exp).view(np.uint32)
    diff = got_b != exp_b
    zero_sign = diff & ((got_b & 0x7FFFFFFF) == 0) & ((exp_b & 0x7FFFFFFF) == 0)
    other = diff & ~zero_sign
    assert not other.any(), (f"{int(other.sum())} elements differ beyond the sign of zero; "
                             f"first at {np.argwhere(other)[:4].tolist()}")
    # the decode keeps -0 (Q6_K, Q4_0, Q5_0 can produce it); Y holds +0 there
    assert not (zero_sign & (got_b != 0)).any()
    print(f"{FMT_NAME[fmt]}: {int(zero_sign.sum())} of {Y.size} outputs are +0 where the "
          f"decode gives -0")


@pytest.mark.parametrize("fmt", FMTS)
def test_rb_random_fused_equals_cache(fmt):
    _plan_is_rb(fmt, 1)
    q = synth.weights(fmt, synth.rng(61, 0, fmt, N), N, K)
    x = synth.activations(synth.rng(61, role=1), M, K)
    qd, xd = to_dev_u8(q), to_dev_f16(x)
    announce("gemm_fused vs cache, random", FMT_NAME[fmt], f"M={M}", f"N={N}", f"K={K}")
    cache = mq.dequant_to_f16(qd, fmt, N, K)
    yc = mq.gemm_f16cache(xd, cache, K, split_k=1)
    yf = mq.gemm_fused(xd, qd, fmt, N, K, split_k=1)
    torch.cuda.synchronize()
    assert torch.equal(yc, yf), "fused and cache GEMMs differ at split 1"
    rows = np.unique(np.concatenate([[0, 255, 256, 1023, 2047],
                                     np.random.default_rng(fmt).choice(M, 11)]))
    w = oracle.dequant_ref(fmt, q, N, K)
    check_gemm(to_host(yf)[rows], x, w, K, f"fused {FMT_NAME[fmt]} random", rows=rows)
