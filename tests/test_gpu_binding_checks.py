"""The Python binding checks the sizes the C ABI cannot see (it receives plain
pointers): an argument too small for the requested N, K or M raises before
anything is enqueued, so a caller's mistake is an exception, not an access
out of bounds.  Each case is followed by a correct call on the same tensors."""

import numpy as np
import pytest

import synth
from gpu_common import announce, dev, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]

import torch  # noqa: E402

import quantized_weight_prefill_q4_amd as mq  # noqa: E402

N, K, M = 96, 512, 40


@pytest.fixture(scope="module")
def q():
    return torch.from_numpy(synth.weights(synth.Q4_K, synth.rng(90), N, K)).to(dev()).reshape(-1)


def _x(dtype=torch.float16, cols=K):
    return torch.randn((M, cols), device=dev()).to(dtype)


def test_dequant_sizes(q):
    announce("binding checks", "dequant")
    with pytest.raises(ValueError, match="wq holds"):
        mq.dequant_to_f16(q[:-1], "q4_k", N, K)
    with pytest.raises(ValueError, match="out must be at least"):
        mq.dequant_to_f16(q, "q4_k", N, K, out=torch.empty((N - 1, K), dtype=torch.float16,
                                                            device=dev()))
    # the kernel writes every row's pad columns up to the row stride, so an
    # [N, K] view at stride K + 64 needs N · (K + 64) elements of storage
    flat = torch.empty(N * (K + 64) - 10, dtype=torch.float16, device=dev())
    with pytest.raises(ValueError, match="out spans"):
        mq.dequant_to_f16(q, "q4_k", N, K, out=flat.as_strided((N, K), (K + 64, 1)))
    whole = torch.empty(N * (K + 64), dtype=torch.float16, device=dev())
    mq.dequant_to_f16(q, "q4_k", N, K, out=whole.as_strided((N, K), (K + 64, 1)))
    with pytest.raises(ValueError, match="wq holds"):
        mq.dequant_to_f16_batch([(q, "q4_k", N, K), (q[:100], "q4_k", N, K)])
    assert mq.dequant_to_f16(q, "q4_k", N, K).shape == (N, K)


def test_gemm_sizes(q):
    announce("binding checks", "gemm")
    w16 = mq.dequant_to_f16(q, "q4_k", N, K)
    x = _x()
    with pytest.raises(ValueError, match="x must be at least"):
        mq.gemm_f16cache(x[:, : K - 8], w16, K)
    with pytest.raises(ValueError, match="w16 must be at least"):
        mq.gemm_f16cache(x, w16[:, : K - 8], K)
    with pytest.raises(ValueError, match="out must be at least"):
        mq.gemm_f16cache(x, w16, K, out=torch.empty((M, N - 1), device=dev()))
    with pytest.raises(ValueError, match="wq holds"):
        mq.gemm_fused(x, q[:-144], "q4_k", N, K)
    with pytest.raises(ValueError, match="x must be at least"):
        mq.gemm_fused(x[:, : K - 256], q, "q4_k", N, K)
    with pytest.raises(ValueError, match="x must be at least"):
        mq.gemm_fused(_x(torch.float32, K - 256), q, "q4_k", N, K)
    y1 = mq.gemm_f16cache(x, w16, K, split_k=1)
    y2 = mq.gemm_fused(x, q, "q4_k", N, K, split_k=1)
    assert torch.equal(y1, y2)


def test_activation_sizes(q):
    announce("binding checks", "convert / quantize / mmq")
    x32 = _x(torch.float32)
    with pytest.raises(ValueError, match="out must be at least"):
        mq.convert_f32_to_f16(x32, out=torch.empty((M, K - 8), dtype=torch.float16, device=dev()))
    with pytest.raises(ValueError, match="x must be at least"):
        mq.convert_f32_to_f16(x32, K + 8)
    with pytest.raises(ValueError, match="xq must be at least"):
        mq.quantize_q8_1(x32, xq=torch.empty((M, K - 16), dtype=torch.int8, device=dev()))
    xq, ds = mq.quantize_q8_1(x32)
    with pytest.raises(ValueError, match="ds holds"):
        mq.gemm_mmq(xq, ds.reshape(-1)[:-2], q, "q4_k", N, K)
    with pytest.raises(ValueError, match="wq holds"):
        mq.gemm_mmq(xq, ds, q[:-1], "q4_k", N, K)
    with pytest.raises(ValueError, match="out must be at least"):
        mq.gemm_mmq(xq, ds, q, "q4_k", N, K, out=torch.empty((M - 1, N), device=dev()))
    y = mq.gemm_mmq(xq, ds, q, "q4_k", N, K)
    assert y.shape == (M, N) and bool(torch.isfinite(y).all())
    assert np.isfinite(mq.convert_f32_to_f16(x32).float().cpu().numpy()).all()
