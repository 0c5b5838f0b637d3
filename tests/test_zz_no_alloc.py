"""mq_gemm_fused_noalloc: the fused GEMM whose K-split partial tiles live in
the library's static device scratch instead of a caller workspace.  Called
through the C ABI and compared with mq_gemm_fused (workspace from torch) bit
for bit: the two run the same plan and kernels.  Two calls in a row, the
second on a smaller problem (the scratch keeps the first call's partials,
which the second must not see), then the rejection of a forced split whose
partials exceed the scratch."""

import pytest

import synth
from gpu_common import announce, needs_gpu, to_dev_f16, to_dev_u8

pytestmark = [pytest.mark.gpu, needs_gpu]

import torch  # noqa: E402

import quantized_weight_prefill_q4_amd as mq  # noqa: E402
from quantized_weight_prefill_q4_amd import _lib  # noqa: E402


def _noalloc(fmt, x, q, y, M, N, K, split_k=0):
    return _lib.lib().mq_gemm_fused_noalloc(
        fmt, x.data_ptr(), x.stride(0), q.data_ptr(), y.data_ptr(), y.stride(0), M, N, K,
        split_k, torch.cuda.current_stream().cuda_stream)


# (fmt, M, N, K): the 7B gate shape at M = 2048 (80 tail tiles of 256 x 256 split
# 3 ways: 62.9 MB of partials, nearly all of the scratch), then a smaller one
# (Q6_K, 128 x 128 tiles split along K).
CASES = [(12, 2048, 18944, 3584), (14, 128, 4096, 4096)]


def test_noalloc_equals_fused_on_two_calls():
    for i, (fmt, M, N, K) in enumerate(CASES):
        need = mq.workspace_bytes(fmt, M, N, K)
        assert 0 < need <= _lib.MQ_NOALLOC_SCRATCH_BYTES
        q = to_dev_u8(synth.weights(fmt, synth.rng(80, i, fmt, N), N, K))
        x = to_dev_f16(synth.activations(synth.rng(80, i, role=1), M, K))
        announce("mq_gemm_fused_noalloc", f"call {i + 1}", f"fmt={fmt}", f"M={M}", f"N={N}",
                 f"K={K}", f"partials={need}")
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=x.device)
        rc = _noalloc(fmt, x, q, y, M, N, K)
        assert rc == _lib.MQ_OK, _lib.lib().mq_strerror(rc)
        ref = mq.gemm_fused(x, q, fmt, N, K)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"call {i + 1}: noalloc and fused differ"


def test_noalloc_rejects_a_split_beyond_the_scratch():
    fmt, M, N, K = 12, 2048, 18944, 3584
    assert mq.workspace_bytes(fmt, M, N, K, 16) > _lib.MQ_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(N * mq.row_bytes(fmt, K), dtype=torch.uint8, device="cuda")
    x = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    announce("mq_gemm_fused_noalloc rejects split 16")
    assert _noalloc(fmt, x, q, y, M, N, K, split_k=16) == _lib.MQ_ERR_SCRATCH
    assert _noalloc(5, x, q, y, M, N, K) == _lib.MQ_ERR_FORMAT
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "a rejected call wrote Y"
