"""The boundary's ordering contract: every call is enqueued on the stream it
is given and keeps no state between calls, so work on two streams at once
(each with its own outputs and workspace) gives exactly what the same calls
give one after another; and a call with caller-provided outputs and
workspace allocates nothing (torch's allocator is left untouched)."""

import numpy as np
import pytest

import synth
from gpu_common import announce, dev, needs_gpu, to_dev_u8

pytestmark = [pytest.mark.gpu, needs_gpu]

import torch  # noqa: E402

import quantized_weight_prefill_q4_amd as mq  # noqa: E402


def _problem(seed, fmt, M, N, K):
    q = to_dev_u8(synth.weights(fmt, synth.rng(seed, 0, fmt, 0), N, K))
    x = torch.from_numpy(synth.activations(synth.rng(seed, role=1), M, K).view(np.float16)).to(dev())
    cache = mq.dequant_to_f16(q, fmt, N, K)
    y1 = torch.empty((M, N), dtype=torch.float32, device=dev())
    y2 = torch.empty((M, N), dtype=torch.float32, device=dev())
    y3 = torch.empty((M, N), dtype=torch.float32, device=dev())
    c2 = torch.empty_like(cache)
    wsb = max(mq.workspace_bytes(0, M, N, K), mq.workspace_bytes(fmt, M, N, K))
    ws = torch.empty(max(1, wsb // 4), dtype=torch.float32, device=dev())
    return dict(fmt=fmt, N=N, K=K, q=q, x=x, cache=cache, y1=y1, y2=y2, y3=y3, c2=c2, ws=ws)


def _run(p, reps):
    for _ in range(reps):
        mq.gemm_f16cache(p["x"], p["cache"], p["K"], out=p["y1"], ws=p["ws"])
        mq.gemm_fused(p["x"], p["q"], p["fmt"], p["N"], p["K"], out=p["y2"], ws=p["ws"])
        mq.dequant_to_f16(p["q"], p["fmt"], p["N"], p["K"], out=p["c2"])
        mq.gemm_f16cache(p["x"], p["c2"], p["K"], out=p["y3"], ws=p["ws"])


def test_two_streams_equal_sequential_and_allocate_nothing():
    a = _problem(60, 12, 2048, 18944, 3584)      # gate-like: K-split tail, workspace in use
    b = _problem(61, 14, 300, 3584, 18944)       # Q6_K, other tiles
    announce("streams", "sequential reference")
    _run(a, 1)
    _run(b, 1)
    torch.cuda.synchronize()
    ref = {k: (a[k].clone(), b[k].clone()) for k in ("y1", "y2", "y3", "c2")}
    for p in (a, b):
        for k in ("y1", "y2", "y3"):
            p[k].fill_(float("nan"))
        p["c2"].fill_(float("nan"))
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    before = torch.cuda.memory_allocated()
    announce("streams", "two streams at once")
    with torch.cuda.stream(sa):
        _run(a, 3)
    with torch.cuda.stream(sb):
        _run(b, 3)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before, "a call allocated through torch"
    for k in ("y1", "y2", "y3"):
        assert torch.equal(a[k], ref[k][0]), f"stream A {k} differs"
        assert torch.equal(b[k], ref[k][1]), f"stream B {k} differs"
    assert torch.equal(a["c2"].view(torch.int16), ref["c2"][0].view(torch.int16))
    assert torch.equal(b["c2"].view(torch.int16), ref["c2"][1].view(torch.int16))
