"""The library's calls under HIP graph capture: the decode, both GEMMs with a
K split (GEMM + fixed-order reduce), the f32-activation GEMM, the activation
convert and the no-alloc fused GEMM are captured once into one graph, which is
replayed three times.  Between replays eager work overwrites every output with
NaN and the host synchronizes; after each replay every output must equal the
eager calls' result bit for bit (the library records no memset nodes; its
outputs are fully rewritten by each call)."""

import numpy as np
import pytest

import synth
from gpu_common import announce, needs_gpu, to_dev_f16, to_dev_u8

pytestmark = [pytest.mark.gpu, needs_gpu]

import torch  # noqa: E402

import quantized_weight_prefill_q4_amd as mq  # noqa: E402
from quantized_weight_prefill_q4_amd import _lib  # noqa: E402


def test_library_calls_replay_in_a_graph():
    M, N, K, fmt = 256, 1024, 4096, synth.Q4_K
    p = mq.gemm_plan(fmt, M, N, K)
    assert p["split"] > 1 and mq.gemm_plan("f16", M, N, K)["split"] > 1   # a reduce in each GEMM
    dev = torch.device("cuda:0")
    q = to_dev_u8(synth.weights(fmt, synth.rng(90, 0, fmt, N), N, K))
    x = to_dev_f16(synth.activations(synth.rng(90, role=1), M, K))
    x32 = torch.randn((M, K), generator=torch.Generator(device=dev).manual_seed(91), device=dev)
    cache = torch.empty((N, mq.cache_ld(K)), dtype=torch.float16, device=dev)
    outs = {n: torch.empty((M, N), dtype=torch.float32, device=dev)
            for n in ("cache", "fused", "xf32", "noalloc")}
    x16 = torch.empty((M, K), dtype=torch.float16, device=dev)
    ws = {n: torch.empty(max(1, b // 4), dtype=torch.float32, device=dev) for n, b in (
        ("cache", mq.workspace_bytes(0, M, N, K)), ("fused", mq.workspace_bytes(fmt, M, N, K)),
        ("xf32", mq.workspace_bytes(0, M, N, K, x_f32=True)))}

    def calls():
        mq.dequant_to_f16(q, fmt, N, K, out=cache)
        mq.gemm_f16cache(x, cache, K, out=outs["cache"], ws=ws["cache"])
        mq.gemm_fused(x, q, fmt, N, K, out=outs["fused"], ws=ws["fused"])
        mq.gemm_f16cache(x32, cache, K, out=outs["xf32"], ws=ws["xf32"])
        mq.convert_f32_to_f16(x32, out=x16)
        rc = _lib.lib().mq_gemm_fused_noalloc(
            fmt, x.data_ptr(), K, q.data_ptr(), outs["noalloc"].data_ptr(), N, M, N, K, 0,
            torch.cuda.current_stream().cuda_stream)
        assert rc == _lib.MQ_OK

    def snapshot():
        torch.cuda.synchronize()
        return {"cache16": cache.clone(), "x16": x16.clone(), **{n: t.clone() for n, t in outs.items()}}

    announce("graph capture", f"M={M} N={N} K={K}", "eager reference")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    ref = snapshot()
    assert torch.equal(ref["noalloc"], ref["fused"])

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        for t in list(outs.values()) + [cache, x16]:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        announce("graph replay", rep)
        g.replay()
        got = snapshot()
        for n, t in ref.items():
            assert torch.equal(got[n].view(torch.int32 if got[n].dtype == torch.float32 else torch.int16),
                               t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)), \
                f"replay {rep}: {n} differs from the eager result"
    del g
