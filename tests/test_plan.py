"""The GEMM planner on the host (no GPU): for every format, path and a grid of
shapes and forced splits, the plan the library would launch has a kernel for
its tile, its grid covers Y exactly once, its K ranges cover K without gaps or
empty ranges and respect what each kernel assumes of them, and its workspace
is what the *_workspace_bytes functions report.

A plan with a tile no kernel implements is the fault class that addresses
tiles past the matrix (the dispatch rejects it; this test makes sure no plan
asks for one)."""

import itertools

import pytest

import quantized_weight_prefill_q4_amd as mq

FMTS = ("f16", "q4_0", "q5_0", "q5_1", "q8_0", "q4_k", "q5_k", "q6_k")
MS = (1, 17, 64, 65, 128, 129, 200, 256, 384, 512, 1000, 1024, 2048, 2304, 4097)
NS = (1, 40, 128, 512, 1000, 3584, 4096, 4608, 14336, 18944, 37888)
KS_BIG = (256, 512, 1024, 3584, 4096, 14336, 18944)
SPLITS = (0, 1, 2, 3, 5, 8, 16)


def _ks(fmt):
    if fmt == "f16":
        return (8, 24, 64, 520) + KS_BIG
    if fmt in ("q4_k", "q5_k", "q6_k"):
        return KS_BIG
    return (32, 96, 160) + KS_BIG


def _check(p, fmt, M, N, K, split_k, path):
    step = 128 if path == "mmq" else 64
    assert p["has_kernel"] == 1, f"no kernel for tile {p['bm']}x{p['bn']}"
    bm, bn = p["bm"], p["bn"]
    assert p["tiles_m"] == -(-M // bm) and p["tiles_n"] == -(-N // bn)
    tiles = p["tiles_m"] * p["tiles_n"]
    assert p["dp_tiles"] + p["tail_tiles"] == tiles
    assert p["k_steps"] == -(-K // step)
    split, per = p["split"], p["steps_per_split"]
    assert 1 <= split <= 16
    if split == 1:
        assert p["tail_tiles"] == 0 and p["ws_bytes"] == (p["ws_bytes"] if path == "f32" else 0)
        assert per == p["k_steps"]
    else:
        assert p["tail_tiles"] > 0
        # ranges [s·per, min((s+1)·per, k_steps)): none empty, all of K covered
        assert (split - 1) * per < p["k_steps"] <= split * per
        if split_k >= 2:
            assert split <= split_k and p["dp_tiles"] == 0
        # the register-expansion kernels (256-column fused tiles)
        q = fmt in ("q4_k", "q5_k") and bn == 256
        pairs = fmt == "q6_k" or (fmt in ("q8_0", "q4_0", "q5_0", "q5_1") and bn == 256
                                  and K % 256 == 0)
        if path == "f16" and q:
            assert per % 4 == 0, "Q4_K/Q5_K 256x256 ranges are whole super-blocks"
        elif path == "f16" and pairs:
            assert per % 2 == 0, "paired k-steps: ranges start even"
        if path != "f32":
            assert p["ws_bytes"] == split * p["tail_tiles"] * bm * bn * 4
    # the grid the launcher computes stays a valid HIP grid
    assert 0 < p["dp_tiles"] + p["tail_tiles"] * split < 2 ** 31


@pytest.mark.parametrize("fmt", FMTS)
def test_every_plan_has_a_kernel_and_covers_y(fmt):
    n = 0
    for M, N, K in itertools.product(MS, NS, _ks(fmt)):
        for split_k in SPLITS:
            if split_k > 1 and M * N >= 2 ** 31:
                continue
            for path in ("f16", "f32"):
                p = mq.gemm_plan(fmt, M, N, K, split_k, path=path)
                _check(p, fmt, M, N, K, split_k, path)
                ws_fn = mq.workspace_bytes(fmt, M, N, K, split_k, x_f32=path == "f32")
                assert p["ws_bytes"] == ws_fn
                n += 1
            if fmt != "f16" and K % 32 == 0:
                p = mq.gemm_plan(fmt, M, N, K, split_k, path="mmq")
                _check(p, fmt, M, N, K, split_k, "mmq")
                assert p["ws_bytes"] == mq.mmq_workspace_bytes(fmt, M, N, K, split_k)
    assert n > 1000


def test_plan_query_rejects():
    from quantized_weight_prefill_q4_amd import _lib
    import ctypes
    L = _lib.lib()
    info = _lib.MqGemmPlanInfo()
    assert L.mq_gemm_plan_query(0, 12, 64, 64, 256, 0, None) == _lib.MQ_ERR_NULL
    assert L.mq_gemm_plan_query(3, 12, 64, 64, 256, 0, ctypes.byref(info)) == _lib.MQ_ERR_FORMAT
    assert L.mq_gemm_plan_query(2, 0, 64, 64, 256, 0, ctypes.byref(info)) == _lib.MQ_ERR_FORMAT
    assert L.mq_gemm_plan_query(0, 12, 64, 64, 100, 0, ctypes.byref(info)) == _lib.MQ_ERR_SHAPE
    assert L.mq_gemm_plan_query(0, 12, 0, 64, 256, 0, ctypes.byref(info)) == _lib.MQ_ERR_SHAPE
    assert L.mq_gemm_plan_query(0, 12, 64, 64, 256, 17, ctypes.byref(info)) == _lib.MQ_ERR_SPLIT


def test_known_plans():
    # the 7B shapes at M = 2048: gate/up on 256x256 (512 whole tiles + 80 split 3 ways),
    # down on 256x256 split twice, q/o on 256x128, k/v on 64x128 split twice
    g = mq.gemm_plan("f16", 2048, 18944, 3584)
    assert (g["bm"], g["bn"], g["dp_tiles"], g["tail_tiles"], g["split"]) == (256, 256, 512, 80, 3)
    d = mq.gemm_plan("f16", 2048, 3584, 18944)
    assert (d["bm"], d["bn"], d["dp_tiles"], d["split"]) == (256, 256, 0, 2)
    q = mq.gemm_plan("f16", 2048, 3584, 3584)
    assert (q["bm"], q["bn"]) == (256, 128)
    k = mq.gemm_plan("f16", 2048, 512, 3584)
    assert (k["bm"], k["bn"], k["split"]) == (64, 128, 2)
