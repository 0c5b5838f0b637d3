"""Parity of mq_dequant_to_f16 (the load-time f16 cache) with the oracle: bit
for bit, on hand-derived blocks, ragged and padded shapes, and every weight
matrix shape of the 7B and Llama-3.1-8B workloads (full compare)."""

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden
from gpu_common import announce, assert_bits_equal, f16_bits, needs_gpu, to_dev_u8
from oracle.encode import concat_blocks, pack_q4k, pack_q6k, pack_q80

pytestmark = [pytest.mark.gpu, needs_gpu]

import quantized_weight_prefill_q4_amd as mq  # noqa: E402

FMT_NAME = {12: "Q4_K", 14: "Q6_K", 8: "Q8_0", 2: "Q4_0", 6: "Q5_0", 7: "Q5_1", 13: "Q5_K"}


def _run(fmt, q, N, K, pad):
    announce("dequant", FMT_NAME[fmt], f"N={N}", f"K={K}", f"pad={pad}")
    out = mq.dequant_to_f16(to_dev_u8(q), fmt, N, K, pad=pad)
    return f16_bits(out)


def _check(fmt, q, N, K, pad=True, what=""):
    got = _run(fmt, q, N, K, pad)
    exp = oracle.cache_ref(fmt, q, N, K, pad=pad)
    assert got.shape == exp.shape
    assert_bits_equal(got, exp, f"{FMT_NAME[fmt]} {N}x{K} {what}")


def test_worked_blocks_from_golden():
    g = read_golden("q4k_worked.txt")
    qs = [(i % 16) | ((15 - i % 16) << 4) for i in range(128)]
    q = []
    for e in range(256):
        c, r = divmod(e, 64)
        b = qs[32 * c + r % 32]
        q.append(b & 15 if r < 32 else b >> 4)
    sc = [int(t) for t in g["scales"][0].split()]
    mn = [int(t) for t in g["mins"][0].split()]
    blk = np.frombuffer(pack_q4k(0x3C00, 0x3800, sc, mn, q), np.uint8)
    w = _run(12, blk, 1, 256, False)[0].view(np.float16).astype(np.float64)
    for tok in g["expect"][0].split():
        e, v = tok.split(":")
        assert w[int(e)] == float(v), tok

    g6 = read_golden("q6k_worked.txt")
    b6 = np.array([(7 * i) & 255 for i in range(128)] + [(37 * i + 5) & 255 for i in range(64)]
                  + [(j - 8) & 255 for j in range(16)] + [0x00, 0x3C], np.uint8)
    w6 = _run(14, b6, 1, 256, False)[0]
    for tok in g6["expect_bits"][0].split():
        e, v = tok.split(":")
        assert int(w6[int(e)]) == int(v, 16), tok

    for row in read_golden("q80_worked.txt")["block"]:
        d_s, q_s, e_s = row.split("|")
        qv = [int(t) for t in q_s.split()]
        exp = [int(t, 16) for t in e_s.split()]
        b8 = np.frombuffer(pack_q80(int(d_s, 16), qv + [0] * (32 - len(qv))), np.uint8)
        w8 = _run(8, b8, 1, 32, False)[0]
        assert [int(x) for x in w8[: len(exp)]] == exp, row

    gd = read_golden("q4k_double_rounding.txt")
    qd = [0] * 256
    qd[0] = int(gd["q0"][0])
    bd = np.frombuffer(pack_q4k(int(gd["d_bits"][0], 16), int(gd["dmin_bits"][0], 16),
                                [int(t) for t in gd["scales"][0].split()],
                                [int(t) for t in gd["mins"][0].split()], qd), np.uint8)
    assert int(_run(12, bd, 1, 256, False)[0, 0]) == 0x3C02


def test_odd_block_alignment_q6k_q80():
    """Q6_K and Q8_0 blocks at every residue mod 16 (2-byte aligned starts)."""
    g = np.random.default_rng(3)
    b6 = concat_blocks([pack_q6k(int(g.integers(0x0400, 0x2000)), g.integers(-32, 32, 16),
                                 g.integers(0, 64, 256)) for _ in range(8)])
    _check(14, b6, 8, 256, pad=False, what="8 single-block rows")
    _check(14, b6, 1, 2048, pad=True, what="one 8-block row")
    b8 = concat_blocks([pack_q80(int(g.integers(0x0001, 0x3000)), g.integers(-128, 128, 32))
                        for _ in range(24)])
    for N, K in ((24, 32), (3, 256), (1, 768), (8, 96)):
        _check(8, b8, N, K, pad=True, what="hand blocks")


@pytest.mark.parametrize("fmt,N,K", [
    (12, 512, 512), (12, 512, 256), (12, 1, 256), (12, 37, 1024), (12, 33, 2048),
    (14, 1, 256), (14, 37, 512), (14, 64, 1024), (14, 7, 18944),
    (8, 1, 32), (8, 5, 96), (8, 37, 1024), (8, 64, 4096 + 32), (8, 3, 2048),
])
@pytest.mark.parametrize("pad", [True, False])
def test_small_and_ragged(fmt, N, K, pad):
    q = synth.weights(fmt, synth.rng(1, 0, fmt, 0), N, K)
    _check(fmt, q, N, K, pad=pad)


def test_explicit_ld_larger_than_cache_rule():
    import torch
    q = synth.weights(12, synth.rng(2), 16, 512)
    out = torch.full((16, 520), float("nan"), dtype=torch.float16, device="cuda:0")
    announce("dequant", "Q4_K", "N=16 K=512 ld=520")
    mq.dequant_to_f16(to_dev_u8(q), 12, 16, 512, out=out)
    got = f16_bits(out)
    assert_bits_equal(got[:, :512], oracle.dequant_ref(12, q, 16, 512), "body")
    assert np.all(got[:, 512:] == 0)


REAL = [
    ("7B q/o", 12, 3584, 3584), ("7B k/v", 12, 512, 3584), ("7B gate/up", 12, 18944, 3584),
    ("7B down", 14, 3584, 18944), ("8B 4096^2", 12, 4096, 4096), ("8B 14336x4096", 12, 14336, 4096),
    ("8B 4096x14336", 12, 4096, 14336), ("8B Q8_0 4096^2", 8, 4096, 4096),
]


@pytest.mark.parametrize("name,fmt,N,K", REAL)
def test_real_shapes_full(name, fmt, N, K):
    q = synth.weights(fmt, synth.rng(5, 0, N % 97, K % 89), N, K)
    _check(fmt, q, N, K, pad=True, what=name)


def test_batch_matches_oracle_across_launches():
    """mq_dequant_to_f16_batch: 28 jobs of all seven formats, padded and
    unpadded, odd row counts — two kernel launches (16 + 12 jobs) with
    workgroups of different jobs and formats in one grid.  Every cache must
    equal the oracle's bit for bit, pad columns +0."""
    shapes = [(12, 3, 256), (14, 5, 512), (8, 7, 96), (12, 130, 2048), (14, 65, 1024),
              (8, 300, 4096), (12, 1, 4096), (14, 2, 256), (8, 33, 32), (12, 17, 3584),
              (2, 11, 512), (6, 9, 2080), (7, 4, 1024), (13, 6, 512)]
    jobs, exp = [], []
    for i in range(28):
        fmt, N, K = shapes[i % len(shapes)]
        pad = i % 3 != 1
        q = synth.weights(fmt, synth.rng(40, 0, fmt, i), N, K)
        jobs.append((to_dev_u8(q), fmt, N, K))
        exp.append((fmt, N, K, pad, oracle.cache_ref(fmt, q, N, K, pad=pad)))
    announce("dequant_batch", f"{len(jobs)} jobs")
    outs = [None] * len(jobs)
    for pad in (True, False):
        idx = [i for i, e in enumerate(exp) if e[3] == pad]
        res = mq.dequant_to_f16_batch([jobs[i] for i in idx], pad=pad)
        for i, r in zip(idx, res):
            outs[i] = r
    for (fmt, N, K, pad, e), o in zip(exp, outs):
        got = f16_bits(o)
        assert got.shape == e.shape
        assert_bits_equal(got, e, f"batch {FMT_NAME[fmt]} {N}x{K} pad={pad}")


def test_batch_of_7b_layer_equals_single_calls():
    """The load phase's use: one layer's 7 weights (q, k, v, o, gate, up in Q4_K,
    down in Q6_K) decoded by one batched call equal the single-call caches bit
    for bit, plus more than 64 jobs (the library's host-side chunk) of a small
    matrix."""
    jobs, singles = [], []
    for mi, (name, fmt, N, K) in enumerate(synth.LAYER_7B):
        q = to_dev_u8(synth.weights(fmt, synth.rng(41, 0, mi, 0), N, K))
        jobs.append((q, fmt, N, K))
        announce("dequant", name, f"N={N}", f"K={K}")
        singles.append(f16_bits(mq.dequant_to_f16(q, fmt, N, K)))
    announce("dequant_batch", "7B layer")
    for got, exp in zip(mq.dequant_to_f16_batch(jobs), singles):
        assert np.array_equal(f16_bits(got), exp)
    q = synth.weights(8, synth.rng(42, 0, 8, 0), 9, 64)
    exp = oracle.cache_ref(8, q, 9, 64, pad=True)
    dq = to_dev_u8(q)
    announce("dequant_batch", "70 jobs")
    for o in mq.dequant_to_f16_batch([(dq, 8, 9, 64)] * 70):
        assert_bits_equal(f16_bits(o), exp, "batch of 70")
