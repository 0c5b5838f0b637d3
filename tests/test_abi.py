"""The C ABI without a GPU: the library loads, exports every function that
include/mq.h declares, agrees with the binding's signatures, and rejects
invalid arguments before launching anything (every call below has at least one
invalid argument, so no HIP call is made)."""

import ctypes
import os
import re

import pytest

import quantized_weight_prefill_q4_amd as mq
from quantized_weight_prefill_q4_amd import _lib
from oracle import cache_ld as oracle_ld, row_bytes as oracle_row_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mq.h")
FAKE = 0x100000   # a 16-byte-aligned address that is never dereferenced
MIS = FAKE + 2    # misaligned


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(mq_\w+)\s*\(([^)]*)\)\s*;", text):
        args = [a for a in m.group(2).split(",") if a.strip() and a.strip() != "void"]
        out[m.group(1)] = len(args)
    return out


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_header_symbols_exported_and_bound(L):
    decl = _declared()
    assert set(decl) == set(_lib.SIGNATURES), "binding and header disagree"
    for name, nargs in decl.items():
        assert hasattr(L, name), f"{name} not exported"
        assert len(_lib.SIGNATURES[name][1]) == nargs, name


def test_format_tables(L):
    assert (L.mq_block_elems(12), L.mq_block_bytes(12)) == (256, 144)
    assert (L.mq_block_elems(14), L.mq_block_bytes(14)) == (256, 210)
    assert (L.mq_block_elems(8), L.mq_block_bytes(8)) == (32, 34)
    # 2 + 16, 2 + 4 + 16, 2 + 2 + 4 + 16, and Q4_K's 144 + 32 bytes of qh
    assert (L.mq_block_elems(2), L.mq_block_bytes(2)) == (32, 18)
    assert (L.mq_block_elems(6), L.mq_block_bytes(6)) == (32, 22)
    assert (L.mq_block_elems(7), L.mq_block_bytes(7)) == (32, 24)
    assert (L.mq_block_elems(13), L.mq_block_bytes(13)) == (256, 176)
    for unknown in (0, 1, 3, 4, 5, 9, 10, 11, 15, 99):
        assert L.mq_block_elems(unknown) == _lib.MQ_ERR_FORMAT
        assert L.mq_block_bytes(unknown) == _lib.MQ_ERR_FORMAT
    for fmt, K in ((12, 3584), (14, 18944), (8, 4096), (12, 256), (8, 32), (2, 4096),
                   (6, 4096), (7, 32), (13, 3584), (13, 256)):
        assert L.mq_row_bytes(fmt, K) == oracle_row_bytes(fmt, K)
    assert L.mq_row_bytes(6, 48) == _lib.MQ_ERR_SHAPE
    assert L.mq_row_bytes(13, 3200) == _lib.MQ_ERR_SHAPE
    assert L.mq_row_bytes(12, 100) == _lib.MQ_ERR_SHAPE
    assert L.mq_row_bytes(99, 256) == _lib.MQ_ERR_FORMAT


@pytest.mark.parametrize("K", [8, 256, 512, 1024, 3584, 4096, 14336, 18944, 2048, 3072])
def test_cache_ld_matches_oracle(L, K):
    assert L.mq_f16cache_ld(K) == oracle_ld(K)


def test_dequant_rejects(L):
    d = L.mq_dequant_to_f16
    assert d(5, FAKE, 4, 256, FAKE, 256, None) == _lib.MQ_ERR_FORMAT
    assert d(12, None, 4, 256, FAKE, 256, None) == _lib.MQ_ERR_NULL
    assert d(12, FAKE, 4, 256, None, 256, None) == _lib.MQ_ERR_NULL
    assert d(12, FAKE, 0, 256, FAKE, 256, None) == _lib.MQ_ERR_SHAPE
    assert d(12, FAKE, 4, 100, FAKE, 104, None) == _lib.MQ_ERR_SHAPE
    assert d(8, FAKE, 4, 48, FAKE, 48, None) == _lib.MQ_ERR_SHAPE
    assert d(12, FAKE, 4, 256, FAKE, 255, None) == _lib.MQ_ERR_LD
    assert d(12, FAKE, 4, 256, FAKE, 260, None) == _lib.MQ_ERR_LD
    assert d(12, MIS, 4, 256, FAKE, 256, None) == _lib.MQ_ERR_ALIGN
    assert d(12, FAKE, 4, 256, MIS, 256, None) == _lib.MQ_ERR_ALIGN


def test_gemm_rejects(L):
    g = L.mq_gemm_f16cache
    ok = dict(X=FAKE, ldx=512, W=FAKE, ldw=512, Y=FAKE, ldy=256, M=64, N=256, K=512,
              ws=None, wsb=0, split=1, s=None)

    def call(**kw):
        a = {**ok, **kw}
        return g(a["X"], a["ldx"], a["W"], a["ldw"], a["Y"], a["ldy"], a["M"], a["N"], a["K"],
                 a["ws"], a["wsb"], a["split"], a["s"])

    # each call carries exactly one defect
    assert call(X=None) == _lib.MQ_ERR_NULL
    assert call(Y=None) == _lib.MQ_ERR_NULL
    assert call(M=0) == _lib.MQ_ERR_SHAPE
    assert call(N=-1) == _lib.MQ_ERR_SHAPE
    assert call(K=100, ldx=104, ldw=104) == _lib.MQ_ERR_SHAPE
    assert call(ldx=500) == _lib.MQ_ERR_LD
    assert call(ldw=520 + 4) == _lib.MQ_ERR_LD
    assert call(ldy=255) == _lib.MQ_ERR_LD
    assert call(X=MIS) == _lib.MQ_ERR_ALIGN
    assert call(W=MIS) == _lib.MQ_ERR_ALIGN
    assert call(split=17) == _lib.MQ_ERR_SPLIT
    assert call(split=-1) == _lib.MQ_ERR_SPLIT
    # forced split without workspace
    assert call(split=4) == _lib.MQ_ERR_WORKSPACE
    need = L.mq_gemm_workspace_bytes(0, 64, 256, 512, 4)
    assert need == 4 * 64 * 256 * 4
    assert call(split=4, ws=FAKE, wsb=need - 1) == _lib.MQ_ERR_WORKSPACE
    assert call(split=4, ws=MIS, wsb=need) == _lib.MQ_ERR_WORKSPACE


def test_fused_rejects(L):
    f = L.mq_gemm_fused
    assert f(5, FAKE, 512, FAKE, FAKE, 256, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_FORMAT
    assert f(0, FAKE, 512, FAKE, FAKE, 256, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_FORMAT
    assert f(12, FAKE, 512, None, FAKE, 256, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_NULL
    assert f(12, FAKE, 512, FAKE, FAKE, 256, 64, 256, 480, None, 0, 1, None) == _lib.MQ_ERR_SHAPE
    assert f(8, FAKE, 64, FAKE, FAKE, 256, 64, 256, 48, None, 0, 1, None) == _lib.MQ_ERR_SHAPE
    assert f(12, FAKE, 512, MIS, FAKE, 256, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_ALIGN
    assert f(12, FAKE, 512, FAKE, FAKE, 256, 64, 256, 512, None, 0, 4, None) == _lib.MQ_ERR_WORKSPACE


def test_xf32_entry_points_reject(L):
    """f32 activations: rows 16-byte aligned (ldx a multiple of 4, not 8) and
    at most MQ_MAX_K apart; the other checks as the f16 entry points."""
    c = L.mq_gemm_f16cache_xf32
    f = L.mq_gemm_fused_xf32
    # (X, ldx, W16, ldw, Y, ldy, M, N, K, ws, wsb, split, stream) with one bad value each
    assert c(FAKE, 514, FAKE, 512, FAKE, 256, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_LD
    assert c(FAKE, 504, FAKE, 512, FAKE, 256, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_LD
    assert c(FAKE, (1 << 21) + 4, FAKE, 512, FAKE, 256, 64, 256, 512, None, 0, 1,
             None) == _lib.MQ_ERR_LD
    assert c(None, 512, FAKE, 512, FAKE, 256, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_NULL
    assert c(MIS, 512, FAKE, 512, FAKE, 256, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_ALIGN
    assert c(FAKE, 512, FAKE, 512, FAKE, 256, 64, 256, 512, None, 0, 4, None) == _lib.MQ_ERR_WORKSPACE
    assert f(5, FAKE, 512, FAKE, FAKE, 256, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_FORMAT
    assert f(12, FAKE, 512, FAKE, FAKE, 256, 64, 256, 480, None, 0, 1, None) == _lib.MQ_ERR_SHAPE
    assert f(12, FAKE, 510, FAKE, FAKE, 256, 64, 256, 256, None, 0, 1, None) == _lib.MQ_ERR_LD
    assert f(12, FAKE, 512, FAKE, FAKE, 255, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_LD
    assert f(13, FAKE, 512, FAKE, MIS, 256, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_ALIGN
    assert f(2, FAKE, 512, FAKE, FAKE, 256, 64, 256, 512, None, 0, 17, None) == _lib.MQ_ERR_SPLIT
    v = L.mq_convert_f32_to_f16
    # (X, ldx, X16, ld16, M, K, stream)
    assert v(None, 512, FAKE, 512, 4, 512, None) == _lib.MQ_ERR_NULL
    assert v(FAKE, 512, None, 512, 4, 512, None) == _lib.MQ_ERR_NULL
    assert v(FAKE, 512, FAKE, 512, 0, 512, None) == _lib.MQ_ERR_SHAPE
    assert v(FAKE, 512, FAKE, 512, 4, 12, None) == _lib.MQ_ERR_SHAPE
    assert v(FAKE, 510, FAKE, 512, 4, 504, None) == _lib.MQ_ERR_LD
    assert v(FAKE, 512, FAKE, 508, 4, 504, None) == _lib.MQ_ERR_LD
    assert v(FAKE, 512, FAKE, 500, 4, 504, None) == _lib.MQ_ERR_LD
    assert v(MIS, 512, FAKE, 512, 4, 512, None) == _lib.MQ_ERR_ALIGN
    assert v(FAKE, 512, MIS, 512, 4, 512, None) == _lib.MQ_ERR_ALIGN


def test_mmq_entry_points_reject(L):
    q = L.mq_quantize_q8_1
    # (X, ldx, Xq, ldq, ds, M, K, stream)
    assert q(None, 512, FAKE, 512, FAKE, 4, 512, None) == _lib.MQ_ERR_NULL
    assert q(FAKE, 512, FAKE, 512, None, 4, 512, None) == _lib.MQ_ERR_NULL
    assert q(FAKE, 512, FAKE, 512, FAKE, 4, 496, None) == _lib.MQ_ERR_SHAPE      # K % 32
    assert q(FAKE, 512, FAKE, 512, FAKE, 0, 512, None) == _lib.MQ_ERR_SHAPE
    assert q(FAKE, 510, FAKE, 512, FAKE, 4, 480, None) == _lib.MQ_ERR_LD         # ldx % 4
    assert q(FAKE, 512, FAKE, 520, FAKE, 4, 512, None) == _lib.MQ_ERR_LD         # ldq % 16
    assert q(FAKE, 512, FAKE, 496, FAKE, 4, 512, None) == _lib.MQ_ERR_LD         # ldq < K
    assert q(FAKE, 512, FAKE, 512, MIS, 4, 512, None) == _lib.MQ_ERR_ALIGN
    g = L.mq_gemm_mmq
    # (fmt, Xq, ldq, ds, wq, Y, ldy, M, N, K, ws, wsb, split, stream)
    assert g(5, FAKE, 512, FAKE, FAKE, FAKE, 256, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_FORMAT
    assert g(0, FAKE, 512, FAKE, FAKE, FAKE, 256, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_FORMAT
    assert g(12, FAKE, 512, None, FAKE, FAKE, 256, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_NULL
    assert g(12, FAKE, 512, FAKE, FAKE, FAKE, 256, 64, 256, 480, None, 0, 1, None) == _lib.MQ_ERR_SHAPE
    assert g(8, FAKE, 512, FAKE, FAKE, FAKE, 256, 64, 256, 48, None, 0, 1, None) == _lib.MQ_ERR_SHAPE
    assert g(8, FAKE, 520, FAKE, FAKE, FAKE, 256, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_LD
    assert g(8, FAKE, 512, FAKE, FAKE, FAKE, 255, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_LD
    assert g(14, FAKE, 512, FAKE, MIS, FAKE, 256, 64, 256, 512, None, 0, 1, None) == _lib.MQ_ERR_ALIGN
    assert g(14, FAKE, 512, FAKE, FAKE, FAKE, 256, 64, 256, 512, None, 0, 17, None) == _lib.MQ_ERR_SPLIT
    assert g(14, FAKE, 512, FAKE, FAKE, FAKE, 256, 64, 256, 512, None, 0, 4, None) == _lib.MQ_ERR_WORKSPACE
    w = L.mq_gemm_mmq_workspace_bytes
    # 128 x 128 tiles, 128-wide k-steps: a forced split of 4 over 4 steps
    assert w(14, 64, 256, 512, 4) == 4 * 2 * 128 * 128 * 4
    assert w(12, 2048, 4096, 4096, 0) == 0                 # 512 tiles: two whole rounds
    # 16 x 33 = 528 tiles: 2 rounds + 16 tiles split min(16, 256/16, 32/2) = 16 ways
    assert w(12, 2048, 4224, 4096, 0) == 16 * 16 * 128 * 128 * 4
    assert w(99, 64, 128, 128, 1) == _lib.MQ_ERR_FORMAT


def test_dequant_batch_rejects(L):
    J = _lib.MqDequantJob
    ok = J(12, 64, 256, 256, FAKE, FAKE)
    f = L.mq_dequant_to_f16_batch
    assert f(None, 0, None) == _lib.MQ_OK            # empty batch: no-op
    assert f(None, 2, None) == _lib.MQ_ERR_NULL
    assert f((J * 1)(ok), -1, None) == _lib.MQ_ERR_SHAPE
    # the first invalid job's code is returned and nothing is launched (a
    # launch without a GPU would report MQ_ERR_HIP instead)
    for bad, code in ((J(5, 64, 256, 256, FAKE, FAKE), _lib.MQ_ERR_FORMAT),
                      (J(12, 64, 100, 256, FAKE, FAKE), _lib.MQ_ERR_SHAPE),
                      (J(12, 64, 256, 200, FAKE, FAKE), _lib.MQ_ERR_LD),
                      (J(12, 64, 256, 256, MIS, FAKE), _lib.MQ_ERR_ALIGN),
                      (J(14, 64, 256, 256, FAKE, None), _lib.MQ_ERR_NULL),
                      (J(8, 0, 32, 32, FAKE, FAKE), _lib.MQ_ERR_SHAPE)):
        arr = (J * 3)(ok, ok, bad)
        assert f(arr, 3, None) == code


def test_workspace_planning(L):
    # k/v projection at M=2048 underfills 256 CUs with 256x128 tiles -> split:
    # the cache GEMM takes 64-row tiles (128 of them, split 2 ways), the fused
    # one 128-row tiles (64, split 4 ways: each weight decoded 16 times, not 32)
    assert L.mq_gemm_workspace_bytes(0, 2048, 512, 3584, 0) == 2 * 128 * 64 * 128 * 4
    for fmt in (8, 12, 14):
        assert L.mq_gemm_workspace_bytes(fmt, 2048, 512, 3584, 0) == 4 * 64 * 128 * 128 * 4
    # with fewer than 64 tiles of 128 rows the fused GEMM keeps 64-row tiles
    assert L.mq_gemm_workspace_bytes(12, 1024, 512, 3584, 0) == \
        L.mq_gemm_workspace_bytes(0, 1024, 512, 3584, 0)
    # gate/up: 8 x 74 tiles of 256 x 256 = two full rounds of 256 plus 80 tiles,
    # which are split 256 // 80 = 3 ways along K
    assert L.mq_gemm_workspace_bytes(0, 2048, 18944, 3584, 0) == 3 * 80 * 256 * 256 * 4
    # every fused weight format takes the same 256 x 256 tiles (same plan);
    # Q6_K's 3-way split of 56 steps is 20, 20, 16 (ranges start even)
    for fmt in (2, 6, 7, 8, 12, 13, 14):
        assert L.mq_gemm_workspace_bytes(fmt, 2048, 18944, 3584, 0) == 3 * 80 * 256 * 256 * 4
    # the Q4_K 256 x 256 kernel stages whole super-blocks: its K ranges are
    # multiples of 4 k-steps, so a requested 7-way split of 20 steps becomes
    # 5 ranges of 4.  The Q8_0 one (K a multiple of 256) pairs k-steps: 7
    # ranges of 3 become 5 of 4 (ranges start even); with K = 1056 (17 steps)
    # Q8_0 keeps the 2 x 2 kernel and 6 ranges of 3, the last of 2
    assert L.mq_gemm_workspace_bytes(12, 300, 32768, 1280, 7) == 5 * 256 * 256 * 256 * 4
    assert L.mq_gemm_workspace_bytes(8, 300, 32768, 1280, 7) == 5 * 256 * 256 * 256 * 4
    assert L.mq_gemm_workspace_bytes(8, 300, 32768, 1056, 7) == 6 * 256 * 256 * 256 * 4
    # Q5_K takes the Q4_K kernel (ranges of whole super-blocks); Q4_0, Q5_0
    # and Q5_1 the Q8_0 one (even starts): 20 steps forced 7 ways -> 5 of 4
    for fmt in (2, 6, 7, 13):
        assert L.mq_gemm_workspace_bytes(fmt, 300, 32768, 1280, 7) == 5 * 256 * 256 * 256 * 4
    # 32 steps forced 3 ways: 11-step ranges become 12 (even) or 12 (whole
    # super-blocks); 3 ranges either way
    for fmt in (2, 8, 13):
        assert L.mq_gemm_workspace_bytes(fmt, 300, 32768, 2048, 3) == 3 * 256 * 256 * 256 * 4
    assert L.mq_gemm_workspace_bytes(12, 300, 32768, 1280, 3) == 3 * 256 * 256 * 256 * 4
    # 4096 x 14336 at M = 1024: 64 tiles of 256 x 256 split 4 ways (ranges of
    # 3584 k fill the compute units); at M = 512 the ranges would be 1792 k, so
    # the plan keeps 256 x 128 tiles (64 of them, split 4 ways)
    assert L.mq_gemm_workspace_bytes(0, 1024, 4096, 14336, 0) == 4 * 64 * 256 * 256 * 4
    assert L.mq_gemm_workspace_bytes(0, 512, 4096, 14336, 0) == 4 * 64 * 256 * 128 * 4
    # more than 3/4 of a round of 256 x 256 tiles: unsplit, no workspace
    assert L.mq_gemm_workspace_bytes(0, 1024, 14336, 4096, 0) == 0
    # q/o: 224 tiles of 256 x 128, one partial round that a split cannot double
    assert L.mq_gemm_workspace_bytes(0, 2048, 3584, 3584, 0) == 0
    assert L.mq_gemm_workspace_bytes(0, 64, 512, 512, 1) == 0
    # forced splits are clamped to the number of 64-wide k-steps
    assert L.mq_gemm_workspace_bytes(0, 64, 128, 128, 16) == 2 * 64 * 128 * 4
    assert L.mq_gemm_workspace_bytes(99, 64, 128, 128, 1) == _lib.MQ_ERR_FORMAT
    # f32 activations, M > 64: X rounded once into the front of the workspace
    # (2048 rows of 3584 halves, already a multiple of 256 bytes), then the
    # f16-activation plan with its split planes behind it
    x16 = 2048 * 3584 * 2
    for fmt in (0, 2, 12, 13, 14):
        assert L.mq_gemm_xf32_workspace_bytes(fmt, 2048, 18944, 3584, 0) == x16 + 3 * 80 * 256 * 256 * 4
    assert L.mq_gemm_xf32_workspace_bytes(12, 2048, 512, 3584, 0) == \
        x16 + L.mq_gemm_workspace_bytes(12, 2048, 512, 3584, 0)
    # padded row stride for the converted X when 2K bytes is a multiple of 2048;
    # 65 rows of 4160 halves = 540800 bytes, rounded up to 540928
    assert L.mq_gemm_xf32_workspace_bytes(0, 65, 4096, 4096, 1) == 540928
    # M <= 64: in-tile conversion, own tiles (64 x 128), split planes only
    assert L.mq_gemm_xf32_workspace_bytes(0, 64, 128, 128, 16) == 2 * 64 * 128 * 4
    assert L.mq_gemm_xf32_workspace_bytes(12, 64, 4096, 4096, 1) == 0
    assert L.mq_gemm_xf32_workspace_bytes(99, 64, 128, 128, 1) == _lib.MQ_ERR_FORMAT


def test_strerror_total(L):
    for code in range(-9, 1):
        assert isinstance(L.mq_strerror(code), bytes)
    assert L.mq_last_hip_error() == 0


def test_binding_errors_are_raised():
    with pytest.raises(mq.MQError) as e:
        _lib.check(_lib.MQ_ERR_LD, "x")
    assert e.value.code == _lib.MQ_ERR_LD
    assert mq.cache_ld(4096) == 4160 and mq.row_bytes("q6_k", 18944) == 15540
