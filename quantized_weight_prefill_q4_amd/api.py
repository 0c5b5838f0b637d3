"""Torch-tensor front end of libmq (argument marshalling only).

Each function takes device tensors, allocates its outputs (and the split-K
workspace) with torch on the tensors' device, and calls the C ABI on torch's
current stream.  Every step of the computation runs in the HIP library; these
wrappers only check dtypes/devices/strides and pass pointers.
"""

from __future__ import annotations

import ctypes
import functools

import torch

from ._lib import (MQ_Q4_0, MQ_Q4_K, MQ_Q5_0, MQ_Q5_1, MQ_Q5_K, MQ_Q6_K, MQ_Q8_0,
                   MqDequantJob, MqGemmPlanInfo, check, lib)

FORMATS = {"q4_0": MQ_Q4_0, "q5_0": MQ_Q5_0, "q5_1": MQ_Q5_1, "q8_0": MQ_Q8_0,
           "q4_k": MQ_Q4_K, "q5_k": MQ_Q5_K, "q6_k": MQ_Q6_K}


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        return FORMATS[fmt.lower()]
    return int(fmt)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need_cuda(t: torch.Tensor, name: str, dtype: torch.dtype) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _row_major_2d(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return t.stride(0)


# The C ABI sees plain pointers; the sizes it cannot check are checked here,
# so that a wrong argument is an exception rather than an access out of bounds.
def _need_shape(t: torch.Tensor, rows: int, cols: int, name: str) -> None:
    if t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{name} must be at least {rows} x {cols}, got {tuple(t.shape)}")


def _need_span(t: torch.Tensor, elems: int, name: str) -> None:
    """t's storage holds `elems` elements from t's first one (rows written at
    the full row stride, e.g. a cache's pad columns)."""
    if t.is_contiguous() and t.numel() >= elems:   # its own elements suffice
        return
    have = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
    if have < elems:
        raise ValueError(f"{name} spans {have} elements, {elems} needed")


# The library's host-only answers (format tables, the stride rule, workspace
# sizes) depend on their arguments alone: each is asked once per argument
# tuple, so a call's checks make no extra round trip into the library.
@functools.lru_cache(maxsize=4096)
def _row_bytes(f: int, K: int) -> int:
    return check(lib().mq_row_bytes(f, K), "mq_row_bytes")


@functools.lru_cache(maxsize=1024)
def _cache_ld(K: int) -> int:
    return check(lib().mq_f16cache_ld(K), "mq_f16cache_ld")


@functools.lru_cache(maxsize=4096)
def _workspace_bytes(f: int, M: int, N: int, K: int, split_k: int, x_f32: bool) -> int:
    fn = "mq_gemm_xf32_workspace_bytes" if x_f32 else "mq_gemm_workspace_bytes"
    return check(getattr(lib(), fn)(f, M, N, K, split_k), fn)


def _need_quant(wq: torch.Tensor, f: int, N: int, K: int) -> None:
    _need_cuda(wq, "wq", torch.uint8)
    if not wq.is_contiguous():
        raise ValueError("wq must be contiguous")
    need = N * _row_bytes(f, K)
    if wq.numel() < need:
        raise ValueError(f"wq holds {wq.numel()} bytes; {N} rows of K = {K} need {need}")


def block_elems(fmt) -> int:
    return check(lib().mq_block_elems(_fmt(fmt)), "mq_block_elems")


def block_bytes(fmt) -> int:
    return check(lib().mq_block_bytes(_fmt(fmt)), "mq_block_bytes")


def row_bytes(fmt, K: int) -> int:
    return _row_bytes(_fmt(fmt), int(K))


def cache_ld(K: int) -> int:
    return _cache_ld(int(K))


def workspace_bytes(fmt, M: int, N: int, K: int, split_k: int = 0, x_f32: bool = False) -> int:
    """Workspace bytes of a GEMM (fmt 0 / "f16": the f16 cache); x_f32 for f32
    activations."""
    f = 0 if fmt in (0, None, "f16") else _fmt(fmt)
    return _workspace_bytes(f, int(M), int(N), int(K), int(split_k), bool(x_f32))


def gemm_plan(fmt, M: int, N: int, K: int, split_k: int = 0, path: str = "f16") -> dict:
    """The launch plan of a GEMM call (host only): path "f16" for
    gemm_f16cache / gemm_fused (fmt 0 / "f16" = the cache), "f32" for their
    f32-activation variants, "mmq" for gemm_mmq."""
    f = 0 if fmt in (0, None, "f16") else _fmt(fmt)
    p = {"f16": 0, "f32": 1, "mmq": 2}[path]
    info = MqGemmPlanInfo()
    check(lib().mq_gemm_plan_query(p, f, M, N, K, split_k, ctypes.byref(info)),
          "mq_gemm_plan_query")
    return {name: getattr(info, name) for name, _ in MqGemmPlanInfo._fields_}


def dequant_to_f16(wq: torch.Tensor, fmt, N: int, K: int, pad: bool = True,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """Decode a quantized N×K weight (uint8, rows contiguous) into an f16 cache
    [N, ld]; ld = cache_ld(K) when pad else K.  Use ``[:, :K]`` for the matrix."""
    f = _fmt(fmt)
    _need_quant(wq, f, N, K)
    ld = cache_ld(K) if pad else K
    if out is None:
        out = torch.empty((N, ld), dtype=torch.float16, device=wq.device)
    else:
        _need_cuda(out, "out", torch.float16)
        ld = _row_major_2d(out, "out")
        _need_shape(out, N, K, "out")
        _need_span(out, N * ld, "out")
    check(lib().mq_dequant_to_f16(f, wq.data_ptr(), N, K, out.data_ptr(), ld, _stream(wq)),
          "mq_dequant_to_f16")
    return out


def dequant_to_f16_batch(jobs, pad: bool = True) -> list[torch.Tensor]:
    """Decode several weights with one library call (launches of up to 16
    jobs each).  ``jobs``: iterable of ``(wq, fmt, N, K)`` or ``(wq, fmt, N, K,
    out)``; returns the caches in order, each as ``dequant_to_f16`` would."""
    jobs = list(jobs)
    arr = (MqDequantJob * max(1, len(jobs)))()
    outs = []
    stream = None
    for i, job in enumerate(jobs):
        wq, fmt, N, K = job[:4]
        out = job[4] if len(job) > 4 else None
        _need_quant(wq, _fmt(fmt), N, K)
        ld = cache_ld(K) if pad else K
        if out is None:
            out = torch.empty((N, ld), dtype=torch.float16, device=wq.device)
        else:
            _need_cuda(out, "out", torch.float16)
            ld = _row_major_2d(out, "out")
            _need_shape(out, N, K, "out")
            _need_span(out, N * ld, "out")
        if stream is None:
            stream = _stream(wq)
        arr[i] = MqDequantJob(_fmt(fmt), N, K, ld, wq.data_ptr(), out.data_ptr())
        outs.append(out)
    check(lib().mq_dequant_to_f16_batch(arr, len(jobs), stream), "mq_dequant_to_f16_batch")
    return outs


def _workspace(fmt_code: int, M: int, N: int, K: int, split_k: int, device,
               x_f32: bool = False) -> torch.Tensor | None:
    nbytes = workspace_bytes(fmt_code, M, N, K, split_k, x_f32)
    if nbytes == 0:
        return None
    return torch.empty(nbytes // 4, dtype=torch.float32, device=device)


def _x_kind(x: torch.Tensor) -> bool:
    """True for f32 activations (the _xf32 entry points), False for f16."""
    if x.dtype == torch.float32:
        _need_cuda(x, "x", torch.float32)
        return True
    _need_cuda(x, "x", torch.float16)
    return False


def gemm_f16cache(x: torch.Tensor, w16: torch.Tensor, K: int | None = None, split_k: int = 0,
                  out: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    """Y[M, N] (f32) = x[:, :K] @ w16[:, :K]^T with x [M, >=K] (f16, or f32
    rounded to f16 inside the kernel), w16 the f16 cache [N, ld]."""
    xf32 = _x_kind(x)
    _need_cuda(w16, "w16", torch.float16)
    ldx = _row_major_2d(x, "x")
    ldw = _row_major_2d(w16, "w16")
    M, N = x.shape[0], w16.shape[0]
    K = x.shape[1] if K is None else K
    _need_shape(x, M, K, "x")
    _need_shape(w16, N, K, "w16")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    else:
        _need_cuda(out, "out", torch.float32)
    ldy = _row_major_2d(out, "out")
    _need_shape(out, M, N, "out")
    if ws is None:
        ws = _workspace(0, M, N, K, split_k, x.device, xf32)
    fn = "mq_gemm_f16cache_xf32" if xf32 else "mq_gemm_f16cache"
    check(getattr(lib(), fn)(x.data_ptr(), ldx, w16.data_ptr(), ldw, out.data_ptr(), ldy,
                             M, N, K, 0 if ws is None else ws.data_ptr(),
                             0 if ws is None else ws.numel() * ws.element_size(),
                             split_k, _stream(x)), fn)
    return out


def gemm_fused(x: torch.Tensor, wq: torch.Tensor, fmt, N: int, K: int | None = None,
               split_k: int = 0, out: torch.Tensor | None = None,
               ws: torch.Tensor | None = None) -> torch.Tensor:
    """Y[M, N] (f32) = x[:, :K] @ dequant(wq)^T, expanding the quantized weight
    in-kernel; x f16, or f32 rounded to f16 inside the kernel."""
    f = _fmt(fmt)
    xf32 = _x_kind(x)
    ldx = _row_major_2d(x, "x")
    M = x.shape[0]
    K = x.shape[1] if K is None else K
    _need_shape(x, M, K, "x")
    _need_quant(wq, f, N, K)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    else:
        _need_cuda(out, "out", torch.float32)
    ldy = _row_major_2d(out, "out")
    _need_shape(out, M, N, "out")
    if ws is None:
        ws = _workspace(f, M, N, K, split_k, x.device, xf32)
    fn = "mq_gemm_fused_xf32" if xf32 else "mq_gemm_fused"
    check(getattr(lib(), fn)(f, x.data_ptr(), ldx, wq.data_ptr(), out.data_ptr(), ldy, M, N, K,
                             0 if ws is None else ws.data_ptr(),
                             0 if ws is None else ws.numel() * ws.element_size(),
                             split_k, _stream(x)), fn)
    return out


def convert_f32_to_f16(x: torch.Tensor, K: int | None = None,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """f16 copy (round to nearest even) of the f32 activations x[:, :K]."""
    _need_cuda(x, "x", torch.float32)
    ldx = _row_major_2d(x, "x")
    M = x.shape[0]
    K = x.shape[1] if K is None else K
    _need_shape(x, M, K, "x")
    if out is None:
        out = torch.empty((M, K), dtype=torch.float16, device=x.device)
    else:
        _need_cuda(out, "out", torch.float16)
    ld16 = _row_major_2d(out, "out")
    _need_shape(out, M, K, "out")
    check(lib().mq_convert_f32_to_f16(x.data_ptr(), ldx, out.data_ptr(), ld16, M, K, _stream(x)),
          "mq_convert_f32_to_f16")
    return out


def quantize_q8_1(x: torch.Tensor, K: int | None = None, xq: torch.Tensor | None = None,
                  ds: torch.Tensor | None = None):
    """Q8_1-style int8 blocks of the f32 activations x[:, :K]: (codes int8
    [M, ldq], factors f32 [M, K/32, 2] = (d, s) per 32-element block)."""
    _need_cuda(x, "x", torch.float32)
    ldx = _row_major_2d(x, "x")
    M = x.shape[0]
    K = x.shape[1] if K is None else K
    _need_shape(x, M, K, "x")
    if xq is None:
        xq = torch.empty((M, (K + 15) // 16 * 16), dtype=torch.int8, device=x.device)
    else:
        _need_cuda(xq, "xq", torch.int8)
    ldq = _row_major_2d(xq, "xq")
    _need_shape(xq, M, K, "xq")
    if ds is None:
        ds = torch.empty((M, K // 32, 2), dtype=torch.float32, device=x.device)
    else:
        _need_cuda(ds, "ds", torch.float32)
        if not ds.is_contiguous() or ds.numel() < M * (K // 32) * 2:
            raise ValueError("ds must be contiguous with M*K/16 floats")
    check(lib().mq_quantize_q8_1(x.data_ptr(), ldx, xq.data_ptr(), ldq, ds.data_ptr(), M, K,
                                 _stream(x)), "mq_quantize_q8_1")
    return xq, ds


def mmq_workspace_bytes(fmt, M: int, N: int, K: int, split_k: int = 0) -> int:
    return check(lib().mq_gemm_mmq_workspace_bytes(_fmt(fmt), M, N, K, split_k),
                 "mq_gemm_mmq_workspace_bytes")


def gemm_mmq(xq: torch.Tensor, ds: torch.Tensor, wq: torch.Tensor, fmt, N: int, K: int,
             split_k: int = 0, out: torch.Tensor | None = None,
             ws: torch.Tensor | None = None) -> torch.Tensor:
    """Y[M, N] (f32): the int8 product of quantize_q8_1's (xq, ds) and the
    quantized weight wq (rows contiguous)."""
    f = _fmt(fmt)
    _need_cuda(xq, "xq", torch.int8)
    _need_cuda(ds, "ds", torch.float32)
    _need_quant(wq, f, N, K)
    if not ds.is_contiguous():
        raise ValueError("ds must be contiguous")
    ldq = _row_major_2d(xq, "xq")
    M = xq.shape[0]
    _need_shape(xq, M, K, "xq")
    if ds.numel() < M * (K // 32) * 2:
        raise ValueError(f"ds holds {ds.numel()} floats; {M * (K // 32) * 2} needed")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    else:
        _need_cuda(out, "out", torch.float32)
    ldy = _row_major_2d(out, "out")
    _need_shape(out, M, N, "out")
    if ws is None:
        nbytes = mmq_workspace_bytes(f, M, N, K, split_k)
        ws = torch.empty(nbytes // 4, dtype=torch.float32, device=xq.device) if nbytes else None
    check(lib().mq_gemm_mmq(f, xq.data_ptr(), ldq, ds.data_ptr(), wq.data_ptr(), out.data_ptr(),
                            ldy, M, N, K, 0 if ws is None else ws.data_ptr(),
                            0 if ws is None else ws.numel() * ws.element_size(), split_k,
                            _stream(xq)), "mq_gemm_mmq")
    return out
