"""ctypes loader for libmq.so (the HIP library).  No fallback: if the library
is missing or does not load, every call raises."""

from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmq.so")

# return codes (include/mq.h)
MQ_OK = 0
MQ_ERR_NULL = -1
MQ_ERR_FORMAT = -2
MQ_ERR_SHAPE = -3
MQ_ERR_LD = -4
MQ_ERR_ALIGN = -5
MQ_ERR_WORKSPACE = -6
MQ_ERR_SPLIT = -7
MQ_ERR_HIP = -8
MQ_ERR_SCRATCH = -9
MQ_NOALLOC_SCRATCH_BYTES = 64 << 20

MQ_Q4_0 = 2
MQ_Q5_0 = 6
MQ_Q5_1 = 7
MQ_Q8_0 = 8
MQ_Q4_K = 12
MQ_Q5_K = 13
MQ_Q6_K = 14

_c_int, _c_i64, _c_size, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p



class MqDequantJob(ctypes.Structure):
    """struct mq_dequant_job of include/mq.h."""
    _fields_ = [("fmt", _c_int), ("N", _c_int), ("K", _c_int), ("ld", _c_int),
                ("wq", _vp), ("w16", _vp)]


class MqGemmPlanInfo(ctypes.Structure):
    """struct mq_gemm_plan_info of include/mq.h."""
    _fields_ = [("bm", _c_int), ("bn", _c_int), ("tiles_m", _c_int), ("tiles_n", _c_int),
                ("k_steps", _c_int), ("dp_tiles", _c_int), ("tail_tiles", _c_int),
                ("split", _c_int), ("steps_per_split", _c_int), ("has_kernel", _c_int),
                ("ws_bytes", _c_i64)]


# name -> (restype, argtypes); mirrors include/mq.h
SIGNATURES = {
    "mq_block_elems": (_c_int, [_c_int]),
    "mq_block_bytes": (_c_int, [_c_int]),
    "mq_row_bytes": (_c_i64, [_c_int, _c_i64]),
    "mq_f16cache_ld": (_c_i64, [_c_i64]),
    "mq_dequant_to_f16": (_c_int, [_c_int, _vp, _c_int, _c_int, _vp, _c_int, _vp]),
    "mq_dequant_to_f16_batch": (_c_int, [ctypes.POINTER(MqDequantJob), _c_int, _vp]),
    "mq_gemm_workspace_bytes": (_c_i64, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "mq_gemm_f16cache": (_c_int, [_vp, _c_int, _vp, _c_int, _vp, _c_int, _c_int, _c_int, _c_int,
                                  _vp, _c_size, _c_int, _vp]),
    "mq_gemm_fused": (_c_int, [_c_int, _vp, _c_int, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                               _vp, _c_size, _c_int, _vp]),
    "mq_gemm_fused_noalloc": (_c_int, [_c_int, _vp, _c_int, _vp, _vp, _c_int, _c_int, _c_int,
                                       _c_int, _c_int, _vp]),
    "mq_gemm_xf32_workspace_bytes": (_c_i64, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "mq_gemm_f16cache_xf32": (_c_int, [_vp, _c_int, _vp, _c_int, _vp, _c_int, _c_int, _c_int,
                                       _c_int, _vp, _c_size, _c_int, _vp]),
    "mq_gemm_fused_xf32": (_c_int, [_c_int, _vp, _c_int, _vp, _vp, _c_int, _c_int, _c_int,
                                    _c_int, _vp, _c_size, _c_int, _vp]),
    "mq_convert_f32_to_f16": (_c_int, [_vp, _c_int, _vp, _c_int, _c_int, _c_int, _vp]),
    "mq_quantize_q8_1": (_c_int, [_vp, _c_int, _vp, _c_int, _vp, _c_int, _c_int, _vp]),
    "mq_gemm_mmq_workspace_bytes": (_c_i64, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "mq_gemm_mmq": (_c_int, [_c_int, _vp, _c_int, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                             _vp, _c_size, _c_int, _vp]),
    "mq_gemm_plan_query": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    ctypes.POINTER(MqGemmPlanInfo)]),
    "mq_strerror": (ctypes.c_char_p, [_c_int]),
    "mq_last_hip_error": (_c_int, []),
}


class MQError(RuntimeError):
    """A libmq call returned a negative status."""

    def __init__(self, code: int, where: str):
        self.code = code
        msg = lib().mq_strerror(code).decode()
        if code == MQ_ERR_HIP:
            msg += f" (hipError {lib().mq_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{code}]")


_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m quantized_weight_prefill_q4_amd.build`")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def check(rc: int, where: str) -> int:
    if rc < 0:
        raise MQError(rc, where)
    return rc
