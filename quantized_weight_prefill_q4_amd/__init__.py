"""Prefill matmul over GGUF block-quantized weights (Q4_K, Q6_K, Q8_0, Q4_0,
Q5_0, Q5_1, Q5_K) for AMD MI355X: a load-time f16 cache with an MFMA GEMM, and
a fused dequant-in-GEMM.

The computation lives in the HIP library ``libmq.so`` (C ABI in
``include/mq.h``); this package only marshals torch tensors into it.
"""

from ._lib import (
    LIB_PATH,
    MQ_Q4_0,
    MQ_Q4_K,
    MQ_Q5_0,
    MQ_Q5_1,
    MQ_Q5_K,
    MQ_Q6_K,
    MQ_Q8_0,
    MQError,
    lib,
)
from .api import (
    FORMATS,
    block_bytes,
    block_elems,
    cache_ld,
    convert_f32_to_f16,
    dequant_to_f16,
    dequant_to_f16_batch,
    gemm_f16cache,
    gemm_fused,
    gemm_mmq,
    gemm_plan,
    mmq_workspace_bytes,
    quantize_q8_1,
    row_bytes,
    workspace_bytes,
)

__all__ = [
    "FORMATS",
    "LIB_PATH",
    "MQ_Q4_0",
    "MQ_Q4_K",
    "MQ_Q5_0",
    "MQ_Q5_1",
    "MQ_Q5_K",
    "MQ_Q6_K",
    "MQ_Q8_0",
    "MQError",
    "block_bytes",
    "block_elems",
    "cache_ld",
    "convert_f32_to_f16",
    "dequant_to_f16",
    "dequant_to_f16_batch",
    "gemm_f16cache",
    "gemm_fused",
    "gemm_mmq",
    "gemm_plan",
    "lib",
    "mmq_workspace_bytes",
    "quantize_q8_1",
    "row_bytes",
    "workspace_bytes",
]
