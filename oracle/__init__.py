"""CPU oracle for the quantized-weight prefill matmul — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP
library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
the GPU library (``quantized_weight_prefill_q4_amd``) and imports nothing from
it; the product path never calls it.

What it computes (sources are the four pages the method is described on):

* ``dequant_ref`` — decode of GGUF Q4_K / Q6_K / Q8_0 (and Q4_0 / Q5_0 / Q5_1
  / Q5_K) blocks into f16 bit patterns.  minfer "05 · 8p — Persistent f16 weight cache + fused
  dequant-in-GEMM", §2 Principle and §3.2 (third site): weights are decoded in
  f32 and rounded once to f16 per element, the same path for the standalone
  dequant and for the fused kernel.
* ``cache_ref`` — that decode placed in a row stride padded by one 128-byte
  line when the f16 row size is a multiple of 2048 bytes (llama.cpp PR #57
  "GEMM weight row padding + one-time K-padded f16 dequant for prefill",
  Summary, second bullet).
* ``gemm_ref`` — Y = X·Wᵀ over the f16 operands, evaluated exactly in f64,
  plus S = |X|·|W|ᵀ for the per-element tolerance 1e-3·S + 1e-5.
* ``mmq`` — the int8 product's own numerics (Fucina "Eager GPU Offload
  Without A Compute Graph", the ik_llama.cpp audit: Q8_1-style activation
  blocks, signed-int8 weights, int8 matrix instructions): ``quantize_q8_1``,
  ``decompose`` (w = α·c − β per format), ``mmq_ref``.
* ``activations_to_f16`` — f32 activations rounded once to f16 (Fucina "Eager
  GPU Offload Without A Compute Graph", quantized linears: f32 activations
  converted to half as the operand tile is staged); the f32-activation GEMM
  is ``gemm_ref`` on that.

Every function is pinned by ``-m "not gpu"`` tests against hand-derived
worked vectors, closed forms, an independent field-wise encoder, exact
rational arithmetic and brute force.
"""

from .f16 import f16_bits_to_float, f32_to_f16_bits, f64_to_f32
from .formats import (
    BLOCK_BYTES,
    BLOCK_ELEMS,
    Q4_0,
    Q4_K,
    Q5_0,
    Q5_1,
    Q5_K,
    Q6_K,
    Q8_0,
    cache_ld,
    cache_ref,
    dequant_ref,
    dequant_scalar,
    q4k_scale_min,
    row_bytes,
)
from . import mmq
from .gemm import (activations_to_f16, activations_to_f16_scalar, gemm_bruteforce, gemm_ref,
                   within_tolerance)

__all__ = [
    "mmq",
    "activations_to_f16",
    "activations_to_f16_scalar",
    "BLOCK_BYTES",
    "BLOCK_ELEMS",
    "Q4_0",
    "Q4_K",
    "Q5_0",
    "Q5_1",
    "Q5_K",
    "Q6_K",
    "Q8_0",
    "cache_ld",
    "cache_ref",
    "dequant_ref",
    "dequant_scalar",
    "f16_bits_to_float",
    "f32_to_f16_bits",
    "f64_to_f32",
    "gemm_bruteforce",
    "gemm_ref",
    "q4k_scale_min",
    "row_bytes",
    "within_tolerance",
]
