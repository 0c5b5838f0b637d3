// The prefill GEMM with f32 activations (Fucina "Eager GPU Offload Without A
// Compute Graph", quantized linears: the callers hold f32 activations, which
// the kernel rounds to f16 while staging the operand tile), and the
// standalone f32 → f16 activation conversion it saves (llama.cpp PR #57,
// batch-size dependence: the separate activation convert is part of what the
// f16 path pays at small M).  Kernels: gemm_kernel.h with XF32 = true.

#include "gemm_kernel.h"

namespace mq {
namespace {

// Chunks of 8 consecutive elements of a row, numbered row-major over
// M × K/8, dealt grid-stride to the threads: per chunk two 16-byte loads and
// one 16-byte store.
__global__ __launch_bounds__(256) void convert_f32_to_f16(const float *__restrict__ X, int ldx,
                                                          uint16_t *__restrict__ X16, int ld16,
                                                          int64_t chunks, int chunks_per_row) {
    for (int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x; id < chunks;
         id += (int64_t)gridDim.x * 256) {
        const int64_t row = id / chunks_per_row;
        const int c = (int)(id - row * chunks_per_row);
        const f32x4 *src = reinterpret_cast<const f32x4 *>(X + row * ldx + 8 * c);
        const f32x4 a = src[0], b = src[1];
        *reinterpret_cast<u32x4 *>(X16 + row * ld16 + 8 * c) =
            u32x4{pack_f16x2(a.x, a.y), pack_f16x2(a.z, a.w), pack_f16x2(b.x, b.y),
                  pack_f16x2(b.z, b.w)};
    }
}

}  // namespace

hipError_t launch_gemm_xf32(int fmt, const float *X, int ldx, const void *W, int64_t ldw,
                            float *Y, int ldy, int M, int N, int K, const GemmPlan &plan,
                            float *ws, hipStream_t stream, bool dry) {
    return launch_gemm_t<true>(fmt, X, ldx, W, ldw, Y, ldy, M, N, K, plan, ws, stream, dry);
}

hipError_t launch_convert_f32_to_f16(const float *X, int ldx, uint16_t *X16, int ld16, int M,
                                     int K, hipStream_t stream) {
    const int cpr = K / 8;
    const int64_t chunks = (int64_t)M * cpr;
    int64_t blocks = (chunks + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;   // grid-stride beyond 2^28 chunks
    hipLaunchKernelGGL(convert_f32_to_f16, dim3((unsigned)blocks), dim3(256), 0, stream, X, ldx,
                       X16, ld16, chunks, cpr);
    return hipGetLastError();
}

}  // namespace mq
