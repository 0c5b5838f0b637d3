// Host-side interface between the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

constexpr int kFmtF16 = 0;  // the f16-cache operand of the GEMM
constexpr int kFmtQ4_0 = 2;
constexpr int kFmtQ5_0 = 6;
constexpr int kFmtQ5_1 = 7;
constexpr int kFmtQ8_0 = 8;
constexpr int kFmtQ4_K = 12;
constexpr int kFmtQ5_K = 13;
constexpr int kFmtQ6_K = 14;

inline int block_elems(int fmt) {
    switch (fmt) {
    case kFmtQ4_0: case kFmtQ5_0: case kFmtQ5_1: case kFmtQ8_0: return 32;
    case kFmtQ4_K: case kFmtQ5_K: case kFmtQ6_K: return 256;
    default: return -1;
    }
}
inline int block_bytes(int fmt) {
    switch (fmt) {
    case kFmtQ4_0: return 18;
    case kFmtQ5_0: return 22;
    case kFmtQ5_1: return 24;
    case kFmtQ8_0: return 34;
    case kFmtQ4_K: return 144;
    case kFmtQ5_K: return 176;
    case kFmtQ6_K: return 210;
    default: return -1;
    }
}

// Decode launcher (arguments already validated).
hipError_t launch_dequant(int fmt, const void *wq, int N, int K, uint16_t *w16, int ld,
                          hipStream_t stream);

// One decode of a batch (arguments already validated).
struct DequantSpec {
    int fmt, N, K, ld;
    const void *wq;
    uint16_t *w16;
};
// Decodes specs[0..n) in launches of up to 16 jobs, in order, on `stream`.
hipError_t launch_dequant_batch(const DequantSpec *specs, int n, hipStream_t stream);

// Launch shape of one GEMM.  Tiles are numbered in raster order; the first
// dp_tiles run over all of K and write Y directly, the remaining tail_tiles
// are each split into `split` K ranges whose f32 partial tiles go to the
// workspace and are summed in a fixed order by a second kernel.
struct GemmPlan {
    int bm, bn;             // block tile (M rows of X, N rows of W)
    int tiles_m, tiles_n;
    int k_steps;            // ceil(K / 64)
    int dp_tiles;           // tiles computed over the whole K
    int tail_tiles;         // tiles split along K (0 when split == 1)
    int split;              // K ranges per tail tile (>= 1)
    int steps_per_split;    // k-steps per range
    int64_t ws_bytes;       // split · tail_tiles · bm · bn · 4, or 0
};

// split_req: 0 = choose, 1..16 = requested partitions (clamped to the k-steps).
// x_f32: the activations are f32 (converted to f16 in the A-tile load).
GemmPlan plan_gemm(int fmt, int M, int N, int K, int split_req, bool x_f32 = false);

// Launch the GEMM (and the split-K reduction when plan.split > 1).
//   W    : uint16 f16 cache when fmt == kFmtF16, else quantized bytes.
//   ldw  : f16 row stride (elements) or quantized row bytes.
//   dry  : launch nothing; hipSuccess iff a kernel implements the plan.
hipError_t launch_gemm(int fmt, const uint16_t *X, int ldx, const void *W, int64_t ldw,
                       float *Y, int ldy, int M, int N, int K, const GemmPlan &plan, float *ws,
                       hipStream_t stream, bool dry = false);

// The same GEMM with f32 activations X (row stride ldx in elements), each
// rounded to f16 as its tile is staged; plan from plan_gemm(..., true).
hipError_t launch_gemm_xf32(int fmt, const float *X, int ldx, const void *W, int64_t ldw,
                            float *Y, int ldy, int M, int N, int K, const GemmPlan &plan,
                            float *ws, hipStream_t stream, bool dry = false);

// The int8 product: Q8_1-style activation blocks (codes Xq, row stride ldq;
// (d, s) pairs ds, [M][K/32]) and the plan and launch of the MMQ kernel.
hipError_t launch_quantize_q8_1(const float *X, int ldx, int8_t *Xq, int ldq, float *ds, int M,
                                int K, hipStream_t stream);
GemmPlan plan_mmq(int M, int N, int K, int split_req);
bool mmq_plan_has_kernel(const GemmPlan &p);   // the int8 kernel's tile is the plan's
hipError_t launch_mmq(int fmt, const int8_t *Xq, int ldq, const float *ds, const void *W,
                      int64_t ldw, float *Y, int ldy, int M, int N, int K, const GemmPlan &plan,
                      float *ws, hipStream_t stream);

// X16[m·ld16 + k] = f16_rne(X[m·ldx + k]) for m < M, k < K (K a multiple of 8).
hipError_t launch_convert_f32_to_f16(const float *X, int ldx, uint16_t *X16, int ld16, int M,
                                     int K, hipStream_t stream);

}  // namespace mq
