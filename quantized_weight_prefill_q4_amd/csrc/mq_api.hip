// C ABI of libmq: argument validation, launch planning, error reporting.
// Every check happens before anything is enqueued, so a rejected call has no
// side effect (Fucina "Eager GPU Offload Without A Compute Graph", ordering
// section: submission failures are reported before return; faults after
// submission surface at the host boundary).

#include "mq.h"
#include "mq_internal.h"

#include <mutex>
#include <stdint.h>

// The K-split partial tiles of mq_gemm_fused_noalloc, for callers that cannot
// allocate.  Each GPU the library runs on holds its own copy for the life of
// the process.  In host code `scratch` names a host-side stand-in: kernels get
// the device address that hipGetSymbolAddress returns for the device
// (scratch_ptr below), never the array's name.
static __device__ __align__(256) float scratch[MQ_NOALLOC_SCRATCH_BYTES / 4];

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

bool quant_fmt(int fmt) { return mq::block_elems(fmt) > 0; }

int check_dims(int M, int N, int K) {
    if (M <= 0 || N <= 0 || K <= 0 || M > MQ_MAX_DIM || N > MQ_MAX_DIM || K > MQ_MAX_K)
        return MQ_ERR_SHAPE;
    return MQ_OK;
}

bool ld_ok(int64_t ld, int64_t K) { return ld >= K && ld % 8 == 0 && ld <= MQ_MAX_K + 64; }

// int8 code rows: 16-byte aligned, at most MQ_MAX_K bytes apart.
bool ldq_ok(int64_t ld, int64_t K) { return ld >= K && ld % 16 == 0 && ld <= MQ_MAX_K; }

// f32 activation rows: 16-byte aligned (ld a multiple of 4), at most MQ_MAX_K
// elements apart (a 256-row tile then spans at most 2^31 bytes).
bool ld32_ok(int64_t ld, int64_t K) { return ld >= K && ld % 4 == 0 && ld <= MQ_MAX_K; }

int hip_status(hipError_t e) {
    if (e == hipSuccess) return MQ_OK;
    g_last_hip_error = (int)e;
    return MQ_ERR_HIP;
}

// Checks of one decode (mq_dequant_to_f16 and each job of a batch).
int check_dequant(int fmt, const void *wq, int N, int K, const uint16_t *w16, int ld) {
    if (!quant_fmt(fmt)) return MQ_ERR_FORMAT;
    if (!wq || !w16) return MQ_ERR_NULL;
    if (check_dims(1, N, K) || K % mq::block_elems(fmt)) return MQ_ERR_SHAPE;
    if (!ld_ok(ld, K)) return MQ_ERR_LD;
    if (!aligned16(wq) || !aligned16(w16)) return MQ_ERR_ALIGN;
    if ((int64_t)N * ld / 8 >= ((int64_t)1 << 31)) return MQ_ERR_SHAPE;
    return MQ_OK;
}

// How a GEMM with f32 activations runs.  Up to kInTileMaxM rows the kernel
// rounds X to f16 while staging its tiles; above, X is converted once into
// the front of the workspace and the f16-activation kernel (with its own
// plan, 256 × 256 tiles included) reads it: every column tile re-reads the
// X panel, so converting inside the tile costs N/BN conversions and twice
// the A-operand bytes per element, against one 6-byte pass.
constexpr int kInTileMaxM = 64;

struct XPlan {
    bool convert_first;
    int ld16;               // row stride of the converted X (convert_first)
    int64_t x16_bytes;      // its workspace bytes, a multiple of 256 (else 0)
    mq::GemmPlan gemm;      // split planes follow the converted X in the workspace
};

XPlan xf32_plan(int fmt, int M, int N, int K, int split_k) {
    XPlan xp;
    xp.convert_first = M > kInTileMaxM;
    if (xp.convert_first) {
        xp.ld16 = (int)mq_f16cache_ld(K);
        xp.x16_bytes = ((int64_t)M * xp.ld16 * 2 + 255) / 256 * 256;
        xp.gemm = mq::plan_gemm(fmt, M, N, K, split_k, false);
    } else {
        xp.ld16 = 0;
        xp.x16_bytes = 0;
        xp.gemm = mq::plan_gemm(fmt, M, N, K, split_k, true);
    }
    return xp;
}

// Device address of `scratch` on the device that owns `stream` (the current
// device for the null stream), looked up once per device with that device
// current and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

int scratch_ptr(hipStream_t stream, void **out) {
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e);
    dev = cur;
    if (stream) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return hip_status(e);
    }
    if (dev < 0 || dev >= kMaxDevices) return hip_status(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return hip_status(e);
        if (!p) return hip_status(hipErrorInvalidSymbol);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MQ_OK;
}

// Shared checks of both GEMM entry points; fills the plan on success.
int check_gemm(int fmt, const void *X, int ldx, const void *W, int64_t ldw_elems, const float *Y,
               int ldy, int M, int N, int K, const void *ws, size_t ws_bytes, int split_k,
               mq::GemmPlan *plan, bool x_f32 = false, XPlan *xplan = nullptr) {
    if (!X || !W || !Y) return MQ_ERR_NULL;
    if (fmt != mq::kFmtF16 && !quant_fmt(fmt)) return MQ_ERR_FORMAT;
    if (int rc = check_dims(M, N, K)) return rc;
    const int step = fmt == mq::kFmtF16 ? 8 : mq::block_elems(fmt);
    if (K % step) return MQ_ERR_SHAPE;
    if (!(x_f32 ? ld32_ok(ldx, K) : ld_ok(ldx, K)) || ldy < N) return MQ_ERR_LD;
    if (fmt == mq::kFmtF16 && !ld_ok(ldw_elems, K)) return MQ_ERR_LD;
    if (!aligned16(X) || !aligned16(W) || !aligned16(Y)) return MQ_ERR_ALIGN;
    if (split_k < 0 || split_k > MQ_MAX_SPLIT_K) return MQ_ERR_SPLIT;
    if (split_k > 1 && (int64_t)M * N >= ((int64_t)1 << 31)) return MQ_ERR_SPLIT;
    int64_t need;
    if (x_f32) {
        *xplan = xf32_plan(fmt, M, N, K, split_k);
        *plan = xplan->gemm;
        need = xplan->x16_bytes + plan->ws_bytes;
    } else {
        *plan = mq::plan_gemm(fmt, M, N, K, split_k);
        need = plan->ws_bytes;
    }
    if (need > 0 && (!ws || !aligned16(ws) || ws_bytes < (size_t)need)) return MQ_ERR_WORKSPACE;
    return MQ_OK;
}

// The f32-activation GEMM: in-tile conversion, or convert into the
// workspace and the f16-activation kernel.
int run_xf32(int fmt, const float *X, int ldx, const void *W, int64_t ldw, float *Y, int ldy,
             int M, int N, int K, void *ws, const XPlan &xp, hipStream_t stream) {
    if (!xp.convert_first)
        return hip_status(mq::launch_gemm_xf32(fmt, X, ldx, W, ldw, Y, ldy, M, N, K, xp.gemm,
                                               (float *)ws, stream));
    uint16_t *x16 = (uint16_t *)ws;
    if (int rc = hip_status(mq::launch_convert_f32_to_f16(X, ldx, x16, xp.ld16, M, K, stream)))
        return rc;
    return hip_status(mq::launch_gemm(fmt, x16, xp.ld16, W, ldw, Y, ldy, M, N, K, xp.gemm,
                                      (float *)((char *)ws + xp.x16_bytes), stream));
}

}  // namespace

extern "C" {

int mq_block_elems(int fmt) {
    const int v = mq::block_elems(fmt);
    return v < 0 ? MQ_ERR_FORMAT : v;
}

int mq_block_bytes(int fmt) {
    const int v = mq::block_bytes(fmt);
    return v < 0 ? MQ_ERR_FORMAT : v;
}

int64_t mq_row_bytes(int fmt, int64_t K) {
    const int be = mq::block_elems(fmt);
    if (be < 0) return MQ_ERR_FORMAT;
    if (K <= 0 || K > MQ_MAX_K || K % be) return MQ_ERR_SHAPE;
    return K / be * mq::block_bytes(fmt);
}

int64_t mq_f16cache_ld(int64_t K) {
    if (K <= 0 || K > MQ_MAX_K) return MQ_ERR_SHAPE;
    return (2 * K) % 2048 == 0 ? K + 64 : K;
}

int mq_dequant_to_f16(int fmt, const void *wq, int N, int K, uint16_t *w16, int ld,
                      void *stream) {
    if (int rc = check_dequant(fmt, wq, N, K, w16, ld)) return rc;
    return hip_status(mq::launch_dequant(fmt, wq, N, K, w16, ld, (hipStream_t)stream));
}

int mq_dequant_to_f16_batch(const mq_dequant_job *jobs, int n, void *stream) {
    if (n < 0) return MQ_ERR_SHAPE;
    if (n == 0) return MQ_OK;
    if (!jobs) return MQ_ERR_NULL;
    for (int i = 0; i < n; ++i) {
        const mq_dequant_job &j = jobs[i];
        if (int rc = check_dequant(j.fmt, j.wq, j.N, j.K, j.w16, j.ld)) return rc;
    }
    constexpr int kChunk = 64;
    mq::DequantSpec specs[kChunk];
    for (int first = 0; first < n; first += kChunk) {
        const int m = n - first < kChunk ? n - first : kChunk;
        for (int i = 0; i < m; ++i) {
            const mq_dequant_job &j = jobs[first + i];
            specs[i] = mq::DequantSpec{j.fmt, j.N, j.K, j.ld, j.wq, j.w16};
        }
        if (int rc = hip_status(mq::launch_dequant_batch(specs, m, (hipStream_t)stream))) return rc;
    }
    return MQ_OK;
}

static int64_t workspace_bytes(int fmt, int M, int N, int K, int split_k, bool x_f32) {
    if (fmt != mq::kFmtF16 && !quant_fmt(fmt)) return MQ_ERR_FORMAT;
    if (int rc = check_dims(M, N, K)) return rc;
    if (K % (fmt == mq::kFmtF16 ? 8 : mq::block_elems(fmt))) return MQ_ERR_SHAPE;
    if (split_k < 0 || split_k > MQ_MAX_SPLIT_K) return MQ_ERR_SPLIT;
    if (split_k > 1 && (int64_t)M * N >= ((int64_t)1 << 31)) return MQ_ERR_SPLIT;
    if (!x_f32) return mq::plan_gemm(fmt, M, N, K, split_k).ws_bytes;
    const XPlan xp = xf32_plan(fmt, M, N, K, split_k);
    return xp.x16_bytes + xp.gemm.ws_bytes;
}

int64_t mq_gemm_workspace_bytes(int fmt, int M, int N, int K, int split_k) {
    return workspace_bytes(fmt, M, N, K, split_k, false);
}

int64_t mq_gemm_xf32_workspace_bytes(int fmt, int M, int N, int K, int split_k) {
    return workspace_bytes(fmt, M, N, K, split_k, true);
}

int mq_gemm_f16cache(const uint16_t *X, int ldx, const uint16_t *W16, int ldw, float *Y,
                     int ldy, int M, int N, int K, void *ws, size_t ws_bytes, int split_k,
                     void *stream) {
    mq::GemmPlan plan;
    if (int rc = check_gemm(mq::kFmtF16, X, ldx, W16, ldw, Y, ldy, M, N, K, ws, ws_bytes,
                            split_k, &plan))
        return rc;
    return hip_status(mq::launch_gemm(mq::kFmtF16, X, ldx, W16, ldw, Y, ldy, M, N, K, plan,
                                      (float *)ws, (hipStream_t)stream));
}

int mq_gemm_fused(int fmt, const uint16_t *X, int ldx, const void *wq, float *Y, int ldy,
                  int M, int N, int K, void *ws, size_t ws_bytes, int split_k, void *stream) {
    if (!quant_fmt(fmt)) return MQ_ERR_FORMAT;
    mq::GemmPlan plan;
    if (int rc = check_gemm(fmt, X, ldx, wq, 0, Y, ldy, M, N, K, ws, ws_bytes, split_k, &plan))
        return rc;
    const int64_t row_bytes = (int64_t)K / mq::block_elems(fmt) * mq::block_bytes(fmt);
    return hip_status(mq::launch_gemm(fmt, X, ldx, wq, row_bytes, Y, ldy, M, N, K, plan,
                                      (float *)ws, (hipStream_t)stream));
}

int mq_gemm_fused_noalloc(int fmt, const uint16_t *X, int ldx, const void *wq, float *Y,
                          int ldy, int M, int N, int K, int split_k, void *stream) {
    if (!quant_fmt(fmt)) return MQ_ERR_FORMAT;
    // the plan's partial tiles must fit the static scratch
    const int64_t need = mq_gemm_workspace_bytes(fmt, M, N, K, split_k);
    if (need < 0) return (int)need;
    if (need > MQ_NOALLOC_SCRATCH_BYTES) return MQ_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0) {
        if (int rc = scratch_ptr((hipStream_t)stream, &ws)) return rc;
    }
    mq::GemmPlan plan;
    if (int rc = check_gemm(fmt, X, ldx, wq, 0, Y, ldy, M, N, K, ws,
                            need > 0 ? (size_t)MQ_NOALLOC_SCRATCH_BYTES : 0, split_k, &plan))
        return rc;
    const int64_t row_bytes = (int64_t)K / mq::block_elems(fmt) * mq::block_bytes(fmt);
    return hip_status(mq::launch_gemm(fmt, X, ldx, wq, row_bytes, Y, ldy, M, N, K, plan,
                                      (float *)ws, (hipStream_t)stream));
}

int mq_gemm_f16cache_xf32(const float *X, int ldx, const uint16_t *W16, int ldw, float *Y,
                          int ldy, int M, int N, int K, void *ws, size_t ws_bytes, int split_k,
                          void *stream) {
    mq::GemmPlan plan;
    XPlan xp;
    if (int rc = check_gemm(mq::kFmtF16, X, ldx, W16, ldw, Y, ldy, M, N, K, ws, ws_bytes,
                            split_k, &plan, true, &xp))
        return rc;
    return run_xf32(mq::kFmtF16, X, ldx, W16, ldw, Y, ldy, M, N, K, ws, xp, (hipStream_t)stream);
}

int mq_gemm_fused_xf32(int fmt, const float *X, int ldx, const void *wq, float *Y, int ldy,
                       int M, int N, int K, void *ws, size_t ws_bytes, int split_k,
                       void *stream) {
    if (!quant_fmt(fmt)) return MQ_ERR_FORMAT;
    mq::GemmPlan plan;
    XPlan xp;
    if (int rc = check_gemm(fmt, X, ldx, wq, 0, Y, ldy, M, N, K, ws, ws_bytes, split_k, &plan,
                            true, &xp))
        return rc;
    const int64_t row_bytes = (int64_t)K / mq::block_elems(fmt) * mq::block_bytes(fmt);
    return run_xf32(fmt, X, ldx, wq, row_bytes, Y, ldy, M, N, K, ws, xp, (hipStream_t)stream);
}

int mq_convert_f32_to_f16(const float *X, int ldx, uint16_t *X16, int ld16, int M, int K,
                          void *stream) {
    if (!X || !X16) return MQ_ERR_NULL;
    if (check_dims(M, 1, K) || K % 8) return MQ_ERR_SHAPE;
    if (!ld32_ok(ldx, K) || !ld_ok(ld16, K)) return MQ_ERR_LD;
    if (!aligned16(X) || !aligned16(X16)) return MQ_ERR_ALIGN;
    return hip_status(mq::launch_convert_f32_to_f16(X, ldx, X16, ld16, M, K, (hipStream_t)stream));
}

int mq_quantize_q8_1(const float *X, int ldx, int8_t *Xq, int ldq, float *ds, int M, int K,
                     void *stream) {
    if (!X || !Xq || !ds) return MQ_ERR_NULL;
    if (check_dims(M, 1, K) || K % 32) return MQ_ERR_SHAPE;
    if (!ld32_ok(ldx, K) || !ldq_ok(ldq, K)) return MQ_ERR_LD;
    if (!aligned16(X) || !aligned16(Xq) || !aligned16(ds)) return MQ_ERR_ALIGN;
    return hip_status(mq::launch_quantize_q8_1(X, ldx, Xq, ldq, ds, M, K, (hipStream_t)stream));
}

int64_t mq_gemm_mmq_workspace_bytes(int fmt, int M, int N, int K, int split_k) {
    if (!quant_fmt(fmt)) return MQ_ERR_FORMAT;
    if (int rc = check_dims(M, N, K)) return rc;
    if (K % mq::block_elems(fmt) || K % 32) return MQ_ERR_SHAPE;
    if (split_k < 0 || split_k > MQ_MAX_SPLIT_K) return MQ_ERR_SPLIT;
    if (split_k > 1 && (int64_t)M * N >= ((int64_t)1 << 31)) return MQ_ERR_SPLIT;
    return mq::plan_mmq(M, N, K, split_k).ws_bytes;
}

int mq_gemm_mmq(int fmt, const int8_t *Xq, int ldq, const float *ds, const void *wq, float *Y,
                int ldy, int M, int N, int K, void *ws, size_t ws_bytes, int split_k,
                void *stream) {
    if (!quant_fmt(fmt)) return MQ_ERR_FORMAT;
    if (!Xq || !ds || !wq || !Y) return MQ_ERR_NULL;
    if (int rc = check_dims(M, N, K)) return rc;
    if (K % mq::block_elems(fmt) || K % 32) return MQ_ERR_SHAPE;
    if (!ldq_ok(ldq, K) || ldy < N) return MQ_ERR_LD;
    if (!aligned16(Xq) || !aligned16(ds) || !aligned16(wq) || !aligned16(Y)) return MQ_ERR_ALIGN;
    if (split_k < 0 || split_k > MQ_MAX_SPLIT_K) return MQ_ERR_SPLIT;
    if (split_k > 1 && (int64_t)M * N >= ((int64_t)1 << 31)) return MQ_ERR_SPLIT;
    const mq::GemmPlan plan = mq::plan_mmq(M, N, K, split_k);
    if (plan.ws_bytes > 0 && (!ws || !aligned16(ws) || ws_bytes < (size_t)plan.ws_bytes))
        return MQ_ERR_WORKSPACE;
    const int64_t row_bytes = (int64_t)K / mq::block_elems(fmt) * mq::block_bytes(fmt);
    return hip_status(mq::launch_mmq(fmt, Xq, ldq, ds, wq, row_bytes, Y, ldy, M, N, K, plan,
                                     (float *)ws, (hipStream_t)stream));
}

int mq_gemm_plan_query(int path, int fmt, int M, int N, int K, int split_k,
                       mq_gemm_plan_info *out) {
    if (!out) return MQ_ERR_NULL;
    if (path < 0 || path > 2) return MQ_ERR_FORMAT;
    const bool mmq = path == 2;
    if (mmq ? !quant_fmt(fmt) : (fmt != mq::kFmtF16 && !quant_fmt(fmt))) return MQ_ERR_FORMAT;
    if (int rc = check_dims(M, N, K)) return rc;
    if (K % (fmt == mq::kFmtF16 ? 8 : mq::block_elems(fmt)) || (mmq && K % 32))
        return MQ_ERR_SHAPE;
    if (split_k < 0 || split_k > MQ_MAX_SPLIT_K) return MQ_ERR_SPLIT;
    if (split_k > 1 && (int64_t)M * N >= ((int64_t)1 << 31)) return MQ_ERR_SPLIT;
    mq::GemmPlan p;
    int64_t x16_bytes = 0;
    bool has_kernel;
    if (mmq) {
        p = mq::plan_mmq(M, N, K, split_k);
        has_kernel = mq::mmq_plan_has_kernel(p);
    } else if (path == 1) {
        const XPlan xp = xf32_plan(fmt, M, N, K, split_k);
        p = xp.gemm;
        x16_bytes = xp.x16_bytes;
        has_kernel = (xp.convert_first
                          ? mq::launch_gemm(fmt, nullptr, 0, nullptr, 0, nullptr, 0, M, N, K, p,
                                            nullptr, nullptr, true)
                          : mq::launch_gemm_xf32(fmt, nullptr, 0, nullptr, 0, nullptr, 0, M, N,
                                                 K, p, nullptr, nullptr, true)) == hipSuccess;
    } else {
        p = mq::plan_gemm(fmt, M, N, K, split_k);
        has_kernel = mq::launch_gemm(fmt, nullptr, 0, nullptr, 0, nullptr, 0, M, N, K, p,
                                     nullptr, nullptr, true) == hipSuccess;
    }
    out->bm = p.bm;
    out->bn = p.bn;
    out->tiles_m = p.tiles_m;
    out->tiles_n = p.tiles_n;
    out->k_steps = p.k_steps;
    out->dp_tiles = p.dp_tiles;
    out->tail_tiles = p.tail_tiles;
    out->split = p.split;
    out->steps_per_split = p.steps_per_split;
    out->has_kernel = has_kernel ? 1 : 0;
    out->ws_bytes = x16_bytes + p.ws_bytes;
    return MQ_OK;
}

const char *mq_strerror(int code) {
    switch (code) {
    case MQ_OK: return "success";
    case MQ_ERR_NULL: return "a required pointer is NULL";
    case MQ_ERR_FORMAT: return "unknown weight format";
    case MQ_ERR_SHAPE: return "M, N or K out of range, or K not a multiple of the block size";
    case MQ_ERR_LD: return "a leading dimension is too small, too large or not a multiple of 8 (4 for f32 rows, 16 for int8 codes)";
    case MQ_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MQ_ERR_WORKSPACE: return "workspace missing, misaligned or smaller than required";
    case MQ_ERR_SPLIT: return "split_k out of range for this problem";
    case MQ_ERR_HIP: return "the HIP runtime rejected a launch";
    case MQ_ERR_SCRATCH: return "the K-split partial tiles exceed the static scratch (MQ_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error code";
    }
}

int mq_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
