/*
 * mq.h — prefill matmul over GGUF block-quantized weights on AMD MI355X (gfx950).
 *
 * The operation (minfer "05 · 8p — Persistent f16 weight cache + fused
 * dequant-in-GEMM", §2 Principle): Y = X·Wᵀ with X the f16 activations of
 * M prefill tokens [M × K], W a quantized weight of N output rows [N × K]
 * and Y in f32 [M × N].  Two shapes of the same product are offered:
 *
 *   1. the persistent f16 cache: mq_dequant_to_f16 decodes W once (at load
 *      time) into an f16 matrix with an optionally padded row stride, and
 *      mq_gemm_f16cache multiplies X by it (f16 products, f32 accumulation);
 *   2. the fused kernel: mq_gemm_fused reads the quantized bytes of W inside
 *      the GEMM and expands them to f16 on the fly, for callers that cannot
 *      spend 2 bytes per weight of extra device memory.
 *
 * Both feed the contraction the same f16 values (§3.3: the fused expansion
 * follows the standalone decode's rounding path; the values are equal, only
 * the sign of an exact zero may differ, which no f32 sum can see).
 *
 * Conventions shared by every entry point
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates device memory, never frees, never synchronizes the host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it in call order and returns immediately; buffers
 *     must stay alive until the stream has passed the call.
 *   - Arguments are validated before anything is enqueued; on any error the
 *     call returns a negative MQ_ERR_* code and has no side effect.
 *   - Faults that happen while a kernel runs are reported by HIP at the
 *     caller's next synchronization, not by these functions.
 *   - Every function is thread-safe; calls on different streams may overlap.
 *   - Weights must not change while an f16 cache built from them is in use
 *     (the cache is derived state; minfer 05 · 8p §2: weights are immutable
 *     after load).
 */
#ifndef MQ_H
#define MQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats, numbered as GGUF types (minfer's type_id 6 is Q5_0, page
 * "79 · Phase-8 coverage batch", §3.6, which fixes the numbering).
 *   MQ_Q8_0: 32 elements in 34 bytes   = f16 d, 32 × int8 q;        w = d·q
 *   MQ_Q4_K: 256 elements in 144 bytes = f16 d, f16 dmin, 12 bytes of eight
 *            6-bit scales + eight 6-bit mins, 128 bytes of 4-bit q;
 *            w = d·sc·q − dmin·m per 32-element sub-block
 *   MQ_Q6_K: 256 elements in 210 bytes = 128 B low 4 bits, 64 B high 2 bits
 *            of 6-bit q, 16 × int8 scales, f16 d;  w = d·s·(q − 32)
 * Four more of the family (minfer 79 · Phase-8 coverage batch, §3.4 and §3.6;
 * minfer 05 · 8p §2 for the Q5_0 layout).  In the 32-element formats element
 * j < 16 is the low nibble of quant byte j and element j + 16 its high nibble;
 * the 5-bit formats add bit j of the 32-bit qh plane as the 16s bit:
 *   MQ_Q4_0: 32 elements in 18 bytes  = f16 d, 16 B q;           w = d·(q − 8)
 *   MQ_Q5_0: 32 elements in 22 bytes  = f16 d, 4 B qh, 16 B q;   w = d·(q − 16)
 *   MQ_Q5_1: 32 elements in 24 bytes  = f16 d, f16 m, 4 B qh, 16 B q;
 *            w = d·q + m
 *   MQ_Q5_K: 256 elements in 176 bytes = Q4_K's d, dmin and 12 scale/min
 *            bytes, 32 B qh, 128 B low 4 bits laid out as Q4_K's; element l
 *            of 32-element sub-block s takes bit s of qh[l] as its 16s bit;
 *            w = d·sc·q − dmin·m as Q4_K
 * A quantized weight of N rows is N rows of K/block_elems blocks each, rows
 * contiguous (row bytes = K/block_elems · block_bytes).  Q8_0, Q6_K, Q4_0 and
 * Q5_0 blocks are only 2-byte aligned inside a row (minfer 05 · 8p §2:
 * alignment of a strided block is stride·g + offset); the library never
 * issues a load that needs more. */
enum {
    MQ_Q4_0 = 2,
    MQ_Q5_0 = 6,
    MQ_Q5_1 = 7,
    MQ_Q8_0 = 8,
    MQ_Q4_K = 12,
    MQ_Q5_K = 13,
    MQ_Q6_K = 14
};

/* Return codes. */
enum {
    MQ_OK = 0,
    MQ_ERR_NULL = -1,      /* a required pointer is NULL */
    MQ_ERR_FORMAT = -2,    /* unknown weight format */
    MQ_ERR_SHAPE = -3,     /* M, N or K <= 0 or too large, or K not a multiple of the block */
    MQ_ERR_LD = -4,        /* a leading dimension is too small, too large or not a
                              multiple of 8 (of 4 for f32 activation rows) */
    MQ_ERR_ALIGN = -5,     /* a pointer is not 16-byte aligned */
    MQ_ERR_WORKSPACE = -6, /* workspace missing or smaller than mq_gemm_workspace_bytes */
    MQ_ERR_SPLIT = -7,     /* split_k outside 0..MQ_MAX_SPLIT_K */
    MQ_ERR_HIP = -8,       /* the HIP runtime rejected a launch; see mq_last_hip_error */
    MQ_ERR_SCRATCH = -9    /* mq_gemm_fused_noalloc: the plan's partial tiles exceed
                              MQ_NOALLOC_SCRATCH_BYTES */
};

/* Limits checked by every entry point. */
#define MQ_MAX_DIM (1 << 24)     /* M and N */
#define MQ_MAX_K (1 << 21)       /* K and every leading dimension */
#define MQ_MAX_SPLIT_K 16
/* Static device scratch of mq_gemm_fused_noalloc, per GPU (64 MiB). */
#define MQ_NOALLOC_SCRATCH_BYTES (64 << 20)

/* Elements per block of `fmt` (32 or 256), or MQ_ERR_FORMAT. */
int mq_block_elems(int fmt);

/* Bytes per block of `fmt` (18, 22, 24, 34, 144, 176, 210), or MQ_ERR_FORMAT. */
int mq_block_bytes(int fmt);

/* Bytes of one quantized row of K elements, or a negative MQ_ERR_* code when
 * the format is unknown or K is not a positive multiple of the block. */
int64_t mq_row_bytes(int fmt, int64_t K);

/* Row stride (elements) of the f16 cache for an inner size K: K + 64 (one
 * 128-byte line) when the f16 row size 2·K bytes is a multiple of 2048, else K
 * (llama.cpp PR #57, Summary, second bullet: pad only when the row aliases at
 * 2048 B).  Negative MQ_ERR_SHAPE when K <= 0 or K > MQ_MAX_K. */
int64_t mq_f16cache_ld(int64_t K);

/* Decode a quantized N×K weight into the f16 cache.
 *   wq  : device, 16-byte aligned, N·mq_row_bytes(fmt, K) bytes, read only.
 *   w16 : device, 16-byte aligned, N·ld f16 (uint16 bit patterns), written:
 *         w16[n·ld + k] = f16 of weight (n, k) for k < K, +0 for K <= k < ld.
 *   ld  : >= K, multiple of 8 (mq_f16cache_ld(K) is the padded choice).
 * Each element is computed in f32 and rounded once to f16 (round to nearest
 * even, subnormals kept, IEEE signed zeros kept): Q4_K and Q5_K as
 * fl32(d·sc·q − dmin·m), Q6_K as (d·s)·(q − 32), Q8_0 as d·q, Q4_0 as
 * d·(q − 8), Q5_0 as d·(q − 16), Q5_1 as fl32(d·q + m) (minfer 05 · 8p §3.2:
 * float math, then one conversion to half).  The result is bit-identical to
 * that definition.
 * One kernel, one pass over the quantized bytes; HBM-bound. */
int mq_dequant_to_f16(int fmt, const void *wq, int N, int K, uint16_t *w16, int ld,
                      void *stream);

/* One weight of a batched decode (see mq_dequant_to_f16_batch); the fields
 * mean what the same-named arguments of mq_dequant_to_f16 mean. */
typedef struct mq_dequant_job {
    int fmt;             /* one of the MQ_Q* formats */
    int N, K;            /* rows; columns, a multiple of the format's block */
    int ld;              /* cache row stride in halves: >= K, multiple of 8 */
    const void *wq;      /* device, 16-byte aligned, N·mq_row_bytes(fmt, K) bytes */
    uint16_t *w16;       /* device, 16-byte aligned, N·ld halves */
} mq_dequant_job;

/* The load-time decode of several weights at once: for each jobs[i], exactly
 * what mq_dequant_to_f16 would write (minfer 05 · 8p §2: every weight is
 * decoded once, when the model is loaded; the decodes are independent).  The
 * jobs are packed, up to 16 per kernel launch, into the launch arguments, so
 * small matrices share a launch instead of each ramping the GPU up and down.
 *   jobs : HOST array of n descriptors, read during the call only.
 *   n    : number of jobs; 0 is a no-op.
 * Every job is checked before anything is enqueued: the first invalid job's
 * MQ_ERR_* code is returned and nothing runs.  Jobs must not overlap in w16;
 * they run in no particular order relative to each other, all on `stream`. */
int mq_dequant_to_f16_batch(const mq_dequant_job *jobs, int n, void *stream);

/* Workspace bytes the GEMM entry points need for this problem: 0 when no
 * tile is split along K, else split · T · BM · BN · 4 for the T tiles that
 * are split (one f32 partial tile per K range, summed in a fixed order so
 * results are deterministic; Fucina "Eager GPU Offload Without A Compute
 * Graph", F16/quantized linears: split-K where the output grid underfills the
 * device, with caller-owned partials).  With split_k = 0 the library runs
 * whole rounds of 256 tiles over all of K and splits only the tiles of a last,
 * partial round; a forced split_k >= 2 splits every tile into at most split_k
 * ranges of whole 64-wide k-steps (fewer when ranges must be longer: the
 * fused Q6_K kernel, and on 256 × 256 tiles with K a multiple of 256 the
 * fused Q8_0 / Q4_0 / Q5_0 / Q5_1 kernel, start ranges on even steps; the
 * fused Q4_K and Q5_K kernels on 256 × 256 tiles on super-block boundaries,
 * i.e. multiples of 4 steps).
 *   fmt     : 0 for mq_gemm_f16cache, else the weight format of mq_gemm_fused.
 *   split_k : 0 = let the library choose (as the GEMM will with the same
 *             arguments), 1 = no split, 2..MQ_MAX_SPLIT_K = forced.
 * Negative MQ_ERR_* on invalid arguments. */
int64_t mq_gemm_workspace_bytes(int fmt, int M, int N, int K, int split_k);

/* Y[M×N] = X[M×K] · W16[N×K]ᵀ on the f16 cache.
 *   X   : device f16, 16-byte aligned, row stride ldx (>= K, multiple of 8).
 *   W16 : device f16, 16-byte aligned, row stride ldw (>= K, multiple of 8);
 *         columns >= K are never read.
 *   Y   : device f32, 16-byte aligned, row stride ldy (>= N); overwritten.
 *   ws  : device workspace of ws_bytes >= mq_gemm_workspace_bytes(0, M, N, K,
 *         split_k); may be NULL when that is 0.
 *   K   : multiple of 8.
 * f16 × f16 products are exact in f32; accumulation is f32 (MFMA).  Accuracy
 * contract: |Y − X·Wᵀ| <= 1e-3·(|X|·|W|ᵀ) + 1e-5 per element. */
int mq_gemm_f16cache(const uint16_t *X, int ldx, const uint16_t *W16, int ldw, float *Y,
                     int ldy, int M, int N, int K, void *ws, size_t ws_bytes, int split_k,
                     void *stream);

/* Y[M×N] = X[M×K] · dequant(Wq)ᵀ with the weight expanded inside the kernel.
 *   fmt : one of the MQ_Q* formats; K a multiple of its block.
 *   wq  : device, 16-byte aligned, N·mq_row_bytes(fmt, K) bytes.
 *   other arguments as mq_gemm_f16cache (ws sized with fmt).
 * The expanded f16 values equal mq_dequant_to_f16's in value (minfer 05 · 8p
 * §3.3: same rounding path); only the sign of an exact zero may differ (the
 * Q6_K, Q4_0 and Q5_0 expansions give +0 where the decode keeps −0).  A signed
 * zero adds nothing to an f32 sum that starts at +0, so with the same X and
 * the same K split the two paths return the same Y bit for bit. */
int mq_gemm_fused(int fmt, const uint16_t *X, int ldx, const void *wq, float *Y, int ldy,
                  int M, int N, int K, void *ws, size_t ws_bytes, int split_k, void *stream);

/* mq_gemm_fused for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, plan, kernels and result as mq_gemm_fused (bit for bit),
 * but the K-split partial tiles go to a static array of the library instead
 * of a caller workspace; nothing is allocated or freed (not by the library,
 * not through torch).
 *   split_k : as mq_gemm_fused.  The automatic plan always fits the scratch
 *             (it splits at most kCUs = 256 tiles of at most 256 × 256 f32, i.e.
 *             exactly MQ_NOALLOC_SCRATCH_BYTES); a forced split whose partial
 *             tiles, mq_gemm_workspace_bytes(fmt, M, N, K, split_k), exceed
 *             MQ_NOALLOC_SCRATCH_BYTES returns MQ_ERR_SCRATCH and runs nothing.
 *   stream  : the scratch used is the one of the device that owns `stream`
 *             (the current device for NULL).  Its address is looked up once
 *             per device, on the first call there, with hipGetSymbolAddress.
 * Each GPU has ONE scratch: calls that may overlap on the same GPU (other
 * streams, other host threads) race on it and must be ordered by the caller.
 * Every partial tile is written in full before it is read, so nothing in it
 * has to start at zero; it keeps the last call's partials.
 * Errors: as mq_gemm_fused, plus MQ_ERR_SCRATCH (and MQ_ERR_HIP if the
 * symbol lookup fails). */
int mq_gemm_fused_noalloc(int fmt, const uint16_t *X, int ldx, const void *wq, float *Y,
                          int ldy, int M, int N, int K, int split_k, void *stream);

/* f32 activations.  Fucina "Eager GPU Offload Without A Compute Graph",
 * quantized linears: the callers hold f32 activations, and the GEMM rounds
 * them to f16 while it stages the operand tile instead of in a separate pass
 * (llama.cpp PR #57, batch-size dependence: that separate convert is part of
 * what the f16 path loses at small M).
 *
 * mq_gemm_f16cache_xf32 / mq_gemm_fused_xf32 compute Y[M×N] = X16·Wᵀ with
 * X16 = f16_rne(X) (round to nearest even, subnormals kept, overflow to
 * ±inf), to the accuracy contract of mq_gemm_f16cache.  Without a K split
 * (split_k = 1) each output sums the same products in the same order as
 * mq_gemm_f16cache / mq_gemm_fused on X16, so the two agree bit for bit; the
 * automatic split may differ, since these kernels use other tiles.
 *   X   : device f32, 16-byte aligned, row stride ldx (>= K, multiple of 4,
 *         <= MQ_MAX_K).
 *   ws  : ws_bytes >= mq_gemm_xf32_workspace_bytes(fmt, M, N, K, split_k).
 *   other arguments and errors as mq_gemm_f16cache / mq_gemm_fused.
 * Two ways to run, chosen by M (the result is the same):
 *   M <= 64: the kernel rounds X to f16 as it stages each A tile (no extra
 *            pass; the workspace holds only K-split planes);
 *   M >  64: X is rounded once into the front of the workspace (M rows of
 *            mq_f16cache_ld(K) halves, rounded up to 256 bytes), then the
 *            f16-activation kernel runs on it.  Every column tile of the
 *            output re-reads the A panel, so in-tile conversion repeats the
 *            rounding N/BN times and doubles the A bytes through the compute
 *            units; one 6-byte-per-element pass is cheaper here. */
int64_t mq_gemm_xf32_workspace_bytes(int fmt, int M, int N, int K, int split_k);

int mq_gemm_f16cache_xf32(const float *X, int ldx, const uint16_t *W16, int ldw, float *Y,
                          int ldy, int M, int N, int K, void *ws, size_t ws_bytes, int split_k,
                          void *stream);

int mq_gemm_fused_xf32(int fmt, const float *X, int ldx, const void *wq, float *Y, int ldy,
                       int M, int N, int K, void *ws, size_t ws_bytes, int split_k,
                       void *stream);

/* The standalone activation convert: X16[m·ld16 + k] = f16_rne(X[m·ldx + k])
 * for m < M, k < K; columns >= K of X16 are not written.  For callers that
 * share one converted X between several GEMMs (one pass instead of one per
 * GEMM).  HBM-bound: 6 bytes per element.
 *   X   : device f32, 16-byte aligned, row stride ldx (>= K, multiple of 4,
 *         <= MQ_MAX_K).
 *   X16 : device f16, 16-byte aligned, row stride ld16 (>= K, multiple of 8).
 *   K   : multiple of 8.
 * Errors: MQ_ERR_NULL, MQ_ERR_SHAPE, MQ_ERR_LD, MQ_ERR_ALIGN, MQ_ERR_HIP. */
int mq_convert_f32_to_f16(const float *X, int ldx, uint16_t *X16, int ld16, int M, int K,
                          void *stream);

/* The int8 ("MMQ") product, a backend with numerics of its own (Fucina
 * "Eager GPU Offload Without A Compute Graph", what the ik_llama.cpp audit
 * contributed: f32 activations quantized once to a Q8_1-style int8 layout
 * with scales and sums, weights unpacked to signed int8, int8 matrix
 * instructions, under a separate parity gate).  Its result differs from the
 * f16 paths' by the activation quantization; it reads the quantized weights
 * directly (no cache).
 *
 * mq_quantize_q8_1: for each row m and 32-element block b of X:
 *   a = max|x|, d = fl32(a / 127), q = the integer nearest fl32(x / d), halves
 *   away from zero (0 when d = 0), s = fl32(d · Σq);
 *   Xq[m·ldq + k] = q (int8), ds[2·(m·K/32 + b)] = d, ds[2·(m·K/32 + b) + 1] = s.
 *   X   : device f32, 16-byte aligned, row stride ldx (>= K, multiple of 4,
 *         <= MQ_MAX_K); finite values.
 *   Xq  : device int8, 16-byte aligned, row stride ldq (>= K, multiple of 16,
 *         <= MQ_MAX_K); columns >= K are not written.
 *   ds  : device f32, 16-byte aligned, M·K/16 floats.
 *   K   : multiple of 32.
 * Errors: MQ_ERR_NULL, MQ_ERR_SHAPE, MQ_ERR_LD, MQ_ERR_ALIGN, MQ_ERR_HIP. */
int mq_quantize_q8_1(const float *X, int ldx, int8_t *Xq, int ldq, float *ds, int M, int K,
                     void *stream);

/* Workspace bytes of mq_gemm_mmq (K-split planes; 0 when nothing is split). */
int64_t mq_gemm_mmq_workspace_bytes(int fmt, int M, int N, int K, int split_k);

/* Y[M×N] = the int8 product of mq_quantize_q8_1's (Xq, ds) and Wq:
 *   each format is split as w = α·c − β (int8 code c, f32 factors exact per
 *   32-element group, per 16 for Q6_K: Q8_0 α = d, c = q; Q4_0 c = q − 8;
 *   Q5_0 c = q − 16; Q5_1 c = q, β = −m; Q4_K / Q5_K α = d·sc, β = dmin·m;
 *   Q6_K α = d·s, c = q − 32), and
 *   Y[m, n] = Σ_b (d_b · Σ_G α_G · I_G − β_b · s_b),  I_G = Σ_{i∈G} c_i·q_i
 *   with I exact (int8 MFMA, i32 accumulation) and the rest in f32.
 * Accuracy contract: |Y − Y_exact| <= 1e-3·S + 1e-5 per element, Y_exact and
 * S = Σ_b (Σ_G |d α I_G| + |β s|) evaluated exactly from the same integers
 * and factors.
 *   fmt : any MQ_Q* format; K a multiple of its block (and of 32).
 *   Xq, ldq, ds : as written by mq_quantize_q8_1 for these M and K.
 *   wq  : device, 16-byte aligned, N·mq_row_bytes(fmt, K) bytes.
 *   Y, ldy, ws, ws_bytes, split_k, stream : as mq_gemm_fused, with
 *         ws_bytes >= mq_gemm_mmq_workspace_bytes(fmt, M, N, K, split_k). */
int mq_gemm_mmq(int fmt, const int8_t *Xq, int ldq, const float *ds, const void *wq, float *Y,
                int ldy, int M, int N, int K, void *ws, size_t ws_bytes, int split_k,
                void *stream);

/* The launch plan of a GEMM call, as the host computes it (no GPU needed, no
 * device call made).  For callers that size workspaces ahead and for tests
 * of the planner.
 *   path    : 0 = mq_gemm_f16cache (fmt 0) / mq_gemm_fused (fmt = format),
 *             1 = their f32-activation variants, 2 = mq_gemm_mmq.
 *   fmt, M, N, K, split_k : as the GEMM call would receive them.
 *   out     : host struct, written on MQ_OK.
 * The plan deals a BM × BN tile of Y to each workgroup: dp_tiles tiles over
 * all of K, then tail_tiles tiles each split into `split` K ranges of
 * steps_per_split k-steps (64 wide; 128 for path 2).  has_kernel is 1 when a
 * kernel implements that tile for this format and 0 otherwise (the GEMM call
 * would return MQ_ERR_HIP without launching).  ws_bytes equals what the
 * matching *_workspace_bytes function returns.
 * Errors: the argument checks of the GEMM call (MQ_ERR_FORMAT, MQ_ERR_SHAPE,
 * MQ_ERR_SPLIT), MQ_ERR_NULL for out, MQ_ERR_FORMAT for an unknown path. */
typedef struct mq_gemm_plan_info {
    int bm, bn;              /* block tile: rows of X, rows of W */
    int tiles_m, tiles_n;    /* ceil(M / bm), ceil(N / bn) */
    int k_steps;             /* ceil(K / step) */
    int dp_tiles;            /* tiles computed over all of K (the first ones) */
    int tail_tiles;          /* tiles split along K */
    int split;               /* K ranges per tail tile (1: no split) */
    int steps_per_split;     /* k-steps per range */
    int has_kernel;          /* 1: a kernel implements (bm, bn) for this format */
    int64_t ws_bytes;        /* workspace the call needs */
} mq_gemm_plan_info;

int mq_gemm_plan_query(int path, int fmt, int M, int N, int K, int split_k,
                       mq_gemm_plan_info *out);

/* Static text for a return code (never NULL). */
const char *mq_strerror(int code);

/* Raw hipError_t of the last MQ_ERR_HIP returned on this thread (0 if none). */
int mq_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MQ_H */
