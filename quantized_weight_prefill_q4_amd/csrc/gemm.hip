// Planning and launch of the prefill GEMM with f16 activations (the kernels
// are in gemm_kernel.h; the f32-activation variants are instantiated in
// gemm_xf32.hip).

#include "gemm_kernel.h"

namespace mq {

GemmPlan plan_gemm(int fmt, int M, int N, int K, int split_req, bool x_f32) {
    GemmPlan p;
    p.bn = 128;
    p.bm = M > 128 ? 256 : (M > 64 ? 128 : 64);
    // The larger 256 × 256 tile moves half the operand bytes per flop through
    // L2 and LDS, which under this part's power limit is time.  It is used
    // with at least one full round of such tiles, or — when even the
    // 256 × 128 grid is less than one round — when fewer 256 × 256 tiles split
    // along K fill at least 7/8 of the compute units while every K range
    // keeps >= 3072 elements (the partial tiles' write, read and reduce are
    // then a small part of the call: the 7B down shape, 3584 × 18944, runs
    // 7% faster than on 224 unsplit 256 × 128 tiles, 4096 × 14336 at
    // M = 1024 with ranges of 3584 7%; q/o, K = 3584 in ranges of 1792,
    // would run 18% slower).  Only for f16 activations: the f32 activation
    // registers do not fit beside 256 accumulators.
    if (!x_f32 && M > 128) {
        const int64_t t256 = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
        const int k64 = (K + 63) / 64;
        int s = t256 >= kCUs ? 1 : (int)(kCUs / t256);
        s = s > 16 ? 16 : s;
        s = s > k64 / 4 ? k64 / 4 : s;
        const int64_t t128 = (int64_t)((M + 255) / 256) * ((N + 127) / 128);
        const bool split_fills =
            t128 < kCUs && s >= 2 && t256 * s >= kCUs * 7 / 8 && K / s >= 3072;
        // More than 3/4 of a round of 256 × 256 tiles also takes them, unsplit:
        // the 256 × 128 grid would be a full round plus a tail of more than
        // 128 tiles, too many to split (14336 × 4096 at M = 1024: 160 -> 139
        // us; 18944 × 3584 at M = 768 -13%; fused -10%).
        if (t256 >= kCUs || split_fills || t256 * 4 > kCUs * 3) p.bn = 256;
    }
    // (Fused formats at M <= 128 keep the 2 × 2 tiles: the register-expansion
    // kernels on 128 × 256 tiles, with about 2.6 times less LDS traffic per
    // flop, measured slower on every M = 128 sweep shape — 4096 × 4096
    // 22.2 -> 26.5 us, 4096 × 14336 34.8 -> 37.6 us — so LDS is not what
    // bounds a small-M step.)
    const bool b32 = fmt == kFmtQ8_0 || fmt == kFmtQ4_0 || fmt == kFmtQ5_0 || fmt == kFmtQ5_1;
    // Narrow outputs (the 256 × 128 grid has at most kCUs / 4 tiles, e.g. the
    // 7B k/v projections, N = 512) with a short K take 64-row tiles: four
    // times the tiles, so a two-way K split instead of eight fills the
    // compute units, with a quarter of the partial-plane traffic (k/v at
    // M = 2048: 30.5 -> 26.2 us).  Not for long K: a 64-row tile's k-loop is
    // latency-bound (M = 512, N = 4096, K = 14336: 78 -> 124 us).  The fused
    // kernels decode the weights once per row tile, so they take 128-row
    // tiles instead while those still number kCUs / 4 (a K split of at most
    // 4): k/v at M = 2048 Q4_K 28.7 -> 26.3 us, Q6_K 36.4 -> 30.5, Q8_0
    // 28.7 -> 27.2; N = 1024 46.3 -> 42.0; M = 512, N = 2048 31.2 -> 28.7.
    if (p.bn == 128 && M > 128 && K <= 4096 &&
        (int64_t)((M + 255) / 256) * ((N + 127) / 128) * 4 <= kCUs) {
        const bool rows128 =
            fmt != kFmtF16 && (int64_t)((M + 127) / 128) * ((N + 127) / 128) * 4 >= kCUs;
        p.bm = rows128 ? 128 : 64;
    }
    p.tiles_m = (M + p.bm - 1) / p.bm;
    p.tiles_n = (N + p.bn - 1) / p.bn;
    const int tiles = p.tiles_m * p.tiles_n;
    const int k64 = (K + 63) / 64;
    p.k_steps = k64;
    // Whole rounds of kCUs tiles run over all of K; a last, partial round of
    // `rem` tiles is split along K into kCUs / rem ranges so that it fills the
    // compute units (at least 256 k per range, at most MQ_MAX_SPLIT_K).  A
    // requested split_k >= 2 splits every tile that many ways.
    int dp = tiles, split = 1;
    if (split_req >= 2) {
        dp = 0;
        split = split_req;
    } else if (split_req == 0) {
        const int rem = tiles % kCUs;
        if (rem > 0) {
            int s = kCUs / rem;
            s = s > 16 ? 16 : s;
            s = s > k64 / 4 ? k64 / 4 : s;
            if (s >= 2) {
                dp = tiles - rem;
                split = s;
            }
        }
    }
    if (split > k64) split = k64;
    int per = (k64 + split - 1) / split;
    // the fused Q6_K loader pairs k-steps (2j, 2j + 1), and so does the fused
    // register-expansion kernel of the 32-element block formats (256-column
    // tiles, K a multiple of 256): ranges start even; the fused Q4_K and
    // Q5_K register-expansion kernels stage whole super-blocks (4 steps)
    const bool pairs = fmt == kFmtQ6_K || (b32 && p.bn == 256 && K % 256 == 0);
    if (pairs && (per & 1) && split > 1) ++per;
    if ((fmt == kFmtQ4_K || fmt == kFmtQ5_K) && p.bn == 256 && split > 1)
        per = (per + 3) / 4 * 4;
    split = (k64 + per - 1) / per;   // no empty range
    if (split == 1) dp = tiles;
    p.dp_tiles = dp;
    p.tail_tiles = tiles - dp;
    p.split = split;
    p.steps_per_split = split > 1 ? per : k64;
    p.ws_bytes = split > 1 ? (int64_t)split * p.tail_tiles * p.bm * p.bn * 4 : 0;
    return p;
}

hipError_t launch_gemm(int fmt, const uint16_t *X, int ldx, const void *W, int64_t ldw, float *Y,
                       int ldy, int M, int N, int K, const GemmPlan &plan, float *ws,
                       hipStream_t stream, bool dry) {
    return launch_gemm_t<false>(fmt, X, ldx, W, ldw, Y, ldy, M, N, K, plan, ws, stream, dry);
}

}  // namespace mq
