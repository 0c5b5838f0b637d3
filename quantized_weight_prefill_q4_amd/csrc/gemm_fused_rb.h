// Fused GEMM kernels that expand Q4_K / Q6_K and the 32-element block
// formats' weights straight into the MFMA operand registers (256 × 256
// tiles).  Included by gemm_kernel.h,
// whose helpers (loaders, swizzle, tile mapping, store_tile) they use.
//
// minfer "05 · 8p — Persistent f16 weight cache + fused dequant-in-GEMM" §2
// and §3.3: the fused shape reads the quantized bytes of each B tile and
// expands them with the standalone decode's arithmetic.

#pragma once

namespace mq {
namespace {

// ---------------------------------------------------------------------------
// Fused Q4_K GEMM on 256 × 256 tiles with the weights expanded straight into
// the MFMA operand registers.
//
// In gemm_kernel the fused loaders expand a k-step's B tile once per
// workgroup and write it to LDS as f16 (32 KB), which the 2×2 waves then read
// back (64 KB per k-step).  Here the 4 waves are laid out 1 × 4: wave w owns
// weight rows 64w .. 64w + 63 of the tile and all 256 activation rows, so
// each weight element is still expanded exactly once per tile, by the lane
// that feeds it to the MFMA.  The raw super-blocks (144 bytes per weight row)
// are staged in LDS a whole 256-element super-block at a time — the tile's
// 256 rows × 144 contiguous bytes, each 16-byte chunk loaded once, so the
// global loads stay whole cache lines — and each lane reads the 16 quant
// bytes and the header of its rows per k-step.  B then costs 9 KB of LDS
// writes and 16 KB of reads per k-step instead of 32 + 64 KB, while the X
// fragment reads double (every wave reads all 256 rows: 128 KB); the global
// bytes are the same.  Measured on the 7B gate shape against the 2×2 fused
// kernel: texture-address stalls −90%, LDS bank conflicts −70%, 2-4% less
// time; the expansion's VALU work (~2.8 instructions per element) is what
// remains between this kernel and the f16-cache GEMM.
//
// Lane l of wave w feeds weight rows 64w + 32f + (l & 31) (f = 0, 1) at
// k = 16kk + 8(l >> 5) + 0..7 of k-slice kk, which are, within the k-step's
// 64-element quarter c4 of the super-block, the low nibbles of quant bytes
// 32c4 + 8(l >> 5) + 0..7 (kk = 0) and 32c4 + 16 + 8(l >> 5) + 0..7 (kk = 1)
// with sub-block 2c4's scale and min, and the high nibbles of the same bytes
// (kk = 2, 3) with sub-block 2c4 + 1's.  The arithmetic is the decode's
// (q4k_chunk), so the expanded values are the cache's bit for bit, and the
// MFMAs see the same operands in the same order as the cache kernel's.
//
// Pipeline: X as in gemm_kernel (two register sets, two LDS stages, loads
// two k-steps ahead).  Raw weights: two super-block buffers; during the four
// k-steps of super-block sb the 2304 chunks of super-block sb + 1 are loaded
// (9 per thread: 3 in each of the first three steps, one step ahead in a
// register set) and written to the other buffer, which is not read before
// the last quarter of super-block sb.  Each k-step reads the next step's raw
// bytes and expands its first k-slice between its own MFMAs; for the last
// quarter that is the next super-block, complete since the third quarter's
// barrier (the fourth quarter writes no part).  K ranges are whole
// super-blocks.
// ---------------------------------------------------------------------------
//
// Q5_K takes the same kernel: its 176-byte super-blocks (the Q4_K header,
// then 32 qh bytes, then the 128 quant bytes) are 11 chunks per row, and the
// lane also reads the 8 qh bytes at the positions of its quant bytes; bit j
// of qh[l] is the 16s bit of element l of sub-block j.
// ---------------------------------------------------------------------------
template <int FMT>
struct KRb;
template <>
struct KRb<kFmtQ4_K> {
    static constexpr int CH = 9, BB = 144, QSC = 1, PER = 3;   // chunks per row, bytes, qs chunk
};
template <>
struct KRb<kFmtQ5_K> {
    static constexpr int CH = 11, BB = 176, QSC = 3, PER = 4;
};

// Chunks [lo, hi) of the thread's CH belong to part c4 (loaded for step c4).
template <int FMT, int C4>
struct RbPart {
    static constexpr int n = KRb<FMT>::CH, per = KRb<FMT>::PER;
    static constexpr int lo = C4 * per < n ? C4 * per : n;
    static constexpr int hi = (C4 + 1) * per < n ? (C4 + 1) * per : n;
};

// Scale and min (as the f32 factors d·sc and dmin·m) of sub-blocks 2c4 and
// 2c4 + 1 from a super-block header (d, dmin, 12 scale bytes).
template <int C4>
__device__ __forceinline__ void q4k_sub_scales(const u32x4 h, float &A0, float &C0, float &A1,
                                               float &C1) {
    uint32_t sc0, m0, sc1, m1;
    if constexpr (C4 < 2) {
        constexpr int s0 = 16 * C4, s1 = s0 + 8;
        sc0 = (h.y >> s0) & 63;
        m0 = (h.z >> s0) & 63;
        sc1 = (h.y >> s1) & 63;
        m1 = (h.z >> s1) & 63;
    } else {
        constexpr int s0 = 16 * (C4 - 2), s1 = s0 + 8;
        sc0 = ((h.w >> s0) & 15) | (((h.y >> (s0 + 6)) & 3) << 4);
        m0 = ((h.w >> (s0 + 4)) & 15) | (((h.z >> (s0 + 6)) & 3) << 4);
        sc1 = ((h.w >> s1) & 15) | (((h.y >> (s1 + 6)) & 3) << 4);
        m1 = ((h.w >> (s1 + 4)) & 15) | (((h.z >> (s1 + 6)) & 3) << 4);
    }
    const float d = f16_bits_to_f32(h.x), dmin = f16_bits_to_f32(h.x >> 16);
    A0 = d * (float)sc0;
    C0 = dmin * (float)m0;
    A1 = d * (float)sc1;
    C1 = dmin * (float)m1;
}

// What a lane needs of its two weight rows for one k-step: the quant bytes
// (qa: bytes 8h.., qb: bytes 16 + 8h.. of the quarter), for Q5_K the qh bytes
// at the same positions shifted right by 2c4 (bit 0 of each byte: sub-block
// 2c4, bit 1: 2c4 + 1), the two sub-blocks' factors, and the expanded
// fragments of k-slice 0.  Read and computed during the previous k-step, so a
// step starts with its first MFMAs.
struct RbRaw {
    u32x2 qa[2], qb[2], ha[2], hb[2];
    float A0[2], C0[2], A1[2], C1[2];
    half8 bf0[2];
};

// The B fragment of k-slice kk of weight row f.
template <int FMT, int KK>
__device__ __forceinline__ half8 q4k_frag(const RbRaw &r, int f) {
    constexpr uint32_t L = 0x0F0F0F0Fu, B = 0x01010101u;
    const u32x2 q = (KK & 1) ? r.qb[f] : r.qa[f];
    uint32_t w0 = (KK < 2) ? (q.x & L) : ((q.x >> 4) & L);
    uint32_t w1 = (KK < 2) ? (q.y & L) : ((q.y >> 4) & L);
    if constexpr (FMT == kFmtQ5_K) {
        const u32x2 hq = (KK & 1) ? r.hb[f] : r.ha[f];
        constexpr int j = KK < 2 ? 0 : 1;
        w0 |= ((hq.x >> j) & B) << 4;
        w1 |= ((hq.y >> j) & B) << 4;
    }
    return __builtin_bit_cast(half8, q4k_chunk(w0, w1, KK < 2 ? r.A0[f] : r.A1[f],
                                               KK < 2 ? r.C0[f] : r.C1[f]));
}

// The raw bytes of weight row part f (rows 64·wave + 32f + lane % 32) for
// quarter C4 of the super-block: its 16-byte head and the lane's quant (and,
// for Q5_K, fifth-bit) bytes.
template <int FMT, int C4>
__device__ __forceinline__ void rb_fetch_row(const u32x4 *Bc, int lane, int wave, int f, RbRaw &r,
                                             u32x4 &hdr) {
    using G = KRb<FMT>;
    const int h = lane >> 5;
    const u32x4 *blk = Bc + (wave * 64 + f * 32 + (lane & 31)) * G::CH;   // the row's block
    hdr = blk[0];
    const u32x2 *q2 = reinterpret_cast<const u32x2 *>(blk + G::QSC + 2 * C4);
    r.qa[f] = q2[h];
    r.qb[f] = q2[2 + h];
    if constexpr (FMT == kFmtQ5_K) {
        const u32x2 *h2 = reinterpret_cast<const u32x2 *>(blk + 1);
        const u32x2 ha = h2[h], hb = h2[2 + h];
        r.ha[f] = u32x2{ha.x >> (2 * C4), ha.y >> (2 * C4)};
        r.hb[f] = u32x2{hb.x >> (2 * C4), hb.y >> (2 * C4)};
    }
}

// Row part f's sub-block scales and mins from its head, and its first
// k-slice's B fragment.
template <int FMT, int C4>
__device__ __forceinline__ void rb_fetch_finish(int f, const u32x4 &hdr, RbRaw &r) {
    q4k_sub_scales<C4>(hdr, r.A0[f], r.C0[f], r.A1[f], r.C1[f]);
    r.bf0[f] = q4k_frag<FMT, 0>(r, f);
}

// The register-expansion steps prepare the operands of k-slice kk + 1 while
// slice kk's 2·FM MFMAs run: A fragment i is read after MFMA i and the two
// expanded B fragments are made after MFMAs FM and FM + 2, so that the wave —
// alone on its SIMD — keeps feeding the matrix pipe instead of stopping for
// one burst of LDS reads and expansion arithmetic (3-5% on the 7B gate|up,
// down and 14336 x 4096 shapes at M = 2048).  Called after MFMA IJ of slice
// kk; load_a(i) reads A fragment i of slice kk + 1, make_b(f) expands B
// fragment f.
// A fragment i (activation rows 32i .. 32i + 31) of k-slice kk from an X stage
// (all the tile's rows, as every wave of these kernels reads).
__device__ __forceinline__ half8 rb_a_frag(const u32x4 *Ac, int kk, int i, int lane) {
    const int r = i * 32 + (lane & 31), c = kk * 2 + (lane >> 5);
    return __builtin_bit_cast(half8, Ac[r * 8 + (c ^ swz<8>(r))]);
}

template <int FM, int IJ, class LoadA, class MakeB>
__device__ __forceinline__ void rb_next_operands(LoadA &&load_a, MakeB &&make_b) {
    static_assert(FM >= 4, "a slice needs FM + 3 MFMAs to place the operands");
    if constexpr (IJ < FM) {
        __builtin_amdgcn_sched_barrier(0);
        load_a(std::integral_constant<int, IJ>());
        __builtin_amdgcn_sched_barrier(0);
    } else if constexpr (IJ == FM || IJ == FM + 2) {
        __builtin_amdgcn_sched_barrier(0);
        make_b(std::integral_constant<int, (IJ - FM) / 2>());
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One k-step of the wave's 256 × 64 tile from X stage Ac and the raw bytes
// `cur` (fetched during the previous step); fetches the next step's raw
// bytes (quarter NC4 of buffer Bnext) into `nxt` between the MFMAs.
template <int FMT, int NC4, int FM, class Slot>
__device__ __forceinline__ void rb_step(const u32x4 *Ac, const u32x4 *Bnext, f32x16 (&acc)[FM][2],
                                        int lane, int wave, const RbRaw &cur, RbRaw &nxt,
                                        Slot &&slot) {
    half8 af[2][FM], bf[2][2];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[0][i] = rb_a_frag(Ac, 0, i, lane);
    bf[0][0] = cur.bf0[0];
    bf[0][1] = cur.bf0[1];
    u32x4 hdr[2];
    static_for<4>([&](auto KK) MQ_INLINE {
        constexpr int kk = KK, c = kk & 1;
        __builtin_amdgcn_sched_barrier(0);
        static_for<2 * FM>([&](auto IJ) MQ_INLINE {
            constexpr int i = IJ / 2, f = IJ % 2, n = kk * 2 * FM + IJ;
            acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[c][i], bf[c][f], acc[i][f], 0, 0,
                                                               0);
            if constexpr (kk + 1 < 4) {
                rb_next_operands<FM, IJ>(
                    [&](auto I) MQ_INLINE { af[c ^ 1][I] = rb_a_frag(Ac, kk + 1, I, lane); },
                    [&](auto F) MQ_INLINE { bf[c ^ 1][F] = q4k_frag<FMT, kk + 1>(cur, F); });
            } else if constexpr (IJ == 0 || IJ == 2) {
                // the last slice spreads the next step's raw fetch the same
                // way: the row parts' reads after MFMAs 0 and 2, their scales
                // and first fragments after MFMAs FM and FM + 2
                __builtin_amdgcn_sched_barrier(0);
                rb_fetch_row<FMT, NC4>(Bnext, lane, wave, IJ / 2, nxt, hdr[IJ / 2]);
                __builtin_amdgcn_sched_barrier(0);
            } else if constexpr (IJ == FM || IJ == FM + 2) {
                __builtin_amdgcn_sched_barrier(0);
                rb_fetch_finish<FMT, NC4>((IJ - FM) / 2, hdr[(IJ - FM) / 2], nxt);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (n & 1) {
                __builtin_amdgcn_sched_barrier(0);
                slot(std::integral_constant<int, n / 2>());
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    });
}

// rb_step with the step's barrier inside: af[0] holds k-slice 0's A
// fragments on entry; mid() — the barrier — runs between slices 2 and 3, and
// slice 3 reads, around the next step's raw fetch, the next step's slice-0 A
// fragments from X stage An into af[0], so the next step starts on operands
// already in registers.
template <int FMT, int NC4, int FM, class Slot, class Mid>
__device__ __forceinline__ void rb_step_x(const u32x4 *Ac, const u32x4 *An, const u32x4 *Bnext,
                                          f32x16 (&acc)[FM][2], half8 (&af)[2][FM], int lane,
                                          int wave, const RbRaw &cur, RbRaw &nxt, Slot &&slot,
                                          Mid &&mid) {
    static_assert(FM >= 4, "a slice needs FM + 3 MFMAs to place the operands");
    half8 bf[2][2];
    bf[0][0] = cur.bf0[0];
    bf[0][1] = cur.bf0[1];
    u32x4 hdr[2];
    static_for<4>([&](auto KK) MQ_INLINE {
        constexpr int kk = KK, c = kk & 1;
        __builtin_amdgcn_sched_barrier(0);
        static_for<2 * FM>([&](auto IJ) MQ_INLINE {
            constexpr int i = IJ / 2, f = IJ % 2, n = kk * 2 * FM + IJ;
            acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[c][i], bf[c][f], acc[i][f], 0, 0,
                                                               0);
            if constexpr (kk + 1 < 4) {
                rb_next_operands<FM, IJ>(
                    [&](auto I) MQ_INLINE { af[c ^ 1][I] = rb_a_frag(Ac, kk + 1, I, lane); },
                    [&](auto F) MQ_INLINE { bf[c ^ 1][F] = q4k_frag<FMT, kk + 1>(cur, F); });
            } else if constexpr (IJ == 0 || IJ == 2) {
                __builtin_amdgcn_sched_barrier(0);
                rb_fetch_row<FMT, NC4>(Bnext, lane, wave, IJ / 2, nxt, hdr[IJ / 2]);
                __builtin_amdgcn_sched_barrier(0);
            } else if constexpr (IJ == FM || IJ == FM + 2) {
                __builtin_amdgcn_sched_barrier(0);
                rb_fetch_finish<FMT, NC4>((IJ - FM) / 2, hdr[(IJ - FM) / 2], nxt);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                // the other positions of the last slice, in order, read the
                // next step's slice-0 A fragments
                constexpr int skip = (IJ > 0) + (IJ > 2) + (IJ > FM) + (IJ > FM + 2);
                constexpr int ia = IJ - skip;
                if constexpr (ia < FM) {
                    __builtin_amdgcn_sched_barrier(0);
                    af[0][ia] = rb_a_frag(An, 0, ia, lane);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (n & 1) {
                __builtin_amdgcn_sched_barrier(0);
                slot(std::integral_constant<int, n / 2>());
                __builtin_amdgcn_sched_barrier(0);
            }
        });
        if constexpr (kk == 2) {
            __builtin_amdgcn_sched_barrier(0);
            mid();
            __builtin_amdgcn_sched_barrier(0);
        }
    });
}

template <int FMT, int BM>
__global__ __launch_bounds__(kThreads, 1) void gemm_q4k_rb_kernel(Args a) {
    static_assert(FMT == kFmtQ4_K || FMT == kFmtQ5_K, "Q4_K or Q5_K");
    using G = KRb<FMT>;
    static_assert(BM == 64 || BM == 128 || BM == 256, "tiles of 64, 128 or 256 rows");
    constexpr int BN = 256, BK = 64, CPR = 8;
    constexpr int FM = BM / 32, FN = 2, TM = BM, TN = 64;
    constexpr int NT = G::CH;   // chunks per thread (256 rows × CH over 256 threads)
    __shared__ u32x4 A0[BM * CPR], A1[BM * CPR];
    __shared__ u32x4 Bq0[256 * G::CH], Bq1[256 * G::CH];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = 0, wn = wave;
    const int pid = blockIdx.x;
    int tile, part = 0;
    if (pid < a.dp_tiles) {
        tile = xcd_remap(pid, a.dp_tiles);
    } else {
        const int j = xcd_remap(pid - a.dp_tiles, (int)gridDim.x - a.dp_tiles);
        const int tt = j % a.tail_tiles;
        tile = a.dp_tiles + tt;
        part = j / a.tail_tiles;
    }
    const bool tail = pid >= a.dp_tiles;
    int tm, tn;
    tile_coords(tile, a.tiles_m, a.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    // A tile at or past the matrix edge has nothing to compute; stopping
    // here keeps every buffer range below built from a positive extent.
    if (m0 >= a.M || n0 >= a.N) return;
    // K ranges are whole super-blocks (the plan's steps_per_split is a
    // multiple of 4, and K of 256)
    const int kt_begin = tail ? part * a.steps_per_split : 0;
    const int kt_end = tail ? min(kt_begin + a.steps_per_split, a.k_steps) : a.k_steps;
    const int sb_end = kt_end >> 2;

    F16Loader<BM> la;
    la.init((const uint16_t *)a.X + (int64_t)m0 * a.ldx, min(BM, a.M - m0), a.ldx, a.K);
    constexpr int NA = decltype(la)::NPART;
    // raw weight chunks: chunk c = thread + 256·i is byte 16(c mod CH) of the
    // super-block of tile row c / CH, and lands at LDS chunk c
    const int rows_valid = min(BN, a.N - n0);
    const __amdgpu_buffer_rsrc_t rsb =
        make_rsrc(a.W + (int64_t)n0 * a.ldw, (uint32_t)(rows_valid * a.ldw));
    uint32_t goff[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int c = (int)threadIdx.x + kThreads * i, r = c / G::CH;
        goff[i] = (uint32_t)(r * a.ldw + 16 * (c - G::CH * r));
    }
    u32x4 bv[2][G::PER];
    RbRaw raw[2];   // raw bytes of the current and the next k-step (index P, 1 − P)
    half8 af[2][FM];   // A fragments, k-slice 0 of a step read during the previous one

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // prologue: super-block kt_begin / 4 whole in its buffer, X step kt_begin
    // in stage 0, X step kt_begin + 1 and part 0 of the next super-block in
    // register set 1
    {
        const int sb0 = kt_begin >> 2, k0 = kt_begin * BK;
        u32x4 t[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) t[i] = buf_load16(rsb, goff[i] + (uint32_t)sb0 * (uint32_t)G::BB);
        la.begin(0, k0, true);
#pragma unroll
        for (int i = 0; i < NA; ++i) la.load(0, i);
        la.begin(1, k0 + BK, kt_begin + 1 < kt_end);
#pragma unroll
        for (int i = 0; i < NA; ++i) la.load(1, i);
        const bool nlive = sb0 + 1 < sb_end;
#pragma unroll
        for (int i = RbPart<FMT, 0>::lo; i < RbPart<FMT, 0>::hi; ++i)
            bv[1][i - RbPart<FMT, 0>::lo] =
                buf_load16(rsb, nlive ? goff[i] + (uint32_t)(sb0 + 1) * (uint32_t)G::BB : kOOB);
#pragma unroll
        for (int i = 0; i < NA; ++i) la.store(0, i, A0);
        u32x4 *B = (sb0 & 1) ? Bq1 : Bq0;
#pragma unroll
        for (int i = 0; i < NT; ++i) B[threadIdx.x + kThreads * i] = t[i];
        sync_lds();
        for (int f = 0; f < 2; ++f) {
            u32x4 hd;
            rb_fetch_row<FMT, 0>(B, lane, wave, f, raw[0], hd);
            rb_fetch_finish<FMT, 0>(f, hd, raw[0]);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) af[0][i] = rb_a_frag(A0, 0, i, lane);
    }

    // Step kt (quarter C4, P = C4 & 1): X as in gemm_kernel; raw weights:
    // slots 0..15 load part (C4 + 1) & 3 of the super-block that step kt + 1
    // writes into set P, slots 8..23 (k-slices 1 and 2) write set 1 − P (part
    // C4 of super-block kt / 4 + 1) to that super-block's buffer; the step's
    // barrier follows slice 2 (rb_step_x).
    auto step = [&](auto C4c, int kt) MQ_INLINE {
        constexpr int C4 = decltype(C4c)::value, P = C4 & 1;
        constexpr int LC = (C4 + 1) & 3;
        constexpr int NL = RbPart<FMT, LC>::hi - RbPart<FMT, LC>::lo;
        constexpr int NS = RbPart<FMT, C4>::hi - RbPart<FMT, C4>::lo;
        constexpr int H = 2 * FM;   // half the step's slots
        u32x4 *An = P ? A0 : A1;
        const int sb = kt >> 2;
        const u32x4 *Bc = (sb & 1) ? Bq1 : Bq0;
        u32x4 *Bn = (sb & 1) ? Bq0 : Bq1;
        // the next step's raw bytes: this super-block's buffer, or for the
        // last quarter the next one's, complete since the previous barrier
        // (the last quarter writes no part)
        static_assert(RbPart<FMT, 3>::lo == RbPart<FMT, 3>::hi, "the last quarter writes no part");
        const u32x4 *Bnext = C4 == 3 ? Bn : Bc;
        const int sbl = (kt + 1) / 4 + 1;
        const uint32_t boff = sbl < sb_end ? (uint32_t)sbl * (uint32_t)G::BB : kOOB;
        la.begin(P, (kt + 2) * BK, kt + 2 < kt_end);
        rb_step_x<FMT, (C4 + 1) & 3>(P ? A1 : A0, An, Bnext, acc, af, lane, wave, raw[P],
                                     raw[1 - P], [&](auto SL) MQ_INLINE {
            constexpr int sl = SL;
            if constexpr (sl < H) {
                constexpr int lo = sl * (NA + NL) / H, hi = (sl + 1) * (NA + NL) / H;
                static_for<hi - lo>([&](auto O) MQ_INLINE {
                    constexpr int o = lo + O;
                    if constexpr (o < NA) la.load(P, o);
                    else bv[P][o - NA] = buf_load16(
                        rsb, boff == kOOB ? kOOB : goff[RbPart<FMT, LC>::lo + o - NA] + boff);
                });
            }
            if constexpr (sl >= H / 2 && sl < H / 2 + H) {
                constexpr int w = sl - H / 2;
                constexpr int lo = w * (NA + NS) / H, hi = (w + 1) * (NA + NS) / H;
                static_for<hi - lo>([&](auto O) MQ_INLINE {
                    constexpr int o = lo + O;
                    if constexpr (o < NA) la.store(1 - P, o, An);
                    else Bn[threadIdx.x + kThreads * (RbPart<FMT, C4>::lo + o - NA)] = bv[1 - P][o - NA];
                });
            }
        }, [&]() MQ_INLINE { sync_lds(); });
    };
    for (int kt = kt_begin; kt < kt_end; kt += 4) {
        step(std::integral_constant<int, 0>(), kt);
        step(std::integral_constant<int, 1>(), kt + 1);
        step(std::integral_constant<int, 2>(), kt + 2);
        step(std::integral_constant<int, 3>(), kt + 3);
    }

    store_tile<BM, BN, FM, FN, TM, TN, 4, (int)sizeof(A0), (int)sizeof(Bq0)>(
        a, acc, tail, part, tile, m0, n0, wm, wn, lane, wave, A0, A1, Bq0, Bq1);
}

// ---------------------------------------------------------------------------
// Fused Q6_K GEMM on 256 × 256 tiles, expanded in the MFMA operand registers
// (the layout of gemm_q4k_rb_kernel: 1 × 4 waves, wave w owns weight rows
// 64w .. 64w + 63 and all 256 activation rows).
//
// A Q6_K super-block of a 256-row tile is 53.8 KB, so two of them do not fit
// in LDS beside the X stages; the unit staged here is a half super-block
// (128 elements, two k-steps), 8 aligned 16-byte chunks per weight row:
// chunks 0-3 the half's 64 low-nibble bytes, 4-5 its 32 high-pair bytes, 6
// the block's 16 scales, 7 the block's last 16 bytes (d in bytes 14-15, so
// no load reaches past the block's last dword).  The
// blocks are only 2-byte aligned, so each chunk is loaded as the 20 aligned
// bytes that contain it and shifted into place (realign16) before its LDS
// write.  Thread t always stages chunk t mod 8 of rows t / 8 + 32i.  Rows
// are 9 chunks apart in LDS: at 8 (128 bytes) the 32 rows one lane group
// reads would share two bank groups; at 144 bytes they spread over 16.
//
// Lane l of wave w feeds weight rows 64w + 32f + (l & 31) at k = 16kk +
// 8(l >> 5) + 0..7 of k-slice kk.  Within quarter c4 = 2h + C2 of the
// super-block these are elements 128h + 64C2 + 16kk + 8(l >> 5) + 0..7, i.e.
// group g = 2C2 + kk/2 and position p = 16(kk & 1) + 8(l >> 5) + 0..7: low
// bits from half bytes 32(kk/2) + p (low nibbles for C2 = 0, high for
// C2 = 1), high bits from half bytes p of the qh part shifted by 2g, scale
// 8h + 4C2 + kk.  Value (d·s)·(q − 32) in f32, as the decode (q6k_chunk).
//
// Pipeline: X as in gemm_kernel.  Raw weights: two half-super-block buffers;
// during the two k-steps of half hx the 8 chunks per thread of half hx + 1
// are loaded (4 per step, one step ahead in a register set) and written to
// the other buffer, last read in half hx − 1.  K ranges start on even steps.
// ---------------------------------------------------------------------------
constexpr int kR6Chunks = 256 * 8;                  // 16-byte chunks of a tile half super-block
constexpr int kR6Stride = 9;                        // LDS chunks per row
constexpr int kR6PerThread = kR6Chunks / kThreads;  // 8
static_assert(kR6PerThread * kThreads == kR6Chunks, "chunks per thread");

// The lane's bytes of one k-step for its two weight rows, and the four
// factors d·s of its k-slices.
struct R6Raw {
    u32x2 ql[2][4], qh[2][2];
    float ds[2][4];
};

// h: the half of the super-block the step lies in; C2: its quarter in the half.
// The low-bit bytes of k-slice KK for the lane's two weight rows.
template <int KK>
__device__ __forceinline__ void r6_fetch_ql(const u32x4 *Bc, int lane, int wave, R6Raw &r) {
    const int hl = lane >> 5;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const u32x2 *q2 =
            reinterpret_cast<const u32x2 *>(Bc + (wave * 64 + f * 32 + (lane & 31)) * kR6Stride);
        r.ql[f][KK] = q2[4 * (KK >> 1) + 2 * (KK & 1) + hl];
    }
}

// Everything of the step but the low-bit bytes of k-slices 1-3 (read during
// the slice before each, r6_fetch_ql).
template <int C2>
__device__ __forceinline__ void r6_fetch(const u32x4 *Bc, int h, int lane, int wave, R6Raw &r) {
    const int hl = lane >> 5;
    r6_fetch_ql<0>(Bc, lane, wave, r);
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const u32x4 *blk = Bc + (wave * 64 + f * 32 + (lane & 31)) * kR6Stride;
        const u32x2 *h2 = reinterpret_cast<const u32x2 *>(blk + 4);
        r.qh[f][0] = h2[hl];
        r.qh[f][1] = h2[2 + hl];
        const uint32_t sw = reinterpret_cast<const uint32_t *>(blk + 6)[2 * h + C2];
        const float d = f16_bits_to_f32(reinterpret_cast<const uint32_t *>(blk + 7)[3] >> 16);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) r.ds[f][kk] = d * (float)(int)(int8_t)(sw >> (8 * kk));
    }
}

template <int C2, int KK>
__device__ __forceinline__ half8 q6k_frag(const R6Raw &r, int f) {
    constexpr uint32_t L = 0x0F0F0F0Fu, H = 0x03030303u;
    constexpr uint32_t n4 = 4 * C2, h2 = 4 * C2 + 2 * (KK >> 1);
    const u32x2 l = r.ql[f][KK], hb = r.qh[f][KK & 1];
    const uint32_t q0 = ((l.x >> n4) & L) | (((hb.x >> h2) & H) << 4);
    const uint32_t q1 = ((l.y >> n4) & L) | (((hb.y >> h2) & H) << 4);
    return __builtin_bit_cast(half8, q6k_chunk(q0, q1, r.ds[f][KK]));
}

template <int C2, int FM, class Slot>
__device__ __forceinline__ void rb6_step(const u32x4 *Ac, const u32x4 *Bc, int h,
                                         f32x16 (&acc)[FM][2], int lane, int wave, Slot &&slot) {
    R6Raw raw;
    r6_fetch<C2>(Bc, h, lane, wave, raw);
    half8 af[2][FM], bf[2][2];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[0][i] = rb_a_frag(Ac, 0, i, lane);
    bf[0][0] = q6k_frag<C2, 0>(raw, 0);
    bf[0][1] = q6k_frag<C2, 0>(raw, 1);
    static_for<4>([&](auto KK) MQ_INLINE {
        constexpr int kk = KK, c = kk & 1;
        __builtin_amdgcn_sched_barrier(0);
        static_for<2 * FM>([&](auto IJ) MQ_INLINE {
            constexpr int i = IJ / 2, f = IJ % 2, n = kk * 2 * FM + IJ;
            acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[c][i], bf[c][f], acc[i][f], 0, 0,
                                                               0);
            if constexpr (kk + 1 < 4)
                rb_next_operands<FM, IJ>(
                    [&](auto I) MQ_INLINE {
                        af[c ^ 1][I] = rb_a_frag(Ac, kk + 1, I, lane);
                        // the next slice's low-bit bytes, FM MFMAs before use
                        if constexpr (I == 0) r6_fetch_ql<kk + 1>(Bc, lane, wave, raw);
                    },
                    [&](auto F) MQ_INLINE { bf[c ^ 1][F] = q6k_frag<C2, kk + 1>(raw, F); });
            if constexpr (n & 1) {
                __builtin_amdgcn_sched_barrier(0);
                slot(std::integral_constant<int, n / 2>());
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    });
}

// r6_fetch in two parts, for placing between MFMAs: the LDS reads (the
// factors' scale word and d in sw, db), then the factors d·s.
template <int C2>
__device__ __forceinline__ void r6_fetch_rows(const u32x4 *Bc, int h, int lane, int wave, R6Raw &r,
                                              uint32_t (&sw)[2], uint32_t (&db)[2]) {
    const int hl = lane >> 5;
    r6_fetch_ql<0>(Bc, lane, wave, r);
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const u32x4 *blk = Bc + (wave * 64 + f * 32 + (lane & 31)) * kR6Stride;
        const u32x2 *h2 = reinterpret_cast<const u32x2 *>(blk + 4);
        r.qh[f][0] = h2[hl];
        r.qh[f][1] = h2[2 + hl];
        sw[f] = reinterpret_cast<const uint32_t *>(blk + 6)[2 * h + C2];
        db[f] = reinterpret_cast<const uint32_t *>(blk + 7)[3] >> 16;
    }
}
__device__ __forceinline__ void r6_fetch_factors(R6Raw &r, const uint32_t (&sw)[2],
                                                 const uint32_t (&db)[2]) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const float d = f16_bits_to_f32(db[f]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) r.ds[f][kk] = d * (float)(int)(int8_t)(sw[f] >> (8 * kk));
    }
}

// rb6_step with the step's barrier inside: on entry raw holds the step's
// bytes (low-bit bytes of k-slice 0 only), af[0] its slice-0 A fragments and
// bf0 its slice-0 B fragments; mid() — the barrier — runs between slices 2
// and 3, and slice 3 prepares the next step (quarter C2N, half hn, raw bytes
// in Bnx, X stage An) in raw, af[0] and bf0, so that it starts on operands
// already in registers.
template <int C2, int C2N, int FM, class Slot, class Mid>
__device__ __forceinline__ void rb6_step_x(const u32x4 *Ac, const u32x4 *Bc, const u32x4 *An,
                                           const u32x4 *Bnx, int hn, f32x16 (&acc)[FM][2],
                                           R6Raw &raw, half8 (&af)[2][FM], half8 (&bf0)[2],
                                           int lane, int wave, Slot &&slot, Mid &&mid) {
    static_assert(FM >= 4, "a slice needs FM + 3 MFMAs to place the operands");
    half8 bf[2][2];
    bf[0][0] = bf0[0];
    bf[0][1] = bf0[1];
    uint32_t sw[2], db[2];
    static_for<4>([&](auto KK) MQ_INLINE {
        constexpr int kk = KK, c = kk & 1;
        __builtin_amdgcn_sched_barrier(0);
        static_for<2 * FM>([&](auto IJ) MQ_INLINE {
            constexpr int i = IJ / 2, f = IJ % 2, n = kk * 2 * FM + IJ;
            acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[c][i], bf[c][f], acc[i][f], 0, 0,
                                                               0);
            if constexpr (kk + 1 < 4) {
                rb_next_operands<FM, IJ>(
                    [&](auto I) MQ_INLINE {
                        af[c ^ 1][I] = rb_a_frag(Ac, kk + 1, I, lane);
                        // the next slice's low-bit bytes, FM MFMAs before use
                        if constexpr (I == 0) r6_fetch_ql<kk + 1>(Bc, lane, wave, raw);
                    },
                    [&](auto F) MQ_INLINE { bf[c ^ 1][F] = q6k_frag<C2, kk + 1>(raw, F); });
            } else if constexpr (IJ == 0) {
                // the last slice's operands are made: the next step's bytes
                __builtin_amdgcn_sched_barrier(0);
                r6_fetch_rows<C2N>(Bnx, hn, lane, wave, raw, sw, db);
                __builtin_amdgcn_sched_barrier(0);
            } else if constexpr (IJ == FM) {
                __builtin_amdgcn_sched_barrier(0);
                r6_fetch_factors(raw, sw, db);
                bf0[0] = q6k_frag<C2N, 0>(raw, 0);
                __builtin_amdgcn_sched_barrier(0);
            } else if constexpr (IJ == FM + 2) {
                __builtin_amdgcn_sched_barrier(0);
                bf0[1] = q6k_frag<C2N, 0>(raw, 1);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                // the other positions, in order: the next step's slice-0 A
                constexpr int skip = (IJ > 0) + (IJ > FM) + (IJ > FM + 2);
                constexpr int ia = IJ - skip;
                if constexpr (ia < FM) {
                    __builtin_amdgcn_sched_barrier(0);
                    af[0][ia] = rb_a_frag(An, 0, ia, lane);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (n & 1) {
                __builtin_amdgcn_sched_barrier(0);
                slot(std::integral_constant<int, n / 2>());
                __builtin_amdgcn_sched_barrier(0);
            }
        });
        if constexpr (kk == 2) {
            __builtin_amdgcn_sched_barrier(0);
            mid();
            __builtin_amdgcn_sched_barrier(0);
        }
    });
}

template <int FMT, int BM>
__global__ __launch_bounds__(kThreads, 1) void gemm_q6k_rb_kernel(Args a) {
    static_assert(FMT == kFmtQ6_K, "Q6_K only");
    static_assert(BM == 64 || BM == 128 || BM == 256, "tiles of 64, 128 or 256 rows");
    constexpr int BN = 256, BK = 64, CPR = 8;
    constexpr int FM = BM / 32, FN = 2, TM = BM, TN = 64;
    __shared__ u32x4 A0[BM * CPR], A1[BM * CPR];
    __shared__ u32x4 Bq0[256 * kR6Stride], Bq1[256 * kR6Stride];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = 0, wn = wave;
    const int pid = blockIdx.x;
    int tile, part = 0;
    if (pid < a.dp_tiles) {
        tile = xcd_remap(pid, a.dp_tiles);
    } else {
        const int j = xcd_remap(pid - a.dp_tiles, (int)gridDim.x - a.dp_tiles);
        const int tt = j % a.tail_tiles;
        tile = a.dp_tiles + tt;
        part = j / a.tail_tiles;
    }
    const bool tail = pid >= a.dp_tiles;
    int tm, tn;
    tile_coords(tile, a.tiles_m, a.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    // A tile at or past the matrix edge has nothing to compute; stopping
    // here keeps every buffer range below built from a positive extent.
    if (m0 >= a.M || n0 >= a.N) return;
    // K ranges start on even steps and (K a multiple of 256) end on even ones
    const int kt_begin = tail ? part * a.steps_per_split : 0;
    const int kt_end = tail ? min(kt_begin + a.steps_per_split, a.k_steps) : a.k_steps;
    const int hx_end = kt_end >> 1;

    F16Loader<BM> la;
    la.init((const uint16_t *)a.X + (int64_t)m0 * a.ldx, min(BM, a.M - m0), a.ldx, a.K);
    constexpr int NA = decltype(la)::NPART;
    // raw weight chunks: the resource starts at the 16-byte boundary at or
    // below the tile's first row; chunk p = thread mod 8 of rows r0 + 32i
    const int rows_valid = min(BN, a.N - n0);
    const int64_t start = (int64_t)n0 * a.ldw;
    const uint32_t shift0 = (uint32_t)(((uintptr_t)a.W + start) & 15);
    const int64_t extent = shift0 + (int64_t)rows_valid * a.ldw;
    const __amdgpu_buffer_rsrc_t rsb =
        make_rsrc(a.W + start - shift0, (uint32_t)((extent + 3) & ~(int64_t)3));
    const int p = (int)threadIdx.x & 7, r0 = (int)threadIdx.x >> 3;
    const uint32_t psrc0 = p < 4 ? 16u * p : (p < 6 ? 128u + 16u * (p - 4) : (p == 6 ? 192u : 194u));
    const uint32_t phalf = p < 4 ? 64u : (p < 6 ? 32u : 0u);   // + phalf·h for half h
    uint32_t roff[kR6PerThread];
#pragma unroll
    for (int i = 0; i < kR6PerThread; ++i) roff[i] = shift0 + (uint32_t)((r0 + 32 * i) * a.ldw) + psrc0;
    uint32_t bv[2][4][5], bsh[2][4];
    // load chunk i of half hx into slot (set, j)
    auto bload = [&](int set, int j, int i, int hx) MQ_INLINE {
        const uint32_t o = hx < hx_end ? roff[i] + (uint32_t)(hx >> 1) * 210u + phalf * (hx & 1)
                                       : kOOB;
        bsh[set][j] = o & 2;
        load5(rsb, o, bv[set][j]);
    };
    auto bstore = [&](int set, int j, int i, u32x4 *buf) MQ_INLINE {
        buf[(r0 + 32 * i) * kR6Stride + p] = realign16(bv[set][j], bsh[set][j]);
    };

    // the step's operands, prepared during the previous step (rb6_step_x)
    R6Raw raw;
    half8 af[2][FM], bf0[2];
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // prologue: half kt_begin / 2 whole in its buffer, X step kt_begin in
    // stage 0, X step kt_begin + 1 and part 0 of the next half in set 1
    {
        const int hx0 = kt_begin >> 1, k0 = kt_begin * BK;
        u32x4 *B = (hx0 & 1) ? Bq1 : Bq0;
        la.begin(0, k0, true);
#pragma unroll
        for (int i = 0; i < NA; ++i) la.load(0, i);
#pragma unroll
        for (int i = 0; i < 4; ++i) bload(0, i, i, hx0);
        la.begin(1, k0 + BK, kt_begin + 1 < kt_end);
#pragma unroll
        for (int i = 0; i < NA; ++i) la.load(1, i);
#pragma unroll
        for (int i = 0; i < 4; ++i) bstore(0, i, i, B);
#pragma unroll
        for (int i = 0; i < 4; ++i) bload(0, i, 4 + i, hx0);
#pragma unroll
        for (int i = 0; i < 4; ++i) bload(1, i, i, hx0 + 1);
#pragma unroll
        for (int i = 0; i < NA; ++i) la.store(0, i, A0);
#pragma unroll
        for (int i = 0; i < 4; ++i) bstore(0, i, 4 + i, B);
        sync_lds();
        r6_fetch<0>(B, hx0 & 1, lane, wave, raw);   // kt_begin is even: quarter 0
#pragma unroll
        for (int i = 0; i < FM; ++i) af[0][i] = rb_a_frag(A0, 0, i, lane);
        bf0[0] = q6k_frag<0, 0>(raw, 0);
        bf0[1] = q6k_frag<0, 0>(raw, 1);
    }

    // Step kt (C2 = kt & 1 = P): slots 0..15 load part 1 − C2 of the half
    // that step kt + 1 writes (half kt/2 + 1 for C2 = 0, kt/2 + 2 for C2 = 1)
    // into set P; slots 8..23 (k-slices 1 and 2) write set 1 − P (part C2 of
    // half kt/2 + 1); the step's barrier follows slice 2 (rb6_step_x), after
    // which the next step's bytes are read: from this half's buffer after
    // quarter 0, from the next half's (complete) after quarter 1.
    auto step = [&](auto C2c, int kt) MQ_INLINE {
        constexpr int C2 = decltype(C2c)::value, P = C2;
        constexpr int H = 2 * FM, NB = 4;   // H: half the step's slots
        u32x4 *An = P ? A0 : A1;
        const int hx = kt >> 1;
        const u32x4 *Bc = (hx & 1) ? Bq1 : Bq0;
        u32x4 *Bn = (hx & 1) ? Bq0 : Bq1;
        const int hl_next = C2 == 0 ? hx + 1 : hx + 2;
        constexpr int lpart = 1 - C2;
        la.begin(P, (kt + 2) * BK, kt + 2 < kt_end);
        constexpr int TOT = NA + NB;
        rb6_step_x<C2, 1 - C2>(
            P ? A1 : A0, Bc, An, C2 == 0 ? Bc : Bn, C2 == 0 ? (hx & 1) : ((hx + 1) & 1), acc, raw,
            af, bf0, lane, wave,
            [&](auto SL) MQ_INLINE {
                constexpr int sl = SL;
                if constexpr (sl < H) {
                    constexpr int lo = sl * TOT / H, hi = (sl + 1) * TOT / H;
                    static_for<hi - lo>([&](auto O) MQ_INLINE {
                        constexpr int o = lo + O;
                        if constexpr (o < NA) la.load(P, o);
                        else bload(P, o - NA, 4 * lpart + (o - NA), hl_next);
                    });
                }
                if constexpr (sl >= H / 2 && sl < H / 2 + H) {
                    constexpr int w = sl - H / 2;
                    constexpr int lo = w * TOT / H, hi = (w + 1) * TOT / H;
                    static_for<hi - lo>([&](auto O) MQ_INLINE {
                        constexpr int o = lo + O;
                        if constexpr (o < NA) la.store(1 - P, o, An);
                        else bstore(1 - P, o - NA, 4 * C2 + (o - NA), Bn);
                    });
                }
            },
            [&]() MQ_INLINE { sync_lds(); });
    };
    for (int kt = kt_begin; kt < kt_end; kt += 2) {
        step(std::integral_constant<int, 0>(), kt);
        step(std::integral_constant<int, 1>(), kt + 1);
    }
    store_tile<BM, BN, FM, FN, TM, TN, 4, (int)sizeof(A0), (int)sizeof(Bq0)>(
        a, acc, tail, part, tile, m0, n0, wm, wn, lane, wave, A0, A1, Bq0, Bq1);
}


// ---------------------------------------------------------------------------
// Fused GEMM for the 32-element block formats (Q8_0, Q4_0, Q5_0, Q5_1) on
// 256 × 256 tiles, expanded in the MFMA operand registers (the layout of
// gemm_q6k_rb_kernel).  For K a multiple of 256 only: a row is then K/256
// runs of 8 blocks (272, 144, 176 or 192 bytes), so every row starts on a
// 16-byte boundary.
//
// The 2×2 loaders read each lane's block as two or three loads (16 + 4 [+ 4]
// or 16 + 16 + 4 aligned bytes), and every one of them touches the 1-2 lines
// of 32 rows: the L1 sees each line two or three times.  Here the unit staged
// in LDS is half a run (4 blocks, two k-steps): the CH aligned 16-byte chunks
// that cover it (a half of 136, 72 or 88 bytes starts 8 bytes into a chunk
// when it is odd), loaded once each, consecutive threads on consecutive
// chunks of a row.  Thread t stages chunks c = t + 256i (i < CH) of the
// tile's 256 × CH, row c / CH, chunk c mod CH, at LDS chunk S·row + chunk mod
// the odd stride S, which spreads the 32 rows a lane group reads over 16
// bank groups.
//
// Lane l of wave w feeds weight rows 64w + 32f + (l & 31) at k = 16kk +
// 8(l >> 5) + 0..7 of k-slice kk.  Within step C2 of the half these are
// block b = 2C2 + kk/2, elements e0 = 16(kk & 1) + 8(l >> 5) + 0..7: for
// Q8_0 the int8 bytes 2 + e0.., else the nibbles of bytes (e0 & 15).. (low
// for kk even) with, for Q5_0 / Q5_1, bits e0.. of qh as the 16s bits.  Block
// b starts at byte BB·b + o of the staged row (o = 8 for odd Q8_0 / Q4_0 /
// Q5_0 halves), so each field sits at a byte offset known at compile time up
// to whole dwords, and is read as one dword or two realigned by 2 bytes.
// Values: Q8_0 d·q (q80_chunk); Q4_0 / Q5_0 d·(q − 8 / 16) as one fma of
// d·q and −8d / −16d, Q5_1 fma(d, q, m): the decode's f32 values (d·q and the
// constant are exact), rounded once to f16.
//
// Pipeline as gemm_q6k_rb_kernel: two half buffers; during the two k-steps
// of half hx the CH chunks per thread of half hx + 1 are loaded (P0, then
// CH − P0, one step ahead in a register set) and written to the other
// buffer, last read in half hx − 1.  K ranges start on even steps.
// ---------------------------------------------------------------------------
template <int FMT>
struct B32Rb;
template <>
struct B32Rb<kFmtQ8_0> {
    static constexpr int BB = 34, CH = 9, S = 9, P0 = 5, QS = 2, QH = 0;
};
template <>
struct B32Rb<kFmtQ4_0> {
    static constexpr int BB = 18, CH = 5, S = 5, P0 = 3, QS = 2, QH = 0;
};
template <>
struct B32Rb<kFmtQ5_0> {
    static constexpr int BB = 22, CH = 6, S = 7, P0 = 3, QS = 6, QH = 2;
};
template <>
struct B32Rb<kFmtQ5_1> {
    static constexpr int BB = 24, CH = 6, S = 7, P0 = 3, QS = 8, QH = 4;
};

// Chunks [lo, hi) of the thread's CH belong to part c.
template <int FMT, int C>
struct B32Part {
    static constexpr int lo = C == 0 ? 0 : B32Rb<FMT>::P0;
    static constexpr int hi = C == 0 ? B32Rb<FMT>::P0 : B32Rb<FMT>::CH;
};

// The 4 bytes at byte offset OFF (even) of a dword-aligned row.
template <int OFF>
__device__ __forceinline__ uint32_t rd32(const uint32_t *rw) {
    static_assert(OFF % 2 == 0, "fields are 2-byte aligned");
    if constexpr (OFF % 4 == 0) return rw[OFF / 4];
    else return __builtin_amdgcn_alignbyte(rw[OFF / 4 + 1], rw[OFF / 4], 2);
}

// The lane's quant dwords of one k-step for its two weight rows (per
// k-slice: bytes for Q8_0, 5- or 4-bit values in bytes otherwise) and the
// two blocks' d and additive constant.
struct B32Raw {
    uint32_t q[2][4][2];
    float d[2][2], c[2][2];
};

// o4: the staged row's first block at dword o4 (0, or 2 for odd halves of
// Q8_0, Q4_0 and Q5_0).
template <int FMT, int C2>
__device__ __forceinline__ void b32_fetch_row(const u32x4 *Bc, int o4, int lane, int wave, int f,
                                              B32Raw &r) {
    using G = B32Rb<FMT>;
    const int hl = lane >> 5;
    {
        const uint32_t *rw =
            reinterpret_cast<const uint32_t *>(Bc + (wave * 64 + f * 32 + (lane & 31)) * G::S) + o4;
        const uint32_t *rh = rw + 2 * hl;   // + 8 bytes for the upper half-wave
        static_for<4>([&](auto KK) MQ_INLINE {
            constexpr int kk = KK, b0 = G::BB * (2 * C2 + (kk >> 1));
            if constexpr (FMT == kFmtQ8_0) {
                constexpr int o = b0 + 2 + 16 * (kk & 1);
                r.q[f][kk][0] = rd32<o>(rh);
                r.q[f][kk][1] = rd32<o + 4>(rh);
            } else {
                constexpr int o = b0 + G::QS, n4 = 4 * (kk & 1);
                uint32_t n0 = (rd32<o>(rh) >> n4) & 0x0F0F0F0Fu;
                uint32_t n1 = (rd32<o + 4>(rh) >> n4) & 0x0F0F0F0Fu;
                if constexpr (FMT != kFmtQ4_0) {
                    const uint32_t hb = rd32<b0 + G::QH>(rw) >> (16 * (kk & 1) + 8 * hl);
                    n0 |= spread4_to_bit4(hb & 15);
                    n1 |= spread4_to_bit4((hb >> 4) & 15);
                }
                r.q[f][kk][0] = n0;
                r.q[f][kk][1] = n1;
            }
        });
        static_for<2>([&](auto BBc) MQ_INLINE {
            constexpr int bb = BBc, b0 = G::BB * (2 * C2 + bb);
            const uint32_t w = rd32<b0>(rw);
            const float d = f16_bits_to_f32(w);
            r.d[f][bb] = d;
            if constexpr (FMT == kFmtQ4_0) r.c[f][bb] = -8.0f * d;
            else if constexpr (FMT == kFmtQ5_0) r.c[f][bb] = -16.0f * d;
            else if constexpr (FMT == kFmtQ5_1) r.c[f][bb] = f16_bits_to_f32(w >> 16);
            else r.c[f][bb] = 0.0f;
        });
    }
}
template <int FMT, int C2>
__device__ __forceinline__ void b32_fetch(const u32x4 *Bc, int o4, int lane, int wave, B32Raw &r) {
#pragma unroll
    for (int f = 0; f < 2; ++f) b32_fetch_row<FMT, C2>(Bc, o4, lane, wave, f, r);
}

template <int FMT, int KK>
__device__ __forceinline__ half8 b32_frag(const B32Raw &r, int f) {
    const float d = r.d[f][KK >> 1];
    if constexpr (FMT == kFmtQ8_0) {
        return __builtin_bit_cast(half8, q80_chunk(r.q[f][KK][0], r.q[f][KK][1], d));
    } else {
        // opaque: the masked bytes stay single v_cvt_f32_ubyteK conversions
        const uint32_t w0 = opaque(r.q[f][KK][0]), w1 = opaque(r.q[f][KK][1]);
        const float c = r.c[f][KK >> 1];
        return __builtin_bit_cast(
            half8, pack8(__builtin_fmaf(d, ubyte_f32<0>(w0), c), __builtin_fmaf(d, ubyte_f32<1>(w0), c),
                         __builtin_fmaf(d, ubyte_f32<2>(w0), c), __builtin_fmaf(d, ubyte_f32<3>(w0), c),
                         __builtin_fmaf(d, ubyte_f32<0>(w1), c), __builtin_fmaf(d, ubyte_f32<1>(w1), c),
                         __builtin_fmaf(d, ubyte_f32<2>(w1), c), __builtin_fmaf(d, ubyte_f32<3>(w1), c)));
    }
}

template <int FMT, int C2, int FM, class Slot>
__device__ __forceinline__ void b32_step(const u32x4 *Ac, const u32x4 *Bc, int o4,
                                         f32x16 (&acc)[FM][2], int lane, int wave, Slot &&slot) {
    B32Raw raw;
    b32_fetch<FMT, C2>(Bc, o4, lane, wave, raw);
    half8 af[2][FM], bf[2][2];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[0][i] = rb_a_frag(Ac, 0, i, lane);
    bf[0][0] = b32_frag<FMT, 0>(raw, 0);
    bf[0][1] = b32_frag<FMT, 0>(raw, 1);
    static_for<4>([&](auto KK) MQ_INLINE {
        constexpr int kk = KK, c = kk & 1;
        __builtin_amdgcn_sched_barrier(0);
        static_for<2 * FM>([&](auto IJ) MQ_INLINE {
            constexpr int i = IJ / 2, f = IJ % 2, n = kk * 2 * FM + IJ;
            acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[c][i], bf[c][f], acc[i][f], 0, 0,
                                                               0);
            if constexpr (kk + 1 < 4)
                rb_next_operands<FM, IJ>(
                    [&](auto I) MQ_INLINE { af[c ^ 1][I] = rb_a_frag(Ac, kk + 1, I, lane); },
                    [&](auto F) MQ_INLINE { bf[c ^ 1][F] = b32_frag<FMT, kk + 1>(raw, F); });
            if constexpr (n & 1) {
                __builtin_amdgcn_sched_barrier(0);
                slot(std::integral_constant<int, n / 2>());
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    });
}

// b32_step with the step's barrier inside (as rb6_step_x): raw, af[0] and
// bf0 hold the step's bytes and slice-0 fragments on entry; slice 3, after
// the barrier, prepares the next step's (quarter C2N, first block at dword
// o4n of buffer Bnx, X stage An).
template <int FMT, int C2, int C2N, int FM, class Slot, class Mid>
__device__ __forceinline__ void b32_step_x(const u32x4 *Ac, const u32x4 *An, const u32x4 *Bnx,
                                           int o4n, f32x16 (&acc)[FM][2], B32Raw &raw,
                                           half8 (&af)[2][FM], half8 (&bf0)[2], int lane,
                                           int wave, Slot &&slot, Mid &&mid) {
    static_assert(FM >= 4, "a slice needs FM + 3 MFMAs to place the operands");
    half8 bf[2][2];
    bf[0][0] = bf0[0];
    bf[0][1] = bf0[1];
    static_for<4>([&](auto KK) MQ_INLINE {
        constexpr int kk = KK, c = kk & 1;
        __builtin_amdgcn_sched_barrier(0);
        static_for<2 * FM>([&](auto IJ) MQ_INLINE {
            constexpr int i = IJ / 2, f = IJ % 2, n = kk * 2 * FM + IJ;
            acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[c][i], bf[c][f], acc[i][f], 0, 0,
                                                               0);
            if constexpr (kk + 1 < 4) {
                rb_next_operands<FM, IJ>(
                    [&](auto I) MQ_INLINE { af[c ^ 1][I] = rb_a_frag(Ac, kk + 1, I, lane); },
                    [&](auto F) MQ_INLINE { bf[c ^ 1][F] = b32_frag<FMT, kk + 1>(raw, F); });
            } else if constexpr (IJ == 0 || IJ == 2) {
                // the last slice's operands are made: the next step's bytes
                __builtin_amdgcn_sched_barrier(0);
                b32_fetch_row<FMT, C2N>(Bnx, o4n, lane, wave, IJ / 2, raw);
                __builtin_amdgcn_sched_barrier(0);
            } else if constexpr (IJ == FM || IJ == FM + 2) {
                __builtin_amdgcn_sched_barrier(0);
                bf0[(IJ - FM) / 2] = b32_frag<FMT, 0>(raw, (IJ - FM) / 2);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                // the other positions, in order: the next step's slice-0 A
                constexpr int skip = (IJ > 0) + (IJ > 2) + (IJ > FM) + (IJ > FM + 2);
                constexpr int ia = IJ - skip;
                if constexpr (ia < FM) {
                    __builtin_amdgcn_sched_barrier(0);
                    af[0][ia] = rb_a_frag(An, 0, ia, lane);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (n & 1) {
                __builtin_amdgcn_sched_barrier(0);
                slot(std::integral_constant<int, n / 2>());
                __builtin_amdgcn_sched_barrier(0);
            }
        });
        if constexpr (kk == 2) {
            __builtin_amdgcn_sched_barrier(0);
            mid();
            __builtin_amdgcn_sched_barrier(0);
        }
    });
}

template <int FMT, int BM>
__global__ __launch_bounds__(kThreads, 1) void gemm_b32_rb_kernel(Args a) {
    using G = B32Rb<FMT>;
    static_assert(BM == 64 || BM == 128 || BM == 256, "tiles of 64, 128 or 256 rows");
    constexpr int BN = 256, BK = 64, CPR = 8;
    constexpr int FM = BM / 32, FN = 2, TM = BM, TN = 64;
    constexpr int HB = 4 * G::BB;                  // bytes of a half run
    constexpr int OODD = (HB % 16) / 4;            // odd halves: first block at this dword
    __shared__ u32x4 A0[BM * CPR], A1[BM * CPR];
    __shared__ u32x4 Bq0[256 * G::S], Bq1[256 * G::S];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = 0, wn = wave;
    const int pid = blockIdx.x;
    int tile, part = 0;
    if (pid < a.dp_tiles) {
        tile = xcd_remap(pid, a.dp_tiles);
    } else {
        const int j = xcd_remap(pid - a.dp_tiles, (int)gridDim.x - a.dp_tiles);
        const int tt = j % a.tail_tiles;
        tile = a.dp_tiles + tt;
        part = j / a.tail_tiles;
    }
    const bool tail = pid >= a.dp_tiles;
    int tm, tn;
    tile_coords(tile, a.tiles_m, a.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    // A tile at or past the matrix edge has nothing to compute; stopping
    // here keeps every buffer range below built from a positive extent.
    if (m0 >= a.M || n0 >= a.N) return;
    // K ranges start on even steps and (K a multiple of 256) end on even ones
    const int kt_begin = tail ? part * a.steps_per_split : 0;
    const int kt_end = tail ? min(kt_begin + a.steps_per_split, a.k_steps) : a.k_steps;
    const int hx_end = kt_end >> 1;

    F16Loader<BM> la;
    la.init((const uint16_t *)a.X + (int64_t)m0 * a.ldx, min(BM, a.M - m0), a.ldx, a.K);
    constexpr int NA = decltype(la)::NPART;
    // raw weight chunks (rows 16-byte aligned): chunk c = t + 256i of the
    // tile's 256 × CH is row c / CH, chunk c mod CH, LDS chunk S·row + that
    const int rows_valid = min(BN, a.N - n0);
    const __amdgpu_buffer_rsrc_t rsb =
        make_rsrc(a.W + (int64_t)n0 * a.ldw, (uint32_t)(rows_valid * a.ldw));
    const int t = (int)threadIdx.x;
    uint32_t roff[G::CH];
    int lpos[G::CH];
#pragma unroll
    for (int i = 0; i < G::CH; ++i) {
        const int c = t + kThreads * i, row = c / G::CH, ch = c - row * G::CH;
        roff[i] = (uint32_t)(row * a.ldw) + 16u * (uint32_t)ch;
        lpos[i] = row * G::S + ch;
    }
    constexpr int NSET = G::P0 > G::CH - G::P0 ? G::P0 : G::CH - G::P0;
    u32x4 bv[2][NSET];
    // load chunk i of half hx into slot (set, j): the half's bytes start at
    // HB·hx, in the chunk at or below it
    auto bload = [&](int set, int j, int i, int hx) MQ_INLINE {
        const uint32_t o = hx < hx_end ? roff[i] + (((uint32_t)HB * (uint32_t)hx) & ~15u) : kOOB;
        bv[set][j] = buf_load16(rsb, o);
    };
    auto bstore = [&](int set, int j, int i, u32x4 *buf) MQ_INLINE { buf[lpos[i]] = bv[set][j]; };

    // Q8_0 and Q5_0 run the step with its barrier inside (b32_step_x; Q4_0
    // and Q5_1 would spill registers there and keep b32_step): the step's
    // operands are then prepared during the previous step
    constexpr bool XS = FMT == kFmtQ8_0 || FMT == kFmtQ5_0;
    B32Raw raw;
    half8 af[2][FM], bf0[2];
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // prologue: half kt_begin / 2 whole in its buffer, X step kt_begin in
    // stage 0, X step kt_begin + 1 and part 0 of the next half in set 1
    {
        const int hx0 = kt_begin >> 1, k0 = kt_begin * BK;
        u32x4 *B = (hx0 & 1) ? Bq1 : Bq0;
        la.begin(0, k0, true);
#pragma unroll
        for (int i = 0; i < NA; ++i) la.load(0, i);
#pragma unroll
        for (int i = 0; i < G::P0; ++i) bload(0, i, i, hx0);
        la.begin(1, k0 + BK, kt_begin + 1 < kt_end);
#pragma unroll
        for (int i = 0; i < NA; ++i) la.load(1, i);
#pragma unroll
        for (int i = 0; i < G::P0; ++i) bstore(0, i, i, B);
#pragma unroll
        for (int i = 0; i < G::CH - G::P0; ++i) bload(0, i, G::P0 + i, hx0);
#pragma unroll
        for (int i = 0; i < G::P0; ++i) bload(1, i, i, hx0 + 1);
#pragma unroll
        for (int i = 0; i < NA; ++i) la.store(0, i, A0);
#pragma unroll
        for (int i = 0; i < G::CH - G::P0; ++i) bstore(0, i, G::P0 + i, B);
        sync_lds();
        if constexpr (XS) {
            b32_fetch<FMT, 0>(B, OODD * (hx0 & 1), lane, wave, raw);   // kt_begin is even
#pragma unroll
            for (int i = 0; i < FM; ++i) af[0][i] = rb_a_frag(A0, 0, i, lane);
            bf0[0] = b32_frag<FMT, 0>(raw, 0);
            bf0[1] = b32_frag<FMT, 0>(raw, 1);
        }
    }

    // Step kt (C2 = kt & 1 = P): slots 0..15 load part 1 − C2 of the half
    // that step kt + 1 writes (half kt/2 + 1 for C2 = 0, kt/2 + 2 for C2 = 1)
    // into set P; slots 16..31 write set 1 − P (part C2 of half kt/2 + 1),
    // or with XS slots 8..23 (k-slices 1 and 2), the step's barrier following
    // slice 2, after which the next step's bytes are read: from this half's
    // buffer after quarter 0, from the next half's (complete) after quarter 1.
    auto step = [&](auto C2c, int kt) MQ_INLINE {
        constexpr int C2 = decltype(C2c)::value, P = C2;
        constexpr int H = 2 * FM;   // half the step's slots
        constexpr int lpart = 1 - C2;
        constexpr int NBL = B32Part<FMT, lpart>::hi - B32Part<FMT, lpart>::lo;
        constexpr int NBS = B32Part<FMT, C2>::hi - B32Part<FMT, C2>::lo;
        u32x4 *An = P ? A0 : A1;
        const int hx = kt >> 1;
        const u32x4 *Bc = (hx & 1) ? Bq1 : Bq0;
        u32x4 *Bn = (hx & 1) ? Bq0 : Bq1;
        const int hl_next = C2 == 0 ? hx + 1 : hx + 2;
        la.begin(P, (kt + 2) * BK, kt + 2 < kt_end);
        if constexpr (!XS) {
            b32_step<FMT, C2>(P ? A1 : A0, Bc, OODD * (hx & 1), acc, lane, wave, [&](auto SL) MQ_INLINE {
                constexpr int sl = SL, half = sl < H ? sl : sl - H;
                constexpr int TOT = NA + (sl < H ? NBL : NBS);
                constexpr int lo = half * TOT / H, hi = (half + 1) * TOT / H;
                static_for<hi - lo>([&](auto O) MQ_INLINE {
                    constexpr int o = lo + O;
                    if constexpr (sl < H) {
                        if constexpr (o < NA) la.load(P, o);
                        else bload(P, o - NA, B32Part<FMT, lpart>::lo + (o - NA), hl_next);
                    } else {
                        if constexpr (o < NA) la.store(1 - P, o, An);
                        else bstore(1 - P, o - NA, B32Part<FMT, C2>::lo + (o - NA), Bn);
                    }
                });
            });
            sync_lds();
            return;
        }
        const int hxn = C2 == 0 ? hx : hx + 1;
        b32_step_x<FMT, C2, 1 - C2>(
            P ? A1 : A0, An, C2 == 0 ? Bc : Bn, OODD * (hxn & 1), acc, raw, af, bf0, lane, wave,
            [&](auto SL) MQ_INLINE {
                constexpr int sl = SL;
                if constexpr (sl < H) {
                    constexpr int lo = sl * (NA + NBL) / H, hi = (sl + 1) * (NA + NBL) / H;
                    static_for<hi - lo>([&](auto O) MQ_INLINE {
                        constexpr int o = lo + O;
                        if constexpr (o < NA) la.load(P, o);
                        else bload(P, o - NA, B32Part<FMT, lpart>::lo + (o - NA), hl_next);
                    });
                }
                if constexpr (sl >= H / 2 && sl < H / 2 + H) {
                    constexpr int w = sl - H / 2;
                    constexpr int lo = w * (NA + NBS) / H, hi = (w + 1) * (NA + NBS) / H;
                    static_for<hi - lo>([&](auto O) MQ_INLINE {
                        constexpr int o = lo + O;
                        if constexpr (o < NA) la.store(1 - P, o, An);
                        else bstore(1 - P, o - NA, B32Part<FMT, C2>::lo + (o - NA), Bn);
                    });
                }
            },
            [&]() MQ_INLINE { sync_lds(); });
    };
    for (int kt = kt_begin; kt < kt_end; kt += 2) {
        step(std::integral_constant<int, 0>(), kt);
        step(std::integral_constant<int, 1>(), kt + 1);
    }
    store_tile<BM, BN, FM, FN, TM, TN, 4, (int)sizeof(A0), (int)sizeof(Bq0)>(
        a, acc, tail, part, tile, m0, n0, wm, wn, lane, wave, A0, A1, Bq0, Bq1);
}

}  // namespace
}  // namespace mq
