// Prefill GEMM Y = X·Wᵀ on gfx950 MFMA, for the f16 cache and for the fused
// (quantized-B) shape.
//
// minfer "05 · 8p — Persistent f16 weight cache + fused dequant-in-GEMM":
// §2 gives both shapes (f16 B operand read from the resident cache; or B
// tiles taken from the quantized bytes and expanded to f16 in registers
// inside the GEMM) and §3.3 requires the fused expansion to follow the
// standalone decode's rounding path exactly.  Fucina "Eager GPU Offload
// Without A Compute Graph" (quantized linears): f16-input matrix-core tiles
// with f32 accumulation, and a K split with fixed-order reduction when the
// output grid leaves compute units idle.
//
// Layout of the work (one workgroup per output tile: 4 wave64s, or 8 for the
// f16-cache tiles narrower than 256 × 256, see gemm_kernel):
//   * block tile BM×BN of Y, k-step 64; X and W are both K-contiguous, so
//     each lane feeds MFMA 8 consecutive k of one row (one 16-byte LDS read);
//   * X and B tiles are double-buffered in LDS as rows of eight 16-byte
//     chunks, chunk index XOR-swizzled by row so that the 32 rows a
//     v_mfma_f32_32x32x16_f16 operand reads land in distinct banks;
//   * global loads go to registers two k-steps ahead and are written to LDS
//     one step ahead; both are spread between the MFMAs of the current step,
//     so the address path and LDS stay busy while the matrix cores run, and
//     only one barrier per k-step is needed;
//   * the waves (2×2, or 4×2 / 2×4 of 8) each own a sub-tile of 32×32 MFMA
//     blocks;
//   * global loads go through buffer resources: rows past M/N and k past K
//     read as zeros, so ragged edges need no branches in the inner loop;
//   * workgroup ids are remapped so consecutive tiles (sharing a W panel)
//     run on the same XCD and hit the same L2.
// The fused B loaders fetch the raw block bytes of a k-step into registers
// (Q4_K with 16-byte loads; Q6_K/Q8_0 blocks are 2-byte aligned, so as
// aligned dwords re-assembled with v_alignbyte), expand them to f16 in
// registers with the decode arithmetic of the standalone dequant kernel, and
// store the f16 tile to LDS: each weight element is expanded once per block
// tile (⌈M/BM⌉ times in all), not once per wave.  Fused Q4_K and Q6_K on
// 256 × 256 tiles have kernels of their own (gemm_q4k_rb_kernel,
// gemm_q6k_rb_kernel, gemm_b32_rb_kernel for the 32-element block formats
// with K a multiple of 256, below) that
// stage raw (half) super-blocks or block runs in LDS and expand them in the
// MFMA operand registers.

#pragma once

#include "mq_device.h"
#include "mq_internal.h"

#include <type_traits>
#include <utility>

namespace mq {
namespace {

constexpr int kThreads = 256;

// Calls f(std::integral_constant<int, I>()) for I = 0 .. N−1, in order, so that
// loop indices are compile-time constants in the body (register arrays
// indexed by them stay in registers).
#define MQ_INLINE __attribute__((always_inline))
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>()), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>());
}

constexpr int kBK = 64;        // k elements per step of the fused (quantized-B) kernels
constexpr int kCUs = 256;      // MI355X compute units
constexpr int kXCDs = 8;

struct Args {
    const void *X;      // activations: f16, or f32 for the XF32 kernels
    const uint8_t *W;   // f16 cache (as bytes) or quantized bytes
    float *Y;           // output
    float *ws;          // partial tiles of the K-split tail tiles
    int64_t ldw;        // f16: elements; quantized: bytes per row
    int ldx, ldy;
    int M, N, K;
    int tiles_m, tiles_n, k_steps, steps_per_split;
    int dp_tiles, tail_tiles;
};

// LDS tiles are rows of CPR 16-byte chunks (CPR = k-step / 8: 8 for a 64-wide
// step, 4 for a 32-wide one); chunk c of row r is stored at position
// c ^ swz<CPR>(r).  The LDS (64 banks of 4 bytes) serves a ds_read_b128 16
// lanes at a time, and the 16 lanes of an MFMA operand read 16 consecutive
// rows at one logical chunk: the swizzle puts them on 16 distinct 16-byte
// bank groups.  It depends only on r mod 16, so a lane that loads rows r0,
// r0 + 32, ... (or r0 + 64, ...) keeps the same chunk.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
    if constexpr (CPR == 8)
        return (r & 7) ^ ((r >> 3) & 1);   // row = 128 B: bank group 8·(r&1) + position
    else
        return (r >> 2) & 3;               // row = 64 B: bank group 4·(r&3) + position
}

// Workgroups are dealt to the 8 XCDs round-robin; give each XCD a contiguous
// range of logical tiles so tiles sharing operands share an L2.
__device__ __forceinline__ int xcd_remap(int pid, int total) {
    const int q = total / kXCDs, r = total - q * kXCDs;
    const int xcd = pid % kXCDs, local = pid / kXCDs;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
}

// Logical tile -> (M tile, N tile).  Tiles are taken in groups of kGroupM
// M-tiles, N-tile by N-tile: the 32 tiles an XCD runs at once then cover
// 4 M-tiles × 8 N-tiles, whose operands (4 X panels + 8 W panels per k-step)
// are shared through that XCD's L2 with fewer misses than 8 × 4 would have.
constexpr int kGroupM = 4;
__device__ __forceinline__ void tile_coords(int tile, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int per_group = kGroupM * tiles_n;
    const int g = tile / per_group, r = tile - g * per_group;
    const int gm = min(kGroupM, tiles_m - g * kGroupM);   // the last group may be narrower
    tn = r / gm;
    tm = g * kGroupM + (r - tn * gm);
}

// ---------------------------------------------------------------------------
// Loaders.  Every operand loader has two register sets (the k-steps in
// flight) and splits a k-step into NPART parts per thread:
//   begin(set, k0, live)  per-step offsets of set `set` for the step at k0
//                         (live == false: a look-ahead past the partition,
//                         every load of the step reads zeros);
//   load(set, i)          issue the global loads of part i into the set;
//   store(set, i, lds)    write part i of the set (expanded to f16) to LDS.
// `set` and `i` are compile-time constants after unrolling.
// ---------------------------------------------------------------------------

// f16 tile of ROWS rows × 64 k: 8 chunks of 16 bytes per row.  Thread t
// takes chunk t % 8 of rows t / 8 + 32·i: a wave load covers 8 whole 128-byte
// row segments, and the thread's chunk keeps one swizzled LDS position.
template <int ROWS, int NTH = kThreads>
struct F16Loader {
    static constexpr int NPART = ROWS * 8 / NTH;
    static constexpr int RSTEP = NTH / 8;   // rows between a thread's parts
    __amdgpu_buffer_rsrc_t rs;
    uint32_t off0;     // byte offset of the thread's chunk at k = 0
    uint32_t stride;   // bytes between its parts
    uint32_t kc;       // k of the chunk within a step
    int lds0;          // LDS slot (16-byte units) of part 0
    int K;
    uint32_t obase[2];
    u32x4 v[2][NPART];

    __device__ void init(const uint16_t *base, int rows_valid, int64_t ld, int K_) {
        K = K_;
        rs = make_rsrc(base, (uint32_t)((rows_valid - 1) * ld * 2 + (int64_t)K_ * 2));
        const int t = threadIdx.x, r0 = t >> 3, c = t & 7;
        off0 = (uint32_t)(r0 * ld * 2 + c * 16);
        stride = (uint32_t)(RSTEP * ld * 2);
        kc = (uint32_t)(c * 8);
        lds0 = r0 * 8 + (c ^ swz<8>(r0));   // swz depends on r mod 16 only
    }
    __device__ __forceinline__ void begin(int set, int k0, bool live) {
        obase[set] = live && (uint32_t)k0 + kc < (uint32_t)K ? off0 + (uint32_t)k0 * 2 : kOOB;
    }
    __device__ __forceinline__ void load(int set, int i) {
        v[set][i] = buf_load16(rs, obase[set] + (uint32_t)i * stride);
    }
    __device__ __forceinline__ void store(int set, int i, u32x4 *lds) const {
        lds[lds0 + i * RSTEP * 8] = v[set][i];
    }
};

// Eight f32 values to one 16-byte chunk of f16.
__device__ __forceinline__ u32x4 pack8(float v0, float v1, float v2, float v3, float v4, float v5,
                                       float v6, float v7) {
    return u32x4{pack_f16x2(v0, v1), pack_f16x2(v2, v3), pack_f16x2(v4, v5), pack_f16x2(v6, v7)};
}

// f32 activations rounded to f16 on their way to LDS (Fucina "Eager GPU
// Offload Without A Compute Graph", quantized linears: f32 activation loads
// converted to half while the operand tile is staged).  Same thread → (row,
// 8-element chunk) map as the f16 loader; a chunk is two 16-byte loads, and
// each element is rounded once, to nearest even, when the chunk is stored.
template <int ROWS>
struct XF32Loader {
    static constexpr int NPART = ROWS * 8 / kThreads;
    static constexpr int RSTEP = kThreads / 8;
    __amdgpu_buffer_rsrc_t rs;
    uint32_t off0, stride, kc;
    int lds0;
    int K;
    uint32_t obase[2];
    u32x4 v[2][NPART][2];

    __device__ void init(const float *base, int rows_valid, int64_t ld, int K_) {
        K = K_;
        rs = make_rsrc(base, (uint32_t)((rows_valid - 1) * ld * 4 + (int64_t)K_ * 4));
        const int t = threadIdx.x, r0 = t >> 3, c = t & 7;
        off0 = (uint32_t)(r0 * ld * 4 + c * 32);
        stride = (uint32_t)(RSTEP * ld * 4);
        kc = (uint32_t)(c * 8);
        lds0 = r0 * 8 + (c ^ swz<8>(r0));
    }
    __device__ __forceinline__ void begin(int set, int k0, bool live) {
        obase[set] = live && (uint32_t)k0 + kc < (uint32_t)K ? off0 + (uint32_t)k0 * 4 : kOOB;
    }
    __device__ __forceinline__ void load(int set, int i) {
        const uint32_t o = obase[set] + (uint32_t)i * stride;
        v[set][i][0] = buf_load16(rs, o);
        v[set][i][1] = buf_load16(rs, o + 16);
    }
    __device__ __forceinline__ void store(int set, int i, u32x4 *lds) const {
        const u32x4 a = v[set][i][0], b = v[set][i][1];
        auto f = [](uint32_t u) { return __builtin_bit_cast(float, u); };
        lds[lds0 + i * RSTEP * 8] = pack8(f(a.x), f(a.y), f(a.z), f(a.w), f(b.x), f(b.y), f(b.z),
                                          f(b.w));
    }
};

// Q4_K: value fl32(A·q − C), A = d·sc, C = dmin·m, for the 8 nibbles of two dwords.
__device__ __forceinline__ u32x4 q4k_chunk(uint32_t w0, uint32_t w1, float A, float C) {
    w0 = opaque(w0);
    w1 = opaque(w1);
    return pack8(__builtin_fmaf(A, ubyte_f32<0>(w0), -C), __builtin_fmaf(A, ubyte_f32<1>(w0), -C),
                 __builtin_fmaf(A, ubyte_f32<2>(w0), -C), __builtin_fmaf(A, ubyte_f32<3>(w0), -C),
                 __builtin_fmaf(A, ubyte_f32<0>(w1), -C), __builtin_fmaf(A, ubyte_f32<1>(w1), -C),
                 __builtin_fmaf(A, ubyte_f32<2>(w1), -C), __builtin_fmaf(A, ubyte_f32<3>(w1), -C));
}

// ---------------------------------------------------------------------------
// Q4_K B loader.  A 64-element k-step is one quarter (c4) of a super-block:
// sub-blocks 2·c4 (low nibbles) and 2·c4 + 1 (high nibbles) of the 32 quant
// bytes at 16 + 32·c4.  Thread (row, p) takes the 16 bytes at 16·p of those.
// ---------------------------------------------------------------------------
template <int ROWS>
struct Q4KLoader {
    static constexpr int NPART = ROWS * 2 / kThreads;
    __amdgpu_buffer_rsrc_t rs;
    uint32_t roff[NPART];
    uint32_t obase[2];
    int c4[2];
    u32x4 hdr[2][NPART], qs[2][NPART];

    __device__ void init(const uint8_t *W, int64_t row_bytes, int n0, int rows_valid, int) {
        rs = make_rsrc(W + (int64_t)n0 * row_bytes, (uint32_t)(rows_valid * row_bytes));
#pragma unroll
        for (int i = 0; i < NPART; ++i) {
            const int r = (i * kThreads + (int)threadIdx.x) >> 1;
            roff[i] = (uint32_t)(r * row_bytes);
        }
    }
    __device__ __forceinline__ void begin(int set, int k0, bool live) {
        c4[set] = (k0 >> 6) & 3;
        obase[set] = live ? (uint32_t)(k0 >> 8) * 144u : kOOB;
    }
    __device__ __forceinline__ void load(int set, int i) {
        const uint32_t o = roff[i] + obase[set];
        hdr[set][i] = buf_load16(rs, o);
        qs[set][i] = buf_load16(rs, o + 16 + 32 * c4[set] + 16 * ((int)threadIdx.x & 1));
    }
    __device__ __forceinline__ void store(int set, int i, u32x4 *lds) const {
        const int p = (int)threadIdx.x & 1, c = c4[set];
        const int r = (i * kThreads + (int)threadIdx.x) >> 1;
        const u32x4 h = hdr[set][i];
        uint32_t sc0, m0, sc1, m1;
        if (c < 2) {  // sub-blocks 2c, 2c+1 < 4: low 6 bits of s[j] / s[j+4]
            const int s0 = 16 * c, s1 = 16 * c + 8;
            sc0 = (h.y >> s0) & 63;
            m0 = (h.z >> s0) & 63;
            sc1 = (h.y >> s1) & 63;
            m1 = (h.z >> s1) & 63;
        } else {      // sub-blocks 4..7: nibbles of s[j+4], top bits of s[j-4] / s[j]
            const int s0 = 16 * (c - 2), s1 = s0 + 8;
            sc0 = ((h.w >> s0) & 15) | (((h.y >> (s0 + 6)) & 3) << 4);
            m0 = ((h.w >> (s0 + 4)) & 15) | (((h.z >> (s0 + 6)) & 3) << 4);
            sc1 = ((h.w >> s1) & 15) | (((h.y >> (s1 + 6)) & 3) << 4);
            m1 = ((h.w >> (s1 + 4)) & 15) | (((h.z >> (s1 + 6)) & 3) << 4);
        }
        const float d = f16_bits_to_f32(h.x), dmin = f16_bits_to_f32(h.x >> 16);
        const float A0 = d * (float)sc0, C0 = dmin * (float)m0;
        const float A1 = d * (float)sc1, C1 = dmin * (float)m1;
        const u32x4 q = qs[set][i];
        const uint32_t L = 0x0F0F0F0Fu;
        u32x4 *row = lds + r * 8;
        const int sw = swz<8>(r);
        row[(2 * p) ^ sw] = q4k_chunk(q.x & L, q.y & L, A0, C0);
        row[(2 * p + 1) ^ sw] = q4k_chunk(q.z & L, q.w & L, A0, C0);
        row[(4 + 2 * p) ^ sw] = q4k_chunk((q.x >> 4) & L, (q.y >> 4) & L, A1, C1);
        row[(5 + 2 * p) ^ sw] = q4k_chunk((q.z >> 4) & L, (q.w >> 4) & L, A1, C1);
    }
};

// 16 bytes at a 2-byte-aligned offset, from the 5 aligned dwords w[0..4]:
// sh = 2 when the field starts at the upper half of w[0], else 0 (one
// v_alignbyte per dword, no select).
__device__ __forceinline__ u32x4 realign16(const uint32_t w[5], uint32_t sh) {
    return u32x4{__builtin_amdgcn_alignbyte(w[1], w[0], sh), __builtin_amdgcn_alignbyte(w[2], w[1], sh),
                 __builtin_amdgcn_alignbyte(w[3], w[2], sh), __builtin_amdgcn_alignbyte(w[4], w[3], sh)};
}

__device__ __forceinline__ void load5(__amdgpu_buffer_rsrc_t rs, uint32_t o, uint32_t w[5]) {
    const uint32_t a = o & ~3u;
    const u32x4 v = buf_load16(rs, a);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
    w[4] = buf_load4(rs, a + 16);
}

// Q6_K: the 8 elements (bytes of q) of two dwords, value (d·s)·(q − 32).
// ds = d·s has at most 18 significant bits, so q·ds (q < 64) and 32·ds are
// exact in f32 and one fma gives the exact (q − 32)·ds, as the decode's
// subtract-then-multiply does, in one instruction less.  Only an exact zero
// may differ in sign (+0 here where the decode keeps −0 for ds < 0); these
// values feed only MFMAs, whose sums start at +0, so Y is the same.
__device__ __forceinline__ u32x4 q6k_chunk(uint32_t q0, uint32_t q1, float ds) {
    q0 = opaque(q0);
    q1 = opaque(q1);
    const float c = -32.0f * ds;
    return pack8(__builtin_fmaf(ds, ubyte_f32<0>(q0), c), __builtin_fmaf(ds, ubyte_f32<1>(q0), c),
                 __builtin_fmaf(ds, ubyte_f32<2>(q0), c), __builtin_fmaf(ds, ubyte_f32<3>(q0), c),
                 __builtin_fmaf(ds, ubyte_f32<0>(q1), c), __builtin_fmaf(ds, ubyte_f32<1>(q1), c),
                 __builtin_fmaf(ds, ubyte_f32<2>(q1), c), __builtin_fmaf(ds, ubyte_f32<3>(q1), c));
}

// ---------------------------------------------------------------------------
// Q6_K B loader.  k-step c4 of a super-block lies in half h = c4/2 and covers
// groups g = 2·(c4&1) and g + 1.  Thread (row, p) takes l = 16p..16p+15 of
// both groups: 16 low-nibble bytes per group, 16 high-bit bytes, 2 scales.
// Blocks are 2-byte aligned, so every field is read as aligned dwords.
// ---------------------------------------------------------------------------
template <int ROWS>
struct Q6KLoader {
    // The two quarters of a 128-element half (c4 = 2h, 2h + 1: consecutive
    // k-steps) use the same ql and qh bytes with other nibbles and bit
    // pairs.  The even quarter loads them; when its set is written to LDS the
    // raw dwords are copied into the other set, and the odd quarter loads only
    // its scales and d.  This needs register set == quarter parity, i.e. every
    // K range starting at an even k-step (the plan rounds Q6_K ranges so).
    static constexpr int NPART = ROWS * 2 / kThreads;
    __amdgpu_buffer_rsrc_t rs;
    uint32_t roff[NPART];
    uint32_t obase[2];
    int c4[2];
    mutable uint32_t wa[2][NPART][5], wb[2][NPART][5], wh[2][NPART][5], odd[2][NPART];
    uint32_t wsa[2][NPART], wsb[2][NPART], wd[2][NPART], osc[2][NPART];

    __device__ void init(const uint8_t *W, int64_t row_bytes, int n0, int rows_valid, int) {
        const int64_t start = (int64_t)n0 * row_bytes;
        const uint32_t shift0 = (uint32_t)(((uintptr_t)W + start) & 15);
        const int64_t extent = shift0 + (int64_t)rows_valid * row_bytes;
        rs = make_rsrc(W + start - shift0, (uint32_t)((extent + 3) & ~(int64_t)3));
#pragma unroll
        for (int i = 0; i < NPART; ++i) {
            const int r = (i * kThreads + (int)threadIdx.x) >> 1;
            roff[i] = shift0 + (uint32_t)(r * row_bytes);
        }
    }
    __device__ __forceinline__ void begin(int set, int k0, bool live) {
        c4[set] = (k0 >> 6) & 3;
        obase[set] = live ? (uint32_t)(k0 >> 8) * 210u : kOOB;
    }
    __device__ __forceinline__ void load(int set, int i) {
        const uint32_t h = c4[set] >> 1, gp = c4[set] & 1, p = (int)threadIdx.x & 1;
        const uint32_t o = roff[i] + obase[set];
        if ((set & 1) == 0) {                 // even quarter: the raw bytes
            odd[set][i] = o & 2;
            load5(rs, o + 64 * h + 16 * p, wa[set][i]);
            load5(rs, o + 64 * h + 32 + 16 * p, wb[set][i]);
            load5(rs, o + 128 + 32 * h + 16 * p, wh[set][i]);
        }
        const uint32_t xs = o + 192 + 8 * h + 4 * gp + p;
        osc[set][i] = xs & 3;
        wsa[set][i] = buf_load4(rs, xs & ~3u);
        wsb[set][i] = buf_load4(rs, (xs + 2) & ~3u);
        wd[set][i] = buf_load4(rs, (o + 208) & ~3u);
    }
    __device__ __forceinline__ void store(int set, int i, u32x4 *lds) const {
        const int p = (int)threadIdx.x & 1;
        const uint32_t gp = c4[set] & 1;
        const uint32_t n4 = gp ? 4 : 0, sh_a = 4 * gp, sh_b = 4 * gp + 2;
        const uint32_t L = 0x0F0F0F0Fu, H = 0x03030303u;
        const int r = (i * kThreads + (int)threadIdx.x) >> 1;
        const uint32_t sh = odd[set][i];   // 0 or 2
        const u32x4 a = realign16(wa[set][i], sh), b = realign16(wb[set][i], sh),
                    hh = realign16(wh[set][i], sh);
        const uint32_t bsa = 8 * osc[set][i], bsb = 8 * ((osc[set][i] + 2) & 3);
        const float sa = (float)(int)(int8_t)((wsa[set][i] >> bsa) & 0xFF);
        const float sbv = (float)(int)(int8_t)((wsb[set][i] >> bsb) & 0xFF);
        const float d = f16_bits_to_f32(__builtin_amdgcn_alignbyte(wd[set][i], wd[set][i], sh));
        const float dsa = d * sa, dsb = d * sbv;
        const uint32_t qa0 = ((a.x >> n4) & L) | (((hh.x >> sh_a) & H) << 4);
        const uint32_t qa1 = ((a.y >> n4) & L) | (((hh.y >> sh_a) & H) << 4);
        const uint32_t qa2 = ((a.z >> n4) & L) | (((hh.z >> sh_a) & H) << 4);
        const uint32_t qa3 = ((a.w >> n4) & L) | (((hh.w >> sh_a) & H) << 4);
        const uint32_t qb0 = ((b.x >> n4) & L) | (((hh.x >> sh_b) & H) << 4);
        const uint32_t qb1 = ((b.y >> n4) & L) | (((hh.y >> sh_b) & H) << 4);
        const uint32_t qb2 = ((b.z >> n4) & L) | (((hh.z >> sh_b) & H) << 4);
        const uint32_t qb3 = ((b.w >> n4) & L) | (((hh.w >> sh_b) & H) << 4);
        u32x4 *row = lds + r * 8;
        const int sw = swz<8>(r);
        row[(2 * p) ^ sw] = q6k_chunk(qa0, qa1, dsa);
        row[(2 * p + 1) ^ sw] = q6k_chunk(qa2, qa3, dsa);
        row[(4 + 2 * p) ^ sw] = q6k_chunk(qb0, qb1, dsb);
        row[(5 + 2 * p) ^ sw] = q6k_chunk(qb2, qb3, dsb);
        if ((set & 1) == 0) {                 // hand the raw bytes to the odd quarter
#pragma unroll
            for (int k = 0; k < 5; ++k) {
                wa[set ^ 1][i][k] = wa[set][i][k];
                wb[set ^ 1][i][k] = wb[set][i][k];
                wh[set ^ 1][i][k] = wh[set][i][k];
            }
            odd[set ^ 1][i] = odd[set][i];
        }
    }
};

// Q8_0: value d·q for the 8 signed bytes of two dwords.
__device__ __forceinline__ u32x4 q80_chunk(uint32_t w0, uint32_t w1, float d) {
    return pack8(d * sbyte_f32<0>(w0), d * sbyte_f32<1>(w0), d * sbyte_f32<2>(w0),
                 d * sbyte_f32<3>(w0), d * sbyte_f32<0>(w1), d * sbyte_f32<1>(w1),
                 d * sbyte_f32<2>(w1), d * sbyte_f32<3>(w1));
}

// ---------------------------------------------------------------------------
// Q8_0 B loader.  A k-step is two 34-byte blocks per row; thread (row, p)
// takes block 2·step + p: f16 d then 32 int8, read as 9 aligned dwords.
// ---------------------------------------------------------------------------
template <int ROWS>
struct Q80Loader {
    static constexpr int NPART = ROWS * 2 / kThreads;
    __amdgpu_buffer_rsrc_t rs;
    uint32_t roff[NPART];
    uint32_t w[2][NPART][9], odd[2][NPART];
    int nb, blk[2];
    bool live_[2];

    __device__ void init(const uint8_t *W, int64_t row_bytes, int n0, int rows_valid, int K) {
        nb = K >> 5;
        const int64_t start = (int64_t)n0 * row_bytes;
        const uint32_t shift0 = (uint32_t)(((uintptr_t)W + start) & 15);
        const int64_t extent = shift0 + (int64_t)rows_valid * row_bytes;
        rs = make_rsrc(W + start - shift0, (uint32_t)((extent + 3) & ~(int64_t)3));
#pragma unroll
        for (int i = 0; i < NPART; ++i) {
            const int r = (i * kThreads + (int)threadIdx.x) >> 1;
            roff[i] = shift0 + (uint32_t)(r * row_bytes);
        }
    }
    __device__ __forceinline__ void begin(int set, int k0, bool live) {
        blk[set] = (k0 >> 5) + ((int)threadIdx.x & 1);
        live_[set] = live && blk[set] < nb;
    }
    __device__ __forceinline__ void load(int set, int i) {
        const uint32_t o = roff[i] + (uint32_t)blk[set] * 34u;
        odd[set][i] = o & 2;
        const uint32_t a = live_[set] ? (o & ~3u) : kOOB;
        const u32x4 v0 = buf_load16(rs, a), v1 = buf_load16(rs, a + 16);
        uint32_t *q = w[set][i];
        q[0] = v0.x; q[1] = v0.y; q[2] = v0.z; q[3] = v0.w;
        q[4] = v1.x; q[5] = v1.y; q[6] = v1.z; q[7] = v1.w;
        q[8] = buf_load4(rs, a + 32);
    }
    __device__ __forceinline__ void store(int set, int i, u32x4 *lds) const {
        const int p = (int)threadIdx.x & 1;
        const int r = (i * kThreads + (int)threadIdx.x) >> 1;
        const bool oh = odd[set][i] != 0;
        const uint32_t *wv = w[set][i];
        const float d = f16_bits_to_f32(oh ? (wv[0] >> 16) : wv[0]);
        uint32_t q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = oh ? wv[j + 1] : shift2(wv[j + 1], wv[j]);
        u32x4 *row = lds + r * 8;
        const int sw = swz<8>(r);
#pragma unroll
        for (int j = 0; j < 4; ++j) row[(4 * p + j) ^ sw] = q80_chunk(q[2 * j], q[2 * j + 1], d);
    }
};

// The 16s bits of 4 consecutive elements, bits 0..3 of b, moved to bit 4 of
// bytes 0..3 (b·(1 + 2^7 + 2^14 + 2^21) puts bit i at bit 8i; the partial
// products do not overlap).
__device__ __forceinline__ uint32_t spread4_to_bit4(uint32_t b) {
    return ((b * 0x00204081u) & 0x01010101u) << 4;
}

// ---------------------------------------------------------------------------
// Q4_0 / Q5_0 / Q5_1 B loader (32-element blocks of 18 / 22 / 24 bytes).  A
// k-step is two blocks per row; thread (row, p) takes block 2·step + p, read
// as the aligned dwords covering it (Q4_0 and Q5_0 blocks are only 2-byte
// aligned — the Q5_0 qh word at byte 2 included, the misalignment the pages
// report — so every field is re-assembled with v_alignbyte).  Element j of a
// block: nibble j % 16 (low for j < 16), plus for Q5_x bit j of qh as 16s bit.
// ---------------------------------------------------------------------------
template <int ROWS, int FMT>
struct Q32Loader {
    static constexpr int NPART = ROWS * 2 / kThreads;
    static constexpr uint32_t BB = FMT == kFmtQ4_0 ? 18 : FMT == kFmtQ5_0 ? 22 : 24;
    static constexpr uint32_t QH = FMT == kFmtQ5_1 ? 4 : 2;    // qh offset (Q5_x)
    static constexpr uint32_t QS = FMT == kFmtQ4_0 ? 2 : FMT == kFmtQ5_0 ? 6 : 8;
    // dwords held: the block plus up to 2 lead bytes needs 5 (Q4_0) or 6; one
    // more (zero) lets dw<T> read its upper neighbour for every field
    static constexpr int NW = 7;
    __amdgpu_buffer_rsrc_t rs;
    uint32_t roff[NPART];
    uint32_t w[2][NPART][NW], sh[2][NPART];
    int nb, blk[2];
    bool live_[2];

    __device__ void init(const uint8_t *W, int64_t row_bytes, int n0, int rows_valid, int K) {
        nb = K >> 5;
        const int64_t start = (int64_t)n0 * row_bytes;
        const uint32_t shift0 = (uint32_t)(((uintptr_t)W + start) & 15);
        const int64_t extent = shift0 + (int64_t)rows_valid * row_bytes;
        rs = make_rsrc(W + start - shift0, (uint32_t)((extent + 3) & ~(int64_t)3));
#pragma unroll
        for (int i = 0; i < NPART; ++i) {
            const int r = (i * kThreads + (int)threadIdx.x) >> 1;
            roff[i] = shift0 + (uint32_t)(r * row_bytes);
        }
    }
    __device__ __forceinline__ void begin(int set, int k0, bool live) {
        blk[set] = (k0 >> 5) + ((int)threadIdx.x & 1);
        live_[set] = live && blk[set] < nb;
    }
    __device__ __forceinline__ void load(int set, int i) {
        const uint32_t o = roff[i] + (uint32_t)blk[set] * BB;
        sh[set][i] = o & 3;                       // 0 or 2: blocks are 2-byte aligned
        const uint32_t a = live_[set] ? (o & ~3u) : kOOB;
        const u32x4 v0 = buf_load16(rs, a);
        uint32_t *q = w[set][i];
        q[0] = v0.x; q[1] = v0.y; q[2] = v0.z; q[3] = v0.w;
        if constexpr (FMT == kFmtQ4_0) {          // 18 + 2 bytes: 5 dwords
            q[4] = buf_load4(rs, a + 16);
            q[5] = 0;
        } else {                                  // 22 or 24 (+ 2) bytes: 6 dwords
            const uint32_t t = a + 16;
            q[4] = buf_load4(rs, t);
            q[5] = buf_load4(rs, t + 4);
        }
        q[6] = 0;
    }
    // dword of the block at even byte offset T (compile-time), from the raw window
    template <uint32_t T>
    __device__ __forceinline__ uint32_t dw(const uint32_t *q, uint32_t s) const {
        const uint32_t lo = __builtin_amdgcn_alignbyte(q[T / 4 + 1], q[T / 4], s);
        if constexpr (T % 4 == 0) {
            return lo;
        } else {
            const uint32_t hi = __builtin_amdgcn_alignbyte(q[T / 4 + 2], q[T / 4 + 1], s);
            return __builtin_amdgcn_alignbyte(hi, lo, 2);
        }
    }
    __device__ __forceinline__ void store(int set, int i, u32x4 *lds) const {
        const int p = (int)threadIdx.x & 1;
        const int r = (i * kThreads + (int)threadIdx.x) >> 1;
        const uint32_t *q = w[set][i];
        const uint32_t s = sh[set][i];
        const uint32_t h0 = dw<0>(q, s);
        const float d = f16_bits_to_f32(h0);
        const uint32_t n0 = dw<QS>(q, s), n1 = dw<QS + 4>(q, s), n2 = dw<QS + 8>(q, s),
                       n3 = dw<QS + 12>(q, s);
        uint32_t qh = 0;
        if constexpr (FMT != kFmtQ4_0) qh = dw<QH>(q, s);
        u32x4 *row = lds + r * 8;
        const int sw = swz<8>(r);
        const uint32_t L = 0x0F0F0F0Fu;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            // elements 8c .. 8c+7: bytes (8c) % 16 .. +7 of the nibble plane
            const uint32_t a0 = c & 1 ? n2 : n0, a1 = c & 1 ? n3 : n1;
            uint32_t w0 = c < 2 ? (a0 & L) : ((a0 >> 4) & L);
            uint32_t w1 = c < 2 ? (a1 & L) : ((a1 >> 4) & L);
            u32x4 v;
            if constexpr (FMT == kFmtQ4_0) {
                w0 = opaque(w0);
                w1 = opaque(w1);
                // d·q and 8d / 16d are exact in f32: one fma gives the
                // decode's exact d·(q − 8) (only an exact zero's sign may
                // differ, which the MFMA sums starting at +0 do not see)
                const float bias = -8.0f * d;
                v = pack8(__builtin_fmaf(d, ubyte_f32<0>(w0), bias), __builtin_fmaf(d, ubyte_f32<1>(w0), bias),
                          __builtin_fmaf(d, ubyte_f32<2>(w0), bias), __builtin_fmaf(d, ubyte_f32<3>(w0), bias),
                          __builtin_fmaf(d, ubyte_f32<0>(w1), bias), __builtin_fmaf(d, ubyte_f32<1>(w1), bias),
                          __builtin_fmaf(d, ubyte_f32<2>(w1), bias), __builtin_fmaf(d, ubyte_f32<3>(w1), bias));
            } else {
                const uint32_t hb = qh >> (8 * c);
                w0 = opaque(w0 | spread4_to_bit4(hb & 15));
                w1 = opaque(w1 | spread4_to_bit4((hb >> 4) & 15));
                if constexpr (FMT == kFmtQ5_0) {
                    const float bias = -16.0f * d;
                    v = pack8(__builtin_fmaf(d, ubyte_f32<0>(w0), bias), __builtin_fmaf(d, ubyte_f32<1>(w0), bias),
                              __builtin_fmaf(d, ubyte_f32<2>(w0), bias), __builtin_fmaf(d, ubyte_f32<3>(w0), bias),
                              __builtin_fmaf(d, ubyte_f32<0>(w1), bias), __builtin_fmaf(d, ubyte_f32<1>(w1), bias),
                              __builtin_fmaf(d, ubyte_f32<2>(w1), bias), __builtin_fmaf(d, ubyte_f32<3>(w1), bias));
                } else {
                    const float m = f16_bits_to_f32(h0 >> 16);
                    v = pack8(__builtin_fmaf(d, ubyte_f32<0>(w0), m), __builtin_fmaf(d, ubyte_f32<1>(w0), m),
                              __builtin_fmaf(d, ubyte_f32<2>(w0), m), __builtin_fmaf(d, ubyte_f32<3>(w0), m),
                              __builtin_fmaf(d, ubyte_f32<0>(w1), m), __builtin_fmaf(d, ubyte_f32<1>(w1), m),
                              __builtin_fmaf(d, ubyte_f32<2>(w1), m), __builtin_fmaf(d, ubyte_f32<3>(w1), m));
                }
            }
            row[(4 * p + c) ^ sw] = v;
        }
    }
};

// ---------------------------------------------------------------------------
// Q5_K B loader: Q4_K's, plus the 16 qh bytes l = 16p .. 16p+15 of the thread:
// bit j of qh[l] is the 16s bit of element l of sub-block j.  Blocks are 176
// bytes, so every load is 16-byte aligned.
// ---------------------------------------------------------------------------
template <int ROWS>
struct Q5KLoader {
    static constexpr int NPART = ROWS * 2 / kThreads;
    __amdgpu_buffer_rsrc_t rs;
    uint32_t roff[NPART];
    uint32_t obase[2];
    int c4[2];
    u32x4 hdr[2][NPART], qh[2][NPART], qs[2][NPART];

    __device__ void init(const uint8_t *W, int64_t row_bytes, int n0, int rows_valid, int) {
        rs = make_rsrc(W + (int64_t)n0 * row_bytes, (uint32_t)(rows_valid * row_bytes));
#pragma unroll
        for (int i = 0; i < NPART; ++i) {
            const int r = (i * kThreads + (int)threadIdx.x) >> 1;
            roff[i] = (uint32_t)(r * row_bytes);
        }
    }
    __device__ __forceinline__ void begin(int set, int k0, bool live) {
        c4[set] = (k0 >> 6) & 3;
        obase[set] = live ? (uint32_t)(k0 >> 8) * 176u : kOOB;
    }
    __device__ __forceinline__ void load(int set, int i) {
        const uint32_t o = roff[i] + obase[set], p = (int)threadIdx.x & 1;
        hdr[set][i] = buf_load16(rs, o);
        qh[set][i] = buf_load16(rs, o + 16 + 16 * p);
        qs[set][i] = buf_load16(rs, o + 48 + 32 * c4[set] + 16 * p);
    }
    __device__ __forceinline__ void store(int set, int i, u32x4 *lds) const {
        const int p = (int)threadIdx.x & 1, c = c4[set];
        const int r = (i * kThreads + (int)threadIdx.x) >> 1;
        const u32x4 h = hdr[set][i];
        uint32_t sc0, m0, sc1, m1;
        if (c < 2) {
            const int s0 = 16 * c, s1 = 16 * c + 8;
            sc0 = (h.y >> s0) & 63;
            m0 = (h.z >> s0) & 63;
            sc1 = (h.y >> s1) & 63;
            m1 = (h.z >> s1) & 63;
        } else {
            const int s0 = 16 * (c - 2), s1 = s0 + 8;
            sc0 = ((h.w >> s0) & 15) | (((h.y >> (s0 + 6)) & 3) << 4);
            m0 = ((h.w >> (s0 + 4)) & 15) | (((h.z >> (s0 + 6)) & 3) << 4);
            sc1 = ((h.w >> s1) & 15) | (((h.y >> (s1 + 6)) & 3) << 4);
            m1 = ((h.w >> (s1 + 4)) & 15) | (((h.z >> (s1 + 6)) & 3) << 4);
        }
        const float d = f16_bits_to_f32(h.x), dmin = f16_bits_to_f32(h.x >> 16);
        const float A0 = d * (float)sc0, C0 = dmin * (float)m0;
        const float A1 = d * (float)sc1, C1 = dmin * (float)m1;
        const u32x4 q = qs[set][i], hq = qh[set][i];
        const uint32_t L = 0x0F0F0F0Fu, B = 0x01010101u, j0 = 2 * c, j1 = 2 * c + 1;
        u32x4 *row = lds + r * 8;
        const int sw = swz<8>(r);
        row[(2 * p) ^ sw] = q4k_chunk((q.x & L) | (((hq.x >> j0) & B) << 4),
                                      (q.y & L) | (((hq.y >> j0) & B) << 4), A0, C0);
        row[(2 * p + 1) ^ sw] = q4k_chunk((q.z & L) | (((hq.z >> j0) & B) << 4),
                                          (q.w & L) | (((hq.w >> j0) & B) << 4), A0, C0);
        row[(4 + 2 * p) ^ sw] = q4k_chunk(((q.x >> 4) & L) | (((hq.x >> j1) & B) << 4),
                                          ((q.y >> 4) & L) | (((hq.y >> j1) & B) << 4), A1, C1);
        row[(5 + 2 * p) ^ sw] = q4k_chunk(((q.z >> 4) & L) | (((hq.z >> j1) & B) << 4),
                                          ((q.w >> 4) & L) | (((hq.w >> j1) & B) << 4), A1, C1);
    }
};

template <int ROWS, int FMT>
struct BLoaderFor;
template <int ROWS> struct BLoaderFor<ROWS, kFmtF16> { typedef F16Loader<ROWS> T; };
template <int ROWS> struct BLoaderFor<ROWS, kFmtQ4_K> { typedef Q4KLoader<ROWS> T; };
template <int ROWS> struct BLoaderFor<ROWS, kFmtQ6_K> { typedef Q6KLoader<ROWS> T; };
template <int ROWS> struct BLoaderFor<ROWS, kFmtQ8_0> { typedef Q80Loader<ROWS> T; };
template <int ROWS> struct BLoaderFor<ROWS, kFmtQ4_0> { typedef Q32Loader<ROWS, kFmtQ4_0> T; };
template <int ROWS> struct BLoaderFor<ROWS, kFmtQ5_0> { typedef Q32Loader<ROWS, kFmtQ5_0> T; };
template <int ROWS> struct BLoaderFor<ROWS, kFmtQ5_1> { typedef Q32Loader<ROWS, kFmtQ5_1> T; };
template <int ROWS> struct BLoaderFor<ROWS, kFmtQ5_K> { typedef Q5KLoader<ROWS> T; };

// Stage boundary: every LDS access of this wave done, then meet the other
// waves.  The barrier is an asm statement with a memory clobber, so the
// compiler moves no LDS access across it, but it carries none of
// __syncthreads' fences, which would also drain the global loads in flight
// for the next k-steps (their waits are placed by the compiler where the
// registers are consumed; global loads into registers complete in order).
__device__ __forceinline__ void sync_lds() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt at their maxima
    asm volatile("s_barrier" ::: "memory");
}

// MFMA operand fragments of one 16-wide k-slice.
template <int FM, int FN, int TM, int TN>
__device__ __forceinline__ void load_frags(const u32x4 *Ac, const u32x4 *Bc, int kk, int wm,
                                           int wn, int lane, half8 (&af)[FM], half8 (&bf)[FN]) {
    const int c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int r = wm * TM + i * 32 + (lane & 31);
        af[i] = __builtin_bit_cast(half8, Ac[r * 8 + (c ^ swz<8>(r))]);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int r = wn * TN + j * 32 + (lane & 31);
        bf[j] = __builtin_bit_cast(half8, Bc[r * 8 + (c ^ swz<8>(r))]);
    }
}

// One MFMA operand fragment (A when IDX < FM, else B fragment IDX − FM) of
// k-slice kk.
template <int FM, int FN, int TM, int TN, int IDX>
__device__ __forceinline__ half8 load_frag(const u32x4 *Ac, const u32x4 *Bc, int kk, int wm, int wn,
                                           int lane) {
    const int c = kk * 2 + (lane >> 5);
    if constexpr (IDX < FM) {
        const int r = wm * TM + IDX * 32 + (lane & 31);
        return __builtin_bit_cast(half8, Ac[r * 8 + (c ^ swz<8>(r))]);
    } else {
        const int r = wn * TN + (IDX - FM) * 32 + (lane & 31);
        return __builtin_bit_cast(half8, Bc[r * 8 + (c ^ swz<8>(r))]);
    }
}

// One 64-wide k-step of MFMAs from LDS stage (Ac, Bc) into the wave's tile,
// with the loaders' work for other steps threaded through it: after every
// second MFMA, slot(integral_constant<s>) runs, s = 0 .. FM·FN·2 − 1.
// Fragments are double-buffered: the LDS reads of k-slice kk+1 are issued
// before the MFMAs of slice kk, or with SPREAD_REQ one after each of slice
// kk's first FM + FN MFMAs, so that a wave with one SIMD to itself never
// stops feeding the matrix pipe for a burst of reads.  Scheduling barriers fix
// the order, so loads and LDS writes are issued between matrix instructions
// instead of in one burst.
template <int FM, int FN, int TM, int TN, bool SPREAD_REQ = false, class Slot>
__device__ __forceinline__ void mma_step(const u32x4 *Ac, const u32x4 *Bc, f32x16 (&acc)[FM][FN],
                                         int wm, int wn, int lane, Slot &&slot) {
    // spreading needs a slice with at least as many MFMAs as fragments
    constexpr bool SPREAD = SPREAD_REQ && FM * FN >= FM + FN;
    half8 af[2][FM], bf[2][FN];
    load_frags<FM, FN, TM, TN>(Ac, Bc, 0, wm, wn, lane, af[0], bf[0]);
    static_for<4>([&](auto KK) MQ_INLINE {
        constexpr int kk = KK, cur = kk & 1;
        if constexpr (!SPREAD && kk + 1 < 4)
            load_frags<FM, FN, TM, TN>(Ac, Bc, kk + 1, wm, wn, lane, af[cur ^ 1], bf[cur ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
        static_for<FM * FN>([&](auto IJ) MQ_INLINE {
            constexpr int i = IJ / FN, j = IJ % FN, n = (kk * FM + i) * FN + j;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[cur][i], bf[cur][j], acc[i][j], 0,
                                                               0, 0);
            // SPREAD: the next slice's fragments one after each of this slice's
            // first FM + FN MFMAs, in the order the next slice first uses them
            // (A0, B0 .. B(FN−1), A1 .. A(FM−1)), instead of in one burst
            if constexpr (SPREAD && kk + 1 < 4 && IJ < FM + FN) {
                constexpr int idx = IJ == 0 ? 0 : (IJ <= FN ? FM + IJ - 1 : IJ - FN);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (idx < FM)
                    af[cur ^ 1][idx] = load_frag<FM, FN, TM, TN, idx>(Ac, Bc, kk + 1, wm, wn, lane);
                else
                    bf[cur ^ 1][idx - FM] =
                        load_frag<FM, FN, TM, TN, idx>(Ac, Bc, kk + 1, wm, wn, lane);
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

// The 256 × 256 f16 step with its barrier inside: one 64-wide k-step from
// LDS stage (Ac, Bc) whose k-slice 0 fragments are already in af[0], bf[0].
// The next slice's fragments are read one after each of a slice's first
// FM + FN MFMAs (as mma_step with SPREAD_REQ); slot(s) runs after every second
// MFMA; mid() — the step's barrier — runs between slices 2 and 3, and slice
// 3's reads are the next step's slice 0 from stage (An, Bn), so that the next
// step starts on operands already in registers instead of waiting on LDS
// after a barrier.
template <int FM, int FN, int TM, int TN, class Slot, class Mid>
__device__ __forceinline__ void mma_step_x(const u32x4 *Ac, const u32x4 *Bc, const u32x4 *An,
                                           const u32x4 *Bn, f32x16 (&acc)[FM][FN],
                                           half8 (&af)[2][FM], half8 (&bf)[2][FN], int wm, int wn,
                                           int lane, Slot &&slot, Mid &&mid) {
    // the next slice's fragments in the order it first uses them (A0, B0 ..
    // B(FN−1), A1 .. A(FM−1)); number u of them is read after MFMA u·NM/NF
    // of the slice (one after each of the first NF MFMAs when NF <= NM)
    constexpr int NM = FM * FN, NF = FM + FN;
    static_for<4>([&](auto KK) MQ_INLINE {
        constexpr int kk = KK, cur = kk & 1;
        __builtin_amdgcn_sched_barrier(0);
        static_for<NM>([&](auto IJ) MQ_INLINE {
            constexpr int i = IJ / FN, j = IJ % FN, n = (kk * FM + i) * FN + j;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[cur][i], bf[cur][j], acc[i][j], 0,
                                                               0, 0);
            static_for<NF>([&](auto U) MQ_INLINE {
                constexpr int u = U;
                if constexpr ((NF <= NM ? u : u * NM / NF) == IJ) {
                    constexpr int idx = u == 0 ? 0 : (u <= FN ? FM + u - 1 : u - FN);
                    constexpr int ks = kk < 3 ? kk + 1 : 0;
                    const u32x4 *Ar = kk < 3 ? Ac : An, *Br = kk < 3 ? Bc : Bn;
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (idx < FM)
                        af[cur ^ 1][idx] = load_frag<FM, FN, TM, TN, idx>(Ar, Br, ks, wm, wn, lane);
                    else
                        bf[cur ^ 1][idx - FM] =
                            load_frag<FM, FN, TM, TN, idx>(Ar, Br, ks, wm, wn, lane);
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
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

// Write a wave's accumulators: a whole tile's part of Y, or a tail range's
// partial tile to slot (part, tail tile) of the workspace.  C layout of a
// 32x32 MFMA block: the lane holds column (lane & 31) and rows
// 8·(r/4) + 4·(lane/32) + r%4 for accumulator element r; rows and columns of
// a partial tile past M/N hold zeros.  S0, S1 (SA bytes each) and S2, S3 (SB
// bytes each): LDS buffers of the workgroup that are idle once the k-loop is
// done (its X and weight stages); NW: waves per workgroup.
template <int BM, int BN, int FM, int FN, int TM, int TN, int NW, int SA, int SB>
__device__ __forceinline__ void store_tile(const Args &a, f32x16 (&acc)[FM][FN], bool tail,
                                           int part, int tile, int m0, int n0, int wm, int wn,
                                           int lane, int wave, u32x4 *S0, u32x4 *S1, u32x4 *S2,
                                           u32x4 *S3) {
    float *out;
    int64_t ldo;
    int rows, cols;
    if (tail) {
        out = a.ws + ((int64_t)part * a.tail_tiles + (tile - a.dp_tiles)) * (BM * BN);
        ldo = BN;
        rows = BM;
        cols = BN;
    } else {
        out = a.Y + (int64_t)m0 * a.ldy + n0;
        ldo = a.ldy;
        rows = a.M - m0;
        cols = a.N - n0;
    }
    const int col_l = lane & 31, row_l = (lane >> 5) * 4;
    constexpr int PS = 36;                 // patch row stride in floats (keeps 16-byte rows)
    constexpr int PB = 32 * PS * 4;        // bytes of one wave's patch
    constexpr int PA = SA / PB, PBB = SB / PB;   // patches in each S0/S1 and S2/S3
    if constexpr (2 * (PA + PBB) >= NW) {
        // Full tile, 16-byte-aligned rows: each 32x32 block goes through a
        // private 32 x 36-float LDS patch of the wave (the waves' patches are
        // dealt over S0, S1, S2, S3 in that order) so that every lane then
        // stores 4 consecutive columns of one row — a quarter of the store
        // instructions of the column-per-lane layout.
        if (rows >= BM && cols >= BN && (ldo & 3) == 0) {
            u32x4 *buf;
            int slot;
            if (wave < PA) {
                buf = S0;
                slot = wave;
            } else if (wave < 2 * PA) {
                buf = S1;
                slot = wave - PA;
            } else if (wave < 2 * PA + PBB) {
                buf = S2;
                slot = wave - 2 * PA;
            } else {
                buf = S3;
                slot = wave - 2 * PA - PBB;
            }
            float *patch = reinterpret_cast<float *>(buf) + slot * (32 * PS);
            sync_lds();              // every wave is done reading the stages
            const int rr = lane >> 3, cc = 4 * (lane & 7);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        patch[((r >> 2) * 8 + row_l + (r & 3)) * PS + col_l] = acc[i][j][r];
                    // lanes read what other lanes wrote: the LDS runs one wave's
                    // instructions in order, so only the compiler must keep them
                    asm volatile("" ::: "memory");
                    float *dst = out + (int64_t)(wm * TM + i * 32 + rr) * ldo + wn * TN + j * 32 + cc;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4 v = *reinterpret_cast<const f32x4 *>(patch + (rr + 8 * q) * PS + cc);
                        f32x4 *o = reinterpret_cast<f32x4 *>(dst + (int64_t)(8 * q) * ldo);
                        // Y and the partial tiles are not read again by the
                        // kernel: streamed out with non-temporal stores they
                        // do not displace operand panels from L2 (7B down on
                        // the f16 cache, 117 MB of partial tiles: 265 -> 250
                        // us; Y: o -3%, gate|up -0.3..-1.2%, fused 14336 x
                        // 4096 -2%, M = 128 -3%)
                        __builtin_nontemporal_store(v, o);
                    }
                    asm volatile("" ::: "memory");
                }
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = wn * TN + j * 32 + col_l;
            if (col >= cols) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * TM + i * 32 + (r >> 2) * 8 + row_l + (r & 3);
                if (row < rows) out[row * ldo + col] = acc[i][j][r];
            }
        }
}

// ---------------------------------------------------------------------------
// The GEMM kernel.  Two LDS stages and two register sets per operand:
// during step j (MFMAs from LDS stage j%2) each thread issues the global
// loads of step j+2 into register set j%2 (first half of the step's slots)
// and writes register set (j+1)%2, the data of step j+1, to LDS stage
// (j+1)%2 (second half).  The barrier at the end of the step publishes that
// stage; it also orders the reads of stage j%2 before its refill at the end
// of step j+1.  A global load thus has from its issue in step j until the
// second half of step j+1 to arrive.  The tiles with f16 activations and at
// least two MFMAs per wave and k-slice move the barrier inside the step
// (mma_step_x): their LDS writes take k-slices 1 and 2, the barrier follows,
// and slice 3 reads the next step's first fragments from the stage just
// published (a load then has 1.25 steps).
// BM × BN: block tile, split over NWV waves.  NWV = 4 (2×2 waves): one wave
// per SIMD, whose register file then holds a 128 × 128 sub-tile's 256
// accumulators (the 256 × 256 tile) or the fused loaders' raw bytes.  NWV = 8
// (4×2 waves, 2×4 for 64-row tiles): two waves per SIMD for the smaller
// f16-cache tiles, which are bound by LDS throughput rather than by the
// matrix cores — the LDS serves about twice the ds_read_b128 bytes per clock
// with two waves per SIMD issuing (measured 210 vs 109 B/clk per CU), which
// outweighs the third more fragment reads of the smaller wave tiles.
// A workgroup either computes a whole tile over all of K or one K range of
// a tail tile (see the plan); the latter writes its f32 partial tile to the
// workspace.
// ---------------------------------------------------------------------------
template <int BM, int BN, int FMT, bool XF32, int NWV = 4>
__global__ __launch_bounds__(64 * NWV, 1) void gemm_kernel(Args a) {
    static_assert(NWV == 4 || (NWV == 8 && BN == 128 && !XF32), "8 waves: tiles of 128 columns");
    constexpr int BK = 64;
    constexpr int WN = NWV == 4 ? 2 : (BM >= 128 ? 2 : 4), WM = NWV / WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int CPR = BK / 8;
    __shared__ u32x4 A0[BM * CPR], A1[BM * CPR];
    __shared__ u32x4 B0[BN * CPR], B1[BN * CPR];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    // Workgroups [0, dp_tiles) take whole tiles; the rest take one K range of
    // a tail tile.  Each group is remapped over the XCDs on its own (dp_tiles
    // is a multiple of 8, so the round-robin dealing of both starts at XCD 0).
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
    const int kt_begin = tail ? part * a.steps_per_split : 0;
    const int kt_end = tail ? min(kt_begin + a.steps_per_split, a.k_steps) : a.k_steps;

    std::conditional_t<XF32, XF32Loader<BM>, F16Loader<BM, 64 * NWV>> la;
    if constexpr (XF32)
        la.init((const float *)a.X + (int64_t)m0 * a.ldx, min(BM, a.M - m0), a.ldx, a.K);
    else
        la.init((const uint16_t *)a.X + (int64_t)m0 * a.ldx, min(BM, a.M - m0), a.ldx, a.K);
    // The fused B loaders are written for 256 threads: with 8 waves, waves
    // 0-3 run them (the condition is uniform per wave) and all 8 stage X.
    // Waves 4-7 still issue the B loads, at out-of-range offsets that read
    // zeros, and skip only the LDS writes: with the loads under a branch the
    // compiler's wait counts had to cover both paths and made the decoding
    // waves wait for the loads of the current step (M = 128: 14336 x 4096
    // Q8_0 41 -> 52 us).
    std::conditional_t<NWV == 4 || FMT != kFmtF16, typename BLoaderFor<BN, FMT>::T,
                       F16Loader<BN, 64 * NWV>>
        lb;
    const bool bw = NWV == 4 || FMT == kFmtF16 ||
                    __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) < kThreads / 64;
    if constexpr (FMT == kFmtF16)
        lb.init((const uint16_t *)a.W + n0 * a.ldw, min(BN, a.N - n0), a.ldw, a.K);
    else
        lb.init(a.W, a.ldw, n0, min(BN, a.N - n0), a.K);
    constexpr int NA = decltype(la)::NPART, NB = decltype(lb)::NPART;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // prologue: step kt_begin in registers and then in stage 0; step
    // kt_begin + 1 in flight in register set 1
    {
        const int k0 = kt_begin * BK;
        const bool has1 = kt_begin + 1 < kt_end;
        la.begin(0, k0, true);
        lb.begin(0, k0, bw);
#pragma unroll
        for (int i = 0; i < NA; ++i) la.load(0, i);
#pragma unroll
        for (int i = 0; i < NB; ++i) lb.load(0, i);
        la.begin(1, k0 + BK, has1);
        lb.begin(1, k0 + BK, has1 && bw);
#pragma unroll
        for (int i = 0; i < NA; ++i) la.load(1, i);
#pragma unroll
        for (int i = 0; i < NB; ++i) lb.load(1, i);
#pragma unroll
        for (int i = 0; i < NA; ++i) la.store(0, i, A0);
#pragma unroll
        for (int i = 0; i < NB; ++i)
            if (bw) lb.store(0, i, B0);
        sync_lds();
    }
    // the f16-activation tiles with at least two MFMAs per wave and k-slice
    // (all but 64 x 128; the f16 cache and the fused formats' 2 x 2 loaders)
    // run the step with its barrier inside (mma_step_x; the 7B down call 3.7%
    // faster, gate|up 0.5%, q|k|v and o 0.5%; fused o 2-5%, 128-row fused
    // Q6_K at M = 128 1.5%; 64 x 128 measured 0.5% slower): their fragment
    // registers live across steps
    constexpr bool XS = !XF32 && FM * FN >= 2;
    half8 xaf[2][FM], xbf[2][FN];
    if constexpr (XS) load_frags<FM, FN, TM, TN>(A0, B0, 0, wm, wn, lane, xaf[0], xbf[0]);

    // Step kt with P = (kt − kt_begin) % 2.  Slots 0 .. H−1 issue the NA + NB
    // loads of step kt+2 into set P; slots H .. 2H−1 write set 1−P (step
    // kt+1) to stage 1−P.  A look-ahead past the partition loads zeros and
    // writes them to a stage that is never read.
    constexpr int H = FM * FN;   // half the slots of a step
    auto step = [&](auto PC, int kt) MQ_INLINE {
        constexpr int P = decltype(PC)::value;
        u32x4 *An = P ? A0 : A1, *Bn = P ? B0 : B1;
        const bool live2 = kt + 2 < kt_end;
        la.begin(P, (kt + 2) * BK, live2);
        lb.begin(P, (kt + 2) * BK, live2 && bw);
        if constexpr (XS) {
            // slots 0 .. H-1 (k-slices 0 and 1) issue the loads of step kt+2
            // into set P; slots H/2 .. 3H/2-1 (slices 1 and 2) write set 1-P
            // to stage 1-P, published by the barrier before slice 3
            mma_step_x<FM, FN, TM, TN>(
                P ? A1 : A0, P ? B1 : B0, An, Bn, acc, xaf, xbf, wm, wn, lane,
                [&](auto SL) MQ_INLINE {
                    constexpr int sl = SL;
                    if constexpr (sl < H) {
                        constexpr int lo = sl * (NA + NB) / H, hi = (sl + 1) * (NA + NB) / H;
                        static_for<hi - lo>([&](auto O) MQ_INLINE {
                            constexpr int o = lo + O;
                            if constexpr (o < NA) la.load(P, o);
                            else lb.load(P, o - NA);
                        });
                    }
                    if constexpr (sl >= H / 2 && sl < H / 2 + H) {
                        constexpr int w = sl - H / 2;
                        constexpr int lo = w * (NA + NB) / H, hi = (w + 1) * (NA + NB) / H;
                        static_for<hi - lo>([&](auto O) MQ_INLINE {
                            constexpr int o = lo + O;
                            if constexpr (o < NA) la.store(1 - P, o, An);
                            else if (bw) lb.store(1 - P, o - NA, Bn);
                        });
                    }
                },
                [&]() MQ_INLINE { sync_lds(); });
            return;
        }
        // the 256 x 256 f16 tile spreads its fragment reads (2.6% on the 7B
        // gate|up and down calls); on the 128-column tiles it measured no gain
        // and 3% slower on the 7B o projection
        constexpr bool SPREAD = BM == 256 && BN == 256 && FMT == kFmtF16;
        mma_step<FM, FN, TM, TN, SPREAD>(P ? A1 : A0, P ? B1 : B0, acc, wm, wn, lane, [&](auto SL) MQ_INLINE {
            constexpr int sl = SL, half = sl < H ? sl : sl - H;
            constexpr int lo = half * (NA + NB) / H, hi = (half + 1) * (NA + NB) / H;
            static_for<hi - lo>([&](auto O) MQ_INLINE {
                constexpr int o = lo + O;
                if constexpr (sl < H) {
                    if constexpr (o < NA) la.load(P, o);
                    else lb.load(P, o - NA);
                } else {
                    if constexpr (o < NA) la.store(1 - P, o, An);
                    else if (bw) lb.store(1 - P, o - NA, Bn);
                }
            });
        });
        sync_lds();
    };
    // A single-exit loop over pairs of steps, then the tail: with exits inside
    // the pair, the compiler keeps the accumulators in VGPRs across the back
    // edge and copies all of them to and from AGPRs on every round.
    int kt = kt_begin;
    for (const int pairs_end = kt_begin + (kt_end - kt_begin) / 2 * 2; kt < pairs_end; kt += 2) {
        step(std::integral_constant<int, 0>(), kt);
        step(std::integral_constant<int, 1>(), kt + 1);
    }
    if (kt < kt_end) step(std::integral_constant<int, 0>(), kt);

    store_tile<BM, BN, FM, FN, TM, TN, NWV, BM * CPR * 16, BN * CPR * 16>(
        a, acc, tail, part, tile, m0, n0, wm, wn, lane, wave, A0, A1, B0, B1);
}

}  // namespace
}  // namespace mq

#include "gemm_fused_rb.h"

namespace mq {
namespace {

// Y tile = Σ_s partial[s] in the order s = 0, 1, ..., S − 1, for every tail
// tile.  Block (tail tile, chunk) handles 1024 consecutive elements of the
// BM × BN partial tile, four per thread.  All S loads of a thread are issued
// before the first add (S is a compile-time constant), so the partials
// stream in parallel instead of one memory latency per partial; each is read
// once (non-temporal loads).
template <int S>
__global__ __launch_bounds__(256) void splitk_reduce(const float *__restrict__ ws,
                                                     int tail_tiles, int dp_tiles, int bm, int bn,
                                                     int tiles_m, int tiles_n,
                                                     float *__restrict__ Y, int ldy, int M, int N) {
    const int chunks = bm * bn / 1024;
    const int tt = blockIdx.x / chunks;
    const int e = (blockIdx.x - tt * chunks) * 1024 + threadIdx.x * 4;
    const int r = e / bn, c = e - r * bn;
    int tm, tn;
    tile_coords(dp_tiles + tt, tiles_m, tiles_n, tm, tn);
    const int row = tm * bm + r, col = tn * bn + c;
    if (row >= M || col >= N) return;
    const int64_t tile_elems = (int64_t)bm * bn, stride = tile_elems * tail_tiles;
    const float *p = ws + tt * tile_elems + e;
    f32x4 v[S];
#pragma unroll
    for (int s = 0; s < S; ++s) v[s] = __builtin_nontemporal_load((const f32x4 *)(p + s * stride));
    f32x4 acc = v[0];
#pragma unroll
    for (int s = 1; s < S; ++s) acc += v[s];
    float *y = Y + (int64_t)row * ldy + col;
    const int n = min(4, N - col);
    if (n == 4 && (ldy & 3) == 0) {   // Y is 16-byte aligned, and so is this row piece
        *(f32x4 *)y = acc;
        return;
    }
    y[0] = acc.x;
    if (n > 1) y[1] = acc.y;
    if (n > 2) y[2] = acc.z;
    if (n > 3) y[3] = acc.w;
}

// The reduce of `split` partial planes (2 .. 16).
template <int S = 2>
hipError_t launch_splitk_reduce(int split, dim3 grid, hipStream_t stream, const float *ws,
                                int tail_tiles, int dp_tiles, int bm, int bn, int tiles_m,
                                int tiles_n, float *Y, int ldy, int M, int N) {
    if constexpr (S <= 16) {
        if (split != S)
            return launch_splitk_reduce<S + 1>(split, grid, stream, ws, tail_tiles, dp_tiles, bm,
                                               bn, tiles_m, tiles_n, Y, ldy, M, N);
        hipLaunchKernelGGL(splitk_reduce<S>, grid, dim3(256), 0, stream, ws, tail_tiles,
                           dp_tiles, bm, bn, tiles_m, tiles_n, Y, ldy, M, N);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

template <int BM, int BN, int FMT, bool XF32>
hipError_t launch_tile(const Args &a, int grid, hipStream_t stream, bool dry) {
    if (dry) return hipSuccess;
    // Tiles of 128 columns on 8 waves: two waves per SIMD double the LDS
    // throughput a step can draw on.  f16 cache: 1.5-4% faster at M = 128
    // and on the 7B q/o shape, no slower elsewhere.  Fused, with 128 or 256
    // rows: 2-5% faster at M = 2048 (q/o, 4096 x 4096; Q4_K, Q6_K, Q8_0),
    // 2-18% at M = 128, no slower elsewhere.  Fused 64-row tiles keep 4
    // waves (8 gained nothing on k/v and lost 3% at N = 1024).
    constexpr int NWV = (BN == 128 && !XF32 && (FMT == kFmtF16 || BM >= 128)) ? 8 : 4;
    hipLaunchKernelGGL((gemm_kernel<BM, BN, FMT, XF32, NWV>), dim3(grid), dim3(64 * NWV), 0, stream,
                       a);
    return hipGetLastError();
}

// The register-expansion fused kernel of format FMT on BM × 256 tiles
// (Q4_K and Q5_K, Q6_K, and the 32-element block formats when K is a
// multiple of 256); hipErrorNotSupported when there is none.
template <int FMT, int BM>
hipError_t launch_rb(const Args &a, int grid, hipStream_t stream, bool dry) {
    if constexpr (FMT == kFmtQ4_K || FMT == kFmtQ5_K) {
        if (dry) return hipSuccess;
        hipLaunchKernelGGL((gemm_q4k_rb_kernel<FMT, BM>), dim3(grid), dim3(kThreads), 0, stream, a);
        return hipGetLastError();
    } else if constexpr (FMT == kFmtQ6_K) {
        if (dry) return hipSuccess;
        hipLaunchKernelGGL((gemm_q6k_rb_kernel<FMT, BM>), dim3(grid), dim3(kThreads), 0, stream, a);
        return hipGetLastError();
    } else if constexpr (FMT == kFmtQ8_0 || FMT == kFmtQ4_0 || FMT == kFmtQ5_0 ||
                         FMT == kFmtQ5_1) {
        if (a.K % 256 != 0) return hipErrorNotSupported;   // rows of whole 8-block runs only
        if (dry) return hipSuccess;
        hipLaunchKernelGGL((gemm_b32_rb_kernel<FMT, BM>), dim3(grid), dim3(kThreads), 0, stream, a);
        return hipGetLastError();
    }
    return hipErrorNotSupported;
}

// The kernel for the plan's exact (BM, BN); a plan no kernel implements is an
// error, never a launch with a mismatched tile (its grid would address tiles
// past the matrix).  dry: only report whether a kernel exists (hipSuccess)
// or not (hipErrorInvalidValue), launching nothing.
template <int FMT, bool XF32>
hipError_t launch_fmt(const Args &a, int bm, int bn, int grid, hipStream_t stream, bool dry) {
    if (bm == 256 && bn == 256) {
        if constexpr (!XF32 && FMT != kFmtF16) {
            if (hipError_t e = launch_rb<FMT, 256>(a, grid, stream, dry); e != hipErrorNotSupported)
                return e;
        }
        if constexpr (!XF32) return launch_tile<256, 256, FMT, XF32>(a, grid, stream, dry);
    } else if (bm == 256 && bn == 128) {
        return launch_tile<256, 128, FMT, XF32>(a, grid, stream, dry);
    } else if (bm == 128 && bn == 128) {
        return launch_tile<128, 128, FMT, XF32>(a, grid, stream, dry);
    } else if (bm == 64 && bn == 128) {
        return launch_tile<64, 128, FMT, XF32>(a, grid, stream, dry);
    }
    return hipErrorInvalidValue;
}

// The plan's kernel for format `fmt` (kFmtF16: the f16 cache), then, for a
// K split, the fixed-order reduction of the tail tiles' partial planes.
// dry: check that the plan has a kernel and launch nothing.
template <bool XF32>
hipError_t launch_gemm_t(int fmt, const void *X, int ldx, const void *W, int64_t ldw, float *Y,
                         int ldy, int M, int N, int K, const GemmPlan &plan, float *ws,
                         hipStream_t stream, bool dry = false) {
    Args a;
    a.X = X;
    a.W = (const uint8_t *)W;
    a.Y = Y;
    a.ws = ws;
    a.ldw = ldw;
    a.ldx = ldx;
    a.ldy = ldy;
    a.M = M;
    a.N = N;
    a.K = K;
    a.tiles_m = plan.tiles_m;
    a.tiles_n = plan.tiles_n;
    a.k_steps = plan.k_steps;
    a.steps_per_split = plan.steps_per_split;
    a.dp_tiles = plan.dp_tiles;
    a.tail_tiles = plan.tail_tiles;
    const int grid = plan.dp_tiles + plan.tail_tiles * plan.split;
    hipError_t e;
    switch (fmt) {
    case kFmtQ4_K: e = launch_fmt<kFmtQ4_K, XF32>(a, plan.bm, plan.bn, grid, stream, dry); break;
    case kFmtQ6_K: e = launch_fmt<kFmtQ6_K, XF32>(a, plan.bm, plan.bn, grid, stream, dry); break;
    case kFmtQ8_0: e = launch_fmt<kFmtQ8_0, XF32>(a, plan.bm, plan.bn, grid, stream, dry); break;
    case kFmtQ4_0: e = launch_fmt<kFmtQ4_0, XF32>(a, plan.bm, plan.bn, grid, stream, dry); break;
    case kFmtQ5_0: e = launch_fmt<kFmtQ5_0, XF32>(a, plan.bm, plan.bn, grid, stream, dry); break;
    case kFmtQ5_1: e = launch_fmt<kFmtQ5_1, XF32>(a, plan.bm, plan.bn, grid, stream, dry); break;
    case kFmtQ5_K: e = launch_fmt<kFmtQ5_K, XF32>(a, plan.bm, plan.bn, grid, stream, dry); break;
    case kFmtF16: e = launch_fmt<kFmtF16, XF32>(a, plan.bm, plan.bn, grid, stream, dry); break;
    default: e = hipErrorInvalidValue; break;
    }
    if (e != hipSuccess || plan.split == 1 || dry) return e;
    const int blocks = plan.tail_tiles * (plan.bm * plan.bn / 1024);
    return launch_splitk_reduce(plan.split, dim3(blocks), stream, ws, plan.tail_tiles,
                                plan.dp_tiles, plan.bm, plan.bn, plan.tiles_m, plan.tiles_n, Y,
                                ldy, M, N);
}

}  // namespace
}  // namespace mq
