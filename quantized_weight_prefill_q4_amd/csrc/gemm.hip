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
// Layout of the work (one 256-thread workgroup = 4 wave64s per output tile):
//   * block tile BM×BN of Y, k-step 64; X and W are both K-contiguous, so
//     each lane feeds MFMA 8 consecutive k of one row (one 16-byte LDS read);
//   * X and B tiles are double-buffered in LDS as rows of eight 16-byte
//     chunks, chunk index XOR-swizzled by row so that the 32 rows a
//     v_mfma_f32_32x32x16_f16 operand reads land in distinct banks;
//   * the next k-step's global loads are issued before the current step's
//     MFMAs and written to LDS after them (one barrier per k-step);
//   * the 2×2 waves each own a (BM/2)×(BN/2) sub-tile of 32×32 MFMA blocks;
//   * global loads go through buffer resources: rows past M/N and k past K
//     read as zeros, so ragged edges need no branches in the inner loop;
//   * workgroup ids are remapped so consecutive tiles (sharing a W panel)
//     run on the same XCD and hit the same L2.
// The fused B loaders fetch the raw block bytes of a k-step straight into
// registers (Q4_K with 16-byte loads; Q6_K/Q8_0 blocks are 2-byte aligned,
// so as aligned dwords re-assembled with v_alignbyte), expand them to f16 in
// registers with the decode arithmetic of the standalone dequant kernel, and
// store the f16 tile to LDS: each weight element is expanded once per block
// tile (⌈M/BM⌉ times in all), not once per wave.

#include "mq_device.h"
#include "mq_internal.h"

#include <type_traits>

namespace mq {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;        // k elements per step of the fused (quantized-B) kernels
constexpr int kCUs = 256;      // MI355X compute units
constexpr int kXCDs = 8;

struct Args {
    const uint16_t *X;
    const uint8_t *W;   // f16 cache (as bytes) or quantized bytes
    float *Y;           // output, or the partial planes when split > 1
    int64_t ldw;        // f16: elements; quantized: bytes per row
    int64_t plane;      // elements between partial planes
    int ldx, ldy;
    int M, N, K;
    int tiles_m, tiles_n, k_steps, steps_per_split;
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

typedef __attribute__((address_space(3))) void lds_void;

// One buffer_load_dwordx4 ... lds: 16 bytes at `voff` of `rs` for every lane,
// landing at LDS byte address `lds` + 16·lane.  Issued as inline asm so the
// compiler's wait-count bookkeeping does not see it: that bookkeeping loses
// track of which LDS stage a DMA writes at the loop head and would drain every
// look-ahead load before the next LDS read.  The waits for these loads are
// placed explicitly (sync_stage).  M0 is set here and not assumed afterwards
// by compiler-generated code (it is a reserved register there).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, const u32x4 *lds) {
    const uint32_t a = (uint32_t)(uintptr_t)(lds_void *)lds;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(a), "v"(voff), "s"(rs) : "m0");
}
#pragma clang diagnostic pop

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
// f16 tile fetched straight into LDS by gfx950's buffer_load_dwordx4 ... lds:
// ROWS × 8·CPR halves per k-step.  One wave instruction fills 64 consecutive
// 16-byte LDS slots, lane l the l-th; slot s holds row s/CPR at physical chunk
// s%CPR, which is logical chunk (s%CPR) ^ swz(row) of that row.  The lanes of
// a row therefore fetch its contiguous bytes in a permuted order, and no
// VGPRs or ds_write instructions are spent on staging.
// ---------------------------------------------------------------------------
template <int ROWS, int CPR>
struct DmaTile {
    static constexpr int RPI = 64 / CPR;                  // rows per wave instruction
    static constexpr int INSTR = ROWS * CPR / kThreads;   // per wave and k-step
    __amdgpu_buffer_rsrc_t rs;
    uint32_t off0;     // lane's byte offset for instruction 0 at k = 0
    uint32_t kc;       // first k of the lane's chunk within a k-step
    uint32_t stride;   // bytes between the row groups of consecutive instructions
    int K, wave;       // wave index, wave-uniform

    __device__ void init(const uint16_t *base, int rows_valid, int64_t ld, int K_) {
        K = K_;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        rs = make_rsrc(base, (uint32_t)((rows_valid - 1) * ld * 2 + (int64_t)K_ * 2));
        // instruction i fills rows 4·RPI·i + RPI·wave + (0 .. RPI-1); this lane
        // fills row r0 + 4·RPI·i at physical chunk lane % CPR, i.e. logical
        // chunk c (the swizzle of r0 + 4·RPI·i equals that of r0)
        const int lane = threadIdx.x & 63;
        const int r0 = wave * RPI + lane / CPR;
        const int c = (lane % CPR) ^ swz<CPR>(r0);
        off0 = (uint32_t)(r0 * ld * 2 + c * 16);
        kc = (uint32_t)(c * 8);
        stride = (uint32_t)(4 * RPI * ld * 2);
    }
    // live == false: a look-ahead past the last k-step; every lane reads out of
    // range and the (already consumed) stage is filled with zeros.
    __device__ __forceinline__ void issue(int k0, u32x4 *stage, bool live = true) const {
        const uint32_t klim = live ? (uint32_t)K : 0u;   // wave-uniform
        const uint32_t o0 = (uint32_t)k0 + kc < klim ? off0 + k0 * 2 : kOOB;
        static_assert(INSTR * 4 * 64 == ROWS * CPR, "tile rows must fill whole instructions");
#pragma unroll
        for (int i = 0; i < INSTR; ++i) dma16(rs, o0 + i * stride, stage + (i * 4 + wave) * 64);
    }
};

// Eight f32 values to one 16-byte chunk of f16.
__device__ __forceinline__ u32x4 pack8(float v0, float v1, float v2, float v3, float v4, float v5,
                                       float v6, float v7) {
    return u32x4{pack_f16x2(v0, v1), pack_f16x2(v2, v3), pack_f16x2(v4, v5), pack_f16x2(v6, v7)};
}

// Q4_K: value fl32(A·q − C), A = d·sc, C = dmin·m, for the 8 nibbles of two dwords.
__device__ __forceinline__ u32x4 q4k_chunk(uint32_t w0, uint32_t w1, float A, float C) {
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
    static constexpr int PER = ROWS * 2 / kThreads;
    __amdgpu_buffer_rsrc_t rs;
    uint32_t roff[PER];
    u32x4 hdr[PER], qs[PER];
    int c4;

    __device__ void init(const uint8_t *W, int64_t row_bytes, int n0, int rows_valid, int) {
        rs = make_rsrc(W + (int64_t)n0 * row_bytes, (uint32_t)(rows_valid * row_bytes));
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int r = (i * kThreads + (int)threadIdx.x) >> 1;
            roff[i] = (uint32_t)(r * row_bytes);
        }
    }
    __device__ __forceinline__ void load(int k0) {
        c4 = (k0 >> 6) & 3;
        const uint32_t sb = (uint32_t)(k0 >> 8) * 144u, p = (int)threadIdx.x & 1;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const uint32_t o = roff[i] + sb;
            hdr[i] = buf_load16(rs, o);
            qs[i] = buf_load16(rs, o + 16 + 32 * c4 + 16 * p);
        }
    }
    __device__ __forceinline__ void store(u32x4 *lds) const {
        const int p = (int)threadIdx.x & 1;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int r = (i * kThreads + (int)threadIdx.x) >> 1;
            const u32x4 h = hdr[i];
            uint32_t sc0, m0, sc1, m1;
            if (c4 < 2) {  // sub-blocks 2c4, 2c4+1 < 4: low 6 bits of s[j] / s[j+4]
                const int s0 = 16 * c4, s1 = 16 * c4 + 8;
                sc0 = (h.y >> s0) & 63;
                m0 = (h.z >> s0) & 63;
                sc1 = (h.y >> s1) & 63;
                m1 = (h.z >> s1) & 63;
            } else {       // sub-blocks 4..7: nibbles of s[j+4], top bits of s[j-4] / s[j]
                const int s0 = 16 * (c4 - 2), s1 = s0 + 8;
                sc0 = ((h.w >> s0) & 15) | (((h.y >> (s0 + 6)) & 3) << 4);
                m0 = ((h.w >> (s0 + 4)) & 15) | (((h.z >> (s0 + 6)) & 3) << 4);
                sc1 = ((h.w >> s1) & 15) | (((h.y >> (s1 + 6)) & 3) << 4);
                m1 = ((h.w >> (s1 + 4)) & 15) | (((h.z >> (s1 + 6)) & 3) << 4);
            }
            const float d = f16_bits_to_f32(h.x), dmin = f16_bits_to_f32(h.x >> 16);
            const float A0 = d * (float)sc0, C0 = dmin * (float)m0;
            const float A1 = d * (float)sc1, C1 = dmin * (float)m1;
            const u32x4 q = qs[i];
            const uint32_t L = 0x0F0F0F0Fu;
            u32x4 *row = lds + r * 8;
            const int sw = swz<8>(r);
            row[(2 * p) ^ sw] = q4k_chunk(q.x & L, q.y & L, A0, C0);
            row[(2 * p + 1) ^ sw] = q4k_chunk(q.z & L, q.w & L, A0, C0);
            row[(4 + 2 * p) ^ sw] = q4k_chunk((q.x >> 4) & L, (q.y >> 4) & L, A1, C1);
            row[(5 + 2 * p) ^ sw] = q4k_chunk((q.z >> 4) & L, (q.w >> 4) & L, A1, C1);
        }
    }
};

// 16 bytes at a 2-byte-aligned offset, from the 5 aligned dwords w[0..4].
__device__ __forceinline__ u32x4 realign16(const uint32_t w[5], bool odd_half) {
    return odd_half ? u32x4{shift2(w[1], w[0]), shift2(w[2], w[1]), shift2(w[3], w[2]),
                            shift2(w[4], w[3])}
                    : u32x4{w[0], w[1], w[2], w[3]};
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

// Q6_K: 4 elements (bytes of q) of one dword, value (d·s)·(q − 32).
__device__ __forceinline__ u32x4 q6k_chunk(uint32_t q0, uint32_t q1, float ds) {
    return pack8(ds * (ubyte_f32<0>(q0) - 32.0f), ds * (ubyte_f32<1>(q0) - 32.0f),
                 ds * (ubyte_f32<2>(q0) - 32.0f), ds * (ubyte_f32<3>(q0) - 32.0f),
                 ds * (ubyte_f32<0>(q1) - 32.0f), ds * (ubyte_f32<1>(q1) - 32.0f),
                 ds * (ubyte_f32<2>(q1) - 32.0f), ds * (ubyte_f32<3>(q1) - 32.0f));
}

// ---------------------------------------------------------------------------
// Q6_K B loader.  k-step c4 of a super-block lies in half h = c4/2 and covers
// groups g = 2·(c4&1) and g + 1.  Thread (row, p) takes l = 16p..16p+15 of
// both groups: 16 low-nibble bytes per group, 16 high-bit bytes, 2 scales.
// Blocks are 2-byte aligned, so every field is read as aligned dwords.
// ---------------------------------------------------------------------------
template <int ROWS>
struct Q6KLoader {
    static constexpr int PER = ROWS * 2 / kThreads;
    __amdgpu_buffer_rsrc_t rs;
    uint32_t roff[PER];
    uint32_t wa[PER][5], wb[PER][5], wh[PER][5], wsa[PER], wsb[PER], wd[PER];
    uint32_t osc[PER], odd[PER];
    int c4;

    __device__ void init(const uint8_t *W, int64_t row_bytes, int n0, int rows_valid, int) {
        const int64_t start = (int64_t)n0 * row_bytes;
        const uint32_t shift0 = (uint32_t)(((uintptr_t)W + start) & 15);
        const int64_t extent = shift0 + (int64_t)rows_valid * row_bytes;
        rs = make_rsrc(W + start - shift0, (uint32_t)((extent + 3) & ~(int64_t)3));
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int r = (i * kThreads + (int)threadIdx.x) >> 1;
            roff[i] = shift0 + (uint32_t)(r * row_bytes);
        }
    }
    __device__ __forceinline__ void load(int k0) {
        c4 = (k0 >> 6) & 3;
        const uint32_t h = c4 >> 1, gp = c4 & 1, p = (int)threadIdx.x & 1;
        const uint32_t sb = (uint32_t)(k0 >> 8) * 210u;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const uint32_t o = roff[i] + sb;
            odd[i] = o & 2;
            load5(rs, o + 64 * h + 16 * p, wa[i]);
            load5(rs, o + 64 * h + 32 + 16 * p, wb[i]);
            load5(rs, o + 128 + 32 * h + 16 * p, wh[i]);
            const uint32_t xs = o + 192 + 8 * h + 4 * gp + p;
            osc[i] = xs & 3;
            wsa[i] = buf_load4(rs, xs & ~3u);
            wsb[i] = buf_load4(rs, (xs + 2) & ~3u);
            wd[i] = buf_load4(rs, (o + 208) & ~3u);
        }
    }
    __device__ __forceinline__ void store(u32x4 *lds) const {
        const int p = (int)threadIdx.x & 1;
        const uint32_t gp = c4 & 1;
        const uint32_t n4 = gp ? 4 : 0, sh_a = 4 * gp, sh_b = 4 * gp + 2;
        const uint32_t L = 0x0F0F0F0Fu, H = 0x03030303u;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int r = (i * kThreads + (int)threadIdx.x) >> 1;
            const bool oh = odd[i] != 0;
            const u32x4 a = realign16(wa[i], oh), b = realign16(wb[i], oh), hh = realign16(wh[i], oh);
            const uint32_t bsa = 8 * osc[i], bsb = 8 * ((osc[i] + 2) & 3);
            const float sa = (float)(int)(int8_t)((wsa[i] >> bsa) & 0xFF);
            const float sbv = (float)(int)(int8_t)((wsb[i] >> bsb) & 0xFF);
            const float d = f16_bits_to_f32(oh ? (wd[i] >> 16) : wd[i]);
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
    static constexpr int PER = ROWS * 2 / kThreads;
    __amdgpu_buffer_rsrc_t rs;
    uint32_t roff[PER];
    uint32_t w[PER][9], odd[PER];
    int nb;

    __device__ void init(const uint8_t *W, int64_t row_bytes, int n0, int rows_valid, int K) {
        nb = K >> 5;
        const int64_t start = (int64_t)n0 * row_bytes;
        const uint32_t shift0 = (uint32_t)(((uintptr_t)W + start) & 15);
        const int64_t extent = shift0 + (int64_t)rows_valid * row_bytes;
        rs = make_rsrc(W + start - shift0, (uint32_t)((extent + 3) & ~(int64_t)3));
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int r = (i * kThreads + (int)threadIdx.x) >> 1;
            roff[i] = shift0 + (uint32_t)(r * row_bytes);
        }
    }
    __device__ __forceinline__ void load(int k0) {
        const int b = (k0 >> 5) + ((int)threadIdx.x & 1);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const uint32_t o = roff[i] + (uint32_t)b * 34u;
            odd[i] = o & 2;
            const uint32_t a = b < nb ? (o & ~3u) : kOOB;
            const u32x4 v0 = buf_load16(rs, a), v1 = buf_load16(rs, a + 16);
            w[i][0] = v0.x; w[i][1] = v0.y; w[i][2] = v0.z; w[i][3] = v0.w;
            w[i][4] = v1.x; w[i][5] = v1.y; w[i][6] = v1.z; w[i][7] = v1.w;
            w[i][8] = buf_load4(rs, a + 32);
        }
    }
    __device__ __forceinline__ void store(u32x4 *lds) const {
        const int p = (int)threadIdx.x & 1;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int r = (i * kThreads + (int)threadIdx.x) >> 1;
            const bool oh = odd[i] != 0;
            const float d = f16_bits_to_f32(oh ? (w[i][0] >> 16) : w[i][0]);
            uint32_t q[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) q[j] = oh ? w[i][j + 1] : shift2(w[i][j + 1], w[i][j]);
            u32x4 *row = lds + r * 8;
            const int sw = swz<8>(r);
#pragma unroll
            for (int j = 0; j < 4; ++j) row[(4 * p + j) ^ sw] = q80_chunk(q[2 * j], q[2 * j + 1], d);
        }
    }
};

template <int ROWS, int FMT>
struct BLoaderFor;
template <int ROWS> struct BLoaderFor<ROWS, kFmtF16> { typedef DmaTile<ROWS, 8> T; };
template <int ROWS> struct BLoaderFor<ROWS, kFmtQ4_K> { typedef Q4KLoader<ROWS> T; };
template <int ROWS> struct BLoaderFor<ROWS, kFmtQ6_K> { typedef Q6KLoader<ROWS> T; };
template <int ROWS> struct BLoaderFor<ROWS, kFmtQ8_0> { typedef Q80Loader<ROWS> T; };

// s_waitcnt immediate: at most n vector-memory operations outstanding, every
// LDS operation done (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8).
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

// Stage boundary: wait until this wave has at most N loads in flight and no
// LDS operation pending, then meet the other waves (N = 0 for LDS-DMA).  The barrier is an asm
// statement with a memory clobber, so the compiler moves no LDS access across
// it, but it carries none of __syncthreads' fences, which would also drain
// the LDS-DMA loads already in flight for the next k-steps.
template <int N>
__device__ __forceinline__ void sync_stage() {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(N));
    asm volatile("s_barrier" ::: "memory");
}

// MFMA operand fragments of one 16-wide k-slice.
template <int FM, int FN, int TM, int TN, int CPR>
__device__ __forceinline__ void load_frags(const u32x4 *Ac, const u32x4 *Bc, int kk, int wm,
                                           int wn, int lane, half8 (&af)[FM], half8 (&bf)[FN]) {
    const int c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int r = wm * TM + i * 32 + (lane & 31);
        af[i] = __builtin_bit_cast(half8, Ac[r * CPR + (c ^ swz<CPR>(r))]);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int r = wn * TN + j * 32 + (lane & 31);
        bf[j] = __builtin_bit_cast(half8, Bc[r * CPR + (c ^ swz<CPR>(r))]);
    }
}

// One k-step (8·CPR wide) of MFMAs from LDS stage (Ac, Bc) into the wave's tile.
// Fragments are double-buffered: the LDS reads of k-slice kk+1 are issued
// before the MFMAs of slice kk (scheduling barriers keep that order), so their
// latency hides behind matrix work.
template <int FM, int FN, int TM, int TN, int CPR>
__device__ __forceinline__ void mma_step(const u32x4 *Ac, const u32x4 *Bc, f32x16 (&acc)[FM][FN],
                                         int wm, int wn, int lane) {
    half8 af[2][FM], bf[2][FN];
    load_frags<FM, FN, TM, TN, CPR>(Ac, Bc, 0, wm, wn, lane, af[0], bf[0]);
#pragma unroll
    for (int kk = 0; kk < CPR / 2; ++kk) {
        const int cur = kk & 1;
        if (kk + 1 < CPR / 2)
            load_frags<FM, FN, TM, TN, CPR>(Ac, Bc, kk + 1, wm, wn, lane, af[cur ^ 1], bf[cur ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[cur][i], bf[cur][j], acc[i][j],
                                                                   0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------------------
// The GEMM kernel.  Three LDS stages form a ring: while step j is multiplied
// from stage j%3, the X tile (and the f16 cache tile) of step j+2 streams into
// stage (j+2)%3 by LDS-DMA.  The fused shape instead loads the raw B bytes of
// step j+1 into registers during step j and expands them into B stage
// (j+1)%3 after the step's MFMAs.  One barrier per k-step.
// PARTIAL: the launch is split along K and writes f32 partial planes (a
// distinct symbol, so profiles tell the two launch kinds apart).
// ---------------------------------------------------------------------------
// BK: k-step width (64, or 32 for the f16 operands when two workgroups share
// a compute unit: 72 KB of LDS and at most 256 registers per wave each).
template <int BM, int BN, int FMT, bool PARTIAL, int BK>
__global__ __launch_bounds__(kThreads, BK == 32 ? 2 : 1) void gemm_kernel(Args a) {
    constexpr int TM = BM / 2, TN = BN / 2;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int CPR = BK / 8;
    constexpr bool kDmaB = FMT == kFmtF16;
    static_assert(kDmaB || BK == 64, "the fused loaders expand 64-wide k-steps");
    __shared__ u32x4 A0[BM * CPR], A1[BM * CPR], A2[BM * CPR];
    __shared__ u32x4 B0[BN * CPR], B1[BN * CPR], B2[BN * CPR];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int t = xcd_remap(blockIdx.x, gridDim.x);
    const int tiles = a.tiles_m * a.tiles_n;
    const int s = t / tiles, tile = t - s * tiles;
    int tm, tn;
    tile_coords(tile, a.tiles_m, a.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kt_begin = s * a.steps_per_split;
    const int kt_end = min(kt_begin + a.steps_per_split, a.k_steps);

    DmaTile<BM, CPR> la;
    la.init(a.X + (int64_t)m0 * a.ldx, min(BM, a.M - m0), a.ldx, a.K);
    typename std::conditional<kDmaB, DmaTile<BN, CPR>, typename BLoaderFor<BN, FMT>::T>::type lb;
    if constexpr (kDmaB)
        lb.init((const uint16_t *)a.W + n0 * a.ldw, min(BN, a.N - n0), a.ldw, a.K);
    else
        lb.init(a.W, a.ldw, n0, min(BN, a.N - n0), a.K);
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // prologue: steps kt_begin and kt_begin + 1 in flight
    const int k0 = kt_begin * BK;
    const bool has_second = kt_begin + 1 < kt_end;
    if constexpr (!kDmaB) lb.load(k0);
    la.issue(k0, A0);
    la.issue(k0 + BK, A1, has_second);
    if constexpr (kDmaB) {
        lb.issue(k0, B0);
        lb.issue(k0 + BK, B1, has_second);
    } else {
        lb.store(B0);
    }

    // Step kt on stage (kt - kt_begin) % 3.  LDS-DMA loads of one wave retire
    // out of issue order (a partial vmcnt wait gave wrong, run-to-run
    // different tiles), so each boundary drains this wave's loads to zero:
    // the DMA of step kt+1, issued at the start of step kt-1, has one k-step
    // of MFMA work to land in.  The fused shape loads the raw B bytes of step
    // kt+1 in registers during step kt and expands them into B stage
    // (kt+1) % 3 after the step's MFMAs.
    auto step = [&](const u32x4 *Ac, const u32x4 *Bc, u32x4 *An, u32x4 *Bn, u32x4 *Bnext,
                    int kt) {
        const bool has1 = kt + 1 < kt_end, has2 = kt + 2 < kt_end;
        sync_stage<0>();
        if constexpr (!kDmaB) {
            if (has1) lb.load((kt + 1) * BK);     // raw B of the next step, before the DMA
        }
        la.issue((kt + 2) * BK, An, has2);
        if constexpr (kDmaB) lb.issue((kt + 2) * BK, Bn, has2);
        mma_step<FM, FN, TM, TN, CPR>(Ac, Bc, acc, wm, wn, lane);
        if constexpr (!kDmaB) {
            if (has1) lb.store(Bnext);
        }
    };
    // A single-exit loop over whole rounds of the three stages, then the tail:
    // with the exits inside the round, the compiler keeps the accumulators in
    // VGPRs across the back edge and copies all of them to and from AGPRs on
    // every round.
    int kt = kt_begin;
    for (const int rounds_end = kt_begin + (kt_end - kt_begin) / 3 * 3; kt < rounds_end; kt += 3) {
        step(A0, B0, A2, B2, B1, kt);
        step(A1, B1, A0, B0, B2, kt + 1);
        step(A2, B2, A1, B1, B0, kt + 2);
    }
    if (kt < kt_end) step(A0, B0, A2, B2, B1, kt);
    if (kt + 1 < kt_end) step(A1, B1, A0, B0, B2, kt + 1);
    // the look-ahead loads of the last steps must land before the workgroup's
    // LDS can be handed to another workgroup
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

    // C layout of a 32x32 MFMA block: lane holds column (lane & 31) and rows
    // 8·(r/4) + 4·(lane/32) + r%4 for accumulator element r.
    float *Yp = PARTIAL ? a.Y + (int64_t)s * a.plane : a.Y;
    const int col_l = lane & 31, row_l = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * TN + j * 32 + col_l;
            if (col >= a.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * TM + i * 32 + (r >> 2) * 8 + row_l + (r & 3);
                if (row < a.M) Yp[(int64_t)row * a.ldy + col] = acc[i][j][r];
            }
        }
}

// Y = Σ_s partial[s] in the order s = 0, 1, ..., split − 1.
__global__ __launch_bounds__(256) void splitk_reduce(const float *__restrict__ ws, int split,
                                                     int64_t plane, float *__restrict__ Y, int ldy,
                                                     int M, int N) {
    const uint32_t idx = blockIdx.x * 256u + threadIdx.x;
    if (idx >= (uint32_t)M * (uint32_t)N) return;
    float acc = ws[idx];
    for (int s = 1; s < split; ++s) acc += ws[(int64_t)s * plane + idx];
    const uint32_t m = idx / (uint32_t)N, n = idx - m * (uint32_t)N;
    Y[(int64_t)m * ldy + n] = acc;
}

// k-step width per operand kind: 32 for the f16 cache (two workgroups per
// compute unit), 64 for the fused kernels
constexpr int bk_for(int fmt) { return fmt == kFmtF16 ? 64 : 64; }

template <int BM, int FMT>
hipError_t launch_tile(const Args &a, int grid, bool partial, hipStream_t stream) {
    constexpr int BK = bk_for(FMT);
    if (partial)
        hipLaunchKernelGGL((gemm_kernel<BM, 128, FMT, true, BK>), dim3(grid), dim3(kThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((gemm_kernel<BM, 128, FMT, false, BK>), dim3(grid), dim3(kThreads), 0,
                           stream, a);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const Args &a, int bm, int grid, bool partial, hipStream_t stream) {
    switch (bm) {
    case 64: return launch_tile<64, FMT>(a, grid, partial, stream);
    case 128: return launch_tile<128, FMT>(a, grid, partial, stream);
    default: return launch_tile<256, FMT>(a, grid, partial, stream);
    }
}

}  // namespace

GemmPlan plan_gemm(int fmt, int M, int N, int K, int split_req) {
    GemmPlan p;
    p.bn = 128;
    p.bm = M > 128 ? 256 : (M > 64 ? 128 : 64);
    p.tiles_m = (M + p.bm - 1) / p.bm;
    p.tiles_n = (N + p.bn - 1) / p.bn;
    // The K split is planned in 64-element units whatever the kernel's k-step,
    // so the f16-cache and fused kernels partition K identically and sum the
    // same products in the same order.
    const int k64 = (K + 63) / 64;
    int split = split_req;
    if (split == 0) {
        split = 1;
        const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
        if (tiles < kCUs && (int64_t)M * N <= (1 << 26)) {
            split = (int)(kCUs / tiles);
            if (split > 16) split = 16;
            const int max_by_k = k64 / 4;   // keep >= 256 k per partition
            if (split > max_by_k) split = max_by_k;
            if (split < 1) split = 1;
        }
    }
    if (split > k64) split = k64;
    const int per64 = (k64 + split - 1) / split;
    p.split = (k64 + per64 - 1) / per64;
    const int bk = bk_for(fmt);
    p.k_steps = (K + bk - 1) / bk;
    p.steps_per_split = per64 * (64 / bk);
    p.ws_bytes = p.split > 1 ? (int64_t)p.split * M * N * 4 : 0;
    return p;
}

hipError_t launch_gemm(int fmt, const uint16_t *X, int ldx, const void *W, int64_t ldw, float *Y,
                       int ldy, int M, int N, int K, const GemmPlan &plan, float *ws,
                       hipStream_t stream) {
    Args a;
    a.X = X;
    a.W = (const uint8_t *)W;
    a.ldw = ldw;
    a.ldx = ldx;
    a.M = M;
    a.N = N;
    a.K = K;
    a.tiles_m = plan.tiles_m;
    a.tiles_n = plan.tiles_n;
    a.k_steps = plan.k_steps;
    a.steps_per_split = plan.steps_per_split;
    if (plan.split > 1) {
        a.Y = ws;
        a.ldy = N;
        a.plane = (int64_t)M * N;
    } else {
        a.Y = Y;
        a.ldy = ldy;
        a.plane = 0;
    }
    const int grid = plan.tiles_m * plan.tiles_n * plan.split;
    const bool partial = plan.split > 1;
    hipError_t e;
    switch (fmt) {
    case kFmtQ4_K: e = launch_fmt<kFmtQ4_K>(a, plan.bm, grid, partial, stream); break;
    case kFmtQ6_K: e = launch_fmt<kFmtQ6_K>(a, plan.bm, grid, partial, stream); break;
    case kFmtQ8_0: e = launch_fmt<kFmtQ8_0>(a, plan.bm, grid, partial, stream); break;
    default: e = launch_fmt<kFmtF16>(a, plan.bm, grid, partial, stream); break;
    }
    if (e != hipSuccess || plan.split == 1) return e;
    const uint32_t total = (uint32_t)M * (uint32_t)N;
    hipLaunchKernelGGL(splitk_reduce, dim3((total + 255) / 256), dim3(256), 0, stream, ws, plan.split,
                       (int64_t)M * N, Y, ldy, M, N);
    return hipGetLastError();
}

}  // namespace mq
