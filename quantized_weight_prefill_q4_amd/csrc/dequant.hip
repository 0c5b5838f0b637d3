// Load-time decode of quantized weights into the persistent f16 cache.
//
// minfer "05 · 8p — Persistent f16 weight cache + fused dequant-in-GEMM":
// §2 (the cache is one f16 copy of each weight, written once) and §3.2 (the
// standalone dequant kernel: float math per element, one conversion to half).
// llama.cpp PR #57, Summary: the cache row may be padded by one 128-byte line.
//
// The pass is HBM-bound (0.56–1.06 B read and 2 B written per element), so
// the kernel is laid out for the memory system, not for arithmetic:
//   * one thread produces one 16-byte run of 8 consecutive f16 outputs, so a
//     wave writes 1 KiB of contiguous cache row per store instruction;
//   * Q4_K blocks (144 B) are 16-byte aligned and are read with 16/8-byte
//     loads; Q6_K (210 B) and Q8_0 (34 B) blocks are only 2-byte aligned, so
//     their bytes are read as the aligned dwords that contain them and
//     re-assembled with v_alignbyte (a dword that holds a requested byte lies
//     on the same page as that byte, so no load can fault).
//   * the pad columns [K, ld) are written as +0 by the tail of the same grid.

#include "mq_device.h"
#include "mq_internal.h"

namespace mq {
namespace {

constexpr uint32_t kThreads = 256;

// 8 bytes at a 2-byte-aligned address as two little-endian dwords.
__device__ __forceinline__ u32x2 load8_a2(const uint8_t *p) {
    const uintptr_t a = (uintptr_t)p;
    const uint32_t *w = (const uint32_t *)(a & ~(uintptr_t)3);
    const uint32_t w0 = w[0], w1 = w[1];
    if (a & 2) {
        const uint32_t w2 = w[2];
        return u32x2{shift2(w1, w0), shift2(w2, w1)};
    }
    return u32x2{w0, w1};
}

__device__ __forceinline__ void store8(uint16_t *o, const float v[8]) {
    *(u32x4 *)o = u32x4{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]), pack_f16x2(v[4], v[5]),
                        pack_f16x2(v[6], v[7])};
}

// Zero one 8-element run of the pad columns [K, ld).
__device__ __forceinline__ void write_pad(uint16_t *out, uint32_t p, uint32_t per_row, uint32_t K,
                                          uint32_t ld) {
    const uint32_t row = p / per_row, c = p - row * per_row;
    *(u32x4 *)(out + (size_t)row * ld + K + 8 * c) = u32x4{0, 0, 0, 0};
}

// Q4_K: 256 elements = 8 sub-blocks of 32; value fl32(d·sc·q − dmin·m).
// Element e takes the low nibble of qs[32·(e/64) + e%32] when e%64 < 32, the
// high nibble otherwise; (sc, m) of sub-block j come from the 12 scale bytes
// (6 bits each; sub-blocks 4..7 split 4 + 2 bits).
__global__ __launch_bounds__(kThreads) void dequant_q4k(const uint8_t *__restrict__ wq,
                                                        uint16_t *__restrict__ out, uint32_t nb,
                                                        uint32_t K, uint32_t ld, uint32_t n_data,
                                                        uint32_t pad_per_row, uint32_t n_total) {
    const uint32_t u = blockIdx.x * kThreads + threadIdx.x;
    if (u >= n_total) return;
    if (u >= n_data) {
        write_pad(out, u - n_data, pad_per_row, K, ld);
        return;
    }
    const uint32_t g = u >> 5, e0 = (u & 31) * 8;
    const uint32_t row = g / nb, kb = g - row * nb;
    const uint8_t *blk = wq + (size_t)g * 144;
    const u32x4 h = *(const u32x4 *)blk;
    const uint32_t c = e0 >> 6, r = e0 & 63, j = e0 >> 5;
    const u32x2 qq = *(const u32x2 *)(blk + 16 + 32 * c + (r & 31));

    const uint32_t sh = 8 * (j & 3);
    const uint32_t s_lo = (h.y >> sh) & 0xFF;   // s[j & 3]
    const uint32_t s_mid = (h.z >> sh) & 0xFF;  // s[(j & 3) + 4]
    const uint32_t s_hi = (h.w >> sh) & 0xFF;   // s[(j & 3) + 8]
    const uint32_t sc = j < 4 ? (s_lo & 63) : ((s_hi & 15) | ((s_lo >> 6) << 4));
    const uint32_t m = j < 4 ? (s_mid & 63) : ((s_hi >> 4) | ((s_mid >> 6) << 4));
    const float A = f16_bits_to_f32(h.x) * (float)sc;          // exact
    const float C = f16_bits_to_f32(h.x >> 16) * (float)m;     // exact

    const uint32_t n4 = (r >= 32) ? 4 : 0;
    const uint32_t w0 = (qq.x >> n4) & 0x0F0F0F0Fu, w1 = (qq.y >> n4) & 0x0F0F0F0Fu;
    float v[8];
    // A·q is exact, so one fused rounding equals fl32(A·q − C).
    v[0] = __builtin_fmaf(A, ubyte_f32<0>(w0), -C);
    v[1] = __builtin_fmaf(A, ubyte_f32<1>(w0), -C);
    v[2] = __builtin_fmaf(A, ubyte_f32<2>(w0), -C);
    v[3] = __builtin_fmaf(A, ubyte_f32<3>(w0), -C);
    v[4] = __builtin_fmaf(A, ubyte_f32<0>(w1), -C);
    v[5] = __builtin_fmaf(A, ubyte_f32<1>(w1), -C);
    v[6] = __builtin_fmaf(A, ubyte_f32<2>(w1), -C);
    v[7] = __builtin_fmaf(A, ubyte_f32<3>(w1), -C);
    store8(out + (size_t)row * ld + kb * 256 + e0, v);
}

// Q6_K: element e = 128h + 32g + l takes its low 4 bits from
// ql[64h + l + 32(g & 1)] (low nibble for g < 2, high for g >= 2), its high 2
// bits from qh[32h + l] >> 2g, and the int8 scale sc[e / 16]; the value is
// (d·sc)·(q − 32) in f32 (exact; IEEE signed zeros kept).
__global__ __launch_bounds__(kThreads) void dequant_q6k(const uint8_t *__restrict__ wq,
                                                        uint16_t *__restrict__ out, uint32_t nb,
                                                        uint32_t K, uint32_t ld, uint32_t n_data,
                                                        uint32_t pad_per_row, uint32_t n_total) {
    const uint32_t u = blockIdx.x * kThreads + threadIdx.x;
    if (u >= n_total) return;
    if (u >= n_data) {
        write_pad(out, u - n_data, pad_per_row, K, ld);
        return;
    }
    const uint32_t g = u >> 5, e0 = (u & 31) * 8;
    const uint32_t row = g / nb, kb = g - row * nb;
    const uint8_t *blk = wq + (size_t)g * 210;
    const uint32_t h = e0 >> 7, grp = (e0 >> 5) & 3, l0 = e0 & 31;
    const u32x2 lo = load8_a2(blk + 64 * h + l0 + 32 * (grp & 1));
    const u32x2 hi = load8_a2(blk + 128 + 32 * h + l0);
    const float s = (float)(int)(int8_t)blk[192 + (e0 >> 4)];
    const float d = f16_bits_to_f32(*(const uint16_t *)(blk + 208));
    const float ds = d * s;  // exact

    const uint32_t n4 = grp >= 2 ? 4 : 0, h2 = 2 * grp;
    const uint32_t q0 = ((lo.x >> n4) & 0x0F0F0F0Fu) | (((hi.x >> h2) & 0x03030303u) << 4);
    const uint32_t q1 = ((lo.y >> n4) & 0x0F0F0F0Fu) | (((hi.y >> h2) & 0x03030303u) << 4);
    float v[8];
    v[0] = ds * (ubyte_f32<0>(q0) - 32.0f);
    v[1] = ds * (ubyte_f32<1>(q0) - 32.0f);
    v[2] = ds * (ubyte_f32<2>(q0) - 32.0f);
    v[3] = ds * (ubyte_f32<3>(q0) - 32.0f);
    v[4] = ds * (ubyte_f32<0>(q1) - 32.0f);
    v[5] = ds * (ubyte_f32<1>(q1) - 32.0f);
    v[6] = ds * (ubyte_f32<2>(q1) - 32.0f);
    v[7] = ds * (ubyte_f32<3>(q1) - 32.0f);
    store8(out + (size_t)row * ld + kb * 256 + e0, v);
}

// Q8_0: 32 elements, value d·q.
__global__ __launch_bounds__(kThreads) void dequant_q80(const uint8_t *__restrict__ wq,
                                                        uint16_t *__restrict__ out, uint32_t nb,
                                                        uint32_t K, uint32_t ld, uint32_t n_data,
                                                        uint32_t pad_per_row, uint32_t n_total) {
    const uint32_t u = blockIdx.x * kThreads + threadIdx.x;
    if (u >= n_total) return;
    if (u >= n_data) {
        write_pad(out, u - n_data, pad_per_row, K, ld);
        return;
    }
    const uint32_t g = u >> 2, p = u & 3;
    const uint32_t row = g / nb, kb = g - row * nb;
    const uint8_t *blk = wq + (size_t)g * 34;
    const float d = f16_bits_to_f32(*(const uint16_t *)blk);
    const u32x2 q = load8_a2(blk + 2 + 8 * p);
    float v[8];
    v[0] = d * sbyte_f32<0>(q.x);
    v[1] = d * sbyte_f32<1>(q.x);
    v[2] = d * sbyte_f32<2>(q.x);
    v[3] = d * sbyte_f32<3>(q.x);
    v[4] = d * sbyte_f32<0>(q.y);
    v[5] = d * sbyte_f32<1>(q.y);
    v[6] = d * sbyte_f32<2>(q.y);
    v[7] = d * sbyte_f32<3>(q.y);
    store8(out + (size_t)row * ld + kb * 32 + 8 * p, v);
}

}  // namespace

hipError_t launch_dequant(int fmt, const void *wq, int N, int K, uint16_t *w16, int ld,
                          hipStream_t stream) {
    const uint32_t be = (uint32_t)block_elems(fmt);
    const uint32_t nb = (uint32_t)K / be;
    const uint32_t n_data = (uint32_t)((uint64_t)N * (uint32_t)K / 8);
    const uint32_t pad_per_row = (uint32_t)(ld - K) / 8;
    const uint32_t n_total = n_data + (uint32_t)N * pad_per_row;
    const dim3 grid((n_total + kThreads - 1) / kThreads), block(kThreads);
    const uint8_t *q = (const uint8_t *)wq;
    switch (fmt) {
    case kFmtQ4_K:
        hipLaunchKernelGGL(dequant_q4k, grid, block, 0, stream, q, w16, nb, (uint32_t)K,
                           (uint32_t)ld, n_data, pad_per_row, n_total);
        break;
    case kFmtQ6_K:
        hipLaunchKernelGGL(dequant_q6k, grid, block, 0, stream, q, w16, nb, (uint32_t)K,
                           (uint32_t)ld, n_data, pad_per_row, n_total);
        break;
    default:
        hipLaunchKernelGGL(dequant_q80, grid, block, 0, stream, q, w16, nb, (uint32_t)K,
                           (uint32_t)ld, n_data, pad_per_row, n_total);
        break;
    }
    return hipGetLastError();
}

}  // namespace mq
