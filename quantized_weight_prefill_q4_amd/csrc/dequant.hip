// Load-time decode of quantized weights into the persistent f16 cache.
//
// minfer "05 · 8p — Persistent f16 weight cache + fused dequant-in-GEMM":
// §2 (the cache is one f16 copy of each weight, written once) and §3.2 (the
// standalone dequant kernel: float math per element, one conversion to half).
// llama.cpp PR #57, Summary: the cache row may be padded by one 128-byte line.
//
// The pass is HBM-bound (0.56–1.06 B read and 2 B written per element), so
// the kernel is laid out for the memory system, not for arithmetic: each
// workgroup stages the contiguous bytes of its blocks in LDS with one 16-byte
// load per 16 input bytes, then every thread decodes four 16-byte runs of
// f16 output, each wave store writing 1 KiB of contiguous cache row.  Q6_K
// (210 B), Q8_0 (34 B), Q4_0 (18 B) and Q5_0 (22 B) blocks are only 2-byte
// aligned (the Q5_0 qh word in particular: minfer "05 · 8p" §2); they are
// read from LDS with 2-byte accesses, and global memory is only read in
// aligned 16-byte chunks.  The pad columns [K, ld) are written as +0 by the
// tail of the grid.  Formats: Q4_K, Q5_K, Q6_K (256-element super-blocks),
// Q4_0, Q5_0, Q5_1, Q8_0 (32-element blocks); decode formulas as in the
// per-format functions below.

#include "mq_device.h"
#include "mq_internal.h"

namespace mq {
namespace {

constexpr uint32_t kThreads = 256;
constexpr uint32_t kChunksPerThread = 4;                        // 16-byte output runs
constexpr uint32_t kChunksPerGroup = kThreads * kChunksPerThread;   // 16 KiB of f16 out

template <int FMT> struct Fmt;
template <> struct Fmt<kFmtQ4_K> { static constexpr uint32_t BE = 256, BB = 144; };
template <> struct Fmt<kFmtQ6_K> { static constexpr uint32_t BE = 256, BB = 210; };
template <> struct Fmt<kFmtQ8_0> { static constexpr uint32_t BE = 32, BB = 34; };
template <> struct Fmt<kFmtQ4_0> { static constexpr uint32_t BE = 32, BB = 18; };
template <> struct Fmt<kFmtQ5_0> { static constexpr uint32_t BE = 32, BB = 22; };
template <> struct Fmt<kFmtQ5_1> { static constexpr uint32_t BE = 32, BB = 24; };
template <> struct Fmt<kFmtQ5_K> { static constexpr uint32_t BE = 256, BB = 176; };

// blocks per workgroup and their staged bytes (plus up to 16 bytes of lead-in)
template <int FMT> constexpr uint32_t group_blocks() { return kChunksPerGroup * 8 / Fmt<FMT>::BE; }
template <int FMT> constexpr uint32_t stage_bytes() { return group_blocks<FMT>() * Fmt<FMT>::BB + 32; }

// little-endian reads from LDS at a 2-byte-aligned address
__device__ __forceinline__ uint32_t lds_u16(const uint8_t *p) { return *(const uint16_t *)p; }
__device__ __forceinline__ uint32_t lds_u32_a2(const uint8_t *p) {
    return lds_u16(p) | (lds_u16(p + 2) << 16);
}

// 8 outputs to the cache with a non-temporal (streaming) store: the cache is
// written once at load and not read back by this pass, so its lines need not
// displace anything in L2 / MALL (measured: 5.28 -> 5.43 TB/s for a 7B load).
__device__ __forceinline__ void store8(uint16_t *o, const float v[8]) {
    __builtin_nontemporal_store(u32x4{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]),
                                      pack_f16x2(v[4], v[5]), pack_f16x2(v[6], v[7])},
                                (u32x4 *)o);
}

// Q4_K, 8 outputs e0..e0+7 of the block at `blk` (16-byte aligned in LDS):
// value fl32(d·sc·q − dmin·m).  Element e takes the low nibble of
// qs[32·(e/64) + e%32] when e%64 < 32, the high nibble otherwise; (sc, m) of
// sub-block j come from the 12 scale bytes (6 bits each; sub-blocks 4..7
// split 4 + 2 bits).
__device__ __forceinline__ void decode_q4k(const uint8_t *blk, uint32_t e0, float v[8]) {
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
    const uint32_t w0 = opaque((qq.x >> n4) & 0x0F0F0F0Fu), w1 = opaque((qq.y >> n4) & 0x0F0F0F0Fu);
    // A·q is exact, so one fused rounding equals fl32(A·q − C)
    v[0] = __builtin_fmaf(A, ubyte_f32<0>(w0), -C);
    v[1] = __builtin_fmaf(A, ubyte_f32<1>(w0), -C);
    v[2] = __builtin_fmaf(A, ubyte_f32<2>(w0), -C);
    v[3] = __builtin_fmaf(A, ubyte_f32<3>(w0), -C);
    v[4] = __builtin_fmaf(A, ubyte_f32<0>(w1), -C);
    v[5] = __builtin_fmaf(A, ubyte_f32<1>(w1), -C);
    v[6] = __builtin_fmaf(A, ubyte_f32<2>(w1), -C);
    v[7] = __builtin_fmaf(A, ubyte_f32<3>(w1), -C);
}

// Q6_K, 8 outputs of the block at `blk` (2-byte aligned in LDS): element
// e = 128h + 32g + l takes its low 4 bits from ql[64h + l + 32(g & 1)] (low
// nibble for g < 2, high for g >= 2), its high 2 bits from qh[32h + l] >> 2g,
// and the int8 scale sc[e / 16]; value (d·sc)·(q − 32) in f32 (exact; IEEE
// signed zeros kept).
__device__ __forceinline__ void decode_q6k(const uint8_t *blk, uint32_t e0, float v[8]) {
    const uint32_t h = e0 >> 7, grp = (e0 >> 5) & 3, l0 = e0 & 31;
    const uint8_t *lo = blk + 64 * h + l0 + 32 * (grp & 1);
    const uint8_t *hi = blk + 128 + 32 * h + l0;
    const uint32_t lo0 = lds_u32_a2(lo), lo1 = lds_u32_a2(lo + 4);
    const uint32_t hi0 = lds_u32_a2(hi), hi1 = lds_u32_a2(hi + 4);
    const float s = (float)(int)(int8_t)blk[192 + (e0 >> 4)];
    const float d = f16_bits_to_f32(lds_u16(blk + 208));
    const float ds = d * s;  // exact
    const uint32_t n4 = grp >= 2 ? 4 : 0, h2 = 2 * grp;
    const uint32_t q0 = opaque(((lo0 >> n4) & 0x0F0F0F0Fu) | (((hi0 >> h2) & 0x03030303u) << 4));
    const uint32_t q1 = opaque(((lo1 >> n4) & 0x0F0F0F0Fu) | (((hi1 >> h2) & 0x03030303u) << 4));
    v[0] = ds * (ubyte_f32<0>(q0) - 32.0f);
    v[1] = ds * (ubyte_f32<1>(q0) - 32.0f);
    v[2] = ds * (ubyte_f32<2>(q0) - 32.0f);
    v[3] = ds * (ubyte_f32<3>(q0) - 32.0f);
    v[4] = ds * (ubyte_f32<0>(q1) - 32.0f);
    v[5] = ds * (ubyte_f32<1>(q1) - 32.0f);
    v[6] = ds * (ubyte_f32<2>(q1) - 32.0f);
    v[7] = ds * (ubyte_f32<3>(q1) - 32.0f);
}

// Q8_0, 8 outputs e0..e0+7 of the block at `blk` (2-byte aligned): value d·q.
__device__ __forceinline__ void decode_q80(const uint8_t *blk, uint32_t e0, float v[8]) {
    const float d = f16_bits_to_f32(lds_u16(blk));
    const uint32_t q0 = lds_u32_a2(blk + 2 + e0), q1 = lds_u32_a2(blk + 6 + e0);
    v[0] = d * sbyte_f32<0>(q0);
    v[1] = d * sbyte_f32<1>(q0);
    v[2] = d * sbyte_f32<2>(q0);
    v[3] = d * sbyte_f32<3>(q0);
    v[4] = d * sbyte_f32<0>(q1);
    v[5] = d * sbyte_f32<1>(q1);
    v[6] = d * sbyte_f32<2>(q1);
    v[7] = d * sbyte_f32<3>(q1);
}

// The 16s bits of 4 consecutive elements, bits 0..3 of b, moved to bit 4 of
// bytes 0..3 (b·(1 + 2^7 + 2^14 + 2^21) puts bit i at bit 8i; no partial
// products overlap).
__device__ __forceinline__ uint32_t spread4_to_bit4(uint32_t b) {
    return ((b * 0x00204081u) & 0x01010101u) << 4;
}

// 8 four-bit quants of a 32-element block (Q4_0 / Q5_0 / Q5_1 nibble plane at
// `qs`): elements e0..e0+7 are bytes (e0 & 15) .. +7, low nibbles for e0 < 16.
__device__ __forceinline__ void nibbles8(const uint8_t *qs, uint32_t e0, uint32_t &w0, uint32_t &w1) {
    const uint8_t *p = qs + (e0 & 15);
    const uint32_t n4 = e0 >= 16 ? 4 : 0;
    w0 = (lds_u32_a2(p) >> n4) & 0x0F0F0F0Fu;
    w1 = (lds_u32_a2(p + 4) >> n4) & 0x0F0F0F0Fu;
}

// Q4_0, 8 outputs of the block at `blk` (2-byte aligned): value d·(q − 8).
__device__ __forceinline__ void decode_q40(const uint8_t *blk, uint32_t e0, float v[8]) {
    const float d = f16_bits_to_f32(lds_u16(blk));
    uint32_t w0, w1;
    nibbles8(blk + 2, e0, w0, w1);
    w0 = opaque(w0);
    w1 = opaque(w1);
    v[0] = d * (ubyte_f32<0>(w0) - 8.0f);
    v[1] = d * (ubyte_f32<1>(w0) - 8.0f);
    v[2] = d * (ubyte_f32<2>(w0) - 8.0f);
    v[3] = d * (ubyte_f32<3>(w0) - 8.0f);
    v[4] = d * (ubyte_f32<0>(w1) - 8.0f);
    v[5] = d * (ubyte_f32<1>(w1) - 8.0f);
    v[6] = d * (ubyte_f32<2>(w1) - 8.0f);
    v[7] = d * (ubyte_f32<3>(w1) - 8.0f);
}

// Q5_0, 8 outputs (block 2-byte aligned): q = nibble + 16·(bit e of qh), value
// d·(q − 16).  qh is read as two 2-byte halves (the block start is only
// 2-byte aligned).
__device__ __forceinline__ void decode_q50(const uint8_t *blk, uint32_t e0, float v[8]) {
    const float d = f16_bits_to_f32(lds_u16(blk));
    const uint32_t hb = lds_u32_a2(blk + 2) >> e0;
    uint32_t w0, w1;
    nibbles8(blk + 6, e0, w0, w1);
    w0 = opaque(w0 | spread4_to_bit4(hb & 15));
    w1 = opaque(w1 | spread4_to_bit4((hb >> 4) & 15));
    v[0] = d * (ubyte_f32<0>(w0) - 16.0f);
    v[1] = d * (ubyte_f32<1>(w0) - 16.0f);
    v[2] = d * (ubyte_f32<2>(w0) - 16.0f);
    v[3] = d * (ubyte_f32<3>(w0) - 16.0f);
    v[4] = d * (ubyte_f32<0>(w1) - 16.0f);
    v[5] = d * (ubyte_f32<1>(w1) - 16.0f);
    v[6] = d * (ubyte_f32<2>(w1) - 16.0f);
    v[7] = d * (ubyte_f32<3>(w1) - 16.0f);
}

// Q5_1, 8 outputs: q as Q5_0, value fl32(d·q + m) (d·q exact, one rounding).
__device__ __forceinline__ void decode_q51(const uint8_t *blk, uint32_t e0, float v[8]) {
    const float d = f16_bits_to_f32(lds_u16(blk)), m = f16_bits_to_f32(lds_u16(blk + 2));
    const uint32_t hb = lds_u32_a2(blk + 4) >> e0;
    uint32_t w0, w1;
    nibbles8(blk + 8, e0, w0, w1);
    w0 = opaque(w0 | spread4_to_bit4(hb & 15));
    w1 = opaque(w1 | spread4_to_bit4((hb >> 4) & 15));
    v[0] = __builtin_fmaf(d, ubyte_f32<0>(w0), m);
    v[1] = __builtin_fmaf(d, ubyte_f32<1>(w0), m);
    v[2] = __builtin_fmaf(d, ubyte_f32<2>(w0), m);
    v[3] = __builtin_fmaf(d, ubyte_f32<3>(w0), m);
    v[4] = __builtin_fmaf(d, ubyte_f32<0>(w1), m);
    v[5] = __builtin_fmaf(d, ubyte_f32<1>(w1), m);
    v[6] = __builtin_fmaf(d, ubyte_f32<2>(w1), m);
    v[7] = __builtin_fmaf(d, ubyte_f32<3>(w1), m);
}

// Q5_K, 8 outputs of the block at `blk` (16-byte aligned): as Q4_K, plus bit j
// (the sub-block) of qh[l] as the 16s bit of element l of sub-block j.
__device__ __forceinline__ void decode_q5k(const uint8_t *blk, uint32_t e0, float v[8]) {
    const u32x4 h = *(const u32x4 *)blk;
    const uint32_t c = e0 >> 6, r = e0 & 63, j = e0 >> 5, l0 = r & 31;
    const u32x2 qq = *(const u32x2 *)(blk + 48 + 32 * c + l0);
    const u32x2 hh = *(const u32x2 *)(blk + 16 + l0);
    const uint32_t sh = 8 * (j & 3);
    const uint32_t s_lo = (h.y >> sh) & 0xFF, s_mid = (h.z >> sh) & 0xFF, s_hi = (h.w >> sh) & 0xFF;
    const uint32_t sc = j < 4 ? (s_lo & 63) : ((s_hi & 15) | ((s_lo >> 6) << 4));
    const uint32_t m = j < 4 ? (s_mid & 63) : ((s_hi >> 4) | ((s_mid >> 6) << 4));
    const float A = f16_bits_to_f32(h.x) * (float)sc;
    const float C = f16_bits_to_f32(h.x >> 16) * (float)m;
    const uint32_t n4 = (r >= 32) ? 4 : 0;
    const uint32_t w0 = opaque(((qq.x >> n4) & 0x0F0F0F0Fu) | (((hh.x >> j) & 0x01010101u) << 4));
    const uint32_t w1 = opaque(((qq.y >> n4) & 0x0F0F0F0Fu) | (((hh.y >> j) & 0x01010101u) << 4));
    // A·q is exact (≤ 22 bits), so one fused rounding equals fl32(A·q − C)
    v[0] = __builtin_fmaf(A, ubyte_f32<0>(w0), -C);
    v[1] = __builtin_fmaf(A, ubyte_f32<1>(w0), -C);
    v[2] = __builtin_fmaf(A, ubyte_f32<2>(w0), -C);
    v[3] = __builtin_fmaf(A, ubyte_f32<3>(w0), -C);
    v[4] = __builtin_fmaf(A, ubyte_f32<0>(w1), -C);
    v[5] = __builtin_fmaf(A, ubyte_f32<1>(w1), -C);
    v[6] = __builtin_fmaf(A, ubyte_f32<2>(w1), -C);
    v[7] = __builtin_fmaf(A, ubyte_f32<3>(w1), -C);
}

// Shape of one decode: the matrix's blocks, its cache, and how the groups of
// 16 KiB of output (data groups first, then the pad-column groups) cover it.
struct DequantJob {
    const uint8_t *wq;
    uint16_t *out;
    uint32_t nb, K, ld, n_blocks, data_groups, pad_per_row, n_pad;
    uint32_t groups_end;   // batch launch: first workgroup of the next job
    int fmt;
};

// LDS stage large enough for any format's group
constexpr uint32_t kStageMax =
    stage_bytes<kFmtQ8_0>() > stage_bytes<kFmtQ6_K>() ? stage_bytes<kFmtQ8_0>() : stage_bytes<kFmtQ6_K>();
static_assert(stage_bytes<kFmtQ4_K>() <= kStageMax && stage_bytes<kFmtQ5_K>() <= kStageMax &&
                  stage_bytes<kFmtQ4_0>() <= kStageMax && stage_bytes<kFmtQ5_0>() <= kStageMax &&
                  stage_bytes<kFmtQ5_1>() <= kStageMax,
              "stage size");

// Workgroup `grp` of a job decodes group_blocks<FMT>() consecutive blocks
// (16 KiB of f16 output).  Phase 1: the blocks' bytes — a contiguous span of
// the weight — are staged in LDS with 16-byte loads from its 16-byte-aligned
// cover (a 16-byte chunk that holds a wanted byte lies on that byte's page,
// so no load can fault; the bytes are read once, with non-temporal loads:
// 1-5% on single 7B / 8B shapes).  Phase 2: each thread decodes kChunksPerThread runs
// of 8 outputs, run u = first + i·256 + thread, so every store instruction of
// a wave writes 1 KiB of contiguous cache row.  Groups past the data write
// the +0 pad columns [K, ld).
template <int FMT>
__device__ __forceinline__ void decode_group(const DequantJob &j, uint32_t grp, u32x4 *stage) {
    constexpr uint32_t BE = Fmt<FMT>::BE, BB = Fmt<FMT>::BB, G = group_blocks<FMT>();
    constexpr uint32_t CPB = BE / 8;   // output runs per block
    const uint32_t tid = threadIdx.x;

    if (grp >= j.data_groups) {   // pad columns
        const uint32_t p0 = (grp - j.data_groups) * kChunksPerGroup;
#pragma unroll
        for (uint32_t i = 0; i < kChunksPerThread; ++i) {
            const uint32_t p = p0 + i * kThreads + tid;
            if (p < j.n_pad) {
                const uint32_t row = p / j.pad_per_row, c = p - row * j.pad_per_row;
                *(u32x4 *)(j.out + (size_t)row * j.ld + j.K + 8 * c) = u32x4{0, 0, 0, 0};
            }
        }
        return;
    }

    const uint32_t g0 = grp * G;
    const uint32_t gcount = min(G, j.n_blocks - g0);
    const size_t begin = (size_t)g0 * BB, end = begin + (size_t)gcount * BB;
    const size_t abegin = begin & ~(size_t)15;
    const uint32_t lead = (uint32_t)(begin - abegin);
    const uint32_t nchunks = (uint32_t)((end - abegin + 15) >> 4);
    const u32x4 *src = (const u32x4 *)(j.wq + abegin);
    constexpr uint32_t kLoads = (stage_bytes<FMT>() / 16 + kThreads - 1) / kThreads;
    u32x4 tmp[kLoads];
#pragma unroll
    for (uint32_t i = 0; i < kLoads; ++i) {
        const uint32_t c = i * kThreads + tid;
        if (c < nchunks) tmp[i] = __builtin_nontemporal_load(src + c);
    }
#pragma unroll
    for (uint32_t i = 0; i < kLoads; ++i) {
        const uint32_t c = i * kThreads + tid;
        if (c < nchunks) stage[c] = tmp[i];
    }
    __syncthreads();

    const uint8_t *bytes = (const uint8_t *)stage + lead;
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        const uint32_t u = i * kThreads + tid;          // run within the group
        const uint32_t gl = u / CPB;                    // block within the group
        if (gl >= gcount) break;
        const uint32_t e0 = (u - gl * CPB) * 8;
        const uint32_t g = g0 + gl;
        const uint32_t row = g / j.nb, kb = g - row * j.nb;
        float v[8];
        const uint8_t *blk = bytes + gl * BB;
        if constexpr (FMT == kFmtQ4_K) decode_q4k(blk, e0, v);
        else if constexpr (FMT == kFmtQ6_K) decode_q6k(blk, e0, v);
        else if constexpr (FMT == kFmtQ8_0) decode_q80(blk, e0, v);
        else if constexpr (FMT == kFmtQ4_0) decode_q40(blk, e0, v);
        else if constexpr (FMT == kFmtQ5_0) decode_q50(blk, e0, v);
        else if constexpr (FMT == kFmtQ5_1) decode_q51(blk, e0, v);
        else decode_q5k(blk, e0, v);
        store8(j.out + (size_t)row * j.ld + kb * BE + e0, v);
    }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(DequantJob j) {
    __shared__ u32x4 stage[stage_bytes<FMT>() / 16];
    decode_group<FMT>(j, blockIdx.x, stage);
}

// Several decodes in one launch (a model load decodes every weight back to
// back; one launch per small matrix leaves most of the GPU idle while it
// ramps up and drains).  The jobs travel by value in the kernel arguments;
// workgroups [groups_end of job i-1, groups_end of job i) belong to job i.
constexpr int kBatchJobs = 16;
struct DequantBatch {
    DequantJob job[kBatchJobs];
    int n;
};

__global__ __launch_bounds__(kThreads) void dequant_batch_kernel(DequantBatch b) {
    __shared__ u32x4 stage[kStageMax / 16];
    const uint32_t bid = blockIdx.x;
    int i = 0;
    while (i + 1 < b.n && bid >= b.job[i].groups_end) ++i;   // uniform scan
    const DequantJob &j = b.job[i];
    const uint32_t grp = bid - (i ? b.job[i - 1].groups_end : 0u);
    switch (j.fmt) {
    case kFmtQ4_K: decode_group<kFmtQ4_K>(j, grp, stage); break;
    case kFmtQ6_K: decode_group<kFmtQ6_K>(j, grp, stage); break;
    case kFmtQ5_K: decode_group<kFmtQ5_K>(j, grp, stage); break;
    case kFmtQ4_0: decode_group<kFmtQ4_0>(j, grp, stage); break;
    case kFmtQ5_0: decode_group<kFmtQ5_0>(j, grp, stage); break;
    case kFmtQ5_1: decode_group<kFmtQ5_1>(j, grp, stage); break;
    default: decode_group<kFmtQ8_0>(j, grp, stage); break;
    }
}

template <int FMT>
DequantJob make_job(const void *wq, int N, int K, uint16_t *w16, int ld) {
    constexpr uint32_t G = group_blocks<FMT>();
    DequantJob j;
    j.wq = (const uint8_t *)wq;
    j.out = w16;
    j.nb = (uint32_t)K / Fmt<FMT>::BE;
    j.K = (uint32_t)K;
    j.ld = (uint32_t)ld;
    j.n_blocks = (uint32_t)N * j.nb;
    j.data_groups = (j.n_blocks + G - 1) / G;
    j.pad_per_row = (uint32_t)(ld - K) / 8;
    j.n_pad = (uint32_t)N * j.pad_per_row;
    j.groups_end = j.data_groups + (j.n_pad + kChunksPerGroup - 1) / kChunksPerGroup;
    j.fmt = FMT;
    return j;
}

DequantJob job_for(int fmt, const void *wq, int N, int K, uint16_t *w16, int ld) {
    switch (fmt) {
    case kFmtQ4_K: return make_job<kFmtQ4_K>(wq, N, K, w16, ld);
    case kFmtQ6_K: return make_job<kFmtQ6_K>(wq, N, K, w16, ld);
    case kFmtQ5_K: return make_job<kFmtQ5_K>(wq, N, K, w16, ld);
    case kFmtQ4_0: return make_job<kFmtQ4_0>(wq, N, K, w16, ld);
    case kFmtQ5_0: return make_job<kFmtQ5_0>(wq, N, K, w16, ld);
    case kFmtQ5_1: return make_job<kFmtQ5_1>(wq, N, K, w16, ld);
    default: return make_job<kFmtQ8_0>(wq, N, K, w16, ld);
    }
}

}  // namespace

hipError_t launch_dequant(int fmt, const void *wq, int N, int K, uint16_t *w16, int ld,
                          hipStream_t stream) {
    const DequantJob j = job_for(fmt, wq, N, K, w16, ld);
    const dim3 grid(j.groups_end), block(kThreads);
    switch (fmt) {
    case kFmtQ4_K: hipLaunchKernelGGL(dequant_kernel<kFmtQ4_K>, grid, block, 0, stream, j); break;
    case kFmtQ6_K: hipLaunchKernelGGL(dequant_kernel<kFmtQ6_K>, grid, block, 0, stream, j); break;
    case kFmtQ5_K: hipLaunchKernelGGL(dequant_kernel<kFmtQ5_K>, grid, block, 0, stream, j); break;
    case kFmtQ4_0: hipLaunchKernelGGL(dequant_kernel<kFmtQ4_0>, grid, block, 0, stream, j); break;
    case kFmtQ5_0: hipLaunchKernelGGL(dequant_kernel<kFmtQ5_0>, grid, block, 0, stream, j); break;
    case kFmtQ5_1: hipLaunchKernelGGL(dequant_kernel<kFmtQ5_1>, grid, block, 0, stream, j); break;
    default: hipLaunchKernelGGL(dequant_kernel<kFmtQ8_0>, grid, block, 0, stream, j); break;
    }
    return hipGetLastError();
}

hipError_t launch_dequant_batch(const DequantSpec *specs, int n, hipStream_t stream) {
    for (int first = 0; first < n; first += kBatchJobs) {
        DequantBatch b;
        b.n = n - first < kBatchJobs ? n - first : kBatchJobs;
        uint32_t total = 0;
        for (int i = 0; i < b.n; ++i) {
            const DequantSpec &sp = specs[first + i];
            b.job[i] = job_for(sp.fmt, sp.wq, sp.N, sp.K, sp.w16, sp.ld);
            total += b.job[i].groups_end;
            b.job[i].groups_end = total;
        }
        for (int i = b.n; i < kBatchJobs; ++i) b.job[i] = b.job[b.n - 1];
        hipLaunchKernelGGL(dequant_batch_kernel, dim3(total), dim3(kThreads), 0, stream, b);
        if (hipError_t e = hipGetLastError()) return e;
    }
    return hipSuccess;
}

}  // namespace mq
