// The int8 ("MMQ") prefill product on gfx950 (Fucina "Eager GPU Offload
// Without A Compute Graph", what the ik_llama.cpp audit contributed: f32
// activations quantized once to a Q8_1-style int8 layout with scales and
// sums, quantized weights unpacked to signed int8, int8 matrix instructions,
// with numerics of its own; minfer "05 · 8p" §1 and "79" §1 name it as the
// int8 prefill GEMM that streams raw quantized bytes).
//
// Numerics (the definition the tests check against):
//   * activations, per row and 32-element block b: a = max|x|,
//     d = fl32(a / 127), q = nearest integer to fl32(x / d), halves away from
//     zero (all 0 when d = 0), s = fl32(d · Σq);
//   * weights, per format: w = α·c − β with an int8 code c and exact f32
//     factors per 32-element group (16 for Q6_K, whose β is 0);
//   * Y[m, n] = Σ_b (d_b · Σ_G α_G·I_G − β_b·s_b), I_G = Σ_{i∈G} c_i·q_i
//     exact (int8 MFMA, i32 accumulation), the rest in f32.
//
// Kernel layout: 256 threads (2×2 wave64s) per 128 × 128 tile of Y, k-step
// 128 (four activation blocks).  The codes of both operands sit in LDS as
// 128-byte rows of eight 16-byte chunks, swizzled as the f16 kernels' tiles;
// the per-block factors sit beside them, (d, s) per activation row and
// (α, β) per weight row — for Q6_K (d, the two int8 group scales).  Per block and 32×32
// fragment: one v_mfma_i32_32x32x32_i8 (two v_mfma_i32_32x32x16_i8 for Q6_K,
// one per scale group, combined as I0·s0 + I1·s1 in integers), then
// acc += float(I)·(d·α) on the VALU; the
// β·s terms of two blocks at a time go through one v_mfma_f32_32x32x2_f32
// (s of the rows against −β of the columns), on the matrix core the int8
// products leave mostly idle.  The per-block scaling still costs 3 VALU
// operations per output per 32 k against 64 int8 multiply-adds in the
// matrix core, so this kernel is VALU-bound.  (The file is compiled with
// MFMA results in VGPRs: the VALU reads them directly.)

#include "gemm_kernel.h"

namespace mq {
namespace {

constexpr int kMmqBM = 128, kMmqBN = 128, kMmqBK = 128;
constexpr int kMmqKB = kMmqBK / 32;   // activation blocks per step

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}

struct MmqArgs {
    const int8_t *Xq;
    const float *ds;    // (d, s) pairs, [M][K/32]
    const uint8_t *W;
    float *Y;
    float *ws;
    int64_t ldw;        // quantized row bytes
    int ldq, ldy;
    int M, N, K;
    int tiles_m, tiles_n, k_steps, steps_per_split;
    int dp_tiles, tail_tiles;
};

// Byte-wise c − off for bytes holding 0 .. 2·off − 1 (off = 8, 16 or 32):
// (c + 0x80 − off) never carries out of its byte; flipping bit 7 then gives
// c − off in two's complement.
template <uint32_t OFF>
__device__ __forceinline__ uint32_t sub_bytes(uint32_t c) {
    constexpr uint32_t k = (0x80u - OFF) * 0x01010101u;
    return (c + k) ^ 0x80808080u;
}

// Q6_K operands swap the middle 8-byte quarters of every 32-byte block, so
// that the low 8 bytes of each lane's 16 cover one 16-element scale group
// and the high 8 bytes the other (see the MMA step).
__device__ __forceinline__ void perm_q6(u32x4 &c0, u32x4 &c1) {
    const uint32_t a2 = c0.z, a3 = c0.w;
    c0.z = c1.x;
    c0.w = c1.y;
    c1.x = a2;
    c1.y = a3;
}

// ---------------------------------------------------------------------------
// Activation quantization: 8 elements per thread, 4 threads per block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quantize_q8_1_kernel(const float *__restrict__ X, int ldx,
                                                            int8_t *__restrict__ Xq, int ldq,
                                                            float *__restrict__ ds, int nblk,
                                                            int64_t chunks, int cpr) {
    // chunks and the grid stride are multiples of 4, so the four threads of
    // one block always run the same iterations together
    for (int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x; id < chunks;
         id += (int64_t)gridDim.x * 256) {
        const int64_t row = id / cpr;
        const int c = (int)(id - row * cpr);
        const f32x4 *src = reinterpret_cast<const f32x4 *>(X + row * ldx + 8 * c);
        const f32x4 lo = src[0], hi = src[1];
        const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(v[j]));
        a = fmaxf(a, __shfl_xor(a, 1));
        a = fmaxf(a, __shfl_xor(a, 2));
        const float d = a / 127.0f;
        int q[8], sum = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int qj = 0;
            if (d != 0.0f) {
                const float t = v[j] / d;
                float r = truncf(t);
                if (fabsf(t - r) >= 0.5f) r += copysignf(1.0f, t);   // halves away from zero
                qj = (int)r;
            }
            q[j] = qj;
            sum += qj;
        }
        sum += __shfl_xor(sum, 1);
        sum += __shfl_xor(sum, 2);
        uint2 packed;
        packed.x = (q[0] & 255) | ((q[1] & 255) << 8) | ((q[2] & 255) << 16) | ((uint32_t)q[3] << 24);
        packed.y = (q[4] & 255) | ((q[5] & 255) << 8) | ((q[6] & 255) << 16) | ((uint32_t)q[7] << 24);
        *reinterpret_cast<uint2 *>(Xq + row * ldq + 8 * c) = packed;
        if ((c & 3) == 0) {
            float2 out;
            out.x = d;
            out.y = d * (float)sum;
            *reinterpret_cast<float2 *>(ds + 2 * (row * nblk + (c >> 2))) = out;
        }
    }
}

// ---------------------------------------------------------------------------
// Loaders: one register set; a part is one 32-element block (activations,
// 32-element weight formats) or a 64-element half step (K-quants, Q6_K).
//   begin(k0, live)     offsets of the step at k0 (live == false: zeros)
//   load(i)             global loads of part i
//   store(i, codes, f)  part i's codes to the LDS code tile and its factors
//                       to the factor tile ([kMmqKB][ROWS] float2)
// ---------------------------------------------------------------------------

template <int ROWS, bool PERM>
struct MmqALoader {
    static constexpr int NPART = ROWS * kMmqKB / kThreads;
    __amdgpu_buffer_rsrc_t rq, rs;
    uint32_t qoff[NPART], soff[NPART];
    int nblk, b0;
    bool live_;
    u32x4 q[NPART][2];
    uint2 f[NPART];

    __device__ void init(const int8_t *Xq, int ldq, const float *ds, int rows_valid, int K) {
        nblk = K >> 5;
        rq = make_rsrc(Xq, (uint32_t)((int64_t)(rows_valid - 1) * ldq + K));
        rs = make_rsrc(ds, (uint32_t)((int64_t)rows_valid * nblk * 8));
#pragma unroll
        for (int i = 0; i < NPART; ++i) {
            const int t = i * kThreads + (int)threadIdx.x, r = t >> 2, j = t & 3;
            qoff[i] = (uint32_t)(r * ldq + 32 * j);
            soff[i] = (uint32_t)((r * nblk + j) * 8);
        }
    }
    __device__ __forceinline__ void begin(int k0, bool live) {
        b0 = k0 >> 5;
        live_ = live;
    }
    __device__ __forceinline__ void load(int i) {
        const int j = ((i * kThreads + (int)threadIdx.x) & 3);
        const bool ok = live_ && b0 + j < nblk;
        const uint32_t o = ok ? qoff[i] + 32u * (uint32_t)b0 : kOOB;
        q[i][0] = buf_load16(rq, o);
        q[i][1] = buf_load16(rq, o + 16);
        f[i] = buf_load8(rs, ok ? soff[i] + 8u * (uint32_t)b0 : kOOB);
    }
    __device__ __forceinline__ void store(int i, u32x4 *codes, float2 *fac) const {
        const int t = i * kThreads + (int)threadIdx.x, r = t >> 2, j = t & 3;
        u32x4 c0 = q[i][0], c1 = q[i][1];
        if constexpr (PERM) perm_q6(c0, c1);
        const int sw = swz<8>(r);
        codes[r * 8 + ((2 * j) ^ sw)] = c0;
        codes[r * 8 + ((2 * j + 1) ^ sw)] = c1;
        fac[j * ROWS + r] = __builtin_bit_cast(float2, f[i]);
    }
};

// Q8_0 / Q4_0 / Q5_0 / Q5_1: one 32-element block per part.  Blocks of 34,
// 18 and 22 bytes are only 2-byte aligned: read as the aligned dwords that
// cover them (up to 2 lead bytes) and re-assembled with v_alignbyte.
template <int ROWS, int FMT>
struct MmqB32Loader {
    static constexpr int NPART = ROWS * kMmqKB / kThreads;
    static constexpr uint32_t BB = FMT == kFmtQ8_0 ? 34 : FMT == kFmtQ4_0 ? 18 : FMT == kFmtQ5_0 ? 22 : 24;
    // dwords held: 32 bytes from the aligned start, Q8_0's 36th, and a zero
    // spare that dw<T> may read as the upper neighbour
    static constexpr int NW = 10;
    __amdgpu_buffer_rsrc_t rs;
    uint32_t roff[NPART];
    int nblk, b0;
    bool live_;
    uint32_t w[NPART][NW], sh[NPART];

    __device__ void init(const uint8_t *W, int64_t row_bytes, int n0, int rows_valid, int K) {
        nblk = K >> 5;
        const int64_t start = (int64_t)n0 * row_bytes;
        const uint32_t shift0 = (uint32_t)(((uintptr_t)W + start) & 15);
        rs = make_rsrc(W + start - shift0,
                       (uint32_t)((shift0 + (int64_t)rows_valid * row_bytes + 3) & ~(int64_t)3));
#pragma unroll
        for (int i = 0; i < NPART; ++i) {
            const int t = i * kThreads + (int)threadIdx.x, r = t >> 2;
            roff[i] = shift0 + (uint32_t)(r * row_bytes);
        }
    }
    __device__ __forceinline__ void begin(int k0, bool live) {
        b0 = k0 >> 5;
        live_ = live;
    }
    __device__ __forceinline__ void load(int i) {
        const int j = (i * kThreads + (int)threadIdx.x) & 3;
        const uint32_t o = roff[i] + (uint32_t)(b0 + j) * BB;
        sh[i] = o & 3;
        const uint32_t a = live_ && b0 + j < nblk ? (o & ~3u) : kOOB;
        const u32x4 v0 = buf_load16(rs, a), v1 = buf_load16(rs, a + 16);
        uint32_t *q = w[i];
        q[0] = v0.x; q[1] = v0.y; q[2] = v0.z; q[3] = v0.w;
        q[4] = v1.x; q[5] = v1.y; q[6] = v1.z; q[7] = v1.w;
        q[8] = FMT == kFmtQ8_0 ? buf_load4(rs, a + 32) : 0u;   // 34 + 2 bytes: 9 dwords
        q[9] = 0;
    }
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
    __device__ __forceinline__ void store(int i, u32x4 *codes, float2 *fac) const {
        const int t = i * kThreads + (int)threadIdx.x, r = t >> 2, j = t & 3;
        const uint32_t *q = w[i];
        const uint32_t s = sh[i];
        const uint32_t h0 = dw<0>(q, s);
        float2 ab;
        ab.x = f16_bits_to_f32(h0);
        ab.y = 0.0f;
        u32x4 c0, c1;
        if constexpr (FMT == kFmtQ8_0) {
            c0 = u32x4{dw<2>(q, s), dw<6>(q, s), dw<10>(q, s), dw<14>(q, s)};
            c1 = u32x4{dw<18>(q, s), dw<22>(q, s), dw<26>(q, s), dw<30>(q, s)};
        } else {
            constexpr uint32_t QS = FMT == kFmtQ4_0 ? 2 : FMT == kFmtQ5_0 ? 6 : 8;
            constexpr uint32_t QH = FMT == kFmtQ5_1 ? 4 : 2;
            const uint32_t L = 0x0F0F0F0Fu;
            const uint32_t n0 = dw<QS>(q, s), n1 = dw<QS + 4>(q, s), n2 = dw<QS + 8>(q, s),
                           n3 = dw<QS + 12>(q, s);
            // elements 0..15: low nibbles of bytes 0..15; 16..31: high nibbles
            uint32_t e[8] = {n0 & L, n1 & L, n2 & L, n3 & L,
                             (n0 >> 4) & L, (n1 >> 4) & L, (n2 >> 4) & L, (n3 >> 4) & L};
            if constexpr (FMT != kFmtQ4_0) {
                const uint32_t qh = dw<QH>(q, s);
#pragma unroll
                for (int k = 0; k < 8; ++k) e[k] |= spread4_to_bit4((qh >> (4 * k)) & 15);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if constexpr (FMT == kFmtQ4_0) e[k] = sub_bytes<8>(e[k]);
                else if constexpr (FMT == kFmtQ5_0) e[k] = sub_bytes<16>(e[k]);
            }
            if constexpr (FMT == kFmtQ5_1) ab.y = -f16_bits_to_f32(h0 >> 16);
            c0 = u32x4{e[0], e[1], e[2], e[3]};
            c1 = u32x4{e[4], e[5], e[6], e[7]};
        }
        const int sw = swz<8>(r);
        codes[r * 8 + ((2 * j) ^ sw)] = c0;
        codes[r * 8 + ((2 * j + 1) ^ sw)] = c1;
        fac[j * ROWS + r] = ab;
    }
};

// Q4_K / Q5_K: a part is the 64-element quarter c of a super-block (its
// sub-blocks 2c and 2c + 1): the 16-byte header, the 32 quant bytes of the
// quarter and, for Q5_K, the 32 qh bytes (bits 2c and 2c + 1).
template <int ROWS, int FMT>
struct MmqBKLoader {
    static constexpr int NPART = ROWS * 2 / kThreads;
    static constexpr uint32_t BB = FMT == kFmtQ4_K ? 144 : 176;
    static constexpr uint32_t QS = FMT == kFmtQ4_K ? 16 : 48;
    __amdgpu_buffer_rsrc_t rs;
    uint32_t roff[NPART];
    uint32_t obase;
    int k0_;
    u32x4 hdr[NPART], qs[NPART][2], qh[NPART][2];

    __device__ void init(const uint8_t *W, int64_t row_bytes, int n0, int rows_valid, int) {
        rs = make_rsrc(W + (int64_t)n0 * row_bytes, (uint32_t)(rows_valid * row_bytes));
#pragma unroll
        for (int i = 0; i < NPART; ++i) {
            const int r = (i * kThreads + (int)threadIdx.x) >> 1;
            roff[i] = (uint32_t)(r * row_bytes);
        }
    }
    __device__ __forceinline__ void begin(int k0, bool live) {
        k0_ = k0;
        obase = live ? (uint32_t)(k0 >> 8) * BB : kOOB;
    }
    __device__ __forceinline__ void load(int i) {
        const uint32_t p = threadIdx.x & 1, c = ((k0_ >> 6) + p) & 3;
        const uint32_t o = roff[i] + obase;
        hdr[i] = buf_load16(rs, o);
        qs[i][0] = buf_load16(rs, o + QS + 32 * c);
        qs[i][1] = buf_load16(rs, o + QS + 32 * c + 16);
        if constexpr (FMT == kFmtQ5_K) {
            qh[i][0] = buf_load16(rs, o + 16);
            qh[i][1] = buf_load16(rs, o + 32);
        }
    }
    __device__ __forceinline__ void store(int i, u32x4 *codes, float2 *fac) const {
        const int p = threadIdx.x & 1, c = ((k0_ >> 6) + p) & 3;
        const int r = (i * kThreads + (int)threadIdx.x) >> 1;
        const u32x4 h = hdr[i];
        // sub-blocks 2c, 2c + 1: scale bytes at 2c, 2c + 1 (c < 2), else the low
        // 6 bits come from bytes 8 + 2(c − 2) .. and the top 2 from bytes
        // 2(c − 2) ..; both read at shift 16·(c & 1), so both are formed and
        // one is selected (a branch here made the compiler spill)
        const int s0 = 16 * (c & 1), s1 = s0 + 8;
        const bool lowq = c < 2;
        const uint32_t y0 = h.y >> s0, z0 = h.z >> s0, w0 = h.w >> s0;
        const uint32_t y1 = h.y >> s1, z1 = h.z >> s1, w1 = h.w >> s1;
        const uint32_t sc0 = lowq ? y0 & 63 : (w0 & 15) | (((y0 >> 6) & 3) << 4);
        const uint32_t m0 = lowq ? z0 & 63 : ((w0 >> 4) & 15) | (((z0 >> 6) & 3) << 4);
        const uint32_t sc1 = lowq ? y1 & 63 : (w1 & 15) | (((y1 >> 6) & 3) << 4);
        const uint32_t m1 = lowq ? z1 & 63 : ((w1 >> 4) & 15) | (((z1 >> 6) & 3) << 4);
        const float d = f16_bits_to_f32(h.x), dmin = f16_bits_to_f32(h.x >> 16);
        const uint32_t L = 0x0F0F0F0Fu;
        const uint32_t qv[8] = {qs[i][0].x, qs[i][0].y, qs[i][0].z, qs[i][0].w,
                                qs[i][1].x, qs[i][1].y, qs[i][1].z, qs[i][1].w};
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            lo[k] = qv[k] & L;
            hi[k] = (qv[k] >> 4) & L;
        }
        if constexpr (FMT == kFmtQ5_K) {
            const uint32_t hv[8] = {qh[i][0].x, qh[i][0].y, qh[i][0].z, qh[i][0].w,
                                    qh[i][1].x, qh[i][1].y, qh[i][1].z, qh[i][1].w};
            const uint32_t B = 0x01010101u;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                lo[k] |= ((hv[k] >> (2 * c)) & B) << 4;
                hi[k] |= ((hv[k] >> (2 * c + 1)) & B) << 4;
            }
        }
        const int sw = swz<8>(r);
        codes[r * 8 + ((4 * p) ^ sw)] = u32x4{lo[0], lo[1], lo[2], lo[3]};
        codes[r * 8 + ((4 * p + 1) ^ sw)] = u32x4{lo[4], lo[5], lo[6], lo[7]};
        codes[r * 8 + ((4 * p + 2) ^ sw)] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        codes[r * 8 + ((4 * p + 3) ^ sw)] = u32x4{hi[4], hi[5], hi[6], hi[7]};
        fac[(2 * p) * ROWS + r] = float2{d * (float)sc0, dmin * (float)m0};
        fac[(2 * p + 1) * ROWS + r] = float2{d * (float)sc1, dmin * (float)m1};
    }
};

// Q6_K: a part is 64 elements, quarter j of a 256-element block (half
// h = j / 2, groups g = 2(j % 2), +1): 64 ql bytes at 64h (low nibbles for
// j even, high for j odd), 32 qh bytes at 128 + 32h (bit pairs 2g), the four
// int8 scales of its 16-element groups and d.  Blocks are 210 bytes, so
// 2-byte aligned: everything is read as aligned dwords and re-assembled.
template <int ROWS>
struct MmqBQ6Loader {
    static constexpr int NPART = ROWS * 2 / kThreads;
    __amdgpu_buffer_rsrc_t rs;
    uint32_t roff[NPART];
    uint32_t obase;
    int k0_;
    uint32_t ql[NPART][17], qh[NPART][9], tail[NPART][3], sh[NPART];

    __device__ void init(const uint8_t *W, int64_t row_bytes, int n0, int rows_valid, int) {
        const int64_t start = (int64_t)n0 * row_bytes;
        const uint32_t shift0 = (uint32_t)(((uintptr_t)W + start) & 15);
        rs = make_rsrc(W + start - shift0,
                       (uint32_t)((shift0 + (int64_t)rows_valid * row_bytes + 3) & ~(int64_t)3));
#pragma unroll
        for (int i = 0; i < NPART; ++i) {
            const int r = (i * kThreads + (int)threadIdx.x) >> 1;
            roff[i] = shift0 + (uint32_t)(r * row_bytes);
        }
    }
    __device__ __forceinline__ void begin(int k0, bool live) {
        k0_ = k0;
        obase = live ? (uint32_t)(k0 >> 8) * 210u : kOOB;
    }
    __device__ __forceinline__ void load(int i) {
        const uint32_t p = threadIdx.x & 1, j = ((k0_ >> 6) + p) & 3, h = j >> 1;
        const uint32_t o = roff[i] + obase;      // block start (kOOB + small when dead)
        sh[i] = o & 3;
        const uint32_t a = obase == kOOB ? kOOB : (o & ~3u);
        const uint32_t aql = a + 64 * h, aqh = a + 128 + 32 * h;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const u32x4 v = buf_load16(rs, aql + 16 * k);
            ql[i][4 * k] = v.x; ql[i][4 * k + 1] = v.y; ql[i][4 * k + 2] = v.z; ql[i][4 * k + 3] = v.w;
        }
        ql[i][16] = buf_load4(rs, aql + 64);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const u32x4 v = buf_load16(rs, aqh + 16 * k);
            qh[i][4 * k] = v.x; qh[i][4 * k + 1] = v.y; qh[i][4 * k + 2] = v.z; qh[i][4 * k + 3] = v.w;
        }
        qh[i][8] = buf_load4(rs, aqh + 32);
        // scales of groups 8h + 2(j % 2) .. +3 (bytes 192 + 8h + 4(j % 2)) and d (208)
        const uint32_t asc = a + 192 + 8 * h + 4 * (j & 1);
        tail[i][0] = buf_load4(rs, asc);
        tail[i][1] = buf_load4(rs, asc + 4);
        // d: block bytes 208..209, inside the aligned dword at a + 208 (its low
        // half when the block starts 4-byte aligned, else its high half)
        tail[i][2] = buf_load4(rs, a + 208);
    }
    __device__ __forceinline__ void store(int i, u32x4 *codes, float2 *fac) const {
        const int p = threadIdx.x & 1, j = ((k0_ >> 6) + p) & 3;
        const int r = (i * kThreads + (int)threadIdx.x) >> 1;
        const uint32_t s = sh[i];
        const bool odd = j & 1;
        const uint32_t L = 0x0F0F0F0Fu, B3 = 0x03030303u;
        const int g0 = 2 * (j & 1);
        uint32_t e[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            // bytes 4k .. 4k + 3 of the quarter: elements l = 4k..4k+3 (k < 8,
            // group g0) or l = 4(k − 8).. (group g0 + 1, ql bytes 32 + l)
            const uint32_t b = __builtin_amdgcn_alignbyte(ql[i][k + 1], ql[i][k], s);
            const uint32_t low = odd ? (b >> 4) & L : b & L;
            const int kk = k & 7;
            const uint32_t hb = __builtin_amdgcn_alignbyte(qh[i][kk + 1], qh[i][kk], s);
            const int g = g0 + (k >> 3);
            e[k] = sub_bytes<32>(low | (((hb >> (2 * g)) & B3) << 4));
        }
        const uint32_t sc = __builtin_amdgcn_alignbyte(tail[i][1], tail[i][0], s);
        const float d = f16_bits_to_f32(s ? tail[i][2] >> 16 : tail[i][2]);
        // factors per 32-element block: d and the two int8 group scales,
        // sign-extended into the halves of one word (the kernel combines the
        // two group dots in integers: I0·s0 + I1·s1, exact)
        auto pair = [](uint32_t lo, uint32_t hi) {
            return __builtin_bit_cast(float, (uint32_t)(int)(int8_t)lo & 0xFFFFu |
                                                 ((uint32_t)(int)(int8_t)hi << 16));
        };
        const float p01 = pair(sc & 255, (sc >> 8) & 255), p23 = pair((sc >> 16) & 255, sc >> 24);
        u32x4 c0 = u32x4{e[0], e[1], e[2], e[3]}, c1 = u32x4{e[4], e[5], e[6], e[7]};
        u32x4 c2 = u32x4{e[8], e[9], e[10], e[11]}, c3 = u32x4{e[12], e[13], e[14], e[15]};
        perm_q6(c0, c1);
        perm_q6(c2, c3);
        const int sw = swz<8>(r);
        codes[r * 8 + ((4 * p) ^ sw)] = c0;
        codes[r * 8 + ((4 * p + 1) ^ sw)] = c1;
        codes[r * 8 + ((4 * p + 2) ^ sw)] = c2;
        codes[r * 8 + ((4 * p + 3) ^ sw)] = c3;
        fac[(2 * p) * ROWS + r] = float2{d, p01};
        fac[(2 * p + 1) * ROWS + r] = float2{d, p23};
    }
};

template <int ROWS, int FMT>
struct MmqBFor;
template <int ROWS> struct MmqBFor<ROWS, kFmtQ8_0> { typedef MmqB32Loader<ROWS, kFmtQ8_0> T; };
template <int ROWS> struct MmqBFor<ROWS, kFmtQ4_0> { typedef MmqB32Loader<ROWS, kFmtQ4_0> T; };
template <int ROWS> struct MmqBFor<ROWS, kFmtQ5_0> { typedef MmqB32Loader<ROWS, kFmtQ5_0> T; };
template <int ROWS> struct MmqBFor<ROWS, kFmtQ5_1> { typedef MmqB32Loader<ROWS, kFmtQ5_1> T; };
template <int ROWS> struct MmqBFor<ROWS, kFmtQ4_K> { typedef MmqBKLoader<ROWS, kFmtQ4_K> T; };
template <int ROWS> struct MmqBFor<ROWS, kFmtQ5_K> { typedef MmqBKLoader<ROWS, kFmtQ5_K> T; };
template <int ROWS> struct MmqBFor<ROWS, kFmtQ6_K> { typedef MmqBQ6Loader<ROWS> T; };

// ---------------------------------------------------------------------------
// The kernel.  Work decode (whole tiles, then K ranges of tail tiles) and
// the XCD-aware tile order are the f16 GEMM's.  Per step: the global loads
// of the next step are issued first, the MMA of this step runs from LDS
// stage st, then the next step's codes and factors are written to stage
// st ^ 1 (never the one being read) and the step ends at a barrier.
// ---------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(kThreads, 1) void mmq_kernel(MmqArgs a) {
    constexpr int BM = kMmqBM, BN = kMmqBN, BK = kMmqBK;
    constexpr int TM = BM / 2, TN = BN / 2, FM = TM / 32, FN = TN / 32;
    constexpr bool Q6 = FMT == kFmtQ6_K;
    constexpr bool BETA = FMT == kFmtQ4_K || FMT == kFmtQ5_K || FMT == kFmtQ5_1;
    __shared__ u32x4 Ac[2][BM * 8], Bc[2][BN * 8];
    // (d, s) of 4 consecutive rows are read as two 16-byte vectors
    __shared__ __align__(16) float2 Af[2][kMmqKB * BM];
    __shared__ __align__(16) float2 Bf[2][kMmqKB * BN];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int pid = blockIdx.x;
    int tile, part = 0;
    if (pid < a.dp_tiles) {
        tile = xcd_remap(pid, a.dp_tiles);
    } else {
        const int j = xcd_remap(pid - a.dp_tiles, (int)gridDim.x - a.dp_tiles);
        tile = a.dp_tiles + j % a.tail_tiles;
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
    const int nblk = a.K >> 5;

    MmqALoader<BM, Q6> la;
    la.init(a.Xq + (int64_t)m0 * a.ldq, a.ldq, a.ds + (int64_t)m0 * nblk * 2, min(BM, a.M - m0),
            a.K);
    typename MmqBFor<BN, FMT>::T lb;
    lb.init(a.W, a.ldw, n0, min(BN, a.N - n0), a.K);
    constexpr int NA = decltype(la)::NPART, NB = decltype(lb)::NPART;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    la.begin(kt_begin * BK, true);
    lb.begin(kt_begin * BK, true);
    static_for<NA>([&](auto I) MQ_INLINE { la.load(I); });
    static_for<NB>([&](auto I) MQ_INLINE { lb.load(I); });
    static_for<NA>([&](auto I) MQ_INLINE { la.store(I, Ac[0], Af[0]); });
    static_for<NB>([&](auto I) MQ_INLINE { lb.store(I, Bc[0], Bf[0]); });
    sync_lds();

    const int rl = lane & 31, hl = lane >> 5;
    for (int kt = kt_begin; kt < kt_end; ++kt) {
        const int st = (kt - kt_begin) & 1;
        const bool more = kt + 1 < kt_end;
        la.begin((kt + 1) * BK, more);
        lb.begin((kt + 1) * BK, more);
        static_for<NA>([&](auto I) MQ_INLINE { la.load(I); });
        static_for<NB>([&](auto I) MQ_INLINE { lb.load(I); });

        const u32x4 *A = Ac[st], *B = Bc[st];
        const float2 *AF = Af[st], *BF = Bf[st];
        static_for<kMmqKB>([&](auto KB) MQ_INLINE {
            constexpr int kb = KB;
            // keep each block's MFMAs beside their scaling: hoisted over all
            // four blocks, their results alone fill the register file
            __builtin_amdgcn_sched_barrier(0);
            const int ch = 2 * kb + hl;
            v4i af[FM], bq[FN];
            float2 bfac[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = wm * TM + 32 * i + rl;
                af[i] = __builtin_bit_cast(v4i, A[r * 8 + (ch ^ swz<8>(r))]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int r = wn * TN + 32 * j + rl;
                bq[j] = __builtin_bit_cast(v4i, B[r * 8 + (ch ^ swz<8>(r))]);
                bfac[j] = BF[kb * BN + r];
            }
            // One fragment at a time: its integer product, then its scaling.
            // (Issuing all of a block's products first needs 64 more VGPRs
            // and halves the waves per SIMD, which measured 1.4x slower: the
            // second wave hides each MFMA's latency better.)
            auto beta = [&](int i, int j) MQ_INLINE {
                if constexpr (BETA && (kb & 1)) {
                    // β·s of blocks kb − 1 (lanes 0–31) and kb (32–63)
                    const int rs = wm * TM + 32 * i + rl, cs = wn * TN + 32 * j + rl;
                    const float sa = AF[(kb - 1 + hl) * BM + rs].y;
                    const float nb = -BF[(kb - 1 + hl) * BN + cs].y;
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(sa, nb, acc[i][j], 0, 0, 0);
                }
                // the scaled accumulator is "used" here, in program order:
                // arithmetic carries no ordering against the scheduling
                // barrier, and left free the compiler issues every block's
                // MFMAs first and holds all their results at once
                asm volatile("" : "+v"(acc[i][j]));
            };
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                // d of the 16 rows this lane holds in a 32x32 block: rows
                // 8·(e/4) + 4·hl + e%4, four runs of 4 consecutive rows
                float dr[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int r0 = wm * TM + 32 * i + 8 * g + 4 * hl;
                    const f32x4 p0 = *reinterpret_cast<const f32x4 *>(&AF[kb * BM + r0]);
                    const f32x4 p1 = *reinterpret_cast<const f32x4 *>(&AF[kb * BM + r0 + 2]);
                    dr[4 * g] = p0.x; dr[4 * g + 1] = p0.z; dr[4 * g + 2] = p1.x; dr[4 * g + 3] = p1.z;
                }
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if constexpr (Q6) {
                        const long alo = __builtin_bit_cast(long, int2{af[i].x, af[i].y});
                        const long ahi = __builtin_bit_cast(long, int2{af[i].z, af[i].w});
                        const long blo = __builtin_bit_cast(long, int2{bq[j].x, bq[j].y});
                        const long bhi = __builtin_bit_cast(long, int2{bq[j].z, bq[j].w});
                        const v16i I0 = __builtin_amdgcn_mfma_i32_32x32x16_i8(alo, blo, v16i{}, 0, 0, 0);
                        const v16i I1 = __builtin_amdgcn_mfma_i32_32x32x16_i8(ahi, bhi, v16i{}, 0, 0, 0);
                        // |I| <= 16·127·32 and |s| <= 32: 24-bit products, and
                        // I0·s0 + I1·s1 < 2^24 converts exactly
                        const int s01 = __builtin_bit_cast(int, bfac[j].y);
                        const int s0 = (s01 << 16) >> 16, s1 = s01 >> 16;
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int t = __mul24(I0[e], s0) + __mul24(I1[e], s1);
                            acc[i][j][e] = __builtin_fmaf((float)t, dr[e] * bfac[j].x, acc[i][j][e]);
                        }
                    } else {
                        const v16i I = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bq[j], v16i{}, 0, 0, 0);
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            acc[i][j][e] = __builtin_fmaf((float)I[e], dr[e] * bfac[j].x, acc[i][j][e]);
                    }
                    beta(i, j);
                }
            }
        });

        static_for<NA>([&](auto I) MQ_INLINE { la.store(I, Ac[st ^ 1], Af[st ^ 1]); });
        static_for<NB>([&](auto I) MQ_INLINE { lb.store(I, Bc[st ^ 1], Bf[st ^ 1]); });
        sync_lds();
    }

    // C layout of a 32x32 block: lane holds column lane & 31 and rows
    // 8·(e/4) + 4·(lane/32) + e%4.  A tail range writes its whole partial
    // tile to slot (part, tail tile) of the workspace.
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
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = wn * TN + 32 * j + rl;
            if (col >= cols) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = wm * TM + 32 * i + 8 * (e >> 2) + 4 * hl + (e & 3);
                if (row < rows) out[(int64_t)row * ldo + col] = acc[i][j][e];
            }
        }
}

template <int FMT>
hipError_t launch_mmq_fmt(const MmqArgs &a, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((mmq_kernel<FMT>), dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_q8_1(const float *X, int ldx, int8_t *Xq, int ldq, float *ds, int M,
                                int K, hipStream_t stream) {
    const int cpr = K / 8;
    const int64_t chunks = (int64_t)M * cpr;
    int64_t blocks = (chunks + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;   // grid-stride beyond 2^28 chunks
    hipLaunchKernelGGL(quantize_q8_1_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, X, ldx,
                       Xq, ldq, ds, K / 32, chunks, cpr);
    return hipGetLastError();
}

bool mmq_plan_has_kernel(const GemmPlan &p) { return p.bm == kMmqBM && p.bn == kMmqBN; }

// The f16 GEMM's rule with 128 × 128 tiles and 128-wide k-steps: whole rounds
// of kCUs tiles over all of K, the last partial round split along K (at
// least two steps per range), or every tile split split_req >= 2 ways.
GemmPlan plan_mmq(int M, int N, int K, int split_req) {
    GemmPlan p;
    p.bm = kMmqBM;
    p.bn = kMmqBN;
    p.tiles_m = (M + p.bm - 1) / p.bm;
    p.tiles_n = (N + p.bn - 1) / p.bn;
    const int tiles = p.tiles_m * p.tiles_n;
    const int ks = (K + kMmqBK - 1) / kMmqBK;
    p.k_steps = ks;
    int dp = tiles, split = 1;
    if (split_req >= 2) {
        dp = 0;
        split = split_req;
    } else if (split_req == 0) {
        const int rem = tiles % kCUs;
        if (rem > 0) {
            int s = kCUs / rem;
            s = s > 16 ? 16 : s;
            s = s > ks / 2 ? ks / 2 : s;
            if (s >= 2) {
                dp = tiles - rem;
                split = s;
            }
        }
    }
    if (split > ks) split = ks;
    const int per = (ks + split - 1) / split;
    split = (ks + per - 1) / per;
    if (split == 1) dp = tiles;
    p.dp_tiles = dp;
    p.tail_tiles = tiles - dp;
    p.split = split;
    p.steps_per_split = split > 1 ? per : ks;
    p.ws_bytes = split > 1 ? (int64_t)split * p.tail_tiles * p.bm * p.bn * 4 : 0;
    return p;
}

hipError_t launch_mmq(int fmt, const int8_t *Xq, int ldq, const float *ds, const void *W,
                      int64_t ldw, float *Y, int ldy, int M, int N, int K, const GemmPlan &plan,
                      float *ws, hipStream_t stream) {
    MmqArgs a;
    a.Xq = Xq;
    a.ds = ds;
    a.W = (const uint8_t *)W;
    a.Y = Y;
    a.ws = ws;
    a.ldw = ldw;
    a.ldq = ldq;
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
    case kFmtQ8_0: e = launch_mmq_fmt<kFmtQ8_0>(a, grid, stream); break;
    case kFmtQ4_0: e = launch_mmq_fmt<kFmtQ4_0>(a, grid, stream); break;
    case kFmtQ5_0: e = launch_mmq_fmt<kFmtQ5_0>(a, grid, stream); break;
    case kFmtQ5_1: e = launch_mmq_fmt<kFmtQ5_1>(a, grid, stream); break;
    case kFmtQ4_K: e = launch_mmq_fmt<kFmtQ4_K>(a, grid, stream); break;
    case kFmtQ5_K: e = launch_mmq_fmt<kFmtQ5_K>(a, grid, stream); break;
    case kFmtQ6_K: e = launch_mmq_fmt<kFmtQ6_K>(a, grid, stream); break;
    default: e = hipErrorInvalidValue; break;
    }
    if (e != hipSuccess || plan.split == 1) return e;
    const int blocks = plan.tail_tiles * (plan.bm * plan.bn / 1024);
    return launch_splitk_reduce(plan.split, dim3(blocks), stream, ws, plan.tail_tiles,
                                plan.dp_tiles, plan.bm, plan.bn, plan.tiles_m, plan.tiles_n, Y,
                                ldy, M, N);
}

}  // namespace mq
