// Device-side helpers shared by the mq kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Value of an f16 bit pattern held in the low 16 bits (exact widening).
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

// Pin a value as an f32 register.  The decode rounds to f32 first and only
// then to f16; left alone, the compiler folds "fma, then convert" into one
// v_fma_mix{lo,hi}_f16, which rounds the exact value straight to f16 and
// differs from the two-step result where the f32 value is an f16 midpoint.
__device__ __forceinline__ float as_f32(float v) {
    asm("" : "+v"(v));
    return v;
}

// Two f32 values rounded to f16 (round to nearest even, subnormals kept) and
// packed low/high into one dword.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    half2v v = {(_Float16)as_f32(lo), (_Float16)as_f32(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// Hide what the optimizer knows about a value's bits.  Applied to a masked
// dword before its bytes are converted, it keeps each conversion a single
// v_cvt_f32_ubyteK: knowing the high nibbles are zero, the optimizer would
// otherwise rewrite "byte k" as a 4-bit field extract plus a conversion.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// Byte k (0..3) of a dword as float (exact); lowers to v_cvt_f32_ubyteK.
template <int k>
__device__ __forceinline__ float ubyte_f32(uint32_t w) {
    return (float)((w >> (8 * k)) & 0xFFu);
}

// Signed byte k (0..3) of a dword as float (exact).
template <int k>
__device__ __forceinline__ float sbyte_f32(uint32_t w) {
    return (float)(int)(int8_t)((w >> (8 * k)) & 0xFFu);
}

// Bytes [2, 6) of the 8-byte little-endian pair (lo, hi).
__device__ __forceinline__ uint32_t shift2(uint32_t hi, uint32_t lo) {
    return __builtin_amdgcn_alignbyte(hi, lo, 2);
}

// Buffer resource over [base, base + bytes) for raw buffer loads: a load whose
// offset is at or past `bytes` returns zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Offset used for a masked-off load (beyond every range this library builds).
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

}  // namespace mq
