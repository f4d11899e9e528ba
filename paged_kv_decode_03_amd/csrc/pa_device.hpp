// Device-side helpers shared by the gfx950 kernels of libpa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// ---- bf16 <-> fp32 -------------------------------------------------------

// Low / high bf16 of a packed pair, widened exactly.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((b >> 16) | 0x40u);
    b += 0x7fffu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

// Two small exact integers held as fp32 -> packed bf16 pair (upper halves).
__device__ __forceinline__ uint32_t pack_bf16_trunc(float lo, float hi) {
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// int8 byte n of w, sign-extended and converted exactly to fp32.
__device__ __forceinline__ float i8_at(uint32_t w, int n) {
    return (float)(int32_t)(int8_t)(uint8_t)(w >> (8 * n));
}

// ---- cross-lane reductions inside 16-lane rows (DPP) ----------------------

// v + the value 4 (resp. 8) lanes round the 16-lane row; applied twice it sums
// the four lanes {l, l^4, l^8, l^12} of a row.
__device__ __forceinline__ float row_ror4_add(float v) {
    return v + __builtin_amdgcn_update_dpp(0.0f, v, 0x124, 0xf, 0xf, false);
}
__device__ __forceinline__ float row_ror8_add(float v) {
    return v + __builtin_amdgcn_update_dpp(0.0f, v, 0x128, 0xf, 0xf, false);
}
// Sum over the 4 lanes of a quad (lanes 4k .. 4k+3): quad_perm [1,0,3,2] then [2,3,0,1].
__device__ __forceinline__ float quad_sum(float v) {
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0xb1, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4e, 0xf, 0xf, false);
    return v;
}

// ---- MFMA ---------------------------------------------------------------

// 16 independent 4x4x4 bf16 products, fp32 accumulate.
// Block b = lane / 4. A_b[i][k]: lane 4b+i holds k = 0..3; B_b[k][j]: lane
// 4b+j holds k = 0..3; D_b[i][j]: lane 4b+j, register i.
__device__ __forceinline__ f32x4 mfma4x4x4bf16(i16x4 a, i16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 0, 0, 0);
}
// 16 independent 4x4x1 fp32 outer products: A_b[i] at lane 4b+i, B_b[j] at
// lane 4b+j, D_b[i][j] at lane 4b+j, register i.
__device__ __forceinline__ f32x4 mfma4x4x1f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

// Four packed bf16 (two dwords) as an MFMA operand.
__device__ __forceinline__ i16x4 as_i16x4(uint32_t lo, uint32_t hi) {
    return __builtin_bit_cast(i16x4, make_uint2(lo, hi));
}

// ---- memory --------------------------------------------------------------

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const void* p) { return *reinterpret_cast<const uint2*>(p); }

// Read-only index data (block tables, lengths, scales): loads through the
// constant address space, which the kernel never writes, become scalar loads
// (s_load, into SGPRs) when the index is wave-uniform.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p, int64_t i) {
    typedef const __attribute__((address_space(4))) T* const_ptr;
    return ((const_ptr)p)[i];   // an address-space cast (C-style cast required)
}

// Wave-uniform value (lets the compiler keep it in an SGPR).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long long uniform64(long long v) {
    const unsigned long long u = (unsigned long long)v;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
}

}  // namespace pa
