// device_common.h -- small device-side helpers shared by the gfx950 kernels of
// libmoe_mxfp4 (vector types, bf16 rounding, E8M0 scale decode, matrix-core
// wrappers).  Written for CDNA4 (gfx950) only: 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// fp32 -> bf16 bits, round half to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}

// E8M0 scale byte b (meaning 2^(b-127)) as the fp32 scale operand of the
// v_cvt_scalef32_* conversions.  b = 0 is the fp32 denormal 2^-127.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
    return __builtin_bit_cast(float, b ? (b << 23) : 0x00400000u);
}

// Eight E2M1 codes (one dword, element 2i in the low nibble of byte i) times
// a power-of-two scale, widened to bf16 / fp16 by the gfx950 conversion unit.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16x8(uint32_t codes, float scale) {
    bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
    bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
    bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
    bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
    bf16x8_t r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

__device__ __forceinline__ f16x8_t fp4x8_to_f16x8(uint32_t codes, float scale) {
    f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 0);
    f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 1);
    f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 2);
    f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 3);
    f16x8_t r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// 16x16x32 matrix-core products with fp32 accumulation.  Lane l supplies
// A[l % 16][8 * (l / 16) + i] and B[8 * (l / 16) + i][l % 16] (i = 0..7) and
// receives C[4 * (l / 16) + r][l % 16] (r = 0..3).
__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f16(f16x8_t a, f16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ f16x8_t as_f16x8(u32x4_t v) { return __builtin_bit_cast(f16x8_t, v); }

}  // namespace moe
