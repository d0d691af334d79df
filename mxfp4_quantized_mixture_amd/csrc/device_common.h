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
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

// fp32 -> bf16 bits, round half to even (finite inputs).
// Workgroup barrier ordering LDS accesses only.  __syncthreads() also
// orders global memory, which makes every wavefront wait for all of its
// outstanding loads (the load counter does not tell loads from stores).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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

// silu(z) = z / (1 + e^-z) with the hardware exp2 and reciprocal (a few ulp;
// z -> -inf gives -0, z -> +inf gives z)
__device__ __forceinline__ float silu_f32(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896341f * z));
}

// fp8 (E4M3) residual terms.  A block of 32 values is written as NT E4M3
// terms, term t + 1 carrying the rounding residual of term t, each with its
// own E8M0 scale 2^s.  s = floor(log2 amax) - 7 puts the block's largest
// magnitude in [128, 256) (E4M3 tops out at 448); an all-zero block gets
// s = 0, and s never drops below -127.
__device__ __forceinline__ int fp8_term_exponent(float amax) {
    int se = amax > 0.f ? (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFF) - 127 - 7 : 0;
    return se < -127 ? -127 : se;
}
// 2^-s for s in [-127, 126]
__device__ __forceinline__ float exp2i_neg(int se) {
    return __builtin_bit_cast(float, (uint32_t)(127 - se) << 23);
}
// 2^s for s in [-127, 127] (2^-127 as the fp32 denormal)
__device__ __forceinline__ float exp2i(int se) {
    return se >= -126 ? __builtin_bit_cast(float, (uint32_t)(127 + se) << 23)
                      : __builtin_bit_cast(float, 0x00400000u);
}
// Four values (already divided by the term scale) -> four E4M3 bytes, round
// to nearest even; |v| < 448 so nothing saturates.
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
    int pk = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, pk, true);
    return (uint32_t)pk;
}
// v[0..3] -= the four E4M3 bytes of q times sc
__device__ __forceinline__ void sub4_fp8(float* v, uint32_t q, float sc) {
    v[0] -= __builtin_amdgcn_cvt_f32_fp8((int)q, 0) * sc;
    v[1] -= __builtin_amdgcn_cvt_f32_fp8((int)q, 1) * sc;
    v[2] -= __builtin_amdgcn_cvt_f32_fp8((int)q, 2) * sc;
    v[3] -= __builtin_amdgcn_cvt_f32_fp8((int)q, 3) * sc;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ f16x8_t as_f16x8(u32x4_t v) { return __builtin_bit_cast(f16x8_t, v); }

}  // namespace moe
