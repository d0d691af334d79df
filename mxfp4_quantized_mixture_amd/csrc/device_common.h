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
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(32 * sizeof(float)))) float f32x32_t;
typedef __attribute__((__vector_size__(6 * sizeof(uint32_t)))) uint32_t u32x6_t;
// (clang extended vectors: any length, sub-vectors by __builtin_shufflevector)
typedef uint32_t u32v4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32v8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32v12_t __attribute__((ext_vector_type(12)));
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

// Workgroup barrier ordering LDS accesses only.  __syncthreads() also
// orders global memory, which makes every wavefront wait for all of its
// outstanding loads (the load counter does not tell loads from stores).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// fp32 -> bf16 bits, round half to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}

// fp32 -> fp16 bits, round to nearest even (the hardware conversion).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Scale exponent s of a group of values with largest magnitude m for fp16
// storage as v 2^-s: m 2^-s in [2^14, 2^15) (s = 0 for m = 0), s clamped to
// [-127, 128] so that s + 127 fits a byte.
__device__ __forceinline__ int y_scale_exponent(float m) {
    if (!(m > 0.f)) return 0;
    const int e = __builtin_amdgcn_frexp_expf(m);      // m = f 2^e, f in [0.5, 1)
    const int s = e - 15;                             // m 2^-s = f 2^15
    return s < -127 ? -127 : (s > 128 ? 128 : s);
}

// E8M0 scale byte b (meaning 2^(b-127)) as the fp32 scale operand of the
// v_cvt_scalef32_* conversions.  b = 0 is the fp32 denormal 2^-127.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
    return __builtin_bit_cast(float, b ? (b << 23) : 0x00400000u);
}

// Eight E2M1 codes (one dword, element 2i in the low nibble of byte i) times
// a power-of-two scale, widened to bf16 by the gfx950 conversion unit.
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

// 16x16x32 matrix-core products with fp32 accumulation.  Lane l supplies
// A[l % 16][8 * (l / 16) + i] and B[8 * (l / 16) + i][l % 16] (i = 0..7) and
// receives C[4 * (l / 16) + r][l % 16] (r = 0..3).
__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

// ---------------------------------------------------------------------------
// fp6 (E2M3) residual terms.  E2M3: 1 sign, 2 exponent (bias 1) and 3
// mantissa bits; magnitudes k/8 (k = 0..7, exponent field 0) and
// 2^(e-1) (1 + m/8) (e = 1..3), largest 7.5.  A block of 32 values is carried
// as kFp6Terms terms, term t + 1 holding the exact fp32 residual of term t,
// each with its own E8M0 scale 2^s.  s is chosen so the term's largest
// magnitude rounds into [4, 7.5]; every element's rounding error is then at
// most 1/16 of that magnitude, so each term removes all but 2^-4 of what is
// left and three terms leave at most 2^-12 of the block's largest magnitude,
// at any magnitude the scales reach (2^-126 .. 2^126).
//
// Codes of a block: element i at bits 6i .. 6i + 5 of 6 dwords, the order in
// which the gfx950 block-scaled products read an fp6 operand (lane (n, g)
// of the 32x32x64 product: column n, K = 32 g .. 32 g + 31).  The hardware
// conversion v_cvt_scalef32_2xpk16_fp6_f32 rounds v / scale to nearest even
// and writes its first source's 16 values to the even elements and its
// second source's to the odd ones (both checked bit for bit with in-bounds
// probes, ties included); its inverse v_cvt_scalef32_pk32_f32_fp6 returns
// code value * scale exactly.
// ---------------------------------------------------------------------------
constexpr int kFp6Terms = 3;

// s in [-126, 126] such that amax * 2^-s, rounded to 4 significant bits, lies
// in [4, 7.5]: floor(log2 amax) - 2, plus 1 when the mantissa is at least
// 1.9375 (which would round to 8, past the largest E2M3 value).  amax = 0
// gives -126 (all codes of the block are then zero).
__device__ __forceinline__ int e2m3_term_exponent(float amax) {
    const uint32_t b = __builtin_bit_cast(uint32_t, amax);
    const int s = (int)(b >> 23) - 129 + ((b & 0x7FFFFFu) >= 0x780000u ? 1 : 0);
    return s < -126 ? -126 : (s > 126 ? 126 : s);
}

// 2^s for s in [-126, 127] (normal fp32)
__device__ __forceinline__ float exp2i_normal(int s) {
    return __builtin_bit_cast(float, (uint32_t)(127 + s) << 23);
}

// The kFp6Terms terms of one 32-element block v (v is left holding the
// final residual): codes[t] (6 dwords) and E8M0 scale bytes sb[t].
__device__ __forceinline__ void fp6_block_terms(float (&v)[32], u32x6_t (&codes)[kFp6Terms],
                                                uint32_t (&sb)[kFp6Terms]) {
#pragma unroll
    for (int t = 0; t < kFp6Terms; ++t) {
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
        const int s = e2m3_term_exponent(amax);
        const float sc = exp2i_normal(s);
        f32x16_t ev, od;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            ev[i] = v[2 * i];
            od[i] = v[2 * i + 1];
        }
        codes[t] = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, sc);
        sb[t] = (uint32_t)(s + 127);
        if (t + 1 < kFp6Terms) {
            const f32x32_t back = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(codes[t], sc);
#pragma unroll
            for (int i = 0; i < 32; ++i) v[i] -= back[i];
        }
    }
}

// One 64-element step of an fp6 term row (kTermStep bytes, as 40 dwords),
// block-major: the step's block h (h = 0, 1) owns the 80 bytes (5 units of
// 16) at 80 h; in them, dwords 6 t .. 6 t + 5 hold the 24 code bytes of its
// term t, dword 18 its three E8M0 scales (term t in byte t), dword 19 is
// zero.  A lane (n, g) of the 32x32x64 product thus reads everything it
// needs of row n -- three fp6 operands and their scales -- as the five
// 16-byte units of block g.
constexpr int kTermStep = 160;
constexpr int kTermHalf = kTermStep / 2;
static_assert(kFp6Terms == 3 && 24 * kFp6Terms + 4 <= kTermHalf && kTermHalf % 16 == 0,
              "term step layout");

__device__ __forceinline__ void fp6_encode_step(float (&v)[64], uint32_t (&out)[kTermStep / 4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float blk[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) blk[i] = v[32 * h + i];
        u32x6_t codes[kFp6Terms];
        uint32_t sb[kFp6Terms];
        fp6_block_terms(blk, codes, sb);
#pragma unroll
        for (int t = 0; t < kFp6Terms; ++t)
#pragma unroll
            for (int w = 0; w < 6; ++w) out[20 * h + 6 * t + w] = codes[t][w];
        out[20 * h + 18] = sb[0] | (sb[1] << 8) | (sb[2] << 16);
        out[20 * h + 19] = 0u;
    }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

}  // namespace moe
