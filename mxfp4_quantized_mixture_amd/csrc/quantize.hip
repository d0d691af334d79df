// quantize.hip -- MXFP4 codec kernels for gfx950.
//
// Format: E2M1 elements (1 sign, 2 exponent, 1 mantissa bit) with one shared
// E8M0 scale per 32-element block ("Tricks from OpenAI gpt-oss you can use
// with transformers", section 6; "Transformers 4.40 のパフォーマンス向上",
// section "MXFP4 とは"; OCP MX named in "MXFP4 기반 MoE 기술 리뷰", section 1).
//
// The encoder works on the bf16 bit fields with integer arithmetic only, so
// no floating-point rounding mode, denormal flushing or fast-math setting can
// change a code.
#include "device_common.h"
#include "launch.h"

namespace moe {

// Shared exponent from the block's largest |bf16| bit pattern (sign cleared;
// the bit patterns of non-negative floats order like their values).
//   amax = (128 + M) * 2^(E - 134) for E > 0.
//   rule 0: s = floor(log2(amax / 6)) = E - 130 + [M >= 64]   (1 + M/128 >= 1.5)
//   rule 1: s = floor(log2(amax)) - 2 = E - 129
// A zero or subnormal maximum lies below 2^-126 and gives s < -127: clamp.
__device__ __forceinline__ int block_scale_exponent(uint32_t amax_bits, int rule) {
    int E = (int)(amax_bits >> 7);
    int M = (int)(amax_bits & 0x7F);
    if (E == 0) return -127;
    int s = rule == 0 ? E - 130 + (M >= 64 ? 1 : 0) : E - 129;
    return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// E2M1 code of the bf16 value v scaled by 2^-s: nearest of
// {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, saturating; sign kept.
// With |v| = sig * 2^e2, 4|v|/2^s = sig * 2^(e2 - s + 2) is compared against
// the doubled midpoints {1,3,5,7,10,14,20} of the grid in quarter units,
// carrying a sticky bit for the shifted-out fraction.
__device__ __forceinline__ uint32_t e2m1_encode(uint32_t v, int s) {
    uint32_t sign = (v >> 15) & 1u;
    uint32_t E = (v >> 7) & 0xFFu;
    uint32_t M = v & 0x7Fu;
    uint32_t sig = E ? (M | 0x80u) : M;
    int e2 = (E ? (int)E : 1) - 134;
    int sh = e2 - s + 2;
    uint32_t v2;  // 2 * (4y), plus 1 if any fraction bit was dropped
    if (sig == 0) {
        v2 = 0;
    } else if (sh >= 0) {
        v2 = sh >= 6 ? 0xFFFFu : (sig << sh) << 1;
    } else {
        int n = -sh > 9 ? 9 : -sh;
        uint32_t qi = sig >> n;
        uint32_t sticky = (sig & ((1u << n) - 1u)) != 0u;
        v2 = (qi << 1) | sticky;
    }
    uint32_t c = (v2 > 2u) + (v2 >= 6u) + (v2 > 10u) + (v2 >= 14u) +
                 (v2 > 20u) + (v2 >= 28u) + (v2 > 40u);
    return (sign << 3) | c;
}

// Four lanes per 32-element block; each lane owns 8 consecutive elements
// (one 16-byte load), so a wavefront reads 1 KiB of contiguous bf16 and writes
// 256 contiguous bytes of codes.
__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(
    const uint16_t* __restrict__ w, uint8_t* __restrict__ q,
    uint8_t* __restrict__ s, int64_t nquads, int rule) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nquads; i += stride) {
        // nquads is a multiple of 4 and stride of 256, so the four lanes of a
        // block are always active together for the shuffles below.
        u32x4_t raw = *reinterpret_cast<const u32x4_t*>(w + i * 8);
        uint32_t amax = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t lo = raw[j] & 0x7FFFu, hi = (raw[j] >> 16) & 0x7FFFu;
            amax = max(amax, max(lo, hi));
        }
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
        const int se = block_scale_exponent(amax, rule);
        uint32_t codes = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            codes |= e2m1_encode(raw[j] & 0xFFFFu, se) << (8 * j);
            codes |= e2m1_encode(raw[j] >> 16, se) << (8 * j + 4);
        }
        reinterpret_cast<uint32_t*>(q)[i] = codes;
        if ((i & 3) == 0) s[i >> 2] = (uint8_t)(se + 127);
    }
}

// Eight elements per lane: one dword of codes -> 8 bf16 (16 bytes).
__global__ __launch_bounds__(256) void mxfp4_dequantize_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
    uint16_t* __restrict__ out, int64_t noct) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < noct; i += stride) {
        uint32_t codes = reinterpret_cast<const uint32_t*>(q)[i];
        float scale = e8m0_to_f32(s[i >> 2]);
        bf16x8_t v = fp4x8_to_bf16x8(codes, scale);
        *reinterpret_cast<u32x4_t*>(out + i * 8) = __builtin_bit_cast(u32x4_t, v);
    }
}

static unsigned grid_for(int64_t work, int per_block) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g > 16384) g = 16384;
    return (unsigned)(g < 1 ? 1 : g);
}

hipError_t launch_quantize(const uint16_t* w, int64_t rows, int64_t K, int rule,
                           uint8_t* q, uint8_t* s, hipStream_t stream) {
    const int64_t nquads = rows * (K / 8);
    hipLaunchKernelGGL(mxfp4_quantize_kernel, dim3(grid_for(nquads, 256)), dim3(256), 0,
                       stream, w, q, s, nquads, rule);
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t K,
                             uint16_t* out, hipStream_t stream) {
    const int64_t noct = rows * (K / 8);
    hipLaunchKernelGGL(mxfp4_dequantize_kernel, dim3(grid_for(noct, 256)), dim3(256), 0,
                       stream, q, s, out, noct);
    return hipGetLastError();
}

}  // namespace moe
