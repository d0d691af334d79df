// quantize.hip -- MXFP4 codec kernels for gfx950.
//
// Format: E2M1 elements (1 sign, 2 exponent, 1 mantissa bit) with one shared
// E8M0 scale per 32-element block ("Tricks from OpenAI gpt-oss you can use
// with transformers", section 6; "Transformers 4.40 のパフォーマンス向上",
// section "MXFP4 とは"; OCP MX named in "MXFP4 기반 MoE 기술 리뷰", section 1).
//
// The scale rules and the stochastic encoder work on the bf16 bit fields
// with integer arithmetic; the nearest-even encoder uses fp32 products that
// are exact (see e2m1_encode_f32).  The element rounding of the stochastic
// encoder follows the reading of the stochastic-rounding recipe that "MXFP4
// 기반 MoE 기술 리뷰" section 2 cites (details in the header).
#include "device_common.h"
#include "launch.h"

namespace moe {

// Shared exponent from the block's largest |bf16| bit pattern (sign cleared;
// the bit patterns of non-negative floats order like their values).
//   amax = (128 + M) * 2^(E - 134) for E > 0.
//   rule 0: s = floor(log2(amax / 6)) = E - 130 + [M >= 64]   (1 + M/128 >= 1.5)
//   rule 1: s = floor(log2(amax)) - 2 = E - 129
//   rule 2: s = ceil(log2(amax / 6))  = E - 129 + [M > 64]    (no element beyond 6)
// A zero or subnormal maximum lies below 2^-126 and gives s < -127: clamp.
__device__ __forceinline__ int block_scale_exponent(uint32_t amax_bits, int rule) {
    int E = (int)(amax_bits >> 7);
    int M = (int)(amax_bits & 0x7F);
    if (E == 0) return -127;
    int s = rule == 0 ? E - 130 + (M >= 64 ? 1 : 0)
                      : rule == 1 ? E - 129 : E - 129 + (M > 64 ? 1 : 0);
    return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// E2M1 code of the bf16 value v scaled by 2^-s: nearest of {0, .5, 1, 1.5,
// 2, 3, 4, 6}, ties to the even code, saturating; sign kept (so -0 and
// negatives that round to zero give 0x8).  y = |v| * 2^-s is exact
// here (a power-of-two multiple of a bf16 value; when it is too small for
// that it lies far below 0.25 and rounds to 0 either way; s <= 126 for any
// finite bf16 maximum, so 2^-s is a normal fp32), and on each binade of the
// grid the nearest code is one round-half-even: 2y below 2 (0, .5, 1, 1.5,
// 2 are 0..4), y + 2 below 4 (2, 3, 4 are codes 4..6), y / 2 + 4 below 6
// (4, 6 are codes 6, 7); ties go to the even integer, which is the code
// with mantissa bit 0.  Saturates at 6 (including an infinite product).
__device__ __forceinline__ uint32_t e2m1_encode_f32(uint32_t v, float inv_scale) {
    const float y = __builtin_bit_cast(float, (v & 0x7FFFu) << 16) * inv_scale;
    float c;
    if (y < 2.0f)
        c = __builtin_rintf(2.0f * y);
    else if (y < 4.0f)
        c = __builtin_rintf(y) + 2.0f;
    else if (y < 6.0f)
        c = __builtin_rintf(0.5f * y) + 4.0f;
    else
        c = 7.0f;
    return ((v >> 12) & 8u) | (uint32_t)c;
}

// SplitMix64: output n >= 1 of the generator whose state starts at `seed`
// (state += 0x9E3779B97F4A7C15 per output; output = the mix64 finalizer of
// java.util.SplittableRandom, also S. Vigna's splitmix64.c).
__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t n) {
    uint64_t z = seed + n * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Stochastic E2M1 code of the bf16 value v scaled by 2^-s, with the draw u in
// [0, 2^24): between the neighbouring grid values lo <= |y| < hi the upper
// one is taken when u < 2^24 (|y| - lo) / (hi - lo); |y| >= 6 saturates; sign
// kept.  Integer form: Y = ceil(4|y| 2^40), in quarter units with 40 fraction
// bits (exact unless 4|y| < 2^-40); the grid {0, 2, 4, 6, 8, 12, 16, 24}
// has steps 2, 4, 8; the threshold ceil((Y - lo) / step * 2^-16) equals
// ceil(2^24 (|y| - lo) / (hi - lo)), and u < x <=> u < ceil(x) for integer u.
__device__ __forceinline__ uint32_t e2m1_encode_stochastic(uint32_t v, int s, uint32_t u) {
    const uint32_t sign = (v >> 15) & 1u;
    const uint32_t E = (v >> 7) & 0xFFu;
    const uint32_t M = v & 0x7Fu;
    const uint32_t sig = E ? (M | 0x80u) : M;
    if (sig == 0) return sign << 3;
    const int sh = (E ? (int)E : 1) - 134 - s + 2;       // 4|y| = sig * 2^sh
    if (sh >= 6) return (sign << 3) | 7u;                 // 4|y| >= 64
    const int t = sh + 40;
    uint64_t Y;
    if (t >= 0) {
        Y = (uint64_t)sig << t;
    } else {
        const int n = -t > 63 ? 63 : -t;
        Y = ((uint64_t)sig >> n) + (((uint64_t)sig & ((1ull << n) - 1ull)) != 0ull);
    }
    const uint64_t one = 1ull << 40;
    if (Y >= 24 * one) return (sign << 3) | 7u;
    uint32_t c;
    uint64_t lo;
    int n;                                                // 16 + log2(step)
    if (Y < 8 * one) {
        c = (uint32_t)(Y >> 41);
        lo = (uint64_t)c << 41;
        n = 17;
    } else if (Y < 16 * one) {
        c = 4u + (uint32_t)((Y - 8 * one) >> 42);
        lo = 8 * one + ((uint64_t)(c - 4u) << 42);
        n = 18;
    } else {
        c = 6u;
        lo = 16 * one;
        n = 19;
    }
    const uint64_t d = Y - lo;
    const uint64_t thr = (d >> n) + ((d & ((1ull << n) - 1ull)) != 0ull);
    return (sign << 3) | (c + ((uint64_t)u < thr ? 1u : 0u));
}

// Four lanes per 32-element block; each lane owns 8 consecutive elements
// (one 16-byte load), so a wavefront reads 1 KiB of contiguous bf16 and writes
// 256 contiguous bytes of codes.  Each thread takes kQuantUnroll grid strides
// at once, all their loads issued before any is encoded (one load in flight
// per thread leaves HBM idle between round trips).
// (stochastic: element e = 8 i + m of the flattened [rows, K] matrix draws
// the top 24 bits of SplitMix64 output e + 1)
constexpr int kQuantUnroll = 4;

template <bool kStochastic>
__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(
    const uint16_t* __restrict__ w, uint8_t* __restrict__ q,
    uint8_t* __restrict__ s, int64_t nquads, int rule, uint64_t seed) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i0 < nquads;
         i0 += kQuantUnroll * stride) {
        // nquads is a multiple of 4 and stride of 256, so the four lanes of a
        // block are always active (or idle) together for the shuffles below.
        u32x4_t raw[kQuantUnroll];
#pragma unroll
        for (int u = 0; u < kQuantUnroll; ++u) {
            const int64_t i = i0 + u * stride;
            raw[u] = i < nquads ? *reinterpret_cast<const u32x4_t*>(w + i * 8)
                                : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kQuantUnroll; ++u) {
            const int64_t i = i0 + u * stride;
            uint32_t amax = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t lo = raw[u][j] & 0x7FFFu, hi = (raw[u][j] >> 16) & 0x7FFFu;
                amax = max(amax, max(lo, hi));
            }
            amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
            amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
            if (i >= nquads) continue;
            const int se = block_scale_exponent(amax, rule);
            uint32_t codes = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (kStochastic) {
                    const uint64_t e0 = (uint64_t)i * 8 + 2 * j;
                    const uint32_t u0 = (uint32_t)(splitmix64(seed, e0 + 1) >> 40);
                    const uint32_t u1 = (uint32_t)(splitmix64(seed, e0 + 2) >> 40);
                    codes |= e2m1_encode_stochastic(raw[u][j] & 0xFFFFu, se, u0) << (8 * j);
                    codes |= e2m1_encode_stochastic(raw[u][j] >> 16, se, u1) << (8 * j + 4);
                } else {
                    const float inv = exp2i_neg(se);
                    codes |= e2m1_encode_f32(raw[u][j] & 0xFFFFu, inv) << (8 * j);
                    codes |= e2m1_encode_f32(raw[u][j] >> 16, inv) << (8 * j + 4);
                }
            }
            reinterpret_cast<uint32_t*>(q)[i] = codes;
            if ((i & 3) == 0) s[i >> 2] = (uint8_t)(se + 127);
        }
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

// Packed code layout for the expert kernels: for each 32-row fragment f and
// each 64-element contraction step t, the fragment's 32 rows x 32 bytes of
// that step are one contiguous 1 KiB chunk, chunks in (f, t) order, the
// first 16 bytes (elements 0..31 of the step) of all 32 rows before the
// second 16 bytes:
//   packed[(f * K/64 + t) * 1024 + 512 h + 16 r + b] = q[(32 f + r) * K/2 + 32 t + 16 h + b]
// (h = 0, 1; b < 16), so lane l = 32 h + r of a wavefront finds its 16 bytes
// at 16 l.  One thread per 16 bytes of output (coalesced writes).
__global__ __launch_bounds__(256) void mxfp4_pack_kernel(const uint8_t* __restrict__ q,
                                                         uint8_t* __restrict__ out,
                                                         int64_t n16, int64_t K) {
    const int64_t steps = K / 64;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < n16; o += stride) {
        const int64_t chunk = o >> 6;              // 1 KiB chunk (f, t)
        const int piece = (int)(o & 63);           // 16-byte piece: half h = piece / 32, row r
        const int64_t f = chunk / steps, t = chunk - f * steps;
        const int64_t src = (32 * f + (piece & 31)) * (K / 2) + 32 * t + 16 * (piece >> 5);
        *reinterpret_cast<u32x4_t*>(out + o * 16) = *reinterpret_cast<const u32x4_t*>(q + src);
    }
}

static unsigned grid_for(int64_t work, int per_block) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g > 16384) g = 16384;
    return (unsigned)(g < 1 ? 1 : g);
}

hipError_t launch_quantize(const uint16_t* w, int64_t rows, int64_t K, int rule, int rounding,
                           uint64_t seed, uint8_t* q, uint8_t* s, hipStream_t stream) {
    const int64_t nquads = rows * (K / 8);
    if (rounding == 1)
        hipLaunchKernelGGL(mxfp4_quantize_kernel<true>, dim3(grid_for(nquads, 256)), dim3(256), 0,
                           stream, w, q, s, nquads, rule, seed);
    else
        hipLaunchKernelGGL(mxfp4_quantize_kernel<false>, dim3(grid_for(nquads, 256)), dim3(256),
                           0, stream, w, q, s, nquads, rule, seed);
    return hipGetLastError();
}

hipError_t launch_pack(const uint8_t* q, int64_t rows, int64_t K, uint8_t* out,
                       hipStream_t stream) {
    const int64_t n16 = rows * (K / 2) / 16;
    hipLaunchKernelGGL(mxfp4_pack_kernel, dim3(grid_for(n16, 256)), dim3(256), 0, stream, q, out,
                       n16, K);
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
