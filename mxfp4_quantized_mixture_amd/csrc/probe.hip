// probe.hip -- achievable-peak microbenchmarks for MI355X (gfx950), the
// ceilings the layer's kernels are compared with next to the published
// peaks: a streaming read of a large buffer (HBM) and a loop of independent
// matrix-core products per operand type.  Built as libmoe_probe.so, apart
// from the layer's library; declared in include/moe_probe.h.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_probe.h"

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;

// Every thread reads 16-byte pieces, 4 independent ones per trip, grid
// stride; the XOR of all it read goes to sink so no load is dropped.
__global__ __launch_bounds__(256) void read_kernel(const u32x4_t* __restrict__ p, size_t n16,
                                                   uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4_t a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= p[i];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// The same bytes read in two orders, to separate the cost of the access
// pattern from that of the bytes: every wavefront (8 per block) reads cpw
// 1 KiB chunks (64 lanes x 16 B), four independent loads per trip.  The
// wavefronts form groups of `group` consecutive ones that interleave their
// chunks: chunk c of member r of group q is chunk (q cpw + c) group + r of the
// buffer.  group = 1: each wavefront streams a private contiguous range (as a
// wavefront that owns whole weight tiles does); group = all wavefronts: the
// grid sweeps the buffer together.  Every index is below nw cpw 64 (nw =
// gridDim.x * 8, group divides nw; checked by the host).
__global__ __launch_bounds__(512) void read_grouped_kernel(const u32x4_t* __restrict__ p, int cpw,
                                                           int group, uint32_t* __restrict__ sink) {
    const int lane = (int)threadIdx.x & 63;
    const size_t w = (size_t)blockIdx.x * 8 + (threadIdx.x >> 6);
    const size_t q = w / (size_t)group, r = w % (size_t)group;
    auto at = [&](int c) { return p[((q * cpw + c) * group + r) * 64 + lane]; };
    u32x4_t acc = {0u, 0u, 0u, 0u};
    int c = 0;
    for (; c + 4 <= cpw; c += 4) {
        const u32x4_t a = at(c), b = at(c + 1), d = at(c + 2), e = at(c + 3);
        acc ^= a ^ b ^ d ^ e;
    }
    for (; c < cpw; ++c) acc ^= at(c);
    sink[w * 64 + lane] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// 8 independent accumulator chains per wave, `iters` trips.  The operands
// are arbitrary register contents (the rate does not depend on values).
template <int KIND>
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* __restrict__ sink) {
    constexpr int NCH = 8;
    const int t = (int)threadIdx.x;
    f32x16_t c[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) c[j][i] = 0.f;
    const i32x8_t a = {t, 1, 2, 3, 4, 5, 6, 7};
    const i32x8_t b = {7, 6, 5, 4, 3, 2, 1, t};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            if constexpr (KIND == MOE_PROBE_FP4_FP4)
                c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[j], 4, 4, 0, 127, 0, 127);
            else if constexpr (KIND == MOE_PROBE_FP4_FP6)
                c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[j], 4, 2, 0, 127, 0, 127);
            else if constexpr (KIND == MOE_PROBE_FP4_FP8)
                c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[j], 4, 0, 0, 127, 0, 127);
            else if constexpr (KIND == MOE_PROBE_FP8_FP8)
                c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[j], 0, 0, 0, 127, 0, 127);
            else if constexpr (KIND == MOE_PROBE_F16)
                c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, u32x4_t{1u, 2u, 3u, (uint32_t)t}),
                                                              __builtin_bit_cast(f16x8_t, u32x4_t{4u, 5u, 6u, 7u}), c[j], 0, 0, 0);
            else
                c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, u32x4_t{1u, 2u, 3u, (uint32_t)t}),
                                                               __builtin_bit_cast(bf16x8_t, u32x4_t{4u, 5u, 6u, 7u}), c[j], 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += c[j][i];
    sink[(size_t)blockIdx.x * blockDim.x + t] = s;
}

}  // namespace

extern "C" {

int moe_probe_read(const void* buf, size_t bytes, int blocks, uint32_t* sink, hipStream_t stream) {
    if (!buf || !sink || blocks < 1 || bytes < 16 || (reinterpret_cast<uintptr_t>(buf) & 15u))
        return 1;
    hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const u32x4_t*>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

int moe_probe_read_grouped(const void* buf, int chunks_per_wave, int blocks, int group,
                          uint32_t* sink, hipStream_t stream) {
    if (!buf || !sink || blocks < 1 || chunks_per_wave < 1 || group < 1 ||
        (reinterpret_cast<uintptr_t>(buf) & 15u) || ((int64_t)blocks * 8) % group != 0)
        return 1;
    hipLaunchKernelGGL(read_grouped_kernel, dim3((unsigned)blocks), dim3(512), 0, stream,
                       static_cast<const u32x4_t*>(buf), chunks_per_wave, group, sink);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

int moe_probe_mfma(int kind, int blocks, int iters, float* sink, hipStream_t stream) {
    if (!sink || blocks < 1 || iters < 0) return 1;
    const dim3 g((unsigned)blocks), b(256);
    switch (kind) {
        case MOE_PROBE_FP4_FP4: hipLaunchKernelGGL(mfma_kernel<MOE_PROBE_FP4_FP4>, g, b, 0, stream, iters, sink); break;
        case MOE_PROBE_FP4_FP6: hipLaunchKernelGGL(mfma_kernel<MOE_PROBE_FP4_FP6>, g, b, 0, stream, iters, sink); break;
        case MOE_PROBE_FP4_FP8: hipLaunchKernelGGL(mfma_kernel<MOE_PROBE_FP4_FP8>, g, b, 0, stream, iters, sink); break;
        case MOE_PROBE_FP8_FP8: hipLaunchKernelGGL(mfma_kernel<MOE_PROBE_FP8_FP8>, g, b, 0, stream, iters, sink); break;
        case MOE_PROBE_F16: hipLaunchKernelGGL(mfma_kernel<MOE_PROBE_F16>, g, b, 0, stream, iters, sink); break;
        case MOE_PROBE_BF16: hipLaunchKernelGGL(mfma_kernel<MOE_PROBE_BF16>, g, b, 0, stream, iters, sink); break;
        default: return 4;
    }
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

double moe_probe_mfma_flops(int kind) {
    // flops of one product: 2 * 32 * 32 * K (K = 64 for the scaled ones, 16 else)
    switch (kind) {
        case MOE_PROBE_FP4_FP4: case MOE_PROBE_FP4_FP6: case MOE_PROBE_FP4_FP8: case MOE_PROBE_FP8_FP8:
            return 2.0 * 32 * 32 * 64;
        case MOE_PROBE_F16: case MOE_PROBE_BF16:
            return 2.0 * 32 * 32 * 16;
        default:
            return 0.0;
    }
}

}  // extern "C"
