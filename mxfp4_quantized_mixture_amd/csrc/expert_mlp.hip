// expert_mlp.hip -- SwiGLU experts on MXFP4 weights by weight streaming, and
// the weighted combine, for gfx950.
//
// Per routed pair p = t*k + j of expert e ("Welcome GPT OSS", section 4:
// SwiGLU experts, softmax-after-topk weights; no shared expert per the talk
// summary's Q&A):  g = Wg_e x_t,  u = Wu_e x_t,  h = silu(g) * u,
// y_p = W2_e h,  out[t] = sum_j w[t, j] * y_p.
// The weights stay MXFP4 in HBM and enter the matrix cores as stored ("Tricks",
// section 8: GEMMs that understand 32-element blocks and their scales; talk
// summary, "Hardware optimisation": store low precision, widen only inside
// the arithmetic).
//
// These kernels serve batches in which experts receive few tokens (decode):
// every touched expert's weights are read once per group of 16 of its pairs,
// and the kernels are bound by that weight stream.  The grouped GEMMs of
// expert_gemm.hip serve the rest (and the shapes these kernels' LDS budget
// does not take).  h travels between the two streaming kernels in fp32.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "stream_device.h"

namespace moe {

template <bool kGateUp, bool kPacked>
__global__ __launch_bounds__(kStreamWaves * 64) void expert_stream_kernel(
    const void* __restrict__ act, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ ws, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted, int D, int F, int E, int k, int bpe,
    float* __restrict__ out) {
    extern __shared__ __align__(16) uint8_t lds_stage[];
    __shared__ int s_row[16];
    expert_stream_body<kGateUp, kPacked, false>(act, wq, ws, offsets, sorted, D, F, E, k, bpe,
                                                out, (int)blockIdx.x, lds_stage, s_row,
                                                [] { return true; });
}

// out[t, d] = bf16( sum_j w[t, j] * y[pos[t*k + j], d] ), slots in order.
// All k slots' positions and weights are loaded first, then all k rows, so
// a thread waits for two memory round trips, not 2 k.
constexpr int kCombineMaxK = 8;
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ y, const float* __restrict__ topk_w,
    const int32_t* __restrict__ pos, int T, int D, int k, uint16_t* __restrict__ out) {
    const int q = D / 4;
    const int64_t n = (int64_t)T * q;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int t = (int)(i / q), d4 = (int)(i % q);
        int pr[kCombineMaxK];
        float wv[kCombineMaxK];
#pragma unroll
        for (int j = 0; j < kCombineMaxK; ++j) {
            if (j < k) {
                pr[j] = pos[t * k + j];
                wv[j] = topk_w[t * k + j];
            }
        }
        f32x4_t v[kCombineMaxK];
#pragma unroll
        for (int j = 0; j < kCombineMaxK; ++j)
            if (j < k) v[j] = *reinterpret_cast<const f32x4_t*>(y + (size_t)pr[j] * D + d4 * 4);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kCombineMaxK; ++j) {
            if (j < k) {
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c] = __builtin_fmaf(wv[j], v[j][c], acc[c]);
            }
        }
        uint2 o;
        o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
        o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
        *reinterpret_cast<uint2*>(out + (size_t)t * D + d4 * 4) = o;
    }
}

// The same combine over y stored in slot order (row t k + j holds the pair
// of slot j of token t, as the streaming down kernel writes it): every
// address is known at once, so a thread waits for one memory round trip.
__global__ __launch_bounds__(256) void combine_slots_kernel(
    const float* __restrict__ y, const float* __restrict__ topk_w, int T, int D, int k,
    uint16_t* __restrict__ out) {
    const int q = D / 4;
    const int64_t n = (int64_t)T * q;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int t = (int)(i / q), d4 = (int)(i % q);
        float wv[kCombineMaxK];
        f32x4_t v[kCombineMaxK];
#pragma unroll
        for (int j = 0; j < kCombineMaxK; ++j) {
            if (j < k) {
                wv[j] = topk_w[t * k + j];
                v[j] = *reinterpret_cast<const f32x4_t*>(y + (size_t)(t * k + j) * D + d4 * 4);
            }
        }
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kCombineMaxK; ++j) {
            if (j < k) {
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c] = __builtin_fmaf(wv[j], v[j][c], acc[c]);
            }
        }
        uint2 o;
        o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
        o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
        *reinterpret_cast<uint2*>(out + (size_t)t * D + d4 * 4) = o;
    }
}

// The same combine over y stored in fp16 with a power-of-two scale per
// (pair, 32-output fragment) (ys byte = s + 127, value = y16 2^s), as the
// grouped GEMM's down kernel writes it: eight outputs per thread (16-byte
// loads and stores; the eight share one scale byte per slot).
__global__ __launch_bounds__(256) void combine16_kernel(
    const uint16_t* __restrict__ y16, const uint8_t* __restrict__ ys,
    const float* __restrict__ topk_w, const int32_t* __restrict__ pos, int T, int D, int k,
    uint16_t* __restrict__ out) {
    const int q = D / 8;
    const int64_t n = (int64_t)T * q;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int t = (int)(i / q), d8 = (int)(i % q);
        int pr[kCombineMaxK];
        float wv[kCombineMaxK];
#pragma unroll
        for (int j = 0; j < kCombineMaxK; ++j) {
            if (j < k) {
                pr[j] = pos[t * k + j];
                wv[j] = topk_w[t * k + j];
            }
        }
        u32x4_t v[kCombineMaxK];
        int sc[kCombineMaxK];
#pragma unroll
        for (int j = 0; j < kCombineMaxK; ++j) {
            if (j < k) {
                v[j] = *reinterpret_cast<const u32x4_t*>(y16 + (size_t)pr[j] * D + d8 * 8);
                sc[j] = (int)ys[(size_t)pr[j] * (D / 32) + (d8 * 8) / 32] - 127;
            }
        }
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kCombineMaxK; ++j) {
            if (j < k) {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const uint32_t bits = (v[j][c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
                    const float yv = __builtin_ldexpf(
                        (float)__builtin_bit_cast(_Float16, (uint16_t)bits), sc[j]);
                    acc[c] = __builtin_fmaf(wv[j], yv, acc[c]);
                }
            }
        }
        u32x4_t o;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            o[c] = f32_to_bf16_rne(acc[2 * c]) | (f32_to_bf16_rne(acc[2 * c + 1]) << 16);
        *reinterpret_cast<u32x4_t*>(out + (size_t)t * D + d8 * 8) = o;
    }
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

constexpr size_t kMaxStreamLds = 158 * 1024;   // of 160 KiB, leaving room for static LDS


MlpPlan plan_mlp(int T, int D, int F, int E, int k) {
    MlpPlan p{};
    p.T = T; p.D = D; p.F = F; p.E = E; p.k = k;
    const size_t P = (size_t)T * k;
    // (the grouped GEMM addresses its buffers with 32-bit byte offsets)
    const size_t k4G = (size_t)1 << 32;
    p.max_tiles = gemm_max_tiles(T, E, k);
    p.gemm_ok = D % 64 == 0 && F % 64 == 0 && D <= kGemmMaxContraction &&
                F <= kGemmMaxContraction && gemm_lds_bytes(D, true) <= kGemmMaxLds &&
                gemm_lds_bytes(F, false) <= kGemmMaxLds && gemm_term_bytes(T, D) < k4G &&
                gemm_h_bytes((int64_t)std::min(P, (size_t)1 << 30), F) < k4G && (size_t)E * F * D < k4G;
    p.stream_ok = stream_lds_bytes(D, 2, 2) <= kMaxStreamLds &&
                  stream_lds_bytes(F, 3, 1) <= kMaxStreamLds && D <= 4096 && F <= 4096;
    // Weight streaming reads every touched expert's weights once per 16 of its
    // pairs; the grouped GEMM stages 128-pair tiles.  Switch once the average
    // expert receives 32 pairs, or when the streaming kernels cannot take the
    // shape.
    p.gemm_auto = p.gemm_ok && (P >= (size_t)32 * E || !p.stream_ok);
    p.packed_ok = p.gemm_ok && p.stream_ok;
    p.off_y = 0;
    // (the grouped GEMM stores y as fp16 plus a scale byte per 32 outputs in
    // the same region: P D 2 + P D / 32 bytes)
    p.off_ys = align256(P * D * sizeof(uint16_t));
    // h: fp32 [P, F] for the streaming kernels, fp6 term rows packed by tile
    // (with 128 rows of slack) for the grouped GEMM; one region sized for
    // either
    p.off_h = align256(std::max(P * D * sizeof(float), p.off_ys + P * D / 32));
    size_t h_bytes = P * F * sizeof(float);
    if (p.gemm_ok) h_bytes = std::max(h_bytes, gemm_h_bytes((int64_t)P, F));
    size_t end = align256(p.off_h + h_bytes);
    if (p.gemm_ok) {
        p.off_xq = end;
        p.off_tiles = align256(p.off_xq + gemm_term_bytes(T, D));
        end = align256(p.off_tiles + sizeof(int32_t) * (2 * (size_t)p.max_tiles + 1));
    }
    p.ws_bytes = end;
    return p;
}

// Blocks per expert for the streaming kernels: about 224 blocks in all (7/8
// of MI355X's 256 CUs, one block per CU, so every block runs in the first
// round) and at least 2 per expert, so untouched experts' CUs are reused by
// the dispatcher; at least 8 tiles (one per wavefront) per block where
// possible.  The weight stream is bound by HBM, not by the CUs streaming it:
// at the 20B decode shape (32 experts) 7 blocks per expert measured 57.1 +
// 36.9 us for gate/up and down against 58.7 + 37.2 us with 8 (and 6: 58.3 +
// 37.7, 5: 56.5 + 40.2, 4: 65.9 + 47.6); the 120B decode shape (128 experts,
// about 112 touched) keeps 2 per expert, about 224 active blocks.
static int stream_blocks_per_expert(int E, int ntiles) {
    int bpe = (224 + E - 1) / E;
    if (bpe < 2) bpe = 2;
    if (bpe > ntiles / kStreamWaves) bpe = ntiles / kStreamWaves;
    return bpe < 1 ? 1 : bpe;
}

static hipError_t launch_combine16(const MlpPlan& p, const uint16_t* y16, const uint8_t* ys,
                                   const float* topk_w, const int32_t* pos, uint16_t* out,
                                   hipEvent_t* events, hipStream_t stream);

// One streaming pass: gate/up (kGateUp, K = D, F output rows per expert) or
// down (K = F, D output rows), blocks sized by stream_blocks_per_expert.
template <bool kGateUp, bool kPacked>
static hipError_t launch_stream(const MlpPlan& p, const void* act, const uint8_t* wq,
                                const uint8_t* ws_, const int32_t* offsets,
                                const int32_t* sorted, float* out, hipStream_t stream) {
    const size_t lds = kGateUp ? stream_lds_bytes(p.D, 2, 2) : stream_lds_bytes(p.F, 3, 1);
    const int bpe = stream_blocks_per_expert(p.E, (kGateUp ? p.F : p.D) / 16);
    if (lds > 65536) {
        const hipError_t er =
            hipFuncSetAttribute(reinterpret_cast<const void*>(&expert_stream_kernel<kGateUp, kPacked>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (er != hipSuccess) return er;
    }
    hipLaunchKernelGGL((expert_stream_kernel<kGateUp, kPacked>), dim3(p.E * bpe),
                       dim3(kStreamWaves * 64), lds, stream, act, wq, ws_, offsets, sorted,
                       p.D, p.F, p.E, p.k, bpe, out);
    return hipSuccess;
}

hipError_t launch_stream_down(const MlpPlan& p, bool packed, const float* h, const uint8_t* w2q,
                              const uint8_t* w2s, const int32_t* offsets, const int32_t* sorted,
                              float* y, hipStream_t stream) {
    return packed ? launch_stream<false, true>(p, h, w2q, w2s, offsets, sorted, y, stream)
                  : launch_stream<false, false>(p, h, w2q, w2s, offsets, sorted, y, stream);
}

int stream_blocks_gate_up(const MlpPlan& p) { return stream_blocks_per_expert(p.E, p.F / 16); }

hipError_t launch_mlp(const MlpPlan& p, int algo, bool packed, const uint16_t* x,
                      const uint8_t* w13q, const uint8_t* w13s, const uint8_t* w2q,
                      const uint8_t* w2s, const float* topk_w, const int32_t* offsets,
                      const int32_t* sorted, const int32_t* pos, uint16_t* out, void* ws,
                      hipEvent_t* events, hipStream_t stream) {
    char* base = static_cast<char*>(ws);
    float* y = reinterpret_cast<float*>(base + p.off_y);
    if (algo == 2 || (algo == 0 && p.gemm_auto)) {
        uint16_t* y16 = reinterpret_cast<uint16_t*>(base + p.off_y);
        uint8_t* ys = reinterpret_cast<uint8_t*>(base + p.off_ys);
        const hipError_t er = launch_mlp_gemm(p, packed, x, w13q, w13s, w2q, w2s, offsets, sorted,
                                              y16, ys, base, events, stream);
        if (er != hipSuccess) return er;
        return launch_combine16(p, y16, ys, topk_w, pos, out, events, stream);
    }
    float* h = reinterpret_cast<float*>(base + p.off_h);
    if (events) {
        const hipError_t er = hipEventRecord(events[0], stream);
        if (er != hipSuccess) return er;
    }
    hipError_t er = packed
        ? launch_stream<true, true>(p, x, w13q, w13s, offsets, sorted, h, stream)
        : launch_stream<true, false>(p, x, w13q, w13s, offsets, sorted, h, stream);
    if (er != hipSuccess) return er;
    if (events) {
        er = hipEventRecord(events[1], stream);
        if (er != hipSuccess) return er;
    }
    er = packed ? launch_stream<false, true>(p, h, w2q, w2s, offsets, sorted, y, stream)
                : launch_stream<false, false>(p, h, w2q, w2s, offsets, sorted, y, stream);
    if (er != hipSuccess) return er;
    return launch_combine_slots(p.T, p.D, p.k, y, topk_w, out, events, stream);
}

static hipError_t launch_combine16(const MlpPlan& p, const uint16_t* y16, const uint8_t* ys,
                                   const float* topk_w, const int32_t* pos, uint16_t* out,
                                   hipEvent_t* events, hipStream_t stream) {
    if (events) {
        const hipError_t er = hipEventRecord(events[2], stream);
        if (er != hipSuccess) return er;
    }
    const int64_t n = (int64_t)p.T * (p.D / 8);
    int64_t gb = (n + 255) / 256;
    if (gb > 8192) gb = 8192;
    hipLaunchKernelGGL(combine16_kernel, dim3((unsigned)gb), dim3(256), 0, stream, y16, ys, topk_w,
                       pos, p.T, p.D, p.k, out);
    if (events) {
        const hipError_t er = hipEventRecord(events[3], stream);
        if (er != hipSuccess) return er;
    }
    return hipGetLastError();
}

hipError_t launch_combine_rows(int T, int D, int k, const float* y, const float* topk_w,
                               const int32_t* pos, uint16_t* out, hipEvent_t* events,
                               hipStream_t stream) {
    if (events) {
        const hipError_t er = hipEventRecord(events[2], stream);
        if (er != hipSuccess) return er;
    }
    const int64_t n = (int64_t)T * (D / 4);
    int64_t gb = (n + 255) / 256;
    if (gb > 8192) gb = 8192;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)gb), dim3(256), 0, stream, y, topk_w, pos,
                       T, D, k, out);
    if (events) {
        const hipError_t er = hipEventRecord(events[3], stream);
        if (er != hipSuccess) return er;
    }
    return hipGetLastError();
}

hipError_t launch_combine_slots(int T, int D, int k, const float* y, const float* topk_w,
                                uint16_t* out, hipEvent_t* events, hipStream_t stream) {
    if (events) {
        const hipError_t er = hipEventRecord(events[2], stream);
        if (er != hipSuccess) return er;
    }
    const int64_t n = (int64_t)T * (D / 4);
    int64_t gb = (n + 255) / 256;
    if (gb > 8192) gb = 8192;
    hipLaunchKernelGGL(combine_slots_kernel, dim3((unsigned)gb), dim3(256), 0, stream, y, topk_w,
                       T, D, k, out);
    if (events) {
        const hipError_t er = hipEventRecord(events[3], stream);
        if (er != hipSuccess) return er;
    }
    return hipGetLastError();
}

}  // namespace moe
