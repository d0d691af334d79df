// expert_mlp.hip -- SwiGLU experts on MXFP4 weights and the weighted combine,
// for gfx950.
//
// Per routed pair p = t*k + j of expert e ("Welcome GPT OSS", section 4:
// SwiGLU experts, softmax-after-topk weights; no shared expert per the talk
// summary's Q&A):  g = Wg_e x_t,  u = Wu_e x_t,  h = silu(g) * u,
// y_p = W2_e h,  out[t] = sum_j w[t, j] * y_p.
// The weights stay MXFP4 in HBM and are widened to bf16 / fp16 in registers
// right before the matrix-core product ("Tricks", section 8: GEMMs that
// understand 32-element blocks and their scales; talk summary, "Hardware
// optimisation": store low precision, upcast at compute).
//
// Weight-streaming kernels (every expert's rows are read once per 16-token
// group): a block owns a range of 16-row weight tiles of one expert; its four
// wavefronts split the contraction dimension, hold their slice of the token
// activations in registers, and reduce through LDS in a fixed order.
//
// K permutation: a "super-step" covers 4 MXFP4 blocks (128 K).  Lane group
// g = lane / 16 owns block 4*ss + g and feeds its 32 elements to four 16x16x32
// products, 8 per product.  The A (weights) and B (activations) operands use
// the same permutation, so the contraction is unchanged, and every lane loads
// one whole 16-byte block of codes plus its one scale byte.
#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kMaxSS = 6;    // super-steps of activations a wave keeps in registers

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// h[row, f] for the rows of expert e (sorted order), fp16.
__global__ __launch_bounds__(256) void gateup_stream_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w13q,
    const uint8_t* __restrict__ w13s, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted, int D, int F, int k, int bpe,
    _Float16* __restrict__ h) {
    __shared__ f32x4_t red[2][4][2][64];
    const int e = blockIdx.x / bpe, part = blockIdx.x % bpe;
    const int row0 = offsets[e];
    const int ne = offsets[e + 1] - row0;
    if (ne <= 0) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int nblk = D / 32;
    const int nss = (nblk + 3) / 4;
    const int ss_beg = nss * wave / 4, ss_end = nss * (wave + 1) / 4;
    const int ntiles = F / 16;
    const int tile_beg = ntiles * part / bpe, tile_end = ntiles * (part + 1) / bpe;
    const size_t rowbytes = (size_t)D / 2;
    const uint8_t* qe = w13q + (size_t)e * 2 * F * rowbytes;
    const uint8_t* se = w13s + (size_t)e * 2 * F * nblk;
    int par = 0;

    for (int tg = 0; tg < ne; tg += 16) {
        const int r = tg + m;
        const bool tok_ok = r < ne;
        const int tok = tok_ok ? sorted[row0 + r] / k : 0;
        const uint16_t* xrow = x + (size_t)tok * D;
        int loaded = -1;
        bf16x8_t xf[kMaxSS][4];
        for (int tile = tile_beg; tile < tile_end; ++tile) {
            f32x4_t acc_g = {0.f, 0.f, 0.f, 0.f}, acc_u = {0.f, 0.f, 0.f, 0.f};
            const uint8_t* qg = qe + (size_t)(tile * 16 + m) * rowbytes;
            const uint8_t* qu = qe + (size_t)(F + tile * 16 + m) * rowbytes;
            const uint8_t* sg = se + (size_t)(tile * 16 + m) * nblk;
            const uint8_t* su = se + (size_t)(F + tile * 16 + m) * nblk;
            for (int kc = ss_beg; kc < ss_end; kc += kMaxSS) {
                if (kc != loaded) {
#pragma unroll
                    for (int i = 0; i < kMaxSS; ++i) {
                        const int blk = (kc + i) * 4 + g;
                        const bool ok = tok_ok && kc + i < ss_end && blk < nblk;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            u32x4_t v = {0u, 0u, 0u, 0u};
                            if (ok) v = *reinterpret_cast<const u32x4_t*>(xrow + blk * 32 + j * 8);
                            xf[i][j] = as_bf16x8(v);
                        }
                    }
                    loaded = kc;
                }
#pragma unroll
                for (int i = 0; i < kMaxSS; ++i) {
                    if (kc + i < ss_end) {
                        const int blk = (kc + i) * 4 + g;
                        u32x4_t wg = {0u, 0u, 0u, 0u}, wu = {0u, 0u, 0u, 0u};
                        uint32_t bg = 127u, bu = 127u;
                        if (blk < nblk) {
                            wg = *reinterpret_cast<const u32x4_t*>(qg + blk * 16);
                            wu = *reinterpret_cast<const u32x4_t*>(qu + blk * 16);
                            bg = sg[blk];
                            bu = su[blk];
                        }
                        const float scg = e8m0_to_f32(bg), scu = e8m0_to_f32(bu);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            acc_g = mfma_bf16(fp4x8_to_bf16x8(wg[j], scg), xf[i][j], acc_g);
                            acc_u = mfma_bf16(fp4x8_to_bf16x8(wu[j], scu), xf[i][j], acc_u);
                        }
                    }
                }
            }
            red[par][wave][0][lane] = acc_g;
            red[par][wave][1][lane] = acc_u;
            __syncthreads();
            if (wave == 0 && tok_ok) {
                f32x4_t sg4 = red[par][0][0][lane], su4 = red[par][0][1][lane];
#pragma unroll
                for (int w = 1; w < 4; ++w) {
                    sg4 += red[par][w][0][lane];
                    su4 += red[par][w][1][lane];
                }
                typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4_t;
                f16x4_t hv;
#pragma unroll
                for (int q = 0; q < 4; ++q) hv[q] = (_Float16)(silu_f32(sg4[q]) * su4[q]);
                *reinterpret_cast<f16x4_t*>(h + (size_t)(row0 + r) * F + tile * 16 + 4 * g) = hv;
            }
            par ^= 1;
        }
    }
}

// y[row, d] = W2_e h[row] (fp32), rows of expert e in sorted order.
__global__ __launch_bounds__(256) void down_stream_kernel(
    const _Float16* __restrict__ h, const uint8_t* __restrict__ w2q,
    const uint8_t* __restrict__ w2s, const int32_t* __restrict__ offsets, int D, int F,
    int bpe, float* __restrict__ y) {
    __shared__ f32x4_t red[2][4][64];
    const int e = blockIdx.x / bpe, part = blockIdx.x % bpe;
    const int row0 = offsets[e];
    const int ne = offsets[e + 1] - row0;
    if (ne <= 0) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int nblk = F / 32;
    const int nss = (nblk + 3) / 4;
    const int ss_beg = nss * wave / 4, ss_end = nss * (wave + 1) / 4;
    const int ntiles = D / 16;
    const int tile_beg = ntiles * part / bpe, tile_end = ntiles * (part + 1) / bpe;
    const size_t rowbytes = (size_t)F / 2;
    const uint8_t* qe = w2q + (size_t)e * D * rowbytes;
    const uint8_t* se = w2s + (size_t)e * D * nblk;
    int par = 0;

    for (int tg = 0; tg < ne; tg += 16) {
        const int r = tg + m;
        const bool tok_ok = r < ne;
        const _Float16* hrow = h + (size_t)(row0 + (tok_ok ? r : 0)) * F;
        int loaded = -1;
        f16x8_t hf[kMaxSS][4];
        for (int tile = tile_beg; tile < tile_end; ++tile) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            const uint8_t* qd = qe + (size_t)(tile * 16 + m) * rowbytes;
            const uint8_t* sd = se + (size_t)(tile * 16 + m) * nblk;
            for (int kc = ss_beg; kc < ss_end; kc += kMaxSS) {
                if (kc != loaded) {
#pragma unroll
                    for (int i = 0; i < kMaxSS; ++i) {
                        const int blk = (kc + i) * 4 + g;
                        const bool ok = tok_ok && kc + i < ss_end && blk < nblk;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            u32x4_t v = {0u, 0u, 0u, 0u};
                            if (ok) v = *reinterpret_cast<const u32x4_t*>(hrow + blk * 32 + j * 8);
                            hf[i][j] = as_f16x8(v);
                        }
                    }
                    loaded = kc;
                }
#pragma unroll
                for (int i = 0; i < kMaxSS; ++i) {
                    if (kc + i < ss_end) {
                        const int blk = (kc + i) * 4 + g;
                        u32x4_t wd = {0u, 0u, 0u, 0u};
                        uint32_t bd = 127u;
                        if (blk < nblk) {
                            wd = *reinterpret_cast<const u32x4_t*>(qd + blk * 16);
                            bd = sd[blk];
                        }
                        const float sc = e8m0_to_f32(bd);
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc = mfma_f16(fp4x8_to_f16x8(wd[j], sc), hf[i][j], acc);
                    }
                }
            }
            red[par][wave][lane] = acc;
            __syncthreads();
            if (wave == 0 && tok_ok) {
                f32x4_t s4 = red[par][0][lane];
#pragma unroll
                for (int w = 1; w < 4; ++w) s4 += red[par][w][lane];
                *reinterpret_cast<f32x4_t*>(y + (size_t)(row0 + r) * D + tile * 16 + 4 * g) = s4;
            }
            par ^= 1;
        }
    }
}

// out[t, d] = bf16( sum_j w[t, j] * y[pos[t*k + j], d] ), slots in order.
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ y, const float* __restrict__ topk_w,
    const int32_t* __restrict__ pos, int T, int D, int k, uint16_t* __restrict__ out) {
    const int q = D / 4;
    const int64_t n = (int64_t)T * q;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int t = (int)(i / q), d4 = (int)(i % q);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
            const int p = t * k + j;
            const float wv = topk_w[p];
            const f32x4_t v = *reinterpret_cast<const f32x4_t*>(y + (size_t)pos[p] * D + d4 * 4);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = __builtin_fmaf(wv, v[c], acc[c]);
        }
        uint2 o;
        o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
        o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
        *reinterpret_cast<uint2*>(out + (size_t)t * D + d4 * 4) = o;
    }
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

MlpPlan plan_mlp(int T, int D, int F, int E, int k) {
    MlpPlan p{};
    p.T = T; p.D = D; p.F = F; p.E = E; p.k = k;
    const size_t P = (size_t)T * k;
    p.off_h = 0;
    p.off_y = align256(P * F * sizeof(_Float16));
    p.ws_bytes = align256(p.off_y + P * D * sizeof(float));
    return p;
}

static int blocks_per_expert(int E, int ntiles) {
    int bpe = (2048 + E - 1) / E;
    if (bpe > ntiles) bpe = ntiles;
    return bpe < 1 ? 1 : bpe;
}

hipError_t launch_mlp(const MlpPlan& p, const uint16_t* x, const uint8_t* w13q,
                      const uint8_t* w13s, const uint8_t* w2q, const uint8_t* w2s,
                      const float* topk_w, const int32_t* offsets, const int32_t* sorted,
                      const int32_t* pos, uint16_t* out, void* ws, hipEvent_t* events,
                      hipStream_t stream) {
    char* base = static_cast<char*>(ws);
    _Float16* h = reinterpret_cast<_Float16*>(base + p.off_h);
    float* y = reinterpret_cast<float*>(base + p.off_y);
    if (events) {
        const hipError_t er = hipEventRecord(events[0], stream);
        if (er != hipSuccess) return er;
    }
    const int bpe1 = blocks_per_expert(p.E, p.F / 16);
    hipLaunchKernelGGL(gateup_stream_kernel, dim3(p.E * bpe1), dim3(256), 0, stream, x, w13q,
                       w13s, offsets, sorted, p.D, p.F, p.k, bpe1, h);
    if (events) {
        const hipError_t er = hipEventRecord(events[1], stream);
        if (er != hipSuccess) return er;
    }
    const int bpe2 = blocks_per_expert(p.E, p.D / 16);
    hipLaunchKernelGGL(down_stream_kernel, dim3(p.E * bpe2), dim3(256), 0, stream, h, w2q, w2s,
                       offsets, p.D, p.F, bpe2, y);
    if (events) {
        const hipError_t er = hipEventRecord(events[2], stream);
        if (er != hipSuccess) return er;
    }
    const int64_t n = (int64_t)p.T * (p.D / 4);
    int64_t gb = (n + 255) / 256;
    if (gb > 8192) gb = 8192;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)gb), dim3(256), 0, stream, y, topk_w, pos,
                       p.T, p.D, p.k, out);
    if (events) {
        const hipError_t er = hipEventRecord(events[3], stream);
        if (er != hipSuccess) return er;
    }
    return hipGetLastError();
}

}  // namespace moe
