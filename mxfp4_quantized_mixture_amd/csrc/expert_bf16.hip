// expert_bf16.hip -- the same SwiGLU expert layer with bf16 expert weights, for
// gfx950: the comparison path of the MXFP4 one.
//
// The pages offer bf16 weights as the fallback where MXFP4 kernels are not
// available, at about four times the weight memory ("Tricks from OpenAI
// gpt-oss", section 7; the Japanese Transformers page, "メモリ削減効果").
// This path computes the layer of "Welcome GPT OSS", section 4 -- for routed
// pair p = t k + j of expert e: g = Wg_e x_t, u = Wu_e x_t, h = silu(g) u,
// y_p = W2_e h, out[t] = sum_j w[t, j] y_p -- on weights that are bf16 as
// stored, so that both paths can be run and measured on the same layer.
//
// Weight streaming, for batches in which experts receive few tokens: block
// b owns a fixed range of 16-row weight tiles of expert b / bpe; each of its
// wavefronts streams whole tiles over the full contraction, 32 elements per
// step, on v_mfma_f32_16x16x32_bf16 (A = 16 weight rows as stored, B = the
// activations of up to 16 of the expert's pairs).  Experts with more pairs
// are taken 16 pairs at a time, the tiles streamed again for each group.
// Nothing is staged in LDS: each lane loads its activation piece next to its
// weight piece (the block's waves read the same activations, which L1 and L2
// serve; the weights are the HBM stream).
//
// Precision: x is bf16 and the products of bf16 operands are exact in fp32,
// so g and u are fp32 sums of exact products.  h is kept in fp32 between the
// two kernels and enters the down products as two bf16 terms, hi = bf16(h)
// and lo = bf16(h - hi) (h - hi is exact in fp32), which leaves an error
// below 2^-17 of |h|.  y stays fp32 until the combine rounds the output to
// bf16.
#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kBf16Waves = 8;
constexpr int kBf16Steps = 4;   // 32-element steps per load batch (two batches in flight)

// bf16 hi + lo of 8 fp32 values (two 16-byte pieces): hi = RNE(v), lo =
// RNE(v - hi)
__device__ __forceinline__ void split2_bf16(const u32x4_t (&raw)[2], bf16x8_t& hi, bf16x8_t& lo) {
    const f32x4_t r0 = __builtin_bit_cast(f32x4_t, raw[0]);
    const f32x4_t r1 = __builtin_bit_cast(f32x4_t, raw[1]);
    const float v[8] = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    u32x4_t h, l;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        uint32_t hb[2], lb[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            hb[q] = f32_to_bf16_rne(v[2 * p + q]);
            lb[q] = f32_to_bf16_rne(v[2 * p + q] - bf16_to_f32(hb[q]));
        }
        h[p] = hb[0] | (hb[1] << 16);
        l[p] = lb[0] | (lb[1] << 16);
    }
    hi = as_bf16x8(h);
    lo = as_bf16x8(l);
}

// kGateUp: A = gate and up tiles of W13 (rows tile, F + tile), B = gathered
//          x rows; epilogue h = silu(g) u -> fp32 [P, F].
// else:    A = W2 tile, B = h rows (two bf16 terms); epilogue y -> fp32 [P, D].
// Lane l (m = l % 16, g = l / 16) loads row m of each tile and column m (pair
// m of the group), K = 32 s + 8 g .. + 7 of step s, and receives outputs
// 4 g .. 4 g + 3 of the tile for pair m.
template <bool kGateUp>
__global__ __launch_bounds__(kBf16Waves * 64) void expert_bf16_kernel(
    const void* __restrict__ act, const uint16_t* __restrict__ w,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted, int D, int F, int k,
    int bpe, float* __restrict__ out) {
    constexpr int NS = kGateUp ? 2 : 1;     // weight tiles per step (gate, up)
    constexpr int NR = kGateUp ? 1 : 2;     // 16-byte activation pieces per step
    constexpr int NB = kBf16Steps;
    const int K = kGateUp ? D : F;
    const int NOUT = kGateUp ? F : D;
    const int R = kGateUp ? 2 * F : D;      // weight rows per expert
    const int ntiles = NOUT / 16;
    const int e = blockIdx.x / bpe, part = blockIdx.x - e * bpe;
    const int ta = (int)((int64_t)ntiles * part / bpe), tb = (int)((int64_t)ntiles * (part + 1) / bpe);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int KS = K / 32;
    const int my_tiles = ta + wave < tb ? (tb - ta - wave + kBf16Waves - 1) / kBf16Waves : 0;
    const int total = my_tiles * KS;        // steps of this wavefront per pair group
    const int row_beg = offsets[e], ne = offsets[e + 1] - row_beg;
    if (ne <= 0 || my_tiles == 0) return;
    const uint16_t* we = w + (size_t)e * R * K;

    struct Batch {
        u32x4_t a[NB][NS];
        u32x4_t b[NB][NR];
    };
    for (int tg = 0; tg < ne; tg += 16) {
        const int row0 = row_beg + tg, nvalid = min(16, ne - tg);
        // this lane's activation row: pair m of the group (the last valid
        // pair for columns past the group: finite, never stored)
        const int pr = row0 + min(m, nvalid - 1);
        const uint8_t* arow = kGateUp
            ? static_cast<const uint8_t*>(act) + (size_t)(sorted[pr] / k) * K * 2
            : static_cast<const uint8_t*>(act) + (size_t)pr * K * 4;
        // Loads are unconditional: steps past the end reload the last step
        // (cache hits), so the compiler never drains the queue at a branch.
        auto fetch = [&](Batch& B, int s0) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int s = min(s0 + i, total - 1);
                const int tile = ta + wave + (s / KS) * kBf16Waves, ks = s - (s / KS) * KS;
                const int kk = 32 * ks + 8 * g;
#pragma unroll
                for (int r = 0; r < NS; ++r)
                    B.a[i][r] = *reinterpret_cast<const u32x4_t*>(
                        we + (size_t)(r * F + 16 * tile + m) * K + kk);
#pragma unroll
                for (int c = 0; c < NR; ++c)
                    B.b[i][c] = *reinterpret_cast<const u32x4_t*>(
                        arow + (size_t)kk * (kGateUp ? 2 : 4) + 16 * c);
            }
        };
        f32x4_t acc[NS];
#pragma unroll
        for (int r = 0; r < NS; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        auto compute = [&](const Batch& B, int s0) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int s = s0 + i;
                if (s < total) {
                    if constexpr (kGateUp) {
                        const bf16x8_t xb = as_bf16x8(B.b[i][0]);
#pragma unroll
                        for (int r = 0; r < NS; ++r) acc[r] = mfma_bf16(as_bf16x8(B.a[i][r]), xb, acc[r]);
                    } else {
                        bf16x8_t hi, lo;
                        split2_bf16(B.b[i], hi, lo);
                        const bf16x8_t wa = as_bf16x8(B.a[i][0]);
                        acc[0] = mfma_bf16(wa, hi, acc[0]);
                        acc[0] = mfma_bf16(wa, lo, acc[0]);
                    }
                    if (s % KS == KS - 1) {           // the tile's contraction is done
                        const int tile = ta + wave + (s / KS) * kBf16Waves;
                        f32x4_t res;
                        if constexpr (kGateUp) {
#pragma unroll
                            for (int q = 0; q < 4; ++q) res[q] = silu_f32(acc[0][q]) * acc[1][q];
                        } else {
                            res = acc[0];
                        }
                        if (m < nvalid)
                            *reinterpret_cast<f32x4_t*>(out + (size_t)(row0 + m) * NOUT + 16 * tile + 4 * g) = res;
#pragma unroll
                        for (int r = 0; r < NS; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    }
                }
            }
        };
        Batch B0, B1;
        fetch(B0, 0);
        fetch(B1, NB);
        for (int s = 0; s < total; s += 2 * NB) {
            compute(B0, s);
            fetch(B0, s + 2 * NB);
            compute(B1, s + NB);
            fetch(B1, s + 3 * NB);
        }
    }
}

size_t bf16_mlp_workspace_bytes(int T, int D, int F, int k) {
    const size_t P = (size_t)T * k;
    return ((P * D * sizeof(float) + 255) & ~(size_t)255) + P * F * sizeof(float);
}

// Blocks per expert: about 256 blocks in all and at least 2 per expert, at
// most one per 8 tiles (one tile per wavefront).
static int bf16_blocks_per_expert(int E, int ntiles) {
    int bpe = (256 + E - 1) / E;
    if (bpe < 2) bpe = 2;
    if (bpe > ntiles / kBf16Waves) bpe = ntiles / kBf16Waves;
    return bpe < 1 ? 1 : bpe;
}

hipError_t launch_mlp_bf16(int T, int D, int F, int E, int k, const uint16_t* x,
                           const uint16_t* w13, const uint16_t* w2, const float* topk_w,
                           const int32_t* offsets, const int32_t* sorted, const int32_t* pos,
                           uint16_t* out, void* ws, hipEvent_t* events, hipStream_t stream) {
    const size_t P = (size_t)T * k;
    float* y = static_cast<float*>(ws);
    float* h = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                        ((P * D * sizeof(float) + 255) & ~(size_t)255));
    hipError_t er;
    if (events && (er = hipEventRecord(events[0], stream)) != hipSuccess) return er;
    hipLaunchKernelGGL(expert_bf16_kernel<true>, dim3(E * bf16_blocks_per_expert(E, F / 16)),
                       dim3(kBf16Waves * 64), 0, stream, x, w13, offsets, sorted, D, F, k,
                       bf16_blocks_per_expert(E, F / 16), h);
    if (events && (er = hipEventRecord(events[1], stream)) != hipSuccess) return er;
    hipLaunchKernelGGL(expert_bf16_kernel<false>, dim3(E * bf16_blocks_per_expert(E, D / 16)),
                       dim3(kBf16Waves * 64), 0, stream, h, w2, offsets, sorted, D, F, k,
                       bf16_blocks_per_expert(E, D / 16), y);
    if ((er = hipGetLastError()) != hipSuccess) return er;
    return launch_combine_rows(T, D, k, y, topk_w, pos, out, events, stream);
}

}  // namespace moe
