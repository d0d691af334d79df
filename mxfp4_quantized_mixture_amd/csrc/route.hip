// route.hip -- token-choice router for gfx950.
//
// Each token picks its k experts by router logit and weights them with a
// softmax taken over the selected logits only ("Welcome GPT OSS", section 4:
// token-choice MoE with softmax-after-topk; k = 4 of 32 or 128 experts per the
// talk summary's architecture block).  The pairs p = t*k + j are then grouped
// by expert with a stable counting sort (histogram, exclusive scan, scatter)
// so that the expert GEMMs read contiguous row ranges.
//
// Kernels:
//   router_logits_kernel   matrix-core logits (fp32 weights as 3 exact bf16
//                          terms), split-K over wavefronts and blocks: decode
//                          batches (T <= 64) and contractions not a multiple
//                          of 64
//   router_gemm_kernel     longer batches: 32- or 64-expert x 256-token tiles
//                          staged through LDS chunk by chunk (whole-line
//                          loads, each weight split once per block), split-K
//                          over blocks only
//   route_topk_kernel      one wavefront per token: k rounds of wave-wide
//                          DPP argmax, softmax over the k, per-chunk histogram
//   route_finish_kernel    few pairs: histogram, scan and scatter in one block
//   route_small_kernel     few tokens (T <= 64): top-k, softmax, histogram,
//                          scan and scatter together in one block
//   route_scan_kernel      many pairs: per-expert scan of the chunk counts
//   route_scatter_kernel   many pairs: expert offsets, stable scatter (ranks
//                          from ballots)
// Nothing uses floating-point atomics, so results are deterministic.
#include <float.h>

#include "device_common.h"
#include "launch.h"
#include "route_device.h"

namespace moe {

// Router logits of longer batches.  Block (bx, by, bz) of 4 wavefronts:
// experts 16 NE bx .. + 16 NE - 1, tokens 256 by .. 256 by + 255,
// contraction chunks [c0, c1) of
// 64 (slice bz of S; slice s writes P[s], slice 0 adds the bias).  Each
// chunk of the fp32 weight rows (16 NE rows) and of x (256 rows) is loaded
// with whole-line loads into registers one chunk ahead; the block then
// splits the weights into their three exact bf16 terms (split3_bf16, the
// terms router_logits_tile forms) and writes terms and x rows to LDS rows of
// kRgPitch bytes (128 + 16: the 16-byte operand reads of 16 consecutive rows
// then hit 16 different bank groups), each weight split once per block.
// Wavefront w owns tokens 64 w .. 64 w + 63 against all the block's experts:
// per 32-wide step NE x 4 tiles x 3 terms of 16x16x32 bf16 products,
// C[expert][token] as in router_logits_tile.  Rows past E or T load clamped
// rows; their results are not stored.
constexpr int kRgK = 64, kRgPitch = 144, kRgTok = 256, kRgWaves = 4, kRgThreads = 64 * kRgWaves;
template <int NE>
struct RouterGemm {
    static constexpr int kExp = 16 * NE;
    static constexpr int kTT = kRgTok / 16 / kRgWaves;       // 16-token tiles per wave
    static constexpr int kGroups = kExp * (kRgK / 8);        // 8-weight groups per chunk
    static constexpr int kWPer = kGroups / kRgThreads;       // per thread
    static constexpr int kXPer = kRgTok * (kRgK / 8) / kRgThreads;  // 16-byte x units per thread
    static constexpr int kLds = (3 * kExp + kRgTok) * kRgPitch;
    static_assert(kGroups % kRgThreads == 0, "even split");
};

template <int NE>
__global__ __launch_bounds__(kRgThreads, 2) void router_gemm_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ br,
    float* __restrict__ P, int T, int D, int E, int S) {
    using G = RouterGemm<NE>;
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int e0 = blockIdx.x * G::kExp, t0 = blockIdx.y * kRgTok, sl = blockIdx.z;
    const int nch = D / kRgK;
    const int c0 = (int)((int64_t)nch * sl / S), c1 = (int)((int64_t)nch * (sl + 1) / S);
    // weight group q = tid + 256 i: row q / 8, weights 8 (q % 8) .. + 7 of the
    // chunk; x unit u = tid + 256 i: row u / 8, elements 8 (u % 8) .. + 7
    int64_t wsrc[G::kWPer], xsrc[G::kXPer];
    int wdst[G::kWPer], xdst[G::kXPer];
#pragma unroll
    for (int i = 0; i < G::kWPer; ++i) {
        const int q = tid + kRgThreads * i, r = q / 8, c = q % 8;
        wsrc[i] = (int64_t)min(e0 + r, E - 1) * D + 8 * c;
        wdst[i] = r * kRgPitch + 16 * c;
    }
#pragma unroll
    for (int i = 0; i < G::kXPer; ++i) {
        const int u = tid + kRgThreads * i, r = u / 8, c = u % 8;
        xsrc[i] = (int64_t)min(t0 + r, T - 1) * D + 8 * c;
        xdst[i] = (3 * G::kExp + r) * kRgPitch + 16 * c;
    }
    struct Stage {
        float4 w[G::kWPer][2];
        u32x4_t x[G::kXPer];
    };
    Stage sa;                                   // the next chunk, loaded during this one
    auto load_chunk = [&](Stage& st, int ch) {
        const int64_t k0 = (int64_t)ch * kRgK;
#pragma unroll
        for (int i = 0; i < G::kWPer; ++i) {
            st.w[i][0] = *reinterpret_cast<const float4*>(wr + wsrc[i] + k0);
            st.w[i][1] = *reinterpret_cast<const float4*>(wr + wsrc[i] + k0 + 4);
        }
#pragma unroll
        for (int i = 0; i < G::kXPer; ++i)
            st.x[i] = *reinterpret_cast<const u32x4_t*>(x + xsrc[i] + k0);
    };
    constexpr int TT = G::kTT;
    f32x4_t acc[NE][TT];
#pragma unroll
    for (int et = 0; et < NE; ++et)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[et][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto run_chunk = [&](Stage& st, int ch) {
        __syncthreads();                        // every wave is done with the previous chunk
#pragma unroll
        for (int i = 0; i < G::kWPer; ++i) {
            const float w[8] = {st.w[i][0].x, st.w[i][0].y, st.w[i][0].z, st.w[i][0].w,
                                st.w[i][1].x, st.w[i][1].y, st.w[i][1].z, st.w[i][1].w};
            bf16x8_t t3[3];
            split3_bf16(w, t3[0], t3[1], t3[2]);
#pragma unroll
            for (int pl = 0; pl < 3; ++pl)
                *reinterpret_cast<u32x4_t*>(lds + pl * G::kExp * kRgPitch + wdst[i]) =
                    __builtin_bit_cast(u32x4_t, t3[pl]);
        }
#pragma unroll
        for (int i = 0; i < G::kXPer; ++i) *reinterpret_cast<u32x4_t*>(lds + xdst[i]) = st.x[i];
        __syncthreads();
        if (ch + 1 < c1) load_chunk(st, ch + 1);
#pragma unroll
        for (int j = 0; j < kRgK / 32; ++j) {
            bf16x8_t xb[TT];
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
                xb[tt] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(
                    lds + (3 * G::kExp + 16 * (TT * wave + tt) + m) * kRgPitch + 64 * j + 16 * g));
#pragma unroll
            for (int et = 0; et < NE; ++et) {
                bf16x8_t wt[3];
#pragma unroll
                for (int pl = 0; pl < 3; ++pl)
                    wt[pl] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(
                        lds + (pl * G::kExp + 16 * et + m) * kRgPitch + 64 * j + 16 * g));
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
                    acc[et][tt] = mfma_bf16(wt[0], xb[tt], acc[et][tt]);
                    acc[et][tt] = mfma_bf16(wt[1], xb[tt], acc[et][tt]);
                    acc[et][tt] = mfma_bf16(wt[2], xb[tt], acc[et][tt]);
                }
            }
        }
    };
    if (c0 < c1) load_chunk(sa, c0);
    for (int ch = c0; ch < c1; ++ch) run_chunk(sa, ch);
    // lane (m, g) of tile (et, tt) holds experts e0 + 16 et + 4 g + r of token
    // t0 + 16 (TT w + tt) + m
    float* Ps = P + (int64_t)sl * T * E;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int t = t0 + 16 * (TT * wave + tt) + m;
        if (t >= T) continue;
#pragma unroll
        for (int et = 0; et < NE; ++et)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = e0 + 16 * et + 4 * g + r;
                if (e < E) Ps[(int64_t)t * E + e] = acc[et][tt][r] + ((br && sl == 0) ? br[e] : 0.f);
            }
    }
}

// Router logits kernel: one tile per block (see router_logits_tile).
template <int TT, int NE, int KB, bool kPipe>
__global__ __launch_bounds__(kRouterWaves * 64) void router_logits_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ br,
    float* __restrict__ P, int T, int D, int E, int S) {
    __shared__ f32x4_t red[kRouterWaves * NE * TT * 64];
    router_logits_tile<TT, NE, KB, kPipe>(x, wr, br, P, T, D, E, S, blockIdx.x, blockIdx.y,
                                          blockIdx.z, red);
}

// One step of a wave-wide argmax over (logit, id) pairs through the DPP
// crossbar: combine with the lane the control selects (identity where there
// is none).
template <int kCtrl, int kRowMask, int kBankMask>
__device__ __forceinline__ void argmax_dpp(float& v, int& i) {
    const float ov = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        __builtin_bit_cast(int, -__builtin_inff()), __builtin_bit_cast(int, v), kCtrl, kRowMask,
        kBankMask, false));
    const int oi = __builtin_amdgcn_update_dpp(0x7FFFFFFF, i, kCtrl, kRowMask, kBankMask, false);
    if (ranks_before(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}

// Top-k of one token's logits held 4 per lane (expert lane + 64 q): k rounds
// of a wave-wide argmax (larger logit, then lower id).  Each round reduces
// within rows of 16 lanes (row shifts by 1, 2, 4, 8), then across rows (row
// broadcasts of lanes 15 and 31), leaving the winner in lane 63.  After round
// j, lane j keeps the j-th selection.
__device__ __forceinline__ void wave_topk(float v0, float v1, float v2, float v3, int E, int k,
                                       float& my_v, int& my_i) {
    const int lane = threadIdx.x & 63;
    float v[4] = {v0, v1, v2, v3};
    my_v = 0.f;
    my_i = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -__builtin_inff();
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = lane + 64 * q;
            if (e < E && ranks_before(v[q], e, bv, bi)) {
                bv = v[q];
                bi = e;
            }
        }
        argmax_dpp<0x111, 0xF, 0xF>(bv, bi);   // row_shr:1
        argmax_dpp<0x112, 0xF, 0xF>(bv, bi);   // row_shr:2
        argmax_dpp<0x114, 0xF, 0xE>(bv, bi);   // row_shr:4
        argmax_dpp<0x118, 0xF, 0xC>(bv, bi);   // row_shr:8
        argmax_dpp<0x142, 0xA, 0xF>(bv, bi);   // row_bcast:15
        argmax_dpp<0x143, 0xC, 0xF>(bv, bi);   // row_bcast:31
        bv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 63));
        bi = __builtin_amdgcn_readlane(bi, 63);
        if (bi >= E) bi = E - 1;              // only reachable with non-finite logits
        if (lane == j) {
            my_v = bv;
            my_i = bi;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (lane + 64 * q == bi) v[q] = -__builtin_inff();
    }
}

// Top-k, softmax over the selected logits and the chunk histogram: one
// wavefront per token of the block's 16-token chunk (logit = the S router
// slices summed in order).
template <int kMaxS>
__global__ __launch_bounds__(kChunkTokens * 64) void route_topk_kernel(
    const float* __restrict__ P, int S, int T, int E, int k, float* __restrict__ logits_out,
    int32_t* __restrict__ ids, float* __restrict__ wts, int32_t* __restrict__ chunk_counts) {
    __shared__ int cnt[kMaxE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kMaxE; i += blockDim.x) cnt[i] = 0;
    const int t = blockIdx.x * kChunkTokens + wave;
    float v[4];
    {
        // unconditional loads (clamped slice, token and expert; the extra
        // values are discarded), so the compiler issues them all at once
        float part[4][kMaxS];
        const int tc = min(t, T - 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ec = min(lane + 64 * q, E - 1);
#pragma unroll
            for (int sp = 0; sp < kMaxS; ++sp)
                part[q][sp] = P[((int64_t)min(sp, S - 1) * T + tc) * E + ec];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float acc = part[q][0];
#pragma unroll
            for (int sp = 1; sp < kMaxS; ++sp)
                if (sp < S) acc += part[q][sp];
            v[q] = acc;
        }
    }
    __syncthreads();                           // cnt cleared
    if (t < T) {
        if (logits_out) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (lane + 64 * q < E) logits_out[(int64_t)t * E + lane + 64 * q] = v[q];
        }
        float my_v;
        int my_i;
        wave_topk(v[0], v[1], v[2], v[3], E, k, my_v, my_i);
        // softmax over the k selected logits; lane 0 holds the largest
        const float top = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_v), 0));
        const float ex = lane < k ? expf(my_v - top) : 0.f;
        float den = 0.f;
        for (int j = 0; j < k; ++j)
            den += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), j));
        if (lane < k) {
            ids[(int64_t)t * k + lane] = my_i;
            wts[(int64_t)t * k + lane] = ex / den;
            atomicAdd(&cnt[my_i], 1);
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) chunk_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// Few pairs (P <= kFinishMaxPairs): one block rebuilds the histogram from the
// ids, scans it and scatters every pair.
__global__ __launch_bounds__(1024) void route_finish_kernel(
    const int32_t* __restrict__ ids, int P, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted, int32_t* __restrict__ pos) {
    __shared__ int cnt[kMaxE];
    __shared__ int pair_e[kFinishMaxPairs];
    __shared__ int seg_base[8 * kMaxE];
    __shared__ int base_e[kMaxE];
    __shared__ int wsum[16];
    const int tid = threadIdx.x;
    for (int i = tid; i < kMaxE; i += blockDim.x) cnt[i] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += blockDim.x) {
        const int e = ids[p];
        pair_e[p] = e;
        atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    const int c = tid < E ? cnt[tid] : 0;
    const int excl = block_exclusive_scan(c, wsum);
    if (tid < E) {
        counts[tid] = c;
        offsets[tid] = excl;
        base_e[tid] = excl;
        if (tid == E - 1) offsets[E] = excl + c;
    }
    __syncthreads();
    scatter_chunk(pair_e, P, 0, base_e, E, seg_base, sorted, pos);
}

template <int K>
__global__ __launch_bounds__(1024) void route_small_kernel(
    const float* __restrict__ P, int S, int T, int E, float* __restrict__ logits_out,
    int32_t* __restrict__ ids, float* __restrict__ wts, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted, int32_t* __restrict__ pos) {
    __shared__ SmallRouteLds lds;
    route_small_body<K, 16>(P, S, T, E, logits_out, ids, wts, counts, offsets, sorted, pos, lds);
}

// Many pairs, step 1: block e scans expert e's chunk counts.  Each thread
// sums a contiguous run of chunks (its loads all in flight), the block scans
// the run sums, and each thread writes its chunks' bases relative to the
// expert's first pair; counts[e] is the total.
__global__ __launch_bounds__(256) void route_scan_kernel(
    const int32_t* __restrict__ chunk_counts, int32_t* __restrict__ chunk_base, int chunks,
    int E, int32_t* __restrict__ counts) {
    __shared__ int wsum[16];
    const int e = blockIdx.x;
    const int per = (chunks + blockDim.x - 1) / blockDim.x;
    const int c0 = threadIdx.x * per;
    const int c1 = c0 + per < chunks ? c0 + per : chunks;
    int run = 0;
    for (int c = c0; c < c1; ++c) run += chunk_counts[(int64_t)c * E + e];
    int base = block_exclusive_scan(run, wsum);
    for (int c = c0; c < c1; ++c) {
        const int v = chunk_counts[(int64_t)c * E + e];
        chunk_base[(int64_t)c * E + e] = base;
        base += v;
    }
    if (threadIdx.x == blockDim.x - 1) counts[e] = base;
}

// Many pairs, step 2: one block per chunk.  The expert offsets (an exclusive
// scan of counts, E <= 256 = blockDim) are recomputed by every block, and
// block 0 writes them out; the chunk's pairs are then scattered stably.
__global__ __launch_bounds__(256) void route_scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ counts, int T, int E, int k, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted, int32_t* __restrict__ pos) {
    __shared__ int chunk_ids[kChunkTokens * kMaxK];
    __shared__ int seg_base[8 * kMaxE];
    __shared__ int base_e[kMaxE];
    __shared__ int wsum[16];
    const int tbeg = blockIdx.x * kChunkTokens;
    const int ntok = T - tbeg < kChunkTokens ? T - tbeg : kChunkTokens;
    const int npairs = ntok * k;
    for (int i = threadIdx.x; i < npairs; i += blockDim.x) chunk_ids[i] = ids[(int64_t)tbeg * k + i];
    const int e = threadIdx.x;
    const int c = e < E ? counts[e] : 0;
    const int excl = block_exclusive_scan(c, wsum);
    if (e < E) {
        base_e[e] = excl + chunk_base[(int64_t)blockIdx.x * E + e];
        if (blockIdx.x == 0) {
            offsets[e] = excl;
            if (e == E - 1) offsets[E] = excl + c;
        }
    }
    __syncthreads();
    scatter_chunk(chunk_ids, npairs, tbeg * k, base_e, E, seg_base, sorted, pos);
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

RoutePlan plan_route(int T, int D, int E, int k) {
    RoutePlan p{};
    p.T = T; p.D = D; p.E = E; p.k = k;
    p.token_tiles = T <= 64 ? 1 : 4;           // 16-token tiles per router block
    // longer batches with whole 64-wide contraction chunks: router_gemm_kernel
    p.gemm_router = T > 64 && D % kRgK == 0;
    // 16-expert tiles per router block: one for decode (latency: many small
    // blocks), several for long batches (each block reads its x rows once for
    // all of them)
    p.expert_tiles = T <= 64 ? 1 : (E > 32 ? 4 : 2);
    const int tiles = ((E + 16 * p.expert_tiles - 1) / (16 * p.expert_tiles)) *
                      ((T + 16 * p.token_tiles - 1) / (16 * p.token_tiles));
    // split the contraction over blocks until ~128 blocks (decode) or ~512
    // blocks (long batches: two per CU) are busy, at most 16 slices, and each
    // wavefront keeps at least one 32-column step
    const int want = T <= 64 ? 128 : 512;
    int S = (want + tiles - 1) / tiles;
    int max_s = (D / 32) / kRouterWaves;
    // router_gemm blocks of 256 tokens and 32 experts when there are at most
    // 32, else 64 (measured: 128 experts x 128 tokens, which reads x once, and
    // a second register stage were both slower)
    p.gemm_router_ne = E <= 32 ? 2 : 4;
    if (p.gemm_router) {
        const int ge = 16 * p.gemm_router_ne;
        const int gt = ((E + ge - 1) / ge) * ((T + kRgTok - 1) / kRgTok);
        S = (want + gt - 1) / gt;
        max_s = D / kRgK;                      // at least one chunk per slice
    }
    if (S > max_s) S = max_s;
    if (S > 16) S = 16;
    p.splits = S < 1 ? 1 : S;
    p.chunks = (T + kChunkTokens - 1) / kChunkTokens;
    size_t off = 0;
    p.off_logits = off;
    off = align256(off + (size_t)p.splits * T * E * sizeof(float));
    p.off_chunk_counts = off;
    off = align256(off + (size_t)p.chunks * E * sizeof(int32_t));
    p.off_chunk_base = off;
    off = align256(off + (size_t)p.chunks * E * sizeof(int32_t));
    p.ws_bytes = off;
    return p;
}

hipError_t launch_route(const RoutePlan& p, const uint16_t* x, const float* wr, const float* br,
                        int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                        int32_t* sorted, int32_t* pos, float* logits_out, void* ws,
                        hipStream_t stream) {
    char* base = static_cast<char*>(ws);
    float* P = reinterpret_cast<float*>(base + p.off_logits);
    int32_t* chunk_counts = reinterpret_cast<int32_t*>(base + p.off_chunk_counts);
    int32_t* chunk_base = reinterpret_cast<int32_t*>(base + p.off_chunk_base);
    {
        const int et = 16 * p.expert_tiles, tt = 16 * p.token_tiles;
        const dim3 g((p.E + et - 1) / et, (p.T + tt - 1) / tt, p.splits);
        if (p.gemm_router) {
            const int ge = 16 * p.gemm_router_ne;
            const dim3 gg((p.E + ge - 1) / ge, (p.T + kRgTok - 1) / kRgTok, p.splits);
            constexpr size_t lds2 = RouterGemm<2>::kLds, lds4 = RouterGemm<4>::kLds;
            if (p.gemm_router_ne == 2)
                hipLaunchKernelGGL((router_gemm_kernel<2>), gg, dim3(kRgThreads), lds2, stream, x,
                                   wr, br, P, p.T, p.D, p.E, p.splits);
            else
                hipLaunchKernelGGL((router_gemm_kernel<4>), gg, dim3(kRgThreads), lds4, stream, x,
                                   wr, br, P, p.T, p.D, p.E, p.splits);
        } else if (p.token_tiles == 1)
            hipLaunchKernelGGL((router_logits_kernel<1, 1, 4, false>), g, dim3(kRouterWaves * 64), 0,
                               stream, x, wr, br, P, p.T, p.D, p.E, p.splits);
        else if (p.expert_tiles == 2)
            hipLaunchKernelGGL((router_logits_kernel<4, 2, 4, false>), g, dim3(kRouterWaves * 64), 0,
                               stream, x, wr, br, P, p.T, p.D, p.E, p.splits);
        else
            hipLaunchKernelGGL((router_logits_kernel<4, 4, 1, true>), g, dim3(kRouterWaves * 64), 0,
                               stream, x, wr, br, P, p.T, p.D, p.E, p.splits);
    }
    if (p.T <= kSmallTokens && p.T * p.E <= kSmallLogits) {
        switch (p.k) {
#define MOE_ROUTE_SMALL(K)                                                                    \
    case K:                                                                                   \
        hipLaunchKernelGGL(route_small_kernel<K>, dim3(1), dim3(1024), 0, stream, P, p.splits, \
                           p.T, p.E, logits_out, ids, w, counts, offsets, sorted, pos);        \
        break;
            MOE_ROUTE_SMALL(1) MOE_ROUTE_SMALL(2) MOE_ROUTE_SMALL(3) MOE_ROUTE_SMALL(4)
            MOE_ROUTE_SMALL(5) MOE_ROUTE_SMALL(6) MOE_ROUTE_SMALL(7) MOE_ROUTE_SMALL(8)
#undef MOE_ROUTE_SMALL
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    // (slice loads are unconditional up to the template's bound: 4 when the
    // router used at most 4 slices)
    if (p.splits <= 4)
        hipLaunchKernelGGL(route_topk_kernel<4>, dim3(p.chunks), dim3(kChunkTokens * 64), 0,
                           stream, P, p.splits, p.T, p.E, p.k, logits_out, ids, w, chunk_counts);
    else
        hipLaunchKernelGGL(route_topk_kernel<16>, dim3(p.chunks), dim3(kChunkTokens * 64), 0,
                           stream, P, p.splits, p.T, p.E, p.k, logits_out, ids, w, chunk_counts);
    const int pairs = p.T * p.k;
    if (pairs <= kFinishMaxPairs) {
        hipLaunchKernelGGL(route_finish_kernel, dim3(1), dim3(1024), 0, stream, ids, pairs, p.E,
                           counts, offsets, sorted, pos);
    } else {
        hipLaunchKernelGGL(route_scan_kernel, dim3(p.E), dim3(256), 0, stream, chunk_counts,
                           chunk_base, p.chunks, p.E, counts);
        hipLaunchKernelGGL(route_scatter_kernel, dim3(p.chunks), dim3(256), 0, stream, ids,
                           chunk_base, counts, p.T, p.E, p.k, offsets, sorted, pos);
    }
    return hipGetLastError();
}

}  // namespace moe
