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
//                          terms), split-K over wavefronts and blocks
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
    const int max_s = (D / 32) / kRouterWaves;
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
        if (p.token_tiles == 1)
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
