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
//   router_partial_kernel  logits as fp32 partial sums over D-slices
//                          (32x32 output tiles, LDS-staged operands)
//   route_topk_kernel      one wavefront per token: sum of the slices + bias,
//                          k rounds of wave-wide argmax, softmax, LDS histogram
//                          per 64-token chunk; with a single chunk it also runs
//                          the scan and the scatter (one launch for decode)
//   route_scan_kernel      per-expert running sums over chunks + block scan
//   route_scatter_kernel   stable scatter: ranks from wavefront ballots
// Nothing uses floating-point atomics, so results are deterministic.
#include <float.h>

#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kRouteTile = 32;     // tokens x experts per router tile
constexpr int kChunkTokens = 64;   // tokens per top-k / histogram chunk
constexpr int kMaxK = 8;
constexpr int kMaxE = 256;

__global__ __launch_bounds__(256) void router_partial_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr,
    float* __restrict__ partial, int T, int D, int E, int splits) {
    __shared__ float xs[kRouteTile][kRouteTile + 1];
    __shared__ float ws[kRouteTile][kRouteTile + 1];
    const int t0 = blockIdx.x * kRouteTile, e0 = blockIdx.y * kRouteTile, sp = blockIdx.z;
    const int nch = D / 32;
    const int c_begin = (int)((int64_t)nch * sp / splits);
    const int c_end = (int)((int64_t)nch * (sp + 1) / splits);
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const int lr = tid >> 3, lc = (tid & 7) * 4;
    float a00 = 0.f, a01 = 0.f, a10 = 0.f, a11 = 0.f;
    for (int c = c_begin; c < c_end; ++c) {
        const int d0 = c * 32;
        const int t = t0 + lr, e = e0 + lr;
        uint2 xv = make_uint2(0u, 0u);
        if (t < T) xv = *reinterpret_cast<const uint2*>(x + (int64_t)t * D + d0 + lc);
        float4 wv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (e < E) wv = *reinterpret_cast<const float4*>(wr + (int64_t)e * D + d0 + lc);
        xs[lr][lc + 0] = bf16_to_f32(xv.x & 0xFFFFu);
        xs[lr][lc + 1] = bf16_to_f32(xv.x >> 16);
        xs[lr][lc + 2] = bf16_to_f32(xv.y & 0xFFFFu);
        xs[lr][lc + 3] = bf16_to_f32(xv.y >> 16);
        ws[lr][lc + 0] = wv.x;
        ws[lr][lc + 1] = wv.y;
        ws[lr][lc + 2] = wv.z;
        ws[lr][lc + 3] = wv.w;
        __syncthreads();
#pragma unroll 8
        for (int dd = 0; dd < 32; ++dd) {
            const float x0 = xs[ty][dd], x1 = xs[ty + 16][dd];
            const float w0 = ws[tx][dd], w1 = ws[tx + 16][dd];
            a00 = __builtin_fmaf(x0, w0, a00);
            a01 = __builtin_fmaf(x0, w1, a01);
            a10 = __builtin_fmaf(x1, w0, a10);
            a11 = __builtin_fmaf(x1, w1, a11);
        }
        __syncthreads();
    }
    float* base = partial + (int64_t)sp * T * E;
    const int ta = t0 + ty, tb = t0 + ty + 16, ea = e0 + tx, eb = e0 + tx + 16;
    if (ta < T && ea < E) base[(int64_t)ta * E + ea] = a00;
    if (ta < T && eb < E) base[(int64_t)ta * E + eb] = a01;
    if (tb < T && ea < E) base[(int64_t)tb * E + ea] = a10;
    if (tb < T && eb < E) base[(int64_t)tb * E + eb] = a11;
}

// (v1, i1) ranks before (v2, i2): larger logit, then lower expert id.
__device__ __forceinline__ bool ranks_before(float v1, int i1, float v2, int i2) {
    return v1 > v2 || (v1 == v2 && i1 < i2);
}

// Exclusive prefix sum over the 256 threads of the block.
__device__ int block_exclusive_scan(int v, int* wsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int n = __shfl_up(incl, off);
        if (lane >= off) incl += n;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    __syncthreads();
    return base + incl - v;
}

// Stable scatter of one chunk of pairs.  ids_lds[i] is the expert of pair
// pair_base + i (i < npairs <= 8 * 64); base_e[e] is where this chunk's first
// pair of expert e goes.  Pairs are handled in 64-wide segments: a segment's
// members of one expert are found with 9 ballots over the expert id bits, and
// each pair's rank is the number of earlier lanes with the same expert.
__device__ void scatter_chunk(const int* ids_lds, int npairs, int pair_base,
                              const int* base_e, int E, int* seg_base,
                              int32_t* __restrict__ sorted, int32_t* __restrict__ pos) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nseg = (npairs + 63) / 64;
    for (int i = threadIdx.x; i < nseg * kMaxE; i += blockDim.x) seg_base[i] = 0;
    __syncthreads();
    int my_e[2], my_rank[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int g = wave + 4 * r;
        my_e[r] = kMaxE;
        my_rank[r] = 0;
        if (g < nseg) {
            const int idx = g * 64 + lane;
            const int e = idx < npairs ? ids_lds[idx] : kMaxE;  // 256 marks an empty lane
            uint64_t same = ~0ull;
#pragma unroll
            for (int b = 0; b < 9; ++b) {
                const bool bit = (e >> b) & 1;
                const uint64_t bal = __ballot(bit);
                same &= bit ? bal : ~bal;
            }
            const int rank = __popcll(same & ((1ull << lane) - 1ull));
            if (e < kMaxE && rank == 0) seg_base[g * kMaxE + e] = __popcll(same);
            my_e[r] = e;
            my_rank[r] = rank;
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int run = base_e[e];
        for (int g = 0; g < nseg; ++g) {
            const int c = seg_base[g * kMaxE + e];
            seg_base[g * kMaxE + e] = run;
            run += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int g = wave + 4 * r;
        if (g < nseg && my_e[r] < kMaxE) {
            const int idx = g * 64 + lane;
            const int dest = seg_base[g * kMaxE + my_e[r]] + my_rank[r];
            sorted[dest] = pair_base + idx;
            pos[pair_base + idx] = dest;
        }
    }
}

template <bool kFused>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ partial, int splits, const float* __restrict__ br, int T,
    int E, int k, int32_t* __restrict__ ids, float* __restrict__ wts,
    float* __restrict__ logits_out, int32_t* __restrict__ chunk_counts,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted, int32_t* __restrict__ pos) {
    __shared__ int cnt[kMaxE];
    __shared__ int chunk_ids[kChunkTokens * kMaxK];
    __shared__ int seg_base[8 * kMaxE];
    __shared__ int base_e[kMaxE];
    __shared__ int wsum[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kMaxE; i += blockDim.x) cnt[i] = 0;
    __syncthreads();
    const int tbeg = blockIdx.x * kChunkTokens;
    for (int tt = wave; tt < kChunkTokens; tt += 4) {
        const int t = tbeg + tt;
        if (t >= T) break;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = lane + 64 * q;
            v[q] = -FLT_MAX;
            if (e < E) {
                float s = 0.f;
                for (int sp = 0; sp < splits; ++sp) s += partial[((int64_t)sp * T + t) * E + e];
                if (br) s += br[e];
                v[q] = s;
                if (logits_out) logits_out[(int64_t)t * E + e] = s;
            }
        }
        bool taken[4] = {false, false, false, false};
        float selv[kMaxK];
        int seli[kMaxK];
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            selv[j] = 0.f;
            seli[j] = 0;
            if (j < k) {
                float bv = -FLT_MAX;
                int bi = 0x7FFFFFFF;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int e = lane + 64 * q;
                    if (e < E && !taken[q] && ranks_before(v[q], e, bv, bi)) {
                        bv = v[q];
                        bi = e;
                    }
                }
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) {
                    const float ov = __shfl_xor(bv, off);
                    const int oi = __shfl_xor(bi, off);
                    if (ranks_before(ov, oi, bv, bi)) {
                        bv = ov;
                        bi = oi;
                    }
                }
                if (bi >= E) bi = E - 1;  // only reachable with non-finite logits
                selv[j] = bv;
                seli[j] = bi;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (lane + 64 * q == bi) taken[q] = true;
            }
        }
        // softmax over the selected logits (selv[0] is the largest)
        float ex[kMaxK];
        float den = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            ex[j] = 0.f;
            if (j < k) {
                ex[j] = expf(selv[j] - selv[0]);
                den += ex[j];
            }
        }
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j < k && lane == j) {
                ids[(int64_t)t * k + j] = seli[j];
                wts[(int64_t)t * k + j] = ex[j] / den;
                atomicAdd(&cnt[seli[j]], 1);
                chunk_ids[tt * k + j] = seli[j];
            }
        }
    }
    __syncthreads();
    if (!kFused) {
        for (int e = tid; e < E; e += blockDim.x)
            chunk_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
        return;
    }
    // Single chunk: the chunk's histogram is the whole histogram.
    const int c = tid < E ? cnt[tid] : 0;
    const int excl = block_exclusive_scan(c, wsum);
    if (tid < E) {
        counts[tid] = c;
        offsets[tid] = excl;
        base_e[tid] = excl;
        if (tid == E - 1) offsets[E] = excl + c;
    }
    __syncthreads();
    const int ntok = T - tbeg < kChunkTokens ? T - tbeg : kChunkTokens;
    scatter_chunk(chunk_ids, ntok * k, tbeg * k, base_e, E, seg_base, sorted, pos);
}

__global__ __launch_bounds__(256) void route_scan_kernel(
    const int32_t* __restrict__ chunk_counts, int32_t* __restrict__ chunk_base, int chunks,
    int E, int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
    __shared__ int wsum[4];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        for (int c = 0; c < chunks; ++c) {
            const int v = chunk_counts[(int64_t)c * E + e];
            chunk_base[(int64_t)c * E + e] = run;
            run += v;
        }
    }
    const int excl = block_exclusive_scan(e < E ? run : 0, wsum);
    if (e < E) {
        counts[e] = run;
        offsets[e] = excl;
        if (e == E - 1) offsets[E] = excl + run;
        for (int c = 0; c < chunks; ++c) chunk_base[(int64_t)c * E + e] += excl;
    }
}

__global__ __launch_bounds__(256) void route_scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ chunk_base, int T, int E,
    int k, int32_t* __restrict__ sorted, int32_t* __restrict__ pos) {
    __shared__ int chunk_ids[kChunkTokens * kMaxK];
    __shared__ int seg_base[8 * kMaxE];
    __shared__ int base_e[kMaxE];
    const int tbeg = blockIdx.x * kChunkTokens;
    const int ntok = T - tbeg < kChunkTokens ? T - tbeg : kChunkTokens;
    const int npairs = ntok * k;
    for (int i = threadIdx.x; i < npairs; i += blockDim.x) chunk_ids[i] = ids[(int64_t)tbeg * k + i];
    for (int e = threadIdx.x; e < E; e += blockDim.x) base_e[e] = chunk_base[(int64_t)blockIdx.x * E + e];
    __syncthreads();
    scatter_chunk(chunk_ids, npairs, tbeg * k, base_e, E, seg_base, sorted, pos);
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

RoutePlan plan_route(int T, int D, int E, int k) {
    RoutePlan p{};
    p.T = T; p.D = D; p.E = E; p.k = k;
    const int tiles = ((T + kRouteTile - 1) / kRouteTile) * ((E + kRouteTile - 1) / kRouteTile);
    int splits = 1024 / (tiles > 0 ? tiles : 1);
    const int nch = D / 32;
    if (splits > nch) splits = nch;
    if (splits > 32) splits = 32;
    if (splits < 1) splits = 1;
    p.splits = splits;
    p.chunks = (T + kChunkTokens - 1) / kChunkTokens;
    size_t off = 0;
    p.off_partial = off;
    off = align256(off + (size_t)splits * T * E * sizeof(float));
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
    float* partial = reinterpret_cast<float*>(base + p.off_partial);
    int32_t* chunk_counts = reinterpret_cast<int32_t*>(base + p.off_chunk_counts);
    int32_t* chunk_base = reinterpret_cast<int32_t*>(base + p.off_chunk_base);
    dim3 g1((p.T + kRouteTile - 1) / kRouteTile, (p.E + kRouteTile - 1) / kRouteTile, p.splits);
    hipLaunchKernelGGL(router_partial_kernel, g1, dim3(256), 0, stream, x, wr, partial, p.T,
                       p.D, p.E, p.splits);
    if (p.chunks == 1) {
        hipLaunchKernelGGL(route_topk_kernel<true>, dim3(1), dim3(256), 0, stream, partial,
                           p.splits, br, p.T, p.E, p.k, ids, w, logits_out, chunk_counts,
                           counts, offsets, sorted, pos);
    } else {
        hipLaunchKernelGGL(route_topk_kernel<false>, dim3(p.chunks), dim3(256), 0, stream,
                           partial, p.splits, br, p.T, p.E, p.k, ids, w, logits_out,
                           chunk_counts, counts, offsets, sorted, pos);
        hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(256), 0, stream, chunk_counts,
                           chunk_base, p.chunks, p.E, counts, offsets);
        hipLaunchKernelGGL(route_scatter_kernel, dim3(p.chunks), dim3(256), 0, stream, ids,
                           chunk_base, p.T, p.E, p.k, sorted, pos);
    }
    return hipGetLastError();
}

}  // namespace moe
