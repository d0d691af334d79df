// route_device.h -- device code of the token-choice router shared by the
// routing kernels (route.hip) and the fused decode front (decode.hip):
// matrix-core router logits by tile, the stable scatter, and the whole
// routing of a few tokens in one block.  See route.hip for the method.
#pragma once

#include "device_common.h"

namespace moe {

constexpr int kChunkTokens = 16;   // tokens per top-k / histogram chunk (one per wavefront)
constexpr int kFinishMaxPairs = 512;  // pairs the single-block finish kernel handles
constexpr int kMaxK = 8;
constexpr int kMaxE = 256;

// Router logits on the matrix cores.  Each fp32 router weight is split
// exactly into three bf16 terms by truncation, w = hi + mid + lo: hi keeps
// the top 16 bits of w, mid the top 16 bits of the (exact) residual, and lo
// the remaining at most 8 significant bits.  The activations are bf16, so the
// three 16x16x32 bf16 products accumulate x . w with fp32 rounding only.
// Grid: (16 * NE)-expert tiles x (16 * TT)-token tiles x S slices of the
// contraction; each block's 4 wavefronts split its slice further and are
// summed through LDS in a fixed order.  Slice s writes its partial tile to
// P[s]; slice 0 adds the bias.  The top-k kernel sums the S slices in order.
// A block's NE expert tiles share its activation loads (x is read once per
// expert tile group, not once per 16 experts); the operands of KB K-steps
// are loaded together, one group of KB steps ahead of their products.
constexpr int kRouterWaves = 4;

__device__ __forceinline__ void split3_bf16(const float (&w)[8], bf16x8_t& hi, bf16x8_t& mid,
                                            bf16x8_t& lo) {
    u32x4_t h, md, l;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        uint32_t hb[2], mb[2], lb[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t u = __builtin_bit_cast(uint32_t, w[2 * p + q]);
            hb[q] = u & 0xFFFF0000u;
            const uint32_t r1 = __builtin_bit_cast(uint32_t, w[2 * p + q] - __builtin_bit_cast(float, hb[q]));
            mb[q] = r1 & 0xFFFF0000u;
            lb[q] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, r1) - __builtin_bit_cast(float, mb[q]));
        }
        h[p] = (hb[0] >> 16) | hb[1];
        md[p] = (mb[0] >> 16) | mb[1];
        l[p] = (lb[0] >> 16) | (lb[1] & 0xFFFF0000u);
    }
    hi = as_bf16x8(h);
    mid = as_bf16x8(md);
    lo = as_bf16x8(l);
}

// One router tile: tile (bx, by, bz) of the grid above, computed by
// wavefronts 0 .. kRouterWaves - 1 of the calling block; red is LDS of
// kRouterWaves * NE * TT * 64 f32x4.  Contains exactly one block barrier.
template <int TT, int NE, int KB, bool kPipe>
__device__ __forceinline__ void router_logits_tile(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ br,
    float* __restrict__ P, int T, int D, int E, int S, int bx, int by, int bz, f32x4_t* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int e0 = bx * 16 * NE, t0 = by * 16 * TT, sl = bz;
    const int nk = D / 32;
    const int part = sl * kRouterWaves + wave, parts = S * kRouterWaves;
    const int k_beg = (int)((int64_t)nk * part / parts), k_end = (int)((int64_t)nk * (part + 1) / parts);
    const float* wrow[NE];
#pragma unroll
    for (int n = 0; n < NE; ++n) wrow[n] = wr + (int64_t)min(e0 + 16 * n + m, E - 1) * D;
    f32x4_t acc[NE][TT];
#pragma unroll
    for (int n = 0; n < NE; ++n)
#pragma unroll
        for (int u = 0; u < TT; ++u) acc[n][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Operands of KB K-steps at a time.  kPipe: loaded one group ahead of
    // the products (two register sets, fixed by unrolling the loop by two
    // groups); otherwise each group's loads are issued together and then
    // used.  Loads are unconditional: steps past the slice, experts past E
    // and tokens past T load clamped, valid addresses (their products are
    // skipped or their rows never stored), so the compiler never drains the
    // queue at a branch.
    struct Ops {
        float4 wa[KB][NE], wb[KB][NE];
        u32x4_t xv[KB][TT];
    };
    auto load = [&](Ops& o, int kk) {
#pragma unroll
        for (int h = 0; h < KB; ++h) {
            const int off = min(kk + h, k_end - 1) * 32 + 8 * g;
#pragma unroll
            for (int n = 0; n < NE; ++n) {
                o.wa[h][n] = *reinterpret_cast<const float4*>(wrow[n] + off);
                o.wb[h][n] = *reinterpret_cast<const float4*>(wrow[n] + off + 4);
            }
#pragma unroll
            for (int u = 0; u < TT; ++u) {
                const int t = min(t0 + 16 * u + m, T - 1);
                o.xv[h][u] = *reinterpret_cast<const u32x4_t*>(x + (int64_t)t * D + off);
            }
        }
    };
    auto compute = [&](const Ops& o, int kk) {
#pragma unroll
        for (int h = 0; h < KB; ++h) {
            if (kk + h < k_end) {
#pragma unroll
                for (int n = 0; n < NE; ++n) {
                    const float w[8] = {o.wa[h][n].x, o.wa[h][n].y, o.wa[h][n].z, o.wa[h][n].w,
                                        o.wb[h][n].x, o.wb[h][n].y, o.wb[h][n].z, o.wb[h][n].w};
                    bf16x8_t hi, mid, lo;
                    split3_bf16(w, hi, mid, lo);
#pragma unroll
                    for (int u = 0; u < TT; ++u) {
                        const bf16x8_t xb = as_bf16x8(o.xv[h][u]);
                        acc[n][u] = mfma_bf16(hi, xb, acc[n][u]);
                        acc[n][u] = mfma_bf16(mid, xb, acc[n][u]);
                        acc[n][u] = mfma_bf16(lo, xb, acc[n][u]);
                    }
                }
            }
        }
    };
    if (k_beg < k_end) {
        if constexpr (kPipe) {
            Ops A, B;
            load(A, k_beg);
            for (int kk = k_beg; kk < k_end; kk += 2 * KB) {
                load(B, kk + KB);
                compute(A, kk);
                load(A, kk + 2 * KB);
                compute(B, kk + KB);
            }
        } else {
            for (int kk = k_beg; kk < k_end; kk += KB) {
                Ops A;
                if (kk + KB <= k_end) {
                    load(A, kk);
                } else {                                // last group: only the slice's steps
#pragma unroll
                    for (int h = 0; h < KB; ++h) {
                        if (kk + h < k_end) {
                            const int off = (kk + h) * 32 + 8 * g;
#pragma unroll
                            for (int n = 0; n < NE; ++n) {
                                A.wa[h][n] = *reinterpret_cast<const float4*>(wrow[n] + off);
                                A.wb[h][n] = *reinterpret_cast<const float4*>(wrow[n] + off + 4);
                            }
#pragma unroll
                            for (int u = 0; u < TT; ++u) {
                                const int t = min(t0 + 16 * u + m, T - 1);
                                A.xv[h][u] = *reinterpret_cast<const u32x4_t*>(x + (int64_t)t * D + off);
                            }
                        }
                    }
                }
                compute(A, kk);
            }
        }
    }
#pragma unroll
    for (int n = 0; n < NE; ++n)
#pragma unroll
        for (int u = 0; u < TT; ++u) red[(wave * NE * TT + n * TT + u) * 64 + lane] = acc[n][u];
    __syncthreads();
    // lane holds C[expert 4g + r][token m] of each (expert, token) tile
    float* Ps = P + (int64_t)sl * T * E;
    for (int nu = wave; nu < NE * TT; nu += kRouterWaves) {
        const int n = nu / TT, u = nu - n * TT;
        f32x4_t sum = red[nu * 64 + lane];
        for (int w2 = 1; w2 < kRouterWaves; ++w2) sum += red[(w2 * NE * TT + nu) * 64 + lane];
        const int t = t0 + 16 * u + m;
        if (t < T) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ee = e0 + 16 * n + 4 * g + r;
                if (ee < E) Ps[(int64_t)t * E + ee] = sum[r] + ((br && sl == 0) ? br[ee] : 0.f);
            }
        }
    }
}

// (v1, i1) ranks before (v2, i2): larger logit, then lower expert id.
__device__ __forceinline__ bool ranks_before(float v1, int i1, float v2, int i2) {
    return v1 > v2 || (v1 == v2 && i1 < i2);
}

// Exclusive prefix sum of v over the block's threads (up to 16 wavefronts).
__device__ inline int block_exclusive_scan(int v, int* wsum) {
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
__device__ inline void scatter_chunk(const int* ids_lds, int npairs, int pair_base,
                              const int* base_e, int E, int* seg_base,
                              int32_t* __restrict__ sorted, int32_t* __restrict__ pos) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nseg = (npairs + 63) / 64;
    for (int i = threadIdx.x; i < nseg * kMaxE; i += blockDim.x) seg_base[i] = 0;
    __syncthreads();
    const int nwaves = blockDim.x >> 6;
    int my_e[2], my_rank[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int g = wave + nwaves * r;
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
        const int g = wave + nwaves * r;
        if (g < nseg && my_e[r] < kMaxE) {
            const int idx = g * 64 + lane;
            const int dest = seg_base[g * kMaxE + my_e[r]] + my_rank[r];
            sorted[dest] = pair_base + idx;
            pos[pair_base + idx] = dest;
        }
    }
}

// Few tokens (T <= kSmallTokens, T E <= kSmallLogits): one block of NW
// wavefronts (16 in route_small_kernel, 8 in the fused decode front) does
// the whole routing.
//  1. Sum the router slices of every (token, expert) logit into LDS, 16
//     slice loads in flight per thread (16 slices of one logit, or 4 slices
//     of four logits when S <= 4); rows are padded to E + 1 floats so that
//     lanes reading one expert of different tokens hit different banks.
//  2. Top-k with one lane per token: wavefront w keeps the best (logit, id)
//     of its slice of experts in registers (insertion into a sorted list of
//     k rounded up to a power of two; larger logit first, then lower id), and
//     the NW lists are merged pairwise through LDS (16 -> 8 -> 4 -> 2 -> 1).
//     The order of the selections is the same total order as repeated
//     argmax.
//  3. Softmax over the k, histogram, scan and stable scatter.
constexpr int kSmallTokens = 64;
constexpr int kSmallLogits = 8192;

// Insert (v, e) into the sorted K-list (bv, bi).
template <int K>
__device__ __forceinline__ void topk_insert(float (&bv)[K], int (&bi)[K], float v, int e) {
#pragma unroll
    for (int s = 0; s < K; ++s) {
        const bool b = ranks_before(v, e, bv[s], bi[s]);
        const float tv = b ? bv[s] : v;
        const int ti = b ? bi[s] : e;
        bv[s] = b ? v : bv[s];
        bi[s] = b ? e : bi[s];
        v = tv;
        e = ti;
    }
}

// (av, ai) = the best K of two lists sorted best first (K a power of two):
// picking the better of a[s] and b[K-1-s] leaves the best K as a bitonic
// sequence, which log2 K compare-exchange stages sort.
template <int K>
__device__ __forceinline__ void topk_merge(float (&av)[K], int (&ai)[K], const float (&bv)[K],
                                           const int (&bi)[K]) {
#pragma unroll
    for (int s = 0; s < K; ++s) {
        const bool b = ranks_before(bv[K - 1 - s], bi[K - 1 - s], av[s], ai[s]);
        av[s] = b ? bv[K - 1 - s] : av[s];
        ai[s] = b ? bi[K - 1 - s] : ai[s];
    }
#pragma unroll
    for (int st = K / 2; st >= 1; st >>= 1) {
#pragma unroll
        for (int s = 0; s < K; ++s) {
            if ((s & st) == 0) {
                const int u = s + st;
                const bool b = ranks_before(av[u], ai[u], av[s], ai[s]);
                const float tv = av[s];
                const int ti = ai[s];
                av[s] = b ? av[u] : av[s];
                ai[s] = b ? ai[u] : ai[s];
                av[u] = b ? tv : av[u];
                ai[u] = b ? ti : ai[u];
            }
        }
    }
}

// Sum the S router slices (S <= kSP) of logits tid, tid + blockDim.x, ...
// of P [S][n] into lg (row t at t (E + 1)) and logits_out.  kU logits per
// round with kU * kSP = 16 loads, all issued before any is used: out-of-range
// slices and logits load a valid address and are discarded (no branches
// around the loads).
template <int kSP>
__device__ __forceinline__ void sum_router_slices(const float* __restrict__ P, int S, int n,
                                                  int E, float* lg,
                                                  float* __restrict__ logits_out) {
    constexpr int kU = 16 / kSP;
    const int tid = threadIdx.x;
    for (int i0 = tid; i0 < n; i0 += kU * blockDim.x) {
        float part[kU][kSP];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int i = min(i0 + u * (int)blockDim.x, n - 1);
#pragma unroll
            for (int sp = 0; sp < kSP; ++sp) part[u][sp] = P[(int64_t)min(sp, S - 1) * n + i];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int i = i0 + u * blockDim.x;
            float acc = part[u][0];
#pragma unroll
            for (int sp = 1; sp < kSP; ++sp) acc = sp < S ? acc + part[u][sp] : acc;
            if (i < n) {
                lg[i + i / E] = acc;
                if (logits_out) logits_out[i] = acc;
            }
        }
    }
}

// LDS of route_small_body
struct SmallRouteLds {
    // logits [T][E + 1], later the merge lists: values [NW / 2][KP][64], ids after them
    float lg[kSmallLogits + kSmallTokens];
    int cnt[kMaxE];
    int pair_e[kSmallTokens * kMaxK];
    int seg_base[8 * kMaxE];
    int base_e[kMaxE];
    int wsum[16];
};

// The whole routing of a few tokens by one block of NW wavefronts (NW = 8 or
// 16; the wavefronts split the experts of the top-k lists, so the
// selections, their order and every output are the same for either).
template <int K, int NW>
__device__ __forceinline__ void route_small_body(
    const float* __restrict__ P, int S, int T, int E, float* __restrict__ logits_out,
    int32_t* __restrict__ ids, float* __restrict__ wts, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted, int32_t* __restrict__ pos,
    SmallRouteLds& L) {
    static_assert(NW == 8 || NW == 16, "wavefronts per block");
    constexpr int k = K;
    constexpr int KP = K <= 1 ? 1 : K <= 2 ? 2 : K <= 4 ? 4 : 8;   // list length, a power of two
    float* lg = L.lg;
    int* cnt = L.cnt;
    int* pair_e = L.pair_e;
    int* seg_base = L.seg_base;
    int* base_e = L.base_e;
    int* wsum = L.wsum;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kMaxE; i += blockDim.x) cnt[i] = 0;
    const int n = T * E;
    if (S <= 4)
        sum_router_slices<4>(P, S, n, E, lg, logits_out);
    else
        sum_router_slices<16>(P, S, n, E, lg, logits_out);
    __syncthreads();

    // 2. top-k, lane = token
    float bv[KP];
    int bi[KP];
#pragma unroll
    for (int s = 0; s < KP; ++s) {
        bv[s] = -__builtin_inff();
        bi[s] = 0x7FFFFFFF;                       // ranks after every real (logit, id)
    }
    const int t = lane;
    {
        const int eg = (E + NW - 1) / NW;
        const int e0 = wave * eg, e1 = min(E, e0 + eg);
        if (t < T)
            for (int e = e0; e < e1; ++e) topk_insert<KP>(bv, bi, lg[t * (E + 1) + e], e);
    }
    float* lv = lg;                               // [NW / 2][KP][64]
    int* li = reinterpret_cast<int*>(lg + (NW / 2) * KP * 64);
    for (int half = NW / 2; half >= 1; half >>= 1) {
        __syncthreads();                          // logits / previous lists no longer read
        if (wave >= half && wave < 2 * half) {
#pragma unroll
            for (int s = 0; s < KP; ++s) {
                lv[((wave - half) * KP + s) * 64 + lane] = bv[s];
                li[((wave - half) * KP + s) * 64 + lane] = bi[s];
            }
        }
        __syncthreads();
        if (wave < half && t < T) {
            float ov[KP];
            int oi[KP];
#pragma unroll
            for (int s = 0; s < KP; ++s) {
                ov[s] = lv[(wave * KP + s) * 64 + lane];
                oi[s] = li[(wave * KP + s) * 64 + lane];
            }
            topk_merge<KP>(bv, bi, ov, oi);
        }
    }
    // 3. softmax over the k selected logits (bv[0] is the largest)
    if (wave == 0 && t < T) {
        float ex[K];
        float den = 0.f;
#pragma unroll
        for (int s = 0; s < K; ++s) {
            ex[s] = expf(bv[s] - bv[0]);
            den += ex[s];
        }
#pragma unroll
        for (int s = 0; s < K; ++s) {
            const int e = bi[s] < E ? bi[s] : E - 1;       // only with non-finite logits
            ids[(int64_t)t * k + s] = e;
            wts[(int64_t)t * k + s] = ex[s] / den;
            pair_e[t * k + s] = e;
        }
    }
    __syncthreads();
    const int npairs = T * k;
    for (int p = tid; p < npairs; p += blockDim.x) atomicAdd(&cnt[pair_e[p]], 1);
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
    scatter_chunk(pair_e, npairs, 0, base_e, E, seg_base, sorted, pos);
}

}  // namespace moe
