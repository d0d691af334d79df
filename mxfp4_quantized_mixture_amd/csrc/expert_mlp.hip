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
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kMaxSS = 6;    // super-steps of activations a wave keeps in registers

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

// ---------------------------------------------------------------------------
// Balanced weight-streaming kernels.
//
// A "unit" is one expert with up to 16 of its tokens (experts with more tokens
// contribute several units).  Work = units x 16-row weight tiles, split evenly
// over the grid; every block builds the unit table from `offsets` itself, so
// no host synchronisation is needed.  For each unit in its range a block
// stages the unit's activation rows in LDS once; each wavefront then owns
// whole tiles over the full contraction dimension (no cross-wave reduction)
// and keeps two batches of weight loads in flight.
// ---------------------------------------------------------------------------

constexpr int kStreamWaves = 8;
constexpr int kMaxWaveTiles = 4;       // tile outputs a wavefront holds in registers

// Staged activations.  The weights enter the matrix cores exactly as stored
// (E2M1 codes + E8M0 block scales, v_mfma_scale_f32_16x16x128_f8f6f4 with an
// fp4 A operand), so the activations must be fp8: each activation row is
// split into NT E4M3 terms, term t+1 carrying the rounding residual of term
// t, each with its own E8M0 scale per 32-element block.  A value with b
// significant bits is represented exactly by ceil(b / 4) terms when it lies
// within 13 binades of its block's largest magnitude (bf16 x: 2 terms;
// fp16 h: 3 terms); smaller elements keep an error below 2^-21 of that
// magnitude.
//
// Operand layouts of the 16x16x128 scaled product (lane l, m = l % 16,
// g = l / 16): A lane holds row m, K = 32 g .. 32 g + 31 (one MXFP4 block,
// low nibble first) and that block's scale; B lane holds column m, bytes
// 0..15 = K 16 g .. 16 g + 15 and bytes 16..31 = K 64 + 16 g .. + 15, and
// the scale of K-block g of column m.  C is as for the 16x16x32 products.
//
// LDS, per unit: data [nss][NT][64 lanes][32 B], then scales [nss][NT][64].

__device__ __forceinline__ f32x4_t mfma_fp4w_fp8x(u32x4_t w, int wscale, const u32x4_t (&b)[2],
                                                 int bscale, f32x4_t c) {
    i32x8_t a8 = {(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
    i32x8_t b8 = {(int)b[0][0], (int)b[0][1], (int)b[0][2], (int)b[0][3],
                  (int)b[1][0], (int)b[1][1], (int)b[1][2], (int)b[1][3]};
    // cbsz = 4: A is fp4 (e2m1); blgp = 0: B is fp8 (e4m3)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 0, 0, wscale, 0, bscale);
}

__device__ __forceinline__ float act_to_f32(uint16_t v, bool is_bf16) {
    return is_bf16 ? __builtin_bit_cast(float, (uint32_t)v << 16)
                   : (float)__builtin_bit_cast(_Float16, v);
}

// Stage the unit's rows (pairs row0 .. row0 + nvalid - 1 in sorted order;
// gathered bf16 x rows for gate/up, contiguous fp16 h rows for down) as NT
// fp8 terms.  One thread per (row, 32-element block); rows past nvalid and
// blocks past K are zero with scale 2^0.
//
// after_loads() runs once every thread has issued the loads of its first
// (row, block), after_convert() once it has converted it: the caller issues
// its weight prefetch there.  Loads complete in issue order as far as the
// wait counter is concerned, so activation loads issued behind a chip-wide
// weight prefetch would wait for all of it.
template <int NT, bool kGather, typename F, typename G>
__device__ void stage_split(const uint16_t* __restrict__ src, const int32_t* __restrict__ sorted,
                            int row0, int nvalid, int k, int K, uint8_t* lds, int* s_row,
                            F&& after_loads, G&& after_convert) {
    if (threadIdx.x < 16)
        s_row[threadIdx.x] = threadIdx.x < nvalid
            ? (kGather ? sorted[row0 + threadIdx.x] / k : row0 + threadIdx.x) : -1;
    __syncthreads();
    const int nblk = K / 32, nss = (nblk + 3) / 4;
    uint8_t* scales = lds + (size_t)nss * NT * 64 * 32;
    const int ntask = nvalid * nblk;
    auto load_task = [&](int task, u32x4_t (&raw)[4]) {
        const int m = task % nvalid, blk = task / nvalid;
        const uint16_t* p = src + (int64_t)s_row[m] * K + blk * 32;
#pragma unroll
        for (int c = 0; c < 4; ++c) raw[c] = *reinterpret_cast<const u32x4_t*>(p + c * 8);
    };
    // Hardware K of element n of block gq is 32 gq + n: lanes 16 * (2 (gq & 1) + n / 16)
    // + m, byte 16 (gq >> 1) + n % 16.
    auto convert_task = [&](int task, const u32x4_t (&raw)[4]) {
        const int m = task % nvalid, blk = task / nvalid;
        const int ss = blk >> 2, gq = blk & 3;
        float v[32];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[c * 8 + 2 * h] = act_to_f32((uint16_t)(raw[c][h] & 0xFFFFu), kGather);
                v[c * 8 + 2 * h + 1] = act_to_f32((uint16_t)(raw[c][h] >> 16), kGather);
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            float amax = 0.f;
#pragma unroll
            for (int n = 0; n < 32; ++n) amax = fmaxf(amax, fabsf(v[n]));
            const int se = fp8_term_exponent(amax);
            const float inv = exp2i_neg(se), sc = exp2i(se);
            uint32_t q[8];
#pragma unroll
            for (int w = 0; w < 8; ++w)
                q[w] = pack4_fp8(v[4 * w] * inv, v[4 * w + 1] * inv, v[4 * w + 2] * inv,
                                 v[4 * w + 3] * inv);
#pragma unroll
            for (int w = 0; w < 8; ++w) sub4_fp8(v + 4 * w, q[w], sc);
            uint8_t* base = lds + ((size_t)(ss * NT + t) * 64) * 32;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int lane = 16 * (2 * (gq & 1) + half) + m;
                u32x4_t w4 = {q[4 * half], q[4 * half + 1], q[4 * half + 2], q[4 * half + 3]};
                *reinterpret_cast<u32x4_t*>(base + lane * 32 + 16 * (gq >> 1)) = w4;
            }
            scales[(ss * NT + t) * 64 + gq * 16 + m] = (uint8_t)(se + 127);
        }
    };
    u32x4_t first[4];
    const int task0 = threadIdx.x;
    load_task(task0 < ntask ? task0 : ntask - 1, first);   // unconditional: see after_loads
    // keeps the caller's loads behind these (and in this loop iteration)
    asm volatile("" ::: "memory");
    // No wavefront issues weight loads before every wavefront has issued its
    // activation loads: the CU's memory pipeline serves requests roughly in
    // issue order, so a late wavefront's activation loads would otherwise
    // queue behind the other wavefronts' prefetches.  (Orders issue only:
    // nothing here waits for a load.)
    lds_barrier();
    after_loads();
    // padding: rows past nvalid (all their blocks) and blocks past K -> zeros,
    // scale 2^0 (disjoint from the live (row, block) entries)
    for (int task = threadIdx.x; task < 16 * nss * 4; task += blockDim.x) {
        const int m = task & 15, blk = task >> 4;
        if (m < nvalid && blk < nblk) continue;
        const int ss = blk >> 2, gq = blk & 3;
        const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            uint8_t* base = lds + ((size_t)(ss * NT + t) * 64) * 32;
#pragma unroll
            for (int half = 0; half < 2; ++half)
                *reinterpret_cast<u32x4_t*>(base + (16 * (2 * (gq & 1) + half) + m) * 32 +
                                            16 * (gq >> 1)) = z;
            scales[(ss * NT + t) * 64 + gq * 16 + m] = 127;
        }
    }
    if (task0 < ntask) convert_task(task0, first);
    after_convert();
    for (int task = task0 + blockDim.x; task < ntask; task += blockDim.x) {
        u32x4_t raw[4];
        load_task(task, raw);
        convert_task(task, raw);
    }
}

template <int NB>
struct WBatch {
    u32x4_t q[NB];
};

// Load NB super-steps (from ss0) of one 16-row weight tile (q: this lane's
// row, see row_base); out-of-range blocks are clamped to the row's last block
// (finite data, multiplied by zero activations).  Block blk of the row is at
// 16 blk, or with packed codes (mxfp4_pack: 32-row fragments, 1 KiB per
// 64-element step, its two 32-element halves 512 bytes apart) at
// 1024 (blk / 2) + 512 (blk % 2) from the row's first piece.
template <int NB, bool kPacked>
__device__ __forceinline__ void load_batch(WBatch<NB>& B, const uint8_t* q, int ss0, int g,
                                           int nblk) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        int blk = (ss0 + i) * 4 + g;
        blk = blk < nblk ? blk : nblk - 1;
        const int off = kPacked ? (blk >> 1) * 1024 + (blk & 1) * 512 : blk * 16;
        B.q[i] = *reinterpret_cast<const u32x4_t*>(q + off);
    }
}

// Where weight row `row` (of a matrix with rowbytes bytes per row) starts for
// load_batch: the row itself, or with packed codes its first 16-byte piece in
// the first chunk of its 32-row fragment (a fragment's first byte is the same
// in both layouts).
template <bool kPacked>
__device__ __forceinline__ const uint8_t* row_base(const uint8_t* q, size_t row, size_t rowbytes) {
    return kPacked ? q + (row & ~(size_t)31) * rowbytes + (row & 31) * 16 : q + row * rowbytes;
}

// The E8M0 scales of a 16-row weight tile are one contiguous 16 * nblk-byte
// run of the [rows, K/32] scale array (16-byte aligned).  A wavefront fetches
// the next tile's runs into registers while it streams the current tile, and
// commits them to its own LDS buffer at the tile switch.
constexpr int kScaleChunks = 2;        // 16-byte chunks per lane: K <= 4096

template <int NS>
struct ScaleRegs {
    u32x4_t v[NS][kScaleChunks];
};

template <int NS>
__device__ __forceinline__ void fetch_scales(ScaleRegs<NS>& S, const uint8_t* const (&run)[NS],
                                             int lane, int nblk) {
#pragma unroll
    for (int r = 0; r < NS; ++r)
#pragma unroll
        for (int c = 0; c < kScaleChunks; ++c) {
            const int idx = lane + 64 * c;    // 16-byte chunk of the 16 * nblk-byte run
            // unconditional (chunks past the run reload its last one): a load
            // under a branch makes the compiler's later waits drain the queue
            S.v[r][c] = *reinterpret_cast<const u32x4_t*>(run[r] + (idx < nblk ? idx : nblk - 1) * 16);
        }
}

template <int NS>
__device__ __forceinline__ void commit_scales(const ScaleRegs<NS>& S, uint8_t* buf, int lane,
                                              int nblk) {
#pragma unroll
    for (int r = 0; r < NS; ++r)
#pragma unroll
        for (int c = 0; c < kScaleChunks; ++c) {
            const int idx = lane + 64 * c;
            if (idx < nblk) *reinterpret_cast<u32x4_t*>(buf + r * 16 * nblk + idx * 16) = S.v[r][c];
        }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// acc += this batch's NB super-steps of the tile times the staged terms;
// wsc is this lane's row of the tile's committed scale run.
template <int NB, int NT>
__device__ __forceinline__ void compute_batch(const WBatch<NB>& B, int ss0, int nss,
                                              const uint8_t* lds, const uint8_t* lds_scales,
                                              const uint8_t* wsc, int lane, int g, int nblk,
                                              f32x4_t& acc) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int ss = ss0 + i;
        if (ss < nss) {
            int blk = ss * 4 + g;
            blk = blk < nblk ? blk : nblk - 1;
            const int wscale = wsc[blk];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint8_t* frag = lds + ((size_t)(ss * NT + t) * 64 + lane) * 32;
                u32x4_t bx[2];
                bx[0] = *reinterpret_cast<const u32x4_t*>(frag);
                bx[1] = *reinterpret_cast<const u32x4_t*>(frag + 16);
                const int bs = lds_scales[(ss * NT + t) * 64 + lane];
                acc = mfma_fp4w_fp8x(B.q[i], wscale, bx, bs, acc);
            }
        }
    }
}

// kGateUp: A = [gate rows; up rows] of W13 (NS = 2), B = x rows (2 fp8 terms),
//          epilogue h = silu(g) * u -> fp16.
// else:    A = W2 rows (NS = 1), B = h rows (3 fp8 terms), epilogue y -> fp32.
//
// A wavefront streams one weight row range at a time: for each of its tiles
// the gate rows over the whole contraction, then the up rows (the gate sums
// wait in registers).  Two concurrent row streams per wavefront, 4 MB apart,
// sustain measurably less HBM bandwidth than one.
//
// Block b streams a fixed range of 16-row tiles of expert b / bpe.  It reads
// the expert's pair range, issues the loads of the first activation rows and
// only then its first weight batches, so the activation staging overlaps the
// weight stream instead of queueing behind it.  The expert's pairs are taken
// 16 at a time (one pass over the tiles per group of 16; decode steps have
// one group); blocks of experts without pairs exit before loading anything.
template <bool kGateUp, bool kPacked>
__global__ __launch_bounds__(kStreamWaves * 64) void expert_stream_kernel(
    const uint16_t* __restrict__ act, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ ws, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted, int D, int F, int E, int k, int bpe,
    void* __restrict__ out) {
    constexpr int NS = kGateUp ? 2 : 1;      // row streams per tile, taken in turn
    constexpr int NT = kGateUp ? 2 : 3;
    constexpr int NB = kGateUp ? 8 : 4;      // super-steps per load batch
    // ring depth: two batches of 8 for gate/up, three of 4 for down
    constexpr int kRing = kGateUp ? 2 : 3;
    extern __shared__ __align__(16) uint8_t lds_stage[];
    __shared__ int s_row[16];
    const int K = kGateUp ? D : F;           // contraction length
    const int NOUT = kGateUp ? F : D;        // output features (per stream)
    const int ntiles = NOUT / 16;
    const int e = blockIdx.x / bpe, part = blockIdx.x - e * bpe;
    const int a = (int)((int64_t)ntiles * part / bpe), b = (int)((int64_t)ntiles * (part + 1) / bpe);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int nblk = K / 32, nss = (nblk + 3) / 4, nbt = (nss + NB - 1) / NB;
    const int seg = NS * nbt;                // steps (load batches) per tile
    const size_t rowbytes = (size_t)K / 2;
    const uint8_t* lds_scales = lds_stage + (size_t)nss * NT * 64 * 32;
    uint8_t* wave_sc = lds_stage + (size_t)nss * NT * 64 * 33 + (size_t)wave * NS * 16 * nblk;
    const uint8_t* wsc = wave_sc + m * nblk;        // this lane's row of the committed run
    const int my_tiles = a + wave < b ? (b - a - wave + kStreamWaves - 1) / kStreamWaves : 0;
    const int steps = my_tiles * seg;
    const uint8_t* qe = wq + (size_t)e * (kGateUp ? 2 * F : D) * rowbytes;
    const uint8_t* se = ws + (size_t)e * (kGateUp ? 2 * F : D) * nblk;

    // (a wavefront without tiles prefetches the block's last tile, so every
    // load is in bounds and unconditional)
    auto tile_at = [&](int j) { return min(a + wave + j * kStreamWaves, b - 1); };
    auto row_of = [&](int s) {
        const int tile = tile_at(s / seg);
        const int r = NS == 1 ? 0 : (s / nbt) % NS;   // up rows follow the F gate rows
        return row_base<kPacked>(qe, (size_t)(r * F + tile * 16 + m), rowbytes);
    };
    auto runs_of = [&](int tile, const uint8_t* (&run)[NS]) {
#pragma unroll
        for (int r = 0; r < NS; ++r) run[r] = se + (size_t)(r * F + tile * 16) * nblk;
    };
    // Ring of weight batches.  Prefetches are unconditional (steps past
    // the end reload the last step's lines, which are cache hits) so the
    // compiler never has to drain the load queue at a branch; only the
    // compute is predicated.
    const int last = steps > 0 ? steps - 1 : 0;
    auto fetch = [&](WBatch<NB>& W, int s) {
        const int sc_ = s < last ? s : last;
        load_batch<NB, kPacked>(W, row_of(sc_), (sc_ % nbt) * NB, g, nblk);
    };
    WBatch<NB> B0, B1, B2;
    ScaleRegs<NS> SR;
    // The first tile's scales and weight batch go out with the activation
    // loads; the rest of the ring once this wavefront has converted its
    // first activation block (a wavefront issuing its whole ring first stalls
    // in load issue and holds up the staging barrier).
    auto prologue_a = [&]() {
        const uint8_t* run[NS];
        runs_of(tile_at(0), run);
        fetch_scales<NS>(SR, run, lane, nblk);
        fetch(B0, 0);
    };
    auto prologue_b = [&]() {
        fetch(B1, 1);
        if constexpr (kRing == 3) fetch(B2, 2);
    };
    const int row_beg = offsets[e], ne = offsets[e + 1] - row_beg;
    if (ne <= 0) return;

    for (int tg = 0; tg < ne; tg += 16) {
        const int row0 = row_beg + tg;
        const int nvalid = min(16, ne - tg);
        if (tg > 0) __syncthreads();           // previous group's rows no longer read
        // the weight prefetch goes out right behind the first activation loads
        stage_split<NT, kGateUp>(act, sorted, row0, nvalid, k, K, lds_stage, s_row, prologue_a,
                                 prologue_b);
        lds_barrier();                         // not __syncthreads: the weight loads stay in flight

        f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, acc_gate = {0.f, 0.f, 0.f, 0.f};
        // The first kMaxWaveTiles tile results stay in registers until the
        // wave has issued its last load: on gfx9 the vector memory counter
        // also covers stores, so an early store makes later load waits wait
        // for its write too (measured: 1.5 us per launch at 3 tiles per
        // wave).  Further tiles (many tiles per wave, when blocks per expert
        // are few) are stored as soon as they are computed.
        typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4_t;
        typedef typename std::conditional<kGateUp, f16x4_t, f32x4_t>::type OutT;
        OutT obuf[kMaxWaveTiles];
        auto epilogue = [&](int s) {
            const int j = s / seg;
            OutT res;
            if constexpr (kGateUp) {
#pragma unroll
                for (int q = 0; q < 4; ++q) res[q] = (_Float16)(silu_f32(acc_gate[q]) * acc[q]);
            } else {
                res = acc;
            }
            if (j < kMaxWaveTiles) {
#pragma unroll
                for (int jj = 0; jj < kMaxWaveTiles; ++jj)
                    if (jj == j) obuf[jj] = res;
            } else if (m < nvalid) {
                const int tile = a + wave + j * kStreamWaves;
                if constexpr (kGateUp)
                    *reinterpret_cast<OutT*>(static_cast<_Float16*>(out) + (size_t)(row0 + m) * F +
                                             tile * 16 + 4 * g) = res;
                else
                    *reinterpret_cast<OutT*>(static_cast<float*>(out) + (size_t)(row0 + m) * D +
                                             tile * 16 + 4 * g) = res;
            }
        };
        auto consume = [&](const WBatch<NB>& W, int s) {
            if (s % seg == 0) {               // tile switch: commit its scales, fetch the next's
                commit_scales<NS>(SR, wave_sc, lane, nblk);
                const int nxt = s + seg < steps ? s + seg : s;
                const uint8_t* run[NS];
                runs_of(tile_at(nxt / seg), run);
                fetch_scales<NS>(SR, run, lane, nblk);
            }
            const int r = NS == 1 ? 0 : (s / nbt) % NS;
            compute_batch<NB, NT>(W, (s % nbt) * NB, nss, lds_stage, lds_scales,
                                  wsc + r * 16 * nblk, lane, g, nblk, acc);
            if (s % nbt == nbt - 1) {         // end of a row range
                if (kGateUp && r == 0) {
                    acc_gate = acc;           // gate sums wait for the up rows
                } else {
                    epilogue(s);
                }
                acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        };
        for (int s = 0; s < steps; s += kRing) {
            consume(B0, s);
            fetch(B0, s + kRing);
            if (s + 1 < steps) consume(B1, s + 1);
            fetch(B1, s + 1 + kRing);
            if constexpr (kRing == 3) {
                if (s + 2 < steps) consume(B2, s + 2);
                fetch(B2, s + 5);
            }
        }
        if (m < nvalid) {
#pragma unroll
            for (int jj = 0; jj < kMaxWaveTiles; ++jj) {
                if (jj < my_tiles) {
                    const int tile = a + wave + jj * kStreamWaves;
                    if constexpr (kGateUp)
                        *reinterpret_cast<OutT*>(static_cast<_Float16*>(out) + (size_t)(row0 + m) * F +
                                                 tile * 16 + 4 * g) = obuf[jj];
                    else
                        *reinterpret_cast<OutT*>(static_cast<float*>(out) + (size_t)(row0 + m) * D +
                                                 tile * 16 + 4 * g) = obuf[jj];
                }
            }
        }
    }
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

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

constexpr size_t kMaxStreamLds = 158 * 1024;   // of 160 KiB, leaving room for static LDS

// Staged fp8 terms of 16 rows of K elements: ceil(K/128) super-steps x NT
// terms x 64 lanes x (32 data bytes + 1 scale byte).
static size_t stream_lds_bytes(int K, int NT, int NS) {
    return (size_t)((K / 32 + 3) / 4) * NT * 64 * 33 + (size_t)kStreamWaves * NS * 16 * (K / 32);
}

MlpPlan plan_mlp(int T, int D, int F, int E, int k) {
    MlpPlan p{};
    p.T = T; p.D = D; p.F = F; p.E = E; p.k = k;
    const size_t P = (size_t)T * k;
    // (the grouped GEMM addresses its buffers with 32-bit byte offsets)
    const size_t k4G = (size_t)1 << 32;
    p.gemm_ok = D % 64 == 0 && F % 64 == 0 && D <= kGemmMaxContraction &&
                F <= kGemmMaxContraction && gemm_lds_bytes(D, true, 1, 4) <= kGemmMaxLds &&
                gemm_lds_bytes(F, false, 1, 4) <= kGemmMaxLds && gemm_term_bytes(T, D, 2) < k4G &&
                P * F * sizeof(_Float16) < k4G && (size_t)E * F * D < k4G;
    // Weight streaming reads every touched expert's weights once per 16 of its
    // pairs; the grouped GEMM stages 128-pair tiles.  Switch once the average
    // expert receives 32 pairs.
    p.gemm_auto = p.gemm_ok && P >= (size_t)32 * E;
    p.stream_ok = stream_lds_bytes(D, 2, 2) <= kMaxStreamLds &&
                  stream_lds_bytes(F, 3, 1) <= kMaxStreamLds && D <= 4096 && F <= 4096;
    p.packed_ok = p.gemm_ok && p.stream_ok;
    p.max_tiles = gemm_max_tiles(T, E, k);
    p.off_y = 0;
    const size_t scratch = align256(P * D * sizeof(float));
    p.off_h = scratch;                         // h [P, F] fp16, both algorithms
    const size_t h_end = align256(p.off_h + P * F * sizeof(_Float16));
    size_t gemm_end = h_end;
    if (p.gemm_ok) {
        p.off_xq = h_end;
        p.off_tiles = align256(p.off_xq + gemm_term_bytes(T, D, 2));
        gemm_end = align256(p.off_tiles + sizeof(int32_t) * (2 * (size_t)p.max_tiles + 1));
    }
    p.ws_bytes = gemm_end;
    return p;
}

// Blocks per expert for the streaming kernels: about 256 blocks in all (one
// per CU of MI355X, so every block runs in the first round) and at least 2
// per expert, so untouched experts' CUs are reused by the dispatcher; at
// least 8 tiles (one per wavefront) per block where possible.
static int stream_blocks_per_expert(int E, int ntiles) {
    int bpe = (256 + E - 1) / E;
    if (bpe < 2) bpe = 2;
    if (bpe > ntiles / kStreamWaves) bpe = ntiles / kStreamWaves;
    return bpe < 1 ? 1 : bpe;
}

static int blocks_per_expert(int E, int ntiles) {
    int bpe = (2048 + E - 1) / E;
    if (bpe > ntiles) bpe = ntiles;
    return bpe < 1 ? 1 : bpe;
}

static hipError_t launch_combine(const MlpPlan& p, const float* y, const float* topk_w,
                                 const int32_t* pos, uint16_t* out, hipEvent_t* events,
                                 hipStream_t stream);

// One streaming pass: gate/up (kGateUp, K = D, F output rows per expert) or
// down (K = F, D output rows), blocks sized by stream_blocks_per_expert.
template <bool kGateUp, bool kPacked>
static hipError_t launch_stream(const MlpPlan& p, const void* act, const uint8_t* wq,
                                const uint8_t* ws_, const int32_t* offsets,
                                const int32_t* sorted, void* out, hipStream_t stream) {
    const size_t lds = kGateUp ? stream_lds_bytes(p.D, 2, 2) : stream_lds_bytes(p.F, 3, 1);
    const int bpe = stream_blocks_per_expert(p.E, (kGateUp ? p.F : p.D) / 16);
    if (lds > 65536) {
        const hipError_t er =
            hipFuncSetAttribute(reinterpret_cast<const void*>(&expert_stream_kernel<kGateUp, kPacked>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (er != hipSuccess) return er;
    }
    hipLaunchKernelGGL((expert_stream_kernel<kGateUp, kPacked>), dim3(p.E * bpe),
                       dim3(kStreamWaves * 64), lds, stream,
                       reinterpret_cast<const uint16_t*>(act), wq, ws_, offsets, sorted, p.D,
                       p.F, p.E, p.k, bpe, out);
    return hipSuccess;
}

hipError_t launch_mlp(const MlpPlan& p, int algo, bool packed, const uint16_t* x,
                      const uint8_t* w13q, const uint8_t* w13s, const uint8_t* w2q,
                      const uint8_t* w2s, const float* topk_w, const int32_t* offsets,
                      const int32_t* sorted, const int32_t* pos, uint16_t* out, void* ws,
                      hipEvent_t* events, hipStream_t stream) {
    char* base = static_cast<char*>(ws);
    _Float16* h = reinterpret_cast<_Float16*>(base + p.off_h);
    float* y = reinterpret_cast<float*>(base + p.off_y);
    const bool gemm = algo == 2 || (algo == 0 && p.gemm_auto);
    if (gemm) {
        const hipError_t er = launch_mlp_gemm(p, packed, x, w13q, w13s, w2q, w2s, offsets, sorted,
                                              y, base, events, stream);
        if (er != hipSuccess) return er;
        return launch_combine(p, y, topk_w, pos, out, events, stream);
    }
    if (events) {
        const hipError_t er = hipEventRecord(events[0], stream);
        if (er != hipSuccess) return er;
    }
    if (p.stream_ok) {
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
    } else {
        const int bpe1 = blocks_per_expert(p.E, p.F / 16);
        hipLaunchKernelGGL(gateup_stream_kernel, dim3(p.E * bpe1), dim3(256), 0, stream, x, w13q,
                           w13s, offsets, sorted, p.D, p.F, p.k, bpe1, h);
        if (events) {
            const hipError_t er = hipEventRecord(events[1], stream);
            if (er != hipSuccess) return er;
        }
        const int bpe2 = blocks_per_expert(p.E, p.D / 16);
        hipLaunchKernelGGL(down_stream_kernel, dim3(p.E * bpe2), dim3(256), 0, stream, h, w2q,
                           w2s, offsets, p.D, p.F, bpe2, y);
    }
    return launch_combine(p, y, topk_w, pos, out, events, stream);
}

static hipError_t launch_combine(const MlpPlan& p, const float* y, const float* topk_w,
                                 const int32_t* pos, uint16_t* out, hipEvent_t* events,
                                 hipStream_t stream) {
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
