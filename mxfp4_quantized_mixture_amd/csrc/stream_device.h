// stream_device.h -- device code of the weight-streaming expert kernels
// (expert_mlp.hip), shared with the fused decode front (decode.hip).
#pragma once

#include <type_traits>

#include "device_common.h"

namespace moe {

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
// tile outputs a wavefront holds in registers until its last load: 8 in the
// streaming kernels (255-256 VGPRs), 6 in the fused decode front (its other
// state would make 8 spill).  Measured at the 120B decode shape (11-12 tiles
// per wavefront): 296.1 us per step with 8 and 297.6 with 6 against 300.3 with 4.
template <bool kFused>
constexpr int kMaxWaveTiles = kFused ? 6 : 8;

// Staged activations.  The weights enter the matrix cores exactly as stored
// (E2M1 codes + E8M0 block scales, v_mfma_scale_f32_16x16x128_f8f6f4 with an
// fp4 A operand), so the activations must be fp8: each activation row is
// split into NT E4M3 terms, term t+1 carrying the exact fp32 rounding
// residual of term t, each with its own E8M0 scale per 32-element block
// (the block's largest magnitude scaled into [128, 256)).  Each term leaves
// at most 2^-4 of an element's remaining magnitude while that lies within 13
// binades of the block's largest, so bf16 x (8 significant bits) is exact
// in 2 terms there and fp32 h keeps a relative error below 2^-12 after 3;
// elements further down keep an absolute error below 2^-21 of the block's
// largest magnitude.  The E8M0 scales reach any fp32 magnitude.
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

// Stage the unit's rows (pairs row0 .. row0 + nvalid - 1 in sorted order;
// gathered bf16 x rows for gate/up, contiguous fp32 h rows for down) as NT
// fp8 terms.  One thread per (row, 32-element block); rows past nvalid and
// blocks past K are zero with scale 2^0.
//
// after_loads() runs once every thread has issued the loads of its first
// (row, block), after_convert() once it has converted it: the caller issues
// its weight prefetch there.  Loads complete in issue order as far as the
// wait counter is concerned, so activation loads issued behind a chip-wide
// weight prefetch would wait for all of it.
// An index another block of the same launch may have just written
// (kCoherent: an agent-scope atomic load, which reads the coherent value
// without invalidating any cache), or a plain load.
template <bool kCoherent>
__device__ __forceinline__ int load_index(const int32_t* p) {
    if constexpr (kCoherent)
        return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        return *p;
}

template <int NT, bool kGather, bool kCoherent = false, typename F, typename G>
__device__ void stage_split(const void* __restrict__ src, const int32_t* __restrict__ sorted,
                            int row0, int nvalid, int k, int K, uint8_t* lds, int* s_row,
                            F&& after_loads, G&& after_convert) {
    if (threadIdx.x < 16)
        s_row[threadIdx.x] = threadIdx.x < nvalid
            ? (kGather ? load_index<kCoherent>(sorted + row0 + threadIdx.x) / k : row0 + threadIdx.x)
            : -1;
    __syncthreads();
    const int nblk = K / 32, nss = (nblk + 3) / 4;
    uint8_t* scales = lds + (size_t)nss * NT * 64 * 32;
    const int ntask = nvalid * nblk;
    // 16-byte loads per 32-element block: bf16 x 4, fp32 h 8
    constexpr int kRaw = kGather ? 4 : 8;
    auto load_task = [&](int task, u32x4_t (&raw)[kRaw]) {
        const int m = task % nvalid, blk = task / nvalid;
        const uint8_t* p = static_cast<const uint8_t*>(src) +
                           ((int64_t)s_row[m] * K + blk * 32) * (kGather ? 2 : 4);
#pragma unroll
        for (int c = 0; c < kRaw; ++c) raw[c] = *reinterpret_cast<const u32x4_t*>(p + 16 * c);
    };
    // Hardware K of element n of block gq is 32 gq + n: lanes 16 * (2 (gq & 1) + n / 16)
    // + m, byte 16 (gq >> 1) + n % 16.
    auto convert_task = [&](int task, const u32x4_t (&raw)[kRaw]) {
        const int m = task % nvalid, blk = task / nvalid;
        const int ss = blk >> 2, gq = blk & 3;
        float v[32];
        if constexpr (kGather) {
#pragma unroll
            for (int c = 0; c < kRaw; ++c) {
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    v[c * 8 + 2 * h] = bf16_to_f32(raw[c][h] & 0xFFFFu);
                    v[c * 8 + 2 * h + 1] = bf16_to_f32(raw[c][h] >> 16);
                }
            }
        } else {
            // (the whole vector is reinterpreted: hipcc miscompiles a
            // bit_cast of a single element of a uint32 vector to float, keeping
            // only part of each load)
#pragma unroll
            for (int c = 0; c < kRaw; ++c) {
                const f32x4_t r = __builtin_bit_cast(f32x4_t, raw[c]);
                v[c * 4] = r[0];
                v[c * 4 + 1] = r[1];
                v[c * 4 + 2] = r[2];
                v[c * 4 + 3] = r[3];
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
    // The loads of the first two rounds of (row, block) tasks are issued
    // before anything else: a round loaded after the caller's weight prefetch
    // would wait for all of it (more than blockDim.x / nblk rows, e.g. 6 or
    // more rows at K = 2880).  Later rounds (12 or more rows at K = 2880) are
    // loaded and converted one after the other.
    u32x4_t first[kRaw], second[kRaw];
    const int task0 = threadIdx.x, task1 = task0 + (int)blockDim.x;
    load_task(task0 < ntask ? task0 : ntask - 1, first);   // unconditional: see after_loads
    if (ntask > (int)blockDim.x)                            // uniform in the block
        load_task(task1 < ntask ? task1 : ntask - 1, second);
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
    if (task1 < ntask) convert_task(task1, second);
    for (int task = task1 + blockDim.x; task < ntask; task += blockDim.x) {
        u32x4_t raw[kRaw];
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
//          epilogue h = silu(g) * u -> fp32.
// else:    A = W2 rows (NS = 1), B = h rows (3 fp8 terms), epilogue y -> fp32
//          (row t k + j for the pair of slot j of token t).
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
//
// kFused (the fused decode front): the block's first weight batch and
// scales are issued before the routing exists; wait_routing() (called by
// every thread) returns true once offsets and sorted have been published,
// false if they never were (the block then exits without reading them); the
// block also exits if its expert has no pairs.  It then reads those indices
// with agent-scope atomic loads, so no cache needs invalidating.  Otherwise the pair range is
// read first and blocks of experts without pairs load nothing.
// vblock is the block's index in the streaming grid; lds_stage (dynamic LDS
// of stream_lds_bytes) and s_row (16 ints) are the block's LDS.
template <bool kGateUp, bool kPacked, bool kFused, typename Wait>
__device__ __forceinline__ void expert_stream_body(
    const void* __restrict__ act, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ ws, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted, int D, int F, int E, int k, int bpe,
    float* __restrict__ out, int vblock, uint8_t* lds_stage, int* s_row, Wait&& wait_routing) {
    constexpr int NS = kGateUp ? 2 : 1;      // row streams per tile, taken in turn
    constexpr int NT = kGateUp ? 2 : 3;
    constexpr int NB = kGateUp ? 8 : 4;      // super-steps per load batch
    // ring depth: two batches of 8 for gate/up, three of 4 for down
    constexpr int kRing = kGateUp ? 2 : 3;
    const int K = kGateUp ? D : F;           // contraction length
    const int NOUT = kGateUp ? F : D;        // output features (per stream)
    const int ntiles = NOUT / 16;
    const int e = vblock / bpe, part = vblock - e * bpe;
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
    if constexpr (kFused) {
        prologue_a();
        if (!wait_routing()) return;
    }
    const int row_beg = load_index<kFused>(offsets + e);
    const int ne = load_index<kFused>(offsets + e + 1) - row_beg;
    if (ne <= 0) return;

    for (int tg = 0; tg < ne; tg += 16) {
        const int row0 = row_beg + tg;
        const int nvalid = min(16, ne - tg);
        if (tg > 0) __syncthreads();           // previous group's rows no longer read
        // Output row of this lane's pair: h in pair (sorted) order, the rows
        // the down kernel reads contiguously; y in slot order (pair p of
        // slot sorted[p] = t k + j at row t k + j), so that the combine finds a
        // token's k rows without the permutation.  (Issued ahead of the group's
        // activation and weight loads, so it is back before any of them is
        // waited for.)
        int orow = row0 + m;
        if constexpr (!kGateUp) orow = sorted[row0 + (m < nvalid ? m : nvalid - 1)];
        // the weight prefetch goes out right behind the first activation loads
        // (fused: the first group's first batch went out before the routing
        // wait, the rest of its ring follows the first conversion as usual)
        stage_split<NT, kGateUp, kFused>(act, sorted, row0, nvalid, k, K, lds_stage, s_row,
                                 [&]() {
                                     if (!kFused || tg > 0) prologue_a();
                                 },
                                 prologue_b);
        lds_barrier();                         // not __syncthreads: the weight loads stay in flight

        f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, acc_gate = {0.f, 0.f, 0.f, 0.f};
        // The first kMaxWaveTiles<kFused> tile results stay in registers until the
        // wave has issued its last load: on gfx9 the vector memory counter
        // also covers stores, so an early store makes later load waits wait
        // for its write too (measured: 1.5 us per launch at 3 tiles per
        // wave).  Further tiles (many tiles per wave, when blocks per expert
        // are few) are stored as soon as they are computed.
        constexpr int kTilesHeld = kMaxWaveTiles<kFused>;
        f32x4_t obuf[kTilesHeld];
        const int ostride = kGateUp ? F : D;
        auto epilogue = [&](int s) {
            const int j = s / seg;
            f32x4_t res;
            if constexpr (kGateUp) {
#pragma unroll
                for (int q = 0; q < 4; ++q) res[q] = silu_f32(acc_gate[q]) * acc[q];
            } else {
                res = acc;
            }
            if (j < kTilesHeld) {
#pragma unroll
                for (int jj = 0; jj < kTilesHeld; ++jj)
                    if (jj == j) obuf[jj] = res;
            } else if (m < nvalid) {
                const int tile = a + wave + j * kStreamWaves;
                *reinterpret_cast<f32x4_t*>(out + (size_t)orow * ostride + tile * 16 + 4 * g) = res;
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
            for (int jj = 0; jj < kTilesHeld; ++jj) {
                if (jj < my_tiles) {
                    const int tile = a + wave + jj * kStreamWaves;
                    *reinterpret_cast<f32x4_t*>(out + (size_t)orow * ostride + tile * 16 + 4 * g) =
                        obuf[jj];
                }
            }
        }
    }
}

// Dynamic LDS of expert_stream_body: staged fp8 terms of 16 rows of K
// elements, ceil(K/128) super-steps x NT terms x 64 lanes x (32 data bytes +
// 1 scale byte), and the wavefronts' committed weight-scale runs.
inline size_t stream_lds_bytes(int K, int NT, int NS) {
    return (size_t)((K / 32 + 3) / 4) * NT * 64 * 33 + (size_t)kStreamWaves * NS * 16 * (K / 32);
}

}  // namespace moe
