// expert_gemm.hip -- the expert MLP as two tiled grouped GEMMs, for batches in
// which experts receive many tokens (prefill), gfx950.
//
// The layer is the one of the weight-streaming kernels ("Welcome GPT OSS",
// section 4: SwiGLU experts; "Tricks", section 8: GEMMs that understand the
// 32-element blocks and their scales).  For each expert e with token rows X_e
// (its routed pairs in sorted order):  [G | U] = X_e W13_e^T,
// H = silu(G) * U,  Y = H W2_e^T;  the weighted combine follows.
//
// Gate/up: v_mfma_scale_f32_32x32x64_f8f6f4.  The MXFP4 weights are its A
// operand exactly as stored (E2M1 codes, E8M0 block scales as the hardware
// scale operand); x is its B operand as 2 fp8 (E4M3) residual terms with their
// own E8M0 block scales, which is exact for bf16.  The epilogue writes
// h = silu(g) * u as fp16 rows.
//
// Down: v_mfma_f32_32x32x16_f16 on h (fp16, as stored) and the W2 codes
// converted to fp16 in registers (v_cvt_scalef32_pk_f16_fp4, one conversion
// per code per tile).  A W2 row's codes are converted with the scales
// 2^(b - bmax + 13), b the block's scale byte and bmax the row's largest, so
// every code of a block within 36 binades of the row's largest is exact in
// fp16 (at most 6 * 2^13); the row's fp32 sums are then scaled by
// 2^(bmax - 140).  Codes of blocks further below keep fp16's rounding, an
// error under 2^-37 of the row's largest weight.
//
// Operand layouts (lane l, n = l % 32, g = l / 32):
//   32x32x64 f8f6f4:
//     A: row n, K = 32 g .. 32 g + 31 (one MXFP4 block, low nibble first) in
//        the first 16 bytes; scale = that block's E8M0 byte.
//     B: column n, bytes 0..15 = K 16 g .. 16 g + 15, bytes 16..31 =
//        K 32 + 16 g .. + 15; scale = K-block g of column n.
//   32x32x16 f16: A row n / B column n, elements 8 g .. 8 g + 7.  A lane's
//     16 code bytes (K = 32 g .. 32 g + 31 of a 64-wide step) feed four
//     products, product j taking elements 32 g + 8 j .. + 7; the h operand is
//     read in the same order.
//   C (both): element i = row 8 (i / 4) + 4 g + i % 4, column n.
//
// Activation term rows (x).  A row of K elements (K % 64 == 0) is S = K / 64
// steps of term_chunk(NT) = NT * 64 + 16 bytes.  Term t's 64 codes sit at
// 64 t in B operand order: [lane group 0: elements 0..15 of block 2s,
// elements 0..15 of block 2s+1][lane group 1: elements 16..31 of block 2s,
// 16..31 of block 2s+1]; byte NT * 64 + 2 t + h holds the E8M0 scale of term
// t of block 2s + h (the rest of the last 16 bytes is padding).  Codes and
// scales of a step travel together, so staging a step is one contiguous copy
// per row.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kGemmRows = 128;      // routed pairs per tile: 4 fragments of 32
constexpr int kXcds = 8;            // MI355X: 8 accelerator complex dies, one L2 each
// Wavefront layouts (row groups x pair groups), measured on the 20B-shaped
// prefill: gate/up 2 x 2 (two blocks per CU), down 4 x 2 (one block of 8).
constexpr int kScaleIters = 8;      // weight-scale copy: K <= 64 lanes x 16 bytes x 8
static_assert(64 * 16 * kScaleIters == kGemmMaxContraction, "scale copy covers every K");

__host__ __device__ constexpr int term_chunk(int NT) { return NT * 64 + 16; }
// LDS row pitch of a 64-element fp16 h step: 128 bytes plus a 16-byte pad
// (an odd number of 16-byte units keeps the operand reads conflict free)
constexpr int kHPitch = 144;

// Direct global -> LDS load of 16 bytes per lane: lane l's 16 bytes at
// base + voff land at LDS byte lds_base + 16 l (lds_base wave-uniform).
// Issued as an opaque instruction so the compiler does not order later LDS
// reads behind it (it cannot tell that they read other buffers); callers
// wait for it with wait_vm_all() before the barrier that publishes the data.
// It writes no registers (m0, which holds the LDS destination, is restored),
// and an untracked memory operation can only make the compiler's own
// memory-counter waits stricter.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, const uint8_t* lds_dst) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_dst);
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(m0v), "v"(voff), "s"(base));
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt not waited for)
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): all but the N most recently issued vector-memory
// operations have completed (the count is kept in issue order)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>)
template <int N, typename Fn, int... I>
__device__ __forceinline__ void static_for_impl(Fn&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------------------
// bf16 rows -> NT fp8 term rows.  One thread per (row, 64-element step).
// ---------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(256) void split_terms_kernel(const uint16_t* __restrict__ src,
                                                          int rows, int K,
                                                          uint8_t* __restrict__ tq) {
    const int S = K / 64;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)rows * S) return;
    const int row = (int)(idx / S), s = (int)(idx - (int64_t)row * S);
    const uint16_t* p = src + (size_t)row * K + (size_t)s * 64;
    uint8_t* o = tq + ((size_t)row * S + s) * term_chunk(NT);
    uint32_t sc_bytes[2] = {0u, 0u};
    // the whole 128-byte step is loaded before any of it is converted
    u32x4_t raws[2][4];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            raws[hb][c] = *reinterpret_cast<const u32x4_t*>(p + hb * 32 + c * 8);
    __builtin_amdgcn_sched_barrier(0);                   // (keep the loads together)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        float v[32];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4_t raw = raws[hb][c];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[c * 8 + 2 * h] = bf16_to_f32(raw[h] & 0xFFFFu);
                v[c * 8 + 2 * h + 1] = bf16_to_f32(raw[h] >> 16);
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
            const int se = fp8_term_exponent(amax);
            const float inv = exp2i_neg(se), sc = exp2i(se);
            uint32_t q[8];
#pragma unroll
            for (int w = 0; w < 8; ++w)
                q[w] = pack4_fp8(v[4 * w] * inv, v[4 * w + 1] * inv, v[4 * w + 2] * inv,
                                 v[4 * w + 3] * inv);
            if (t + 1 < NT) {
#pragma unroll
                for (int w = 0; w < 8; ++w) sub4_fp8(v + 4 * w, q[w], sc);
            }
            *reinterpret_cast<u32x4_t*>(o + t * 64 + 16 * hb) = u32x4_t{q[0], q[1], q[2], q[3]};
            *reinterpret_cast<u32x4_t*>(o + t * 64 + 32 + 16 * hb) = u32x4_t{q[4], q[5], q[6], q[7]};
            const int byte = 2 * t + hb;
            sc_bytes[byte >> 2] |= (uint32_t)(se + 127) << (8 * (byte & 3));
        }
    }
    *reinterpret_cast<u32x4_t*>(o + NT * 64) = u32x4_t{sc_bytes[0], sc_bytes[1], 0u, 0u};
}

// ---------------------------------------------------------------------------
// Tile table: expert e's pairs [offsets[e], offsets[e+1]) in tiles of
// kGemmRows, experts in order.  tiles[2 i] = first sorted row of tile i,
// tiles[2 i + 1] = e | rows << 16; tiles[2 max_tiles] = number of tiles.
// One block of 256 threads (E <= 256).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm_tiles_kernel(const int32_t* __restrict__ offsets,
                                                         int E, int max_tiles,
                                                         int32_t* __restrict__ tiles) {
    __shared__ int part[256];
    const int e = threadIdx.x;
    const int beg = e < E ? offsets[e] : 0;
    const int ne = e < E ? offsets[e + 1] - beg : 0;
    const int c = (ne + kGemmRows - 1) / kGemmRows;
    part[e] = c;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {        // inclusive scan
        const int v = e >= d ? part[e - d] : 0;
        __syncthreads();
        part[e] += v;
        __syncthreads();
    }
    const int first = part[e] - c;
    for (int j = 0; j < c && first + j < max_tiles; ++j) {
        const int rows = min(kGemmRows, ne - j * kGemmRows);
        tiles[2 * (first + j)] = beg + j * kGemmRows;
        tiles[2 * (first + j) + 1] = e | (rows << 16);
    }
    if (e == 255) tiles[2 * max_tiles] = min(part[255], max_tiles);
}

// ---------------------------------------------------------------------------
// Grouped GEMM.  Block = one tile of kGemmRows pairs x one column range of
// output fragments (32 outputs each).  WR row groups x WP pair groups of
// wavefronts; each owns 128 / WP pairs (NB = 4 / WP B fragments) and
// kWaveFrags output fragments:
//   gate/up (4 x 1, two blocks per CU): 1 feature fragment -> 2 A
//            fragments (its gate and up rows) x all 4 pair fragments (no
//            two wavefronts load the same weights), epilogue h = silu(g) * u
//            written as fp16 rows;
//   down (8 x 1, one block per CU): 2 output fragments -> 2 A fragments,
//            each converted code serving the wave's 4 pair fragments (the
//            conversions do not overlap the products, so their number per
//            product matters), epilogue y (fp32).
// The contraction runs in stages of kStage 64-wide steps: activations go
// global -> LDS by direct loads one stage ahead, weights global ->
// registers two stages ahead, with one barrier per stage.
// ---------------------------------------------------------------------------
// kPacked: wq in the mxfp4_pack layout (a fragment's 32 rows x 32 bytes of
// one step are a contiguous 1 KiB chunk: 16-byte piece 32 h + r holds half h
// of row r), so lane (n, g)'s A piece of step st is the 16 bytes at
// 16 lane + 1024 st from the fragment's first chunk.
template <bool kGateUp, int kStage, int WR, int WP, bool kPacked>
__global__ __launch_bounds__(64 * WR * WP, 8 / (WR * WP)) void expert_gemm_kernel(
    const uint8_t* __restrict__ bq, const int32_t* __restrict__ sorted, int k,
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc,
    const int32_t* __restrict__ tiles, int max_tiles, int ntl, int K, int NOUT, int F,
    _Float16* __restrict__ h, float* __restrict__ y) {
    constexpr int NT = 2;                               // x terms (gate/up)
    // A fragments per wave: gate/up the gate and up rows of 4 / WR feature
    // fragments (a block covers 4), down 16 / WR (a block covers 16)
    constexpr int NA = kGateUp ? 8 / WR : 16 / WR;
    constexpr int kGemmThreads = 64 * WR * WP;
    constexpr int NB = 4 / WP;                          // B fragments (32 pairs) per wave
    static_assert(WR * WP <= 8 && (kGateUp ? 4 % WR == 0 : 16 % WR == 0), "wavefront layout");
    constexpr int kWaveFrags = kGateUp ? NA / 2 : NA;   // output fragments per wave
    // A step of an activation row: kStepBytes in global memory (x: the
    // terms and scales of one step chunk; h: 64 fp16 values), kChunk in LDS
    // (h: plus a pad unit, loaded as a copy of the step's last 16 bytes).
    constexpr int kChunk = kGateUp ? term_chunk(NT) : kHPitch;
    constexpr int kStepBytes = kGateUp ? kChunk : 128;
    // LDS slot of one step: the 128 rows' step chunks, row-major.  The row
    // pitch kChunk = 144 bytes (9 units of 16) keeps both the staging copy
    // and the operand reads (lanes n = 0..15 at 16-byte units 9 n mod 16)
    // free of bank conflicts.
    constexpr int kSlotBytes = kGemmRows * kChunk;
    constexpr int kRowPieces = kChunk / 16;
    constexpr int kPieces = (kGemmRows * kRowPieces + kGemmThreads - 1) / kGemmThreads;
    constexpr int kBufBytes = kStage * kSlotBytes;      // one stage of activation steps
    // Activation loads run one stage ahead through two LDS buffers.  (Two
    // stages ahead gains nothing: the compiler's own wait for the weight
    // registers at the start of a stage does not count the direct-to-LDS
    // loads, which are opaque to it, and so also drains the newer ones.)
    constexpr int kBufs = 2;
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ int s_src[kGemmRows];
    __shared__ int s_rmax[WR][NA][32];                  // (down) bmax of each A fragment row

    // Work item L = m-tile * ntl + column tile.  The dispatcher deals blocks
    // to the 8 XCDs round robin (block b -> XCD b % 8), each XCD with its own
    // L2; give every XCD one contiguous range of work items so the blocks
    // sharing a tile's activations (same m-tile) or an expert's weights (same
    // expert, neighbouring m-tiles) run on one L2.
    const int work = tiles[2 * max_tiles] * ntl;
    const int chunk = (work + kXcds - 1) / kXcds;
    const int xi = blockIdx.x / kXcds;
    const int L = (blockIdx.x % kXcds) * chunk + xi;
    if (xi >= chunk || L >= work) return;
    const int mt = L / ntl, nt = L - mt * ntl;
    const int row0 = tiles[2 * mt], info = tiles[2 * mt + 1];
    const int e = info & 0xFFFF, nvalid = info >> 16;
    // (the wave index through readfirstlane: the compiler then knows it is
    // uniform, keeps what derives from it in scalar registers and branches
    // on it with scalar branches)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave / WP, wp = wave % WP;           // this wave's row group and pair group
    const int n = lane & 31, g = lane >> 5;
    const int S = K / 64;
    const size_t RB = (size_t)S * kStepBytes;           // bytes per activation row

    // Rows past the tile's pairs repeat its last pair (their results are not stored).
    if (tid < kGemmRows) {
        const int i = row0 + (tid < nvalid ? tid : nvalid - 1);
        s_src[tid] = kGateUp ? sorted[i] / k : i;
    }

    // This block's output fragments [fa, fb); this wave's [wf0, wf0 + wcnt).
    const int nfrag = NOUT / 32;
    // (gate/up: 4 fragments, two whole 64-feature steps of h, per block;
    // down: an even split)
    const int fa = kGateUp ? nt * 4 : (int)((int64_t)nfrag * nt / ntl);
    const int fb = kGateUp ? min(fa + 4, nfrag) : (int)((int64_t)nfrag * (nt + 1) / ntl);
    const int wf0 = fa + wr * kWaveFrags;
    const int wcnt = max(0, min(kWaveFrags, fb - wf0));
    const int R = kGateUp ? 2 * F : NOUT;               // weight rows per expert
    const int nblk = K / 32;
    uint32_t aoff[NA];                                  // byte offset of this lane's A piece in wq
    // The E8M0 scales of a 32-row weight fragment are one contiguous,
    // 16-byte aligned run of 32 * nblk = K bytes; each wave copies its
    // fragments' runs into its own LDS area once.
    // (the WP wavefronts of a row group share one copy, made by wp == 0)
    uint8_t* wave_sc = lds + kBufs * kBufBytes + (size_t)wr * NA * K;
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        // gate/up: a < kWaveFrags the gate rows of fragment wf0 + a, then the up rows
        const int slot = kGateUp ? a % kWaveFrags : a;
        const int f = slot < wcnt ? wf0 + slot : fa;    // idle fragments recompute fragment fa
        const int frow = (kGateUp && a >= kWaveFrags ? F : 0) + 32 * f;
        // (the fragment's first byte is the same in both layouts)
        aoff[a] = kPacked ? (uint32_t)(((size_t)e * R + frow) * (size_t)(K / 2) + 16 * lane)
                          : (uint32_t)(((size_t)e * R + frow + n) * (size_t)(K / 2) + 16 * g);
    }
    // Direct global -> LDS loads (lane l writes 16 bytes at the wave-uniform
    // destination + 16 l), all issued before the prologue barrier, so the
    // copy is one memory round trip and holds no registers.
    auto copy_weight_scales = [&]() {
        if (wp != 0) return;
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            const int slot = kGateUp ? a % kWaveFrags : a;
            const int f = slot < wcnt ? wf0 + slot : fa;
            const int frow = (kGateUp && a >= kWaveFrags ? F : 0) + 32 * f;
            const uint8_t* run = wsc + ((size_t)e * R + frow) * nblk;
#pragma unroll
            for (int it = 0; it < kScaleIters; ++it) {
                const int i = lane + 64 * it;
                if (64 * it < K / 16 && i < K / 16)
                    dma16(wsc, (uint32_t)((size_t)(run - wsc) + 16 * i), wave_sc + a * K + 16 * 64 * it);
            }
        }
    };
    // this lane's scale bytes: row n of each fragment, block 2 s + g at + 2 s
    const uint8_t* my_sc = wave_sc + n * nblk + g;
    uint8_t* dummy = lds + kBufs * kBufBytes + (size_t)WR * NA * K + (wave & 7) * 1024;
    __syncthreads();

    // Staging: piece p = tid + kGemmThreads c (p < 128 kRowPieces) is 16-byte piece
    // p % kRowPieces of row p / kRowPieces's step chunk, loaded straight into
    // byte 16 p of the LDS slot (direct global -> LDS loads: a wave's 64
    // pieces land contiguously at a wave-uniform destination).
    uint32_t gsrc[kPieces];                             // byte offsets in bq (< 4 GiB)
#pragma unroll
    for (int c = 0; c < kPieces; ++c) {
        const int p = min(tid + kGemmThreads * c, kGemmRows * kRowPieces - 1);
        const int r = p / kRowPieces;
        const int piece = min(p - r * kRowPieces, kStepBytes / 16 - 1);
        gsrc[c] = (uint32_t)((size_t)s_src[r] * RB + 16 * piece);
    }

    f32x16_t acc[NA][NB];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][j][i] = 0.f;

    // Stage i = steps kStage i .. kStage i + kStage - 1: its activation
    // steps in LDS buffer i % 2, its weight fragments in register slot i % 3.
    // The weights (read by every pair tile of the expert, mostly from beyond
    // L2) are loaded two stages ahead, the activations one stage ahead.
    using AStage = u32x4_t[kStage][NA];
    AStage a_ring[3];
    const int nst = S / kStage;                         // whole stages; a partial one may follow

    // stage i's activation steps -> LDS buffer i % 2 (steps clamped)
    auto load_act = [&](int i) {
#pragma unroll
        for (int kk = 0; kk < kStage; ++kk) {
            const uint32_t so = (uint32_t)min(i * kStage + kk, S - 1) * kStepBytes;
            uint8_t* slot = lds + (i & 1) * kBufBytes + kk * kSlotBytes;
            // (a wave whose pieces lie past the slot, in the last round, loads
            // a duplicate into its dummy area: no branches in the loop)
#pragma unroll
            for (int c = 0; c < kPieces; ++c) {
                const bool real = kGemmThreads * c + wave * 64 < kGemmRows * kRowPieces;
                dma16(bq, gsrc[c] + so, real ? slot + 16 * (kGemmThreads * c + wave * 64) : dummy);
            }
        }
    };
    // stage i's weight fragments -> dst (steps clamped).  Issued after the
    // activation loads they travel with (the compiler barrier keeps them
    // there), so waiting until only kALoads operations are outstanding
    // leaves exactly these in flight.
    constexpr int kALoads = kStage * NA;
    auto load_a = [&](int i, AStage& dst) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int kk = 0; kk < kStage; ++kk) {
            const uint32_t st = (uint32_t)min(i * kStage + kk, S - 1);
#pragma unroll
            for (int a = 0; a < NA; ++a)
                dst[kk][a] = *reinterpret_cast<const u32x4_t*>(
                    wq + (aoff[a] + (kPacked ? 1024u : 32u) * st));
        }
    };
    // Products of one stage, software-pipelined over its kStage x NB x NT
    // operand groups (step kk, pair fragment j, term t): group q + 1's B
    // operand is read from LDS while group q's NA products run, so two
    // groups' operands (8 registers each) are live.
    struct Frag {
        u32x4_t lo, hi;
        uint32_t sw;                                    // scale word, byte 2 (t % 2) selected
    };
    auto read_frag = [&](int buf, int kk, int j, int t, Frag& fr) {
        // this lane's row (pair 32 j + n) of the step: term t's bytes of lane
        // group g at 64 t + 32 g, its term scales (byte 2 t + g) at NT * 64
        const uint8_t* row = lds + buf * kBufBytes + kk * kSlotBytes + (32 * (wp * NB + j) + n) * kChunk;
        fr.sw = reinterpret_cast<const uint32_t*>(row + NT * 64)[t >> 1] >> (8 * g);
        fr.lo = *reinterpret_cast<const u32x4_t*>(row + 64 * t + 32 * g);
        fr.hi = *reinterpret_cast<const u32x4_t*>(row + 64 * t + 32 * g + 16);
    };
    auto mfma_frag = [&](const AStage& a_cur, int kk, int j, auto tc, const Frag& fr,
                         const int (&as)[NA]) {
        constexpr int t = decltype(tc)::value;
        const i32x8_t b8 = {(int)fr.lo[0], (int)fr.lo[1], (int)fr.lo[2], (int)fr.lo[3],
                            (int)fr.hi[0], (int)fr.hi[1], (int)fr.hi[2], (int)fr.hi[3]};
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            const i32x8_t a8 = {(int)a_cur[kk][a][0], (int)a_cur[kk][a][1],
                                (int)a_cur[kk][a][2], (int)a_cur[kk][a][3], 0, 0, 0, 0};
            // cbsz = 4: A is fp4 (E2M1); blgp = 0: B is fp8 (E4M3);
            // B scale = byte 2 (t % 2) of its (shifted) scale word
            acc[a][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                a8, b8, acc[a][j], 4, 0, 0, as[a], 2 * (t & 1), (int)fr.sw);
        }
    };
    // nsteps (<= kStage) steps of the stage in buffer buf with weights a_cur,
    // first step s0; after_first() runs once the first group's products are
    // issued
    auto compute_stage = [&](int buf, int s0, int nsteps, const AStage& a_cur,
                             auto&& after_first) {
      if constexpr (kGateUp) {
        constexpr int kGroups = kStage * NB * NT;
        Frag fr[2];
        int as[kStage][NA];
#pragma unroll
        for (int kk = 0; kk < kStage; ++kk)
#pragma unroll
            for (int a = 0; a < NA; ++a) as[kk][a] = my_sc[a * K + 2 * min(s0 + kk, S - 1)];
        read_frag(buf, 0, 0, 0, fr[0]);
        static_for<kGroups>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            constexpr int kk = q / (NB * NT), j = (q / NT) % NB, t = q % NT;
            if (kk < nsteps) {
                if constexpr (q + 1 < kGroups) {
                    constexpr int q1 = q + 1;
                    if (q1 / (NB * NT) < nsteps)
                        read_frag(buf, q1 / (NB * NT), (q1 / NT) % NB, q1 % NT, fr[q1 & 1]);
                }
                __builtin_amdgcn_sched_barrier(0);
                // (a pair fragment past the tile's pairs, as in an expert's
                // last tile, has no products to compute: its results are
                // never stored; the branch is uniform in the wavefront)
                if (32 * (wp * NB + j) < nvalid)
                    mfma_frag(a_cur, kk, j, std::integral_constant<int, t>{}, fr[q & 1], as[kk]);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (q == 0) {
                    after_first();
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        });
      } else {
        // Sub-step u = (step kk, jj): the NA x NB products over elements
        // 8 jj .. 8 jj + 7 of each lane's 32.  Sub-step u + 1's h operands
        // (all NB pair fragments) are read from LDS and its A fragments
        // converted while sub-step u's products run.
        constexpr int kSub = kStage * 4;
        float sc[kStage][NA];                           // conversion scales (rewritten bytes)
#pragma unroll
        for (int kk = 0; kk < kStage; ++kk)
#pragma unroll
            for (int a = 0; a < NA; ++a)
                sc[kk][a] = __builtin_bit_cast(float, (uint32_t)my_sc[a * K + 2 * min(s0 + kk, S - 1)] << 23);
        f16x8_t af[2][NA], bf[2][NB];
        auto convert = [&](auto uc, f16x8_t(&dst)[NA]) {
            constexpr int kk = decltype(uc)::value / 4, jj = decltype(uc)::value % 4;
#pragma unroll
            for (int a = 0; a < NA; ++a) {
                const uint32_t w = a_cur[kk][a][jj];
                // byte i's two codes (low nibble first) -> elements 2 i, 2 i + 1
                const u32x4_t v = {
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc[kk][a], 0)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc[kk][a], 1)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc[kk][a], 2)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc[kk][a], 3))};
                dst[a] = __builtin_bit_cast(f16x8_t, v);
            }
        };
        auto read_b = [&](int u, f16x8_t(&dst)[NB]) {
            // pair 32 (wp NB + j) + n of step u / 4: elements 32 g + 8 (u % 4) .. + 7
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const uint8_t* row = lds + buf * kBufBytes + (u / 4) * kSlotBytes +
                                     (32 * (wp * NB + j) + n) * kChunk;
                dst[j] = *reinterpret_cast<const f16x8_t*>(row + 64 * g + 16 * (u % 4));
            }
        };
        convert(std::integral_constant<int, 0>{}, af[0]);
        read_b(0, bf[0]);
        static_for<kSub>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            if (u / 4 < nsteps) {
                if constexpr (u + 1 < kSub) {
                    if ((u + 1) / 4 < nsteps) {
                        read_b(u + 1, bf[(u + 1) & 1]);
                        convert(std::integral_constant<int, u + 1>{}, af[(u + 1) & 1]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    // (pair fragments past the tile's pairs: no products)
                    if (32 * (wp * NB + j) < nvalid) {
#pragma unroll
                        for (int a = 0; a < NA; ++a)
                            acc[a][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                af[u & 1][a], bf[u & 1][j], acc[a][j], 0, 0, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (u == 0) {
                    after_first();
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        });
      }
    };

    // prologue: weight scales and stage 0 in LDS, stage 0's and 1's weights
    // in registers; wait for all but stage 1's weights (the direct loads
    // land in LDS before the counter drops)
    copy_weight_scales();
    load_act(0);
    load_a(0, a_ring[0]);
    load_a(1, a_ring[1]);
    wait_vm<kALoads>();
    lds_barrier();
    if constexpr (!kGateUp) {
        // Down: each A fragment row's largest scale byte bmax; the row's
        // scale bytes b are rewritten in place as max(0, b - bmax + 140), the
        // fp32 biased exponent of its conversion scale 2^(b - bmax + 13)
        // (0: the scale is 0, the codes are more than 139 binades down).
        // The WP wavefronts of a row group share its copy; wp == 0 rewrites.
        if (wp == 0) {
#pragma unroll
            for (int a = 0; a < NA; ++a) {
                uint8_t* run = wave_sc + a * K + n * nblk;
                int mx = 0;
                for (int b = g; b < nblk; b += 2) mx = max(mx, (int)run[b]);
                mx = max(mx, __shfl_xor(mx, 32));
                for (int b = g; b < nblk; b += 2) run[b] = (uint8_t)max(0, (int)run[b] - mx + 140);
                if (g == 0) s_rmax[wr][a][n] = mx;
            }
        }
        lds_barrier();
    }
    // Stage i: products from buffer i % 2 and slot i % 3, with stage i + 1's
    // activations and stage i + 2's weights issued right after the first
    // group of them (buffer (i + 1) % 2 was last read in stage i - 1, slot
    // (i + 2) % 3 likewise).  The wait at the end leaves only stage i + 2's
    // weights in flight: activations get almost one stage to land, weights
    // almost two.  The loop takes three stages per trip, without branches,
    // so that every register slot keeps one fixed set of registers.
    //
    // The count in wait_vm<kALoads> holds only where the weight loads of
    // the stage are live.  After the loop they are not (no later stage reads
    // them), the compiler drops them, and the count would then leave
    // activation loads in flight; the (at most two) stages after the loop
    // therefore wait for everything.
    auto run_stage = [&](int i, auto rc, auto tail) {
        constexpr int r = decltype(rc)::value;
        compute_stage(i & 1, i * kStage, kStage, a_ring[r], [&]() {
            load_act(i + 1);
            load_a(i + 2, a_ring[(r + 2) % 3]);
        });
        if constexpr (decltype(tail)::value)
            wait_vm_all();
        else
            wait_vm<kALoads>();
        lds_barrier();
    };
    using Loop = std::false_type;
    using Tail = std::true_type;
    int i0 = 0;
    for (; i0 + 3 <= nst; i0 += 3) {
        run_stage(i0, std::integral_constant<int, 0>{}, Loop{});
        run_stage(i0 + 1, std::integral_constant<int, 1>{}, Loop{});
        run_stage(i0 + 2, std::integral_constant<int, 2>{}, Loop{});
    }
    if (i0 < nst) run_stage(i0, std::integral_constant<int, 0>{}, Tail{});
    if (i0 + 1 < nst) run_stage(i0 + 1, std::integral_constant<int, 1>{}, Tail{});
    if constexpr (kStage > 1) {
        if (nst * kStage < S) {                         // partial last stage, slot nst % 3
            const int s0 = nst * kStage, ns = S - s0;
            switch (nst % 3) {
                case 0: compute_stage(nst & 1, s0, ns, a_ring[0], []() {}); break;
                case 1: compute_stage(nst & 1, s0, ns, a_ring[1], []() {}); break;
                default: compute_stage(nst & 1, s0, ns, a_ring[2], []() {}); break;
            }
        }
    }
    // (the last stages' clamped prefetches may still be in flight; the LDS
    // is reused below and released at exit)
    wait_vm_all();

    if constexpr (kGateUp) {
        // h = silu(g) * u, rounded to fp16, for the wave's kWaveFrags feature
        // fragments (features 32 wf0 .. 32 (wf0 + kWaveFrags) - 1).  Lanes n
        // and n + 32 hold the features of pair n; the wave assembles its
        // pairs' 64 kWaveFrags-byte row pieces in LDS (free now), then writes
        // them with contiguous 16-byte stores.
        typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4_t;
        constexpr int kWavePairs = 32 * NB;
        constexpr int kRowPieces16 = 4 * kWaveFrags;    // 16-byte pieces of a row piece
        constexpr int kRowPitch = 16 * (kRowPieces16 + 1);
        __syncthreads();                                // every wave is done with the stage buffers
        uint8_t* wst = lds + wave * (kWavePairs * kRowPitch);
        if (wcnt > 0) {
#pragma unroll
            for (int ff = 0; ff < kWaveFrags; ++ff) {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    uint8_t* prow = wst + (32 * j + n) * kRowPitch + 64 * ff;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        // features 32 ff + 8 w + 4 g .. + 3 (C elements 4 w .. 4 w + 3)
                        f16x4_t hv;
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            hv[c] = (_Float16)(silu_f32(acc[ff][j][4 * w + c]) *
                                               acc[kWaveFrags + ff][j][4 * w + c]);
                        *reinterpret_cast<f16x4_t*>(prow + 2 * (8 * w + 4 * g)) = hv;
                    }
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // pairs wp * kWavePairs .. + kWavePairs - 1 of the tile
            const int pr0 = wp * kWavePairs;
            for (int pc = lane; pc < kWavePairs * kRowPieces16; pc += 64) {
                const int pr = pc / kRowPieces16, piece = pc % kRowPieces16;
                if (pr0 + pr < nvalid)
                    *reinterpret_cast<u32x4_t*>(h + (size_t)(row0 + pr0 + pr) * F + 32 * wf0 + 8 * piece) =
                        *reinterpret_cast<const u32x4_t*>(wst + pr * kRowPitch + 16 * piece);
            }
        }
    } else {
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            if (a >= wcnt) break;
            const int f = wf0 + a;
            // element i (feature row 8 (i / 4) + 4 g + i % 4 of the fragment)
            // is scaled by 2^(bmax of that row - 140)
            int ex[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) ex[i] = s_rmax[wr][a][8 * (i / 4) + 4 * g + i % 4] - 140;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int r = 32 * (wp * NB + j) + n;
                if (r < nvalid) {
                    float* orow = y + (size_t)(row0 + r) * NOUT + 32 * f + 4 * g;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        f32x4_t o;
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            o[c] = __builtin_amdgcn_ldexpf(acc[a][j][4 * w + c], ex[4 * w + c]);
                        *reinterpret_cast<f32x4_t*>(orow + 8 * w) = o;
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

int gemm_max_tiles(int T, int E, int k) {
    const int64_t P = (int64_t)T * k;
    const int64_t busy = P < E ? P : E;
    return (int)((P + busy * (kGemmRows - 1) + kGemmRows - 1) / kGemmRows);
}

size_t gemm_term_bytes(int rows, int K, int NT) {
    return (size_t)rows * (K / 64) * term_chunk(NT);
}

// Blocks for up to max_tiles x ntl work items, a multiple of the XCD count.
static int64_t gemm_grid(int max_tiles, int ntl) {
    const int64_t w = (int64_t)max_tiles * ntl;
    return (w + kXcds - 1) / kXcds * kXcds;
}

static int gemm_col_tiles(int NOUT, int frags_per_block) {
    return (NOUT / 32 + frags_per_block - 1) / frags_per_block;
}

// Dynamic LDS of expert_gemm_kernel: two stage buffers of activation steps,
// the weight scales of the block's A fragments (K bytes each; gate/up 8,
// down 16), and 8 KiB of dummy destinations for the staging.
size_t gemm_lds_bytes(int K, bool gate_up, int stage, int wr) {
    const int pitch = gate_up ? term_chunk(2) : kHPitch;
    const int frags = gate_up ? 8 : 16;                 // A fragments per block
    return (size_t)2 * stage * kGemmRows * pitch + (size_t)frags * K + 8 * 1024;
}


template <bool kGateUp, int kStage, int WR, int WP, bool kPacked>
static hipError_t launch_gemm(const MlpPlan& p, const uint8_t* bq, const int32_t* sorted,
                              const uint8_t* wq, const uint8_t* ws, const int32_t* tiles,
                              int K, int NOUT, _Float16* h, float* y, hipStream_t stream) {
    const int ntl = gemm_col_tiles(NOUT, kGateUp ? 4 : 16);
    size_t lds = gemm_lds_bytes(K, kGateUp, kStage, WR);
    if (kGateUp)                                        // epilogue staging of the h rows
        lds = std::max(lds, (size_t)(WR * WP) * 32 * (4 / WP) * 16 * (4 * (4 / WR) + 1));
    if (lds > 65536) {
        const hipError_t er = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&expert_gemm_kernel<kGateUp, kStage, WR, WP, kPacked>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (er != hipSuccess) return er;
    }
    hipLaunchKernelGGL((expert_gemm_kernel<kGateUp, kStage, WR, WP, kPacked>),
                       dim3((unsigned)gemm_grid(p.max_tiles, ntl)), dim3(64 * WR * WP), lds,
                       stream, bq, sorted, p.k, wq, ws, tiles, p.max_tiles, ntl, K, NOUT, p.F,
                       h, y);
    return hipSuccess;
}


hipError_t launch_mlp_gemm(const MlpPlan& p, bool packed, const uint16_t* x, const uint8_t* w13q,
                           const uint8_t* w13s, const uint8_t* w2q, const uint8_t* w2s,
                           const int32_t* offsets, const int32_t* sorted, float* y, char* base,
                           hipEvent_t* events, hipStream_t stream) {
    uint8_t* xq = reinterpret_cast<uint8_t*>(base + p.off_xq);
    _Float16* h = reinterpret_cast<_Float16*>(base + p.off_h);
    int32_t* tiles = reinterpret_cast<int32_t*>(base + p.off_tiles);
    hipLaunchKernelGGL(gemm_tiles_kernel, dim3(1), dim3(256), 0, stream, offsets, p.E,
                       p.max_tiles, tiles);
    const int64_t nsplit = (int64_t)p.T * (p.D / 64);
    hipLaunchKernelGGL(split_terms_kernel<2>, dim3((unsigned)((nsplit + 255) / 256)), dim3(256), 0,
                       stream, x, p.T, p.D, xq);
    if (events) {
        const hipError_t er = hipEventRecord(events[0], stream);
        if (er != hipSuccess) return er;
    }
    hipError_t er;
    er = packed ? launch_gemm<true, 1, 4, 1, true>(p, xq, sorted, w13q, w13s, tiles, p.D, p.F, h,
                                                   nullptr, stream)
                : launch_gemm<true, 1, 4, 1, false>(p, xq, sorted, w13q, w13s, tiles, p.D, p.F, h,
                                                    nullptr, stream);
    if (er != hipSuccess) return er;
    if (events) {
        er = hipEventRecord(events[1], stream);
        if (er != hipSuccess) return er;
    }
    const uint8_t* hb = reinterpret_cast<const uint8_t*>(h);
    er = packed ? launch_gemm<false, 1, 8, 1, true>(p, hb, nullptr, w2q, w2s, tiles, p.F, p.D,
                                                    nullptr, y, stream)
                : launch_gemm<false, 1, 8, 1, false>(p, hb, nullptr, w2q, w2s, tiles, p.F, p.D,
                                                     nullptr, y, stream);
    if (er != hipSuccess) return er;
    return hipGetLastError();
}

}  // namespace moe
