// expert_gemm.hip -- the expert MLP as two tiled grouped GEMMs, for batches in
// which experts receive many tokens (prefill), gfx950.
//
// The layer is the one of the weight-streaming kernels ("Welcome GPT OSS",
// section 4: SwiGLU experts; "Tricks", section 8: GEMMs that understand the
// 32-element blocks and their scales).  For each expert e with token rows X_e
// (its routed pairs in sorted order):  [G | U] = X_e W13_e^T,
// H = silu(G) * U,  Y = H W2_e^T;  the weighted combine follows.
//
// Both GEMMs run on v_mfma_scale_f32_32x32x64_f8f6f4.  The MXFP4 weights are
// its A operand exactly as stored (E2M1 codes, with the E8M0 block scales as
// the hardware A scale), so no weight is ever widened.  The activations -- x
// for gate/up, h for down -- are its B operand in fp6 (E2M3): each row is
// carried as 3 residual terms with their own E8M0 scale per 32-element block
// (fp6_block_terms in device_common.h), which leaves an error below 2^-12 of
// each block's largest magnitude whatever that magnitude is; fp4 x fp6
// products issue at twice the fp8 rate.  The gate/up epilogue computes
// h = silu(g) * u in fp32 and writes it straight away as fp6 term rows.
//
// Operand layouts (lane l, n = l % 32, g = l / 32), checked bit for bit with
// in-bounds probes on gfx950:
//   A (fp4): row n, K = 32 g .. 32 g + 31 (one MXFP4 block, low nibble
//       first) in the first 16 bytes; scale = that block's E8M0 byte.
//   B (fp6): column n, K = 32 g .. 32 g + 31, element i at bits 6 i of 6
//       dwords; scale = K-block g of column n.
//   C: element i = row 8 (i / 4) + 4 g + i % 4, column n.
//
// Activation term rows: a row of K elements (K % 64 == 0) is K / 64 steps of
// kTermStep = 160 bytes in the layout fp6_encode_step writes: per step its
// two 32-blocks one after the other, each as its 3 terms' codes and then
// their scale bytes (80 bytes), so a lane's operands of a step are the 80
// bytes of its block.  x is stored by token, row after row (the gate/up GEMM
// gathers a tile's rows).  h, which the gate/up epilogue writes tile by tile,
// is stored tile by tile, step-major within a tile: the tile whose n pairs
// start at sorted row r0 owns chunks r0 S .. (r0 + n) S - 1, step s of its
// row p is chunk r0 S + s n + p, and each chunk's 16-byte units are already
// rotated as the LDS staging wants them (row_rot below).  The down GEMM thus
// stages a step with contiguous 1 KiB loads; its loads for rows p >= n of a
// short tile read the next chunks of the region (which holds 128 rows of
// slack past its P rows): finite fp6 codes in product columns that are
// never stored, and the products of one column do not involve the others.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kGemmRows = 128;      // routed pairs per tile: 4 fragments of 32
constexpr int kXcds = 8;            // MI355X: 8 accelerator complex dies, one L2 each
constexpr int kScaleIters = 8;      // weight-scale copy: K <= 64 lanes x 16 bytes x 8
static_assert(64 * 16 * kScaleIters == kGemmMaxContraction, "scale copy covers every K");
// LDS row pitch of a staged step: its 160 bytes, 10 units of 16 bytes.  Row
// r's units are rotated by rot(r) = (r / 8) mod 2 (unit u at position
// (u + rot(r)) mod 10): the 128-bit operand reads of 16 consecutive rows (one
// unit each) then hit 16 different groups of 4 banks (with 64 banks of 4
// bytes), as an odd pitch with a pad unit would, without staging the pad.
// (rot depends on the lane only: row 32 j + n has rot (n / 8) mod 2.)
constexpr int kStepPitch = kTermStep;
__device__ __forceinline__ int row_rot(int r) { return (r >> 3) & 1; }
// gate/up epilogue: h of the block's 128 pairs x 128 features in fp32, rows
// of kHRow floats
constexpr int kHRow = 132;
// down epilogue: each wave's 128 pairs x 64 outputs of fp16 y, rows of
// kYPitch bytes (128 + 16: 16-byte aligned rows, at most 2-way bank
// conflicts for the 8-byte writes)
constexpr int kYPitch = 144;

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
// Tile table: expert e's pairs [offsets[e], offsets[e+1]) in tiles of
// kGemmRows, experts in order.  tiles[2 i] = first sorted row of tile i,
// tiles[2 i + 1] = e | rows << 16; tiles[2 max_tiles] = number of tiles.
// Computed by one block of 256 threads (E <= 256), with 256 ints of LDS at part.
// ---------------------------------------------------------------------------
__device__ void gemm_tile_table(const int32_t* __restrict__ offsets, int E, int max_tiles,
                                int32_t* __restrict__ tiles, int* part) {
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
// bf16 rows -> fp6 term rows, one thread per (row, 64-element step) item; the
// grid's extra first block computes the tile table (one launch fewer; as the
// first block dispatched it runs beside the conversion, not after it).
//
// Rows are contiguous (K % 64 == 0), so item i reads the 128 bytes at 128 i
// of src and writes the 160 bytes at 160 i of tq: a wavefront's 64 items are
// one contiguous 8 KiB range in and one 10 KiB range out.  A whole wavefront
// moves them with whole-line accesses (lane l: 16 bytes at 16 l + 1024 c) and
// regroups them by item through its own LDS area: items at a pitch of 144
// bytes going in (the 16-byte accesses of 16 lanes at 16 different items hit
// 16 different groups of 4 banks), 160 going out (at most 2 lanes per group;
// the area of 10 KiB per wavefront lets four blocks share a CU).  The wavefront at
// the end of the range, with fewer than 64 items, moves each item by itself.
// ---------------------------------------------------------------------------
constexpr int kSplitInPitch = 144;
constexpr int kSplitOutPitch = kTermStep;
constexpr int kSplitWaves = 4;
constexpr int kSplitWaveLds = 64 * kSplitOutPitch;   // the in and out layouts share it
static_assert(64 * kSplitInPitch <= kSplitWaveLds && kSplitWaveLds % 16 == 0, "split LDS");

__global__ __launch_bounds__(64 * kSplitWaves) void split_terms_kernel(
    const uint16_t* __restrict__ src, int rows, int K, uint8_t* __restrict__ tq,
    const int32_t* __restrict__ offsets, int E, int max_tiles, int32_t* __restrict__ tiles) {
    __shared__ __align__(16) uint8_t lds[kSplitWaves * kSplitWaveLds];
    if (blockIdx.x == 0) {
        gemm_tile_table(offsets, E, max_tiles, tiles, reinterpret_cast<int*>(lds));
        return;
    }
    const int S = K / 64;
    const int64_t n = (int64_t)rows * S;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t i0 = ((int64_t)(blockIdx.x - 1) * kSplitWaves + wave) * 64;
    if (i0 >= n) return;
    const int64_t idx = i0 + lane;
    const bool whole = i0 + 64 <= n;                  // uniform in the wavefront
    uint8_t* wl = lds + wave * kSplitWaveLds;
    const uint8_t* in = reinterpret_cast<const uint8_t*>(src);
    // the whole 128-byte step is loaded before any of it is converted
    u32x4_t raw[8];
    if (whole) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
            raw[c] = *reinterpret_cast<const u32x4_t*>(in + (size_t)i0 * 128 + 1024 * c + 16 * lane);
        // unit lane % 8 of item 8 c + lane / 8
#pragma unroll
        for (int c = 0; c < 8; ++c)
            *reinterpret_cast<u32x4_t*>(wl + (8 * c + (lane >> 3)) * kSplitInPitch + 16 * (lane & 7)) =
                raw[c];
        // (a wavefront reads back only what it wrote: LDS operations of one
        // wavefront complete in order)
#pragma unroll
        for (int c = 0; c < 8; ++c)
            raw[c] = *reinterpret_cast<const u32x4_t*>(wl + lane * kSplitInPitch + 16 * c);
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c)
            raw[c] = idx < n ? *reinterpret_cast<const u32x4_t*>(in + (size_t)idx * 128 + 16 * c)
                             : u32x4_t{0u, 0u, 0u, 0u};
    }
    __builtin_amdgcn_sched_barrier(0);
    float v[64];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            v[8 * c + 2 * h] = bf16_to_f32(raw[c][h] & 0xFFFFu);
            v[8 * c + 2 * h + 1] = bf16_to_f32(raw[c][h] >> 16);
        }
    uint32_t out[kTermStep / 4];
    fp6_encode_step(v, out);
    if (whole) {
        // (every lane's reads of the area above returned before the
        // conversion, which used them, so its own item may overwrite it)
#pragma unroll
        for (int w = 0; w < kTermStep / 16; ++w)
            *reinterpret_cast<u32x4_t*>(wl + lane * kSplitOutPitch + 16 * w) =
                u32x4_t{out[4 * w], out[4 * w + 1], out[4 * w + 2], out[4 * w + 3]};
        // (at pitch 160 the area holds the range as it is stored: 16-byte
        // unit u = 64 c + lane is at 16 u in both)
        static_assert(kSplitOutPitch == kTermStep, "the area is the stored range");
        uint8_t* o = tq + (size_t)i0 * kTermStep;
#pragma unroll
        for (int c = 0; c < kTermStep / 16; ++c) {
            const int u = 64 * c + lane;
            *reinterpret_cast<u32x4_t*>(o + 16 * u) = *reinterpret_cast<const u32x4_t*>(wl + 16 * u);
        }
    } else if (idx < n) {
        uint8_t* o = tq + (size_t)idx * kTermStep;
#pragma unroll
        for (int w = 0; w < kTermStep / 16; ++w)
            *reinterpret_cast<u32x4_t*>(o + 16 * w) =
                u32x4_t{out[4 * w], out[4 * w + 1], out[4 * w + 2], out[4 * w + 3]};
    }
}

// ---------------------------------------------------------------------------
// Grouped GEMM.  Block = one tile of kGemmRows pairs x one column range of
// output fragments (32 outputs each), WR wavefronts.  Each wavefront owns
// two A fragments against all 4 pair fragments of the tile:
//   gate/up: the gate and the up rows of one feature fragment (a block
//            covers WR fragments: with WR = 4, two whole 64-feature steps of
//            h); epilogue h = silu(g) * u -> fp6 term rows;
//   down:    two output fragments (a block covers 2 WR); epilogue y (fp16
//            with a power-of-two scale per pair and 32-output fragment).
// No two wavefronts load the same weights, and a wavefront without a live
// fragment (the last column range of an odd count) skips its products.
// The contraction runs in 64-wide steps: activation steps go global -> LDS
// by direct loads one step ahead (two LDS buffers), weights global ->
// registers two steps ahead (a ring of three register slots), with one
// barrier per step.
// ---------------------------------------------------------------------------
// kPacked: wq in the mxfp4_pack layout (a fragment's 32 rows x 32 bytes of
// one step are a contiguous 1 KiB chunk: 16-byte piece 32 h + r holds half h
// of row r), so lane (n, g)'s A piece of step st is the 16 bytes at
// 16 lane + 1024 st from the fragment's first chunk.
template <bool kGateUp, int WR, bool kPacked>
__global__ __launch_bounds__(64 * WR, 8 / WR) void expert_gemm_kernel(
    const uint8_t* __restrict__ bq, const int32_t* __restrict__ sorted, int k,
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc,
    const int32_t* __restrict__ tiles, int max_tiles, int ntl, int K, int NOUT, int F,
    uint8_t* __restrict__ hq, uint16_t* __restrict__ y16, uint8_t* __restrict__ ys) {
    constexpr int NT = kFp6Terms;
    static_assert(NT == 3, "the first fragment's products are written out for three terms");
    constexpr int NA = 2;                               // A fragments per wave
    constexpr int NB = kGemmRows / 32;                  // pair fragments per wave
    constexpr int kThreads = 64 * WR;
    constexpr int kBlockFrags = kGateUp ? WR : 2 * WR;  // output fragments per block
    // LDS slot of one step: the 128 rows' step chunks, row pitch kStepPitch,
    // units rotated per row (row_rot)
    constexpr int kSlotBytes = kGemmRows * kStepPitch;
    constexpr int kRowPieces = kStepPitch / 16;
    constexpr int kPieces = (kGemmRows * kRowPieces + kThreads - 1) / kThreads;
    constexpr int kBufs = 2;
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ int s_src[kGemmRows];

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
    const int n = lane & 31, g = lane >> 5;
    const int S = K / 64;
    const size_t RB = (size_t)S * kTermStep;            // bytes per activation term row

    // Rows past the tile's pairs repeat its last pair (their results are not stored).
    if (tid < kGemmRows) {
        const int i = row0 + (tid < nvalid ? tid : nvalid - 1);
        s_src[tid] = kGateUp ? sorted[i] / k : i;
    }

    // This block's output fragments [fa, fb); this wave's first, wf0, and
    // its number of live ones, wcnt (0 .. 1 for gate/up, 0 .. 2 for down).
    const int nfrag = NOUT / 32;
    const int fa = nt * kBlockFrags;
    const int fb = min(fa + kBlockFrags, nfrag);
    const int wf0 = fa + (kGateUp ? wave : 2 * wave);
    const int wcnt = max(0, min(kGateUp ? 1 : 2, fb - wf0));
    const int R = kGateUp ? 2 * F : NOUT;               // weight rows per expert
    const int nblk = K / 32;
    // fragment row of A fragment a (gate/up: a = 0 the gate rows, a = 1 the
    // up rows); a dead fragment loads fragment fa (its products are skipped)
    auto frag_row = [&](int a) {
        if constexpr (kGateUp) return (a == 1 ? F : 0) + 32 * (wcnt > 0 ? wf0 : fa);
        else return 32 * (a < wcnt ? wf0 + a : fa);
    };
    uint32_t aoff[NA];                                  // byte offset of this lane's A piece in wq
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        const int frow = frag_row(a);
        // (the fragment's first byte is the same in both layouts)
        aoff[a] = kPacked ? (uint32_t)(((size_t)e * R + frow) * (size_t)(K / 2) + 16 * lane)
                          : (uint32_t)(((size_t)e * R + frow + n) * (size_t)(K / 2) + 16 * g);
    }
    // The E8M0 scales of a 32-row weight fragment are one contiguous,
    // 16-byte aligned run of 32 * nblk = K bytes; each wave copies its
    // fragments' runs into its own LDS area once, by direct global -> LDS
    // loads (lane l writes 16 bytes at the wave-uniform destination + 16 l),
    // all issued before the prologue barrier: one memory round trip.
    uint8_t* wave_sc = lds + kBufs * kSlotBytes + (size_t)wave * NA * K;
    auto copy_weight_scales = [&]() {
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            const uint8_t* run = wsc + ((size_t)e * R + frag_row(a)) * nblk;
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
    uint8_t* dummy = lds + kBufs * kSlotBytes + (size_t)WR * NA * K + (wave & 7) * 1024;
    __syncthreads();

    // Staging: LDS unit p = tid + kThreads c (p < 128 kRowPieces) of the slot
    // is position p % kRowPieces of row p / kRowPieces, which holds unit
    // (position - row_rot) mod 10 of that row's step chunk; the 16 bytes are
    // loaded straight into byte 16 p of the slot (a wave's 64 pieces land
    // contiguously at a wave-uniform destination).  gate/up gathers the
    // tile's x rows; down reads byte 16 p of the tile's h step run.
    uint32_t gsrc[kPieces];                             // byte offsets in bq (< 4 GiB)
#pragma unroll
    for (int c = 0; c < kPieces; ++c) {
        const int p = min(tid + kThreads * c, kGemmRows * kRowPieces - 1);
        if constexpr (kGateUp) {
            const int r = p / kRowPieces;
            const int q = p - r * kRowPieces + kRowPieces - row_rot(r);
            const int piece = q >= kRowPieces ? q - kRowPieces : q;
            gsrc[c] = (uint32_t)((size_t)s_src[r] * RB + 16 * piece);
        } else {
            gsrc[c] = (uint32_t)((size_t)row0 * RB + 16 * p);
        }
    }

    f32x16_t acc[NA][NB];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][j][i] = 0.f;

    // Step i: its activation chunks in LDS buffer i % 2, its weight pieces in
    // register slot i % 3.  The weights (read by every pair tile of the
    // expert, mostly from beyond L2) are loaded two steps ahead, the
    // activations one step ahead.
    using AStep = u32x4_t[NA];
    AStep a_ring[3];

    // step i's activation chunks -> LDS buffer i % 2 (steps clamped)
    auto load_act = [&](int i) {
        const uint32_t so = (uint32_t)min(i, S - 1) * (kGateUp ? kTermStep : nvalid * kTermStep);
        uint8_t* slot = lds + (i & 1) * kSlotBytes;
        // (with 4 wavefronts the slot's 1280 pieces are exactly 5 rounds;
        // with other block sizes a wave whose pieces lie past the slot, in
        // the last round, loads a duplicate into its dummy area: no branches
        // in the loop)
#pragma unroll
        for (int c = 0; c < kPieces; ++c) {
            const bool real = kThreads * c + wave * 64 < kGemmRows * kRowPieces;
            dma16(bq, gsrc[c] + so, real ? slot + 16 * (kThreads * c + wave * 64) : dummy);
        }
    };
    // step i's weight pieces -> dst (steps clamped).  Issued after the
    // activation loads they travel with (the compiler barrier keeps them
    // there), so waiting until only NA operations are outstanding leaves
    // exactly these in flight.
    auto load_a = [&](int i, AStep& dst) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        const uint32_t st = (uint32_t)min(i, S - 1);
#pragma unroll
        for (int a = 0; a < NA; ++a)
            dst[a] = *reinterpret_cast<const u32x4_t*>(wq + (aoff[a] + (kPacked ? 1024u : 32u) * st));
    };
    // Products of one step, software-pipelined over its NB pair fragments:
    // fragment j + 1's B operands are read from LDS while fragment j's
    // NT x NA products run.  A lane's operands of fragment j are the five
    // units 5 g .. 5 g + 4 of its row (pair 32 j + n): dwords 6 t .. 6 t + 5
    // the codes of term t, dword 18 the terms' scales (term t in byte t).
    // The units sit at their rotated places, position (u + rot) mod 10:
    // only unit 9 (g = 1, rot = 1) wraps round, to position 0.
    // (held as one 12-dword and one 8-dword vector, so that each term's six
    // dwords are consecutive registers that the loads write directly)
    struct Frag {
        u32v12_t a;                                     // dwords 0 .. 11: terms 0, 1
        u32v8_t b;                                      // dwords 12 .. 19: term 2, scales
    };
    const int uoff = 16 * (5 * g + row_rot(n));
    const int uoff4 = g & row_rot(n) ? 0 : uoff + 64;
    auto read_frag = [&](int buf, int j, Frag& fr) {
        const uint8_t* row = lds + buf * kSlotBytes + (32 * j + n) * kStepPitch;
        const u32v4_t r0 = *reinterpret_cast<const u32v4_t*>(row + uoff);
        const u32v4_t r1 = *reinterpret_cast<const u32v4_t*>(row + uoff + 16);
        const u32v4_t r2 = *reinterpret_cast<const u32v4_t*>(row + uoff + 32);
        const u32v4_t r3 = *reinterpret_cast<const u32v4_t*>(row + uoff + 48);
        const u32v4_t r4 = *reinterpret_cast<const u32v4_t*>(row + uoff4);
        const u32v8_t r01 = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
        const u32v8_t r22 = __builtin_shufflevector(r2, r2, 0, 1, 2, 3, 0, 1, 2, 3);
        fr.a = __builtin_shufflevector(r01, r22, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11);
        fr.b = __builtin_shufflevector(r3, r4, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto mfma_frag = [&](const AStep& a_cur, int j, auto tc, const Frag& fr, const int (&as)[NA]) {
        constexpr int t = decltype(tc)::value;
        i32x8_t b8;
        if constexpr (t == 0)
            b8 = i32x8_t{(int)fr.a[0], (int)fr.a[1], (int)fr.a[2], (int)fr.a[3], (int)fr.a[4], (int)fr.a[5], 0, 0};
        else if constexpr (t == 1)
            b8 = i32x8_t{(int)fr.a[6], (int)fr.a[7], (int)fr.a[8], (int)fr.a[9], (int)fr.a[10], (int)fr.a[11], 0, 0};
        else
            b8 = i32x8_t{(int)fr.b[0], (int)fr.b[1], (int)fr.b[2], (int)fr.b[3], (int)fr.b[4], (int)fr.b[5], 0, 0};
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            // (dead fragments: no products; the branch is uniform)
            if (kGateUp ? wcnt > 0 : a < wcnt) {
                const i32x8_t a8 = {(int)a_cur[a][0], (int)a_cur[a][1], (int)a_cur[a][2],
                                    (int)a_cur[a][3], 0, 0, 0, 0};
                // cbsz = 4: A is fp4 (E2M1); blgp = 2: B is fp6 (E2M3);
                // B scale = byte t of the scale dword
                acc[a][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    a8, b8, acc[a][j], 4, 2, 0, as[a], t, (int)fr.b[6]);
            }
        }
    };
    // the step in buffer buf with weights a_cur, step index st; after_first()
    // runs once the first term's products are issued
    auto compute_step = [&](int buf, int st, const AStep& a_cur, auto&& after_first) {
        Frag fr[2];
        int as[NA];
#pragma unroll
        for (int a = 0; a < NA; ++a) as[a] = my_sc[a * K + 2 * st];
        read_frag(buf, 0, fr[0]);
        static_for<NB>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if constexpr (j + 1 < NB) read_frag(buf, j + 1, fr[(j + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (j == 0) {
                // (every tile has a pair in its first fragment)
                // (the wave's issue priority is raised while it issues
                // products and lowered while it issues loads and waits, so
                // the SIMD's other wave gets the issue slots it needs for
                // its products first)
                __builtin_amdgcn_s_setprio(1);
                mfma_frag(a_cur, 0, std::integral_constant<int, 0>{}, fr[0], as);
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_setprio(0);
                after_first();
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_setprio(1);
                mfma_frag(a_cur, 0, std::integral_constant<int, 1>{}, fr[0], as);
                mfma_frag(a_cur, 0, std::integral_constant<int, 2>{}, fr[0], as);
            } else if (32 * j < nvalid) {
                // (a pair fragment past the tile's pairs, as in an expert's
                // last tile, has no products to compute: its results are
                // never stored; the branch is uniform in the wavefront)
                static_for<NT>([&](auto tc) { mfma_frag(a_cur, j, tc, fr[j & 1], as); });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // prologue: weight scales and step 0 in LDS, step 0's and 1's weights in
    // registers; wait for all but step 1's weights (the direct loads land in
    // LDS before the counter drops)
    copy_weight_scales();
    load_act(0);
    load_a(0, a_ring[0]);
    load_a(1, a_ring[1]);
    wait_vm<NA>();
    lds_barrier();
    // Step i: products from buffer i % 2 and slot i % 3, with step i + 1's
    // activations and step i + 2's weights issued right after the first
    // group of them (buffer (i + 1) % 2 was last read in step i - 1, slot
    // (i + 2) % 3 likewise).  The wait at the end leaves only step i + 2's
    // weights in flight: activations get almost one step to land, weights
    // almost two.  The loop takes three steps per trip, without branches,
    // so that every register slot keeps one fixed set of registers.
    //
    // The count in wait_vm<NA> holds only where the weight loads of the step
    // are live.  After the loop they are not (no later step reads them), the
    // compiler drops them, and the count would then leave activation loads
    // in flight; the (at most two) steps after the loop therefore wait for
    // everything.
    auto run_step = [&](int i, auto rc, auto tail) {
        constexpr int r = decltype(rc)::value;
        compute_step(i & 1, i, a_ring[r], [&]() {
            load_act(i + 1);
            load_a(i + 2, a_ring[(r + 2) % 3]);
        });
        __builtin_amdgcn_s_setprio(0);
        if constexpr (decltype(tail)::value)
            wait_vm_all();
        else
            wait_vm<NA>();
        lds_barrier();
    };
    using Loop = std::false_type;
    using Tail = std::true_type;
    int i0 = 0;
    for (; i0 + 3 <= S; i0 += 3) {
        run_step(i0, std::integral_constant<int, 0>{}, Loop{});
        run_step(i0 + 1, std::integral_constant<int, 1>{}, Loop{});
        run_step(i0 + 2, std::integral_constant<int, 2>{}, Loop{});
    }
    if (i0 < S) run_step(i0, std::integral_constant<int, 0>{}, Tail{});
    if (i0 + 1 < S) run_step(i0 + 1, std::integral_constant<int, 1>{}, Tail{});
    // (the last steps' clamped prefetches may still be in flight; the LDS
    // is reused below and released at exit)
    wait_vm_all();

    if constexpr (kGateUp) {
        // h = silu(g) * u in fp32 for the block's 128 pairs x 32 WR features
        // (wave w: features 32 w .. 32 w + 31, C element i of pair fragment
        // j = feature 8 (i / 4) + 4 g + i % 4 of pair 32 j + n), gathered in
        // LDS (free now), then one thread per (pair, 64-feature step) turns
        // its 64 values into the pair's 160-byte fp6 step chunk, units rotated.
        // The chunks go back to LDS, in the order they have in the tile's h
        // run (each step's nvalid chunks contiguous), and the block copies them
        // out with whole-line stores (measured 0.7-1.1 % faster than storing
        // each thread's chunk directly, 16 bytes in each of 64 chunks per
        // instruction).
        static_assert(WR % 2 == 0 && WR * 32 <= kHRow, "epilogue layout: whole 64-feature steps");
        static_assert(kGemmRows * (WR / 2) == kThreads, "one chunk per thread");
        __syncthreads();                                // every wave is done with the stage buffers
        float* hb = reinterpret_cast<float*>(lds);
        if (wcnt > 0) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    f32x4_t hv;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        hv[c] = silu_f32(acc[0][j][4 * w + c]) * acc[1][j][4 * w + c];
                    *reinterpret_cast<f32x4_t*>(hb + (32 * j + n) * kHRow + 32 * wave + 8 * w + 4 * g) = hv;
                }
        }
        __syncthreads();
        const int nsteps = (fb - fa) / 2;               // F % 64 == 0: whole steps
        const int Sh = F / 64;
        const int p = tid / (WR / 2), hs = tid % (WR / 2);
        const bool live = p < nvalid && hs < nsteps;
        uint32_t out[kTermStep / 4];
        if (live) {
            float v[64];
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const f32x4_t q4 = *reinterpret_cast<const f32x4_t*>(hb + p * kHRow + 64 * hs + 4 * c);
                v[4 * c] = q4[0]; v[4 * c + 1] = q4[1]; v[4 * c + 2] = q4[2]; v[4 * c + 3] = q4[3];
            }
            fp6_encode_step(v, out);
        }
        __syncthreads();                                // hb is no longer read
        // chunk p of step hs at (hs 128 + p) 160 (the first WR/2 x 20 KiB of LDS)
        uint8_t* cb = lds;
        if (live) {
            uint8_t* o = cb + ((size_t)hs * kGemmRows + p) * kTermStep;
            const int rot = row_rot(p);
#pragma unroll
            for (int w = 0; w < kRowPieces; ++w) {
                const int pos = w + rot < kRowPieces ? w + rot : w + rot - kRowPieces;
                *reinterpret_cast<u32x4_t*>(o + 16 * pos) =
                    u32x4_t{out[4 * w], out[4 * w + 1], out[4 * w + 2], out[4 * w + 3]};
            }
        }
        __syncthreads();
        // step hs of the tile: chunks (row0 Sh + (fa / 2 + hs) nvalid + p) 160, p < nvalid
        const int units = nvalid * kRowPieces;          // 16-byte units per step
        for (int u = tid; u < nsteps * units; u += kThreads) {
            const int h = u / units, uu = u - h * units;
            *reinterpret_cast<u32x4_t*>(
                hq + ((size_t)row0 * Sh + (size_t)(fa / 2 + h) * nvalid) * kTermStep + 16 * uu) =
                *reinterpret_cast<const u32x4_t*>(cb + (size_t)h * kGemmRows * kTermStep + 16 * uu);
        }
    } else {
        // y in fp16 with one power-of-two scale per (pair, 32-output fragment):
        // the fragment's largest magnitude m is brought into [2^14, 2^15) (an
        // exact ldexp), so every value keeps fp16's 11-bit precision relative to
        // m (those more than 24 binades below m fall into fp16's subnormals),
        // and no y overflows or underflows whatever its range.  Lane (n, g) holds
        // 16 of the fragment's 32 outputs of pair 32 j + n, lane (n, 1 - g) the
        // other 16.
        //
        // The wave's 128 pairs x 64 outputs go through LDS first (rows of
        // kYPitch bytes, free once every wave is past its last step), so that
        // each global store instruction writes 8 whole 128-byte rows instead of
        // 16 bytes in each of 32 rows (measured 6 % faster at both prefill
        // shapes).
        __syncthreads();                                // every wave is done with the stage buffers
        uint8_t* ytile = lds + (size_t)wave * kGemmRows * kYPitch;
        int sc[NA][NB];
#pragma unroll
        for (int a = 0; a < NA; ++a) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                float m = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(acc[a][j][i]));
                m = fmaxf(m, __shfl_xor(m, 32));
                const int sj = y_scale_exponent(m);
                sc[a][j] = sj;
                // element i: output 32 a + 8 (i / 4) + 4 g + i % 4 of the wave's 64,
                // pair 32 j + n
                uint8_t* trow = ytile + (32 * j + n) * kYPitch + 2 * (32 * a + 4 * g);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uint32_t h2[2];
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        h2[c] = f32_to_f16_bits(__builtin_ldexpf(acc[a][j][4 * w + 2 * c], -sj)) |
                                (f32_to_f16_bits(__builtin_ldexpf(acc[a][j][4 * w + 2 * c + 1], -sj)) << 16);
                    *reinterpret_cast<u32x2_t*>(trow + 16 * w) = u32x2_t{h2[0], h2[1]};
                }
            }
        }
        // (a wave reads back only what it wrote: LDS operations of one wave
        // complete in order, and the compiler waits for the writes' data)
        // scale bytes: f = wf0 and wf0 + 1 are adjacent (wf0 even) in the row
        // of NOUT / 32 bytes (even: NOUT % 64 == 0)
        if (g == 0 && wcnt > 0) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int r = 32 * j + n;
                if (r < nvalid) {
                    uint8_t* srow = ys + (size_t)(row0 + r) * (NOUT / 32) + wf0;
                    if (wcnt == 2)
                        *reinterpret_cast<uint16_t*>(srow) =
                            (uint16_t)((sc[0][j] + 127) | ((sc[1][j] + 127) << 8));
                    else
                        srow[0] = (uint8_t)(sc[0][j] + 127);
                }
            }
        }
        // lane l: 16 bytes (outputs 8 (l % 8) .. + 7 of the wave's 64) of
        // pair 8 q + l / 8
        const int cq = lane & 7;
        if (8 * cq < 32 * wcnt) {
#pragma unroll 4
            for (int q = 0; q < kGemmRows / 8; ++q) {
                const int r = 8 * q + (lane >> 3);
                if (r < nvalid) {
                    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ytile + r * kYPitch + 16 * cq);
                    *reinterpret_cast<u32x4_t*>(y16 + (size_t)(row0 + r) * NOUT + 32 * wf0 + 8 * cq) = v;
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

size_t gemm_term_bytes(int rows, int K) {
    return (size_t)rows * (K / 64) * kTermStep;
}

size_t gemm_h_bytes(int64_t P, int F) {
    return gemm_term_bytes((int)(P + kGemmRows), F);
}

// Blocks for up to max_tiles x ntl work items, a multiple of the XCD count.
static int64_t gemm_grid(int max_tiles, int ntl) {
    const int64_t w = (int64_t)max_tiles * ntl;
    return (w + kXcds - 1) / kXcds * kXcds;
}

// Wavefronts per block: gate/up 4 (two blocks per CU, 128 features each),
// down 4 (256 outputs each).
constexpr int kGateUpWaves = 4;
constexpr int kDownWaves = 4;

// Dynamic LDS of expert_gemm_kernel: two step buffers of activation chunks,
// the weight scales of the block's 2 WR A fragments (K bytes each), 8 KiB of
// dummy destinations for the staging; the epilogues reuse it (gate/up for its
// fp32 h tile, down for its waves' fp16 y tiles) and need at least that much.
size_t gemm_lds_bytes(int K, bool gate_up) {
    const int wr = gate_up ? kGateUpWaves : kDownWaves;
    size_t b = (size_t)2 * kGemmRows * kStepPitch + (size_t)2 * wr * K + 8 * 1024;
    if (gate_up) b = std::max(b, (size_t)kGemmRows * kHRow * sizeof(float));
    else b = std::max(b, (size_t)wr * kGemmRows * kYPitch);
    return b;
}

template <bool kGateUp, int WR, bool kPacked>
static hipError_t launch_gemm(const MlpPlan& p, const uint8_t* bq, const int32_t* sorted,
                              const uint8_t* wq, const uint8_t* ws, const int32_t* tiles,
                              int K, int NOUT, uint8_t* hq, uint16_t* y16, uint8_t* ys,
                              hipStream_t stream) {
    constexpr int kBlockFrags = kGateUp ? WR : 2 * WR;
    const int ntl = (NOUT / 32 + kBlockFrags - 1) / kBlockFrags;
    const size_t lds = gemm_lds_bytes(K, kGateUp);
    if (lds > 65536) {
        const hipError_t er = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&expert_gemm_kernel<kGateUp, WR, kPacked>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (er != hipSuccess) return er;
    }
    hipLaunchKernelGGL((expert_gemm_kernel<kGateUp, WR, kPacked>),
                       dim3((unsigned)gemm_grid(p.max_tiles, ntl)), dim3(64 * WR), lds, stream,
                       bq, sorted, p.k, wq, ws, tiles, p.max_tiles, ntl, K, NOUT, p.F, hq, y16,
                       ys);
    return hipSuccess;
}

hipError_t launch_mlp_gemm(const MlpPlan& p, bool packed, const uint16_t* x, const uint8_t* w13q,
                           const uint8_t* w13s, const uint8_t* w2q, const uint8_t* w2s,
                           const int32_t* offsets, const int32_t* sorted, uint16_t* y16,
                           uint8_t* ys, char* base,
                           hipEvent_t* events, hipStream_t stream) {
    uint8_t* xq = reinterpret_cast<uint8_t*>(base + p.off_xq);
    uint8_t* hq = reinterpret_cast<uint8_t*>(base + p.off_h);
    int32_t* tiles = reinterpret_cast<int32_t*>(base + p.off_tiles);
    const int64_t nsplit = (int64_t)p.T * (p.D / 64);
    constexpr int kSplitThreads = 64 * kSplitWaves;
    hipLaunchKernelGGL(split_terms_kernel,
                       dim3((unsigned)((nsplit + kSplitThreads - 1) / kSplitThreads + 1)),
                       dim3(kSplitThreads), 0,
                       stream, x, p.T, p.D, xq, offsets, p.E, p.max_tiles, tiles);
    if (events) {
        const hipError_t er = hipEventRecord(events[0], stream);
        if (er != hipSuccess) return er;
    }
    hipError_t er;
    er = packed ? launch_gemm<true, kGateUpWaves, true>(p, xq, sorted, w13q, w13s, tiles, p.D,
                                                        p.F, hq, nullptr, nullptr, stream)
                : launch_gemm<true, kGateUpWaves, false>(p, xq, sorted, w13q, w13s, tiles, p.D,
                                                         p.F, hq, nullptr, nullptr, stream);
    if (er != hipSuccess) return er;
    if (events) {
        er = hipEventRecord(events[1], stream);
        if (er != hipSuccess) return er;
    }
    er = packed ? launch_gemm<false, kDownWaves, true>(p, hq, nullptr, w2q, w2s, tiles, p.F, p.D,
                                                       nullptr, y16, ys, stream)
                : launch_gemm<false, kDownWaves, false>(p, hq, nullptr, w2q, w2s, tiles, p.F, p.D,
                                                        nullptr, y16, ys, stream);
    if (er != hipSuccess) return er;
    return hipGetLastError();
}

}  // namespace moe
