// decode.hip -- the fused decode front for gfx950: the router and the gate/up
// weight stream of the MXFP4 MoE layer in one launch.
//
// In a decode step the router ("Welcome GPT OSS", section 4: token-choice
// top-k with softmax over the selected logits) is a few microseconds of
// latency-bound work, and until it is done no expert knows its tokens.  The
// weights, though, do not depend on the routing: here the expert blocks issue
// their first weight batches first and only then wait for the routing, so
// the routing's latency overlaps the start of the weight stream (the pages
// ask that kernels be measured on the real workload, batch size included:
// "Tricks from OpenAI gpt-oss", section 4).
//
// One launch, three roles by block index:
//   [0, NL)        router tiles: the partial logits of router_logits_tile
//                  (the same tiles and arithmetic as moe_route), then one
//                  arrival on the control block;
//   NL             the routing block: waits for the NL arrivals, then runs
//                  route_small_body (top-k, softmax, histogram, scan, stable
//                  scatter: the same outputs as moe_route, bit for bit) and
//                  publishes them;
//   NL + 1 + b     gate/up block b of the weight-streaming kernel: issues its
//                  first weight batch, waits for the routing, then runs as
//                  expert_stream_kernel's block b (reading the routing's
//                  indices with agent-scope atomic loads).
// Blocks that wait only wait for blocks of lower index, which the dispatcher
// places first, so the launch needs no co-residency guarantee.  Every wait is
// bounded (spin_limit polls): a wait that gives up sets the sticky error word
// of the control block, and the routing block then publishes an empty
// routing (no pairs for any expert, identity permutation) so that every later
// kernel stays in bounds.
//
// Control block (4 ints at the start of the workspace, zeroed by
// moe_layer_decode_init): arrivals, ready (1 = routing published, 2 = given
// up), passed (expert blocks past their wait), error.  A completed call
// leaves the first three at zero: the routing block clears the arrivals once
// it has seen all of them, and the last expert block past its wait clears
// ready and passed.
#include <algorithm>

#include "device_common.h"
#include "launch.h"
#include "route_device.h"
#include "stream_device.h"

namespace moe {

namespace {

enum { kArrive = 0, kReady = 1, kPassed = 2, kErr = 3 };
static_assert(kErr == kDecodeCtlErr, "error word index");

__device__ __forceinline__ int ctl_load(int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ctl_store(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll *p until it is at least `target`, at most spin_limit times after the
// first look (about 0.1 us apart); returns the last value read.
__device__ __forceinline__ int wait_at_least(int* p, int target, int spin_limit) {
    int v = ctl_load(p);
    for (int i = 0; v < target && i < spin_limit; ++i) {
        __builtin_amdgcn_s_sleep(4);
        v = ctl_load(p);
    }
    return v;
}

// Every thread's global writes so far have reached L2 (each wave waits for
// all its memory operations) before anything the block does after the
// barrier; the caller's thread 0 then publishes with an agent-scope release
// (one L2 write-back for the block).
__device__ __forceinline__ void publish_block() {
    __builtin_amdgcn_s_waitcnt(0);      // every memory operation of this wave done
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
}

}  // namespace

template <int K, bool kPacked>
__global__ __launch_bounds__(kStreamWaves * 64) void decode_front_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ br,
    float* __restrict__ P, int rx, int ry, int S, int T, int D, int F, int E,
    int32_t* __restrict__ ids, float* __restrict__ wts, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted, int32_t* __restrict__ pos,
    const uint8_t* __restrict__ w13q, const uint8_t* __restrict__ w13s, int bpe,
    float* __restrict__ h, int* __restrict__ ctl, int spin_limit) {
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ int s_row[16];
    __shared__ int s_flag;
    const int NL = rx * ry * S;
    const int b = blockIdx.x, tid = threadIdx.x;

    if (b < NL) {
        // router tile (bx, by, bz) on wavefronts 0 .. 3; the others meet the
        // tile's one block barrier
        const int bx = b % rx, by = (b / rx) % ry, bz = b / (rx * ry);
        if ((tid >> 6) < kRouterWaves)
            router_logits_tile<1, 1, 4, false>(x, wr, br, P, T, D, E, S, bx, by, bz,
                                               reinterpret_cast<f32x4_t*>(lds));
        else
            __syncthreads();
        publish_block();
        if (tid == 0) __hip_atomic_fetch_add(&ctl[kArrive], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    if (b == NL) {
        // (thread 0's acquire invalidates this CU's L1 and its L2's stale
        // lines, which all of the block's loads after the barrier go through)
        if (tid == 0) {
            s_flag = wait_at_least(&ctl[kArrive], NL, spin_limit) >= NL;
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
        const bool ok = s_flag;
        if (ok) {
            route_small_body<K, kStreamWaves>(P, S, T, E, nullptr, ids, wts, counts, offsets,
                                              sorted, pos, *reinterpret_cast<SmallRouteLds*>(lds));
        } else {
            // given up: an empty routing keeps the later kernels in bounds
            const int npairs = T * K;
            for (int i = tid; i <= E; i += blockDim.x) {
                offsets[i] = 0;
                if (i < E) counts[i] = 0;
            }
            for (int i = tid; i < npairs; i += blockDim.x) {
                ids[i] = 0;
                wts[i] = 0.f;
                sorted[i] = i;
                pos[i] = i;
            }
        }
        publish_block();
        if (tid == 0) {
            if (ok) {
                ctl_store(&ctl[kArrive], 0);        // every router block has arrived
            } else {
                __hip_atomic_fetch_or(&ctl[kErr], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __hip_atomic_store(&ctl[kReady], ok ? 1 : 2, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }

    const int nexp = E * bpe;
    auto wait_routing = [&]() -> bool {
        if (tid == 0) {
            const int v = wait_at_least(&ctl[kReady], 1, spin_limit);
            if (v != 1)
                __hip_atomic_fetch_or(&ctl[kErr], 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (__hip_atomic_fetch_add(&ctl[kPassed], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                nexp - 1) {
                ctl_store(&ctl[kPassed], 0);
                ctl_store(&ctl[kReady], 0);
            }
            s_flag = v == 1;
        }
        __syncthreads();
        return s_flag != 0;
    };
    expert_stream_body<true, kPacked, true>(x, w13q, w13s, offsets, sorted, D, F, E, K, bpe, h,
                                            b - NL - 1, lds, s_row, wait_routing);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

DecodePlan plan_decode(int T, int D, int F, int E, int k) {
    DecodePlan p{};
    p.route = plan_route(T, D, E, k);
    p.mlp = plan_mlp(T, D, F, E, k);
    p.ok = T <= kSmallTokens && T * E <= kSmallLogits && p.mlp.stream_ok &&
           p.route.token_tiles == 1 && p.route.expert_tiles == 1;
    p.router_blocks = ((E + 15) / 16) * ((T + 15) / 16) * p.route.splits;
    p.gate_up_bpe = stream_blocks_gate_up(p.mlp);
    p.off_partials = kDecodeCtlBytes;
    p.off_mlp = align256(p.off_partials + (size_t)p.route.splits * T * E * sizeof(float));
    // the streaming path's part of the MLP workspace: y, then fp32 h
    p.ws_bytes = p.off_mlp + align256(p.mlp.off_h + (size_t)T * k * F * sizeof(float));
    return p;
}

hipError_t decode_init(void* ws, hipStream_t stream) {
    return hipMemsetAsync(ws, 0, kDecodeCtlBytes, stream);
}

template <int K, bool kPacked>
static hipError_t launch_front(const DecodePlan& p, const uint16_t* x, const float* wr,
                               const float* br, const uint8_t* w13q, const uint8_t* w13s,
                               int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                               int32_t* sorted, int32_t* pos, char* base, int spin_limit,
                               hipStream_t stream) {
    const int T = p.mlp.T, D = p.mlp.D, E = p.mlp.E;
    size_t lds = stream_lds_bytes(D, 2, 2);
    lds = std::max(lds, sizeof(SmallRouteLds));
    lds = std::max(lds, (size_t)kRouterWaves * 64 * sizeof(f32x4_t));
    auto* kern = &decode_front_kernel<K, kPacked>;
    if (lds > 65536) {
        const hipError_t er = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                                  (int)lds);
        if (er != hipSuccess) return er;
    }
    const int blocks = p.router_blocks + 1 + E * p.gate_up_bpe;
    float* P = reinterpret_cast<float*>(base + p.off_partials);
    float* h = reinterpret_cast<float*>(base + p.off_mlp + p.mlp.off_h);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kStreamWaves * 64), lds, stream, x, wr,
                       br, P, (E + 15) / 16, (T + 15) / 16, p.route.splits, T, D, p.mlp.F, E,
                       ids, w, counts, offsets, sorted, pos, w13q, w13s, p.gate_up_bpe, h,
                       reinterpret_cast<int*>(base), spin_limit);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodePlan& p, bool packed, const uint16_t* x, const float* wr,
                         const float* br, const uint8_t* w13q, const uint8_t* w13s,
                         const uint8_t* w2q, const uint8_t* w2s, int32_t* ids, float* w,
                         int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* pos,
                         uint16_t* out, void* ws, int spin_limit, hipEvent_t* events,
                         hipStream_t stream) {
    char* base = static_cast<char*>(ws);
    hipError_t er;
    if (events && (er = hipEventRecord(events[0], stream)) != hipSuccess) return er;
    switch (p.mlp.k * 2 + (packed ? 1 : 0)) {
#define MOE_DECODE_FRONT(KK)                                                                  \
    case KK * 2:                                                                              \
        er = launch_front<KK, false>(p, x, wr, br, w13q, w13s, ids, w, counts, offsets, sorted, \
                                     pos, base, spin_limit, stream);                          \
        break;                                                                                \
    case KK * 2 + 1:                                                                          \
        er = launch_front<KK, true>(p, x, wr, br, w13q, w13s, ids, w, counts, offsets, sorted,  \
                                    pos, base, spin_limit, stream);                           \
        break;
        MOE_DECODE_FRONT(1) MOE_DECODE_FRONT(2) MOE_DECODE_FRONT(3) MOE_DECODE_FRONT(4)
        MOE_DECODE_FRONT(5) MOE_DECODE_FRONT(6) MOE_DECODE_FRONT(7) MOE_DECODE_FRONT(8)
#undef MOE_DECODE_FRONT
        default: return hipErrorInvalidValue;
    }
    if (er != hipSuccess) return er;
    if (events && (er = hipEventRecord(events[1], stream)) != hipSuccess) return er;
    float* y = reinterpret_cast<float*>(base + p.off_mlp + p.mlp.off_y);
    const float* h = reinterpret_cast<const float*>(base + p.off_mlp + p.mlp.off_h);
    er = launch_stream_down(p.mlp, packed, h, w2q, w2s, offsets, sorted, y, stream);
    if (er != hipSuccess) return er;
    return launch_combine_slots(p.mlp.T, p.mlp.D, p.mlp.k, y, w, out, events, stream);
}

}  // namespace moe
