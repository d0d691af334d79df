// launch.h -- internal launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_quantize(const uint16_t* w, int64_t rows, int64_t K, int rule, int rounding,
                           uint64_t seed, uint8_t* q, uint8_t* s, hipStream_t stream);
hipError_t launch_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t K,
                             uint16_t* out, hipStream_t stream);
hipError_t launch_pack(const uint8_t* q, int64_t rows, int64_t K, uint8_t* out,
                       hipStream_t stream);

struct RoutePlan {
    int T, D, E, k;
    int token_tiles;   // 16-token tiles per router block
    int expert_tiles;  // 16-expert tiles per router block
    int splits;        // slices of the router contraction (partial logits summed in order)
    int chunks;        // token chunks of the top-k / histogram pass
    size_t off_logits, off_chunk_counts, off_chunk_base, ws_bytes;
};
RoutePlan plan_route(int T, int D, int E, int k);
hipError_t launch_route(const RoutePlan& p, const uint16_t* x, const float* wr, const float* br,
                        int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                        int32_t* sorted, int32_t* pos, float* logits_out, void* ws,
                        hipStream_t stream);

// Workspace of moe_expert_mlp: y (fp32 [P, D], both paths) followed by the
// scratch of whichever path runs (the two share one region).
struct MlpPlan {
    int T, D, F, E, k;
    bool gemm_ok;        // grouped-GEMM path possible: D % 64 == 0 and F % 64 == 0
    bool gemm_auto;      // grouped-GEMM path chosen when the caller leaves it open
    bool stream_ok;      // the streaming kernels take the shape (their LDS budget)
    bool packed_ok;      // packed weights accepted: both algorithms take the shape
    int max_tiles;       // upper bound of 128-pair tiles over all experts
    size_t off_y;
    size_t off_h;                                    // h fp16 [P, F]
    size_t off_xq, off_tiles;                        // grouped GEMM: x terms, tile table
    size_t ws_bytes;
};
MlpPlan plan_mlp(int T, int D, int F, int E, int k);
// algo: 0 = automatic, 1 = weight streaming, 2 = grouped GEMM (requires gemm_ok);
// packed: w13q and w2q in the mxfp4_pack layout (requires packed_ok)
hipError_t launch_mlp(const MlpPlan& p, int algo, bool packed, const uint16_t* x, const uint8_t* w13q,
                      const uint8_t* w13s, const uint8_t* w2q, const uint8_t* w2s,
                      const float* topk_w, const int32_t* offsets, const int32_t* sorted,
                      const int32_t* pos, uint16_t* out, void* ws, hipEvent_t* events,
                      hipStream_t stream);

// grouped-GEMM path (expert_gemm.hip)
int gemm_max_tiles(int T, int E, int k);
size_t gemm_term_bytes(int rows, int K, int NT);
size_t gemm_lds_bytes(int K, bool gate_up, int stage, int wr);
constexpr size_t kGemmMaxLds = 157 * 1024;    // of 160 KiB; the rest is static LDS
constexpr int kGemmMaxContraction = 8192;      // D and F limit of the grouped GEMM
hipError_t launch_mlp_gemm(const MlpPlan& p, bool packed, const uint16_t* x, const uint8_t* w13q,
                           const uint8_t* w13s, const uint8_t* w2q, const uint8_t* w2s,
                           const int32_t* offsets, const int32_t* sorted, float* y, char* base,
                           hipEvent_t* events, hipStream_t stream);

}  // namespace moe
