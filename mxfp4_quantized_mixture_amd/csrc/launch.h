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
    bool gemm_router;   // longer batches: router_gemm_kernel
    int gemm_router_ne; // its 16-expert tiles per block (2 or 4)
};
RoutePlan plan_route(int T, int D, int E, int k);
hipError_t launch_route(const RoutePlan& p, const uint16_t* x, const float* wr, const float* br,
                        int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                        int32_t* sorted, int32_t* pos, float* logits_out, void* ws,
                        hipStream_t stream);

// Workspace of moe_expert_mlp: y (fp32 [P, D] in slot order for weight streaming; fp16
// [P, D] plus a scale byte per 32 outputs for the grouped GEMM), h (fp32 [P, F]
// for weight streaming, fp6 term rows for the grouped GEMM: one region),
// then the grouped GEMM's x term rows and tile table.
struct MlpPlan {
    int T, D, F, E, k;
    bool gemm_ok;        // grouped-GEMM path possible (D, F % 64 == 0, LDS, 32-bit offsets)
    bool gemm_auto;      // grouped-GEMM path chosen when the caller leaves it open
    bool stream_ok;      // the streaming kernels take the shape (their LDS budget)
    bool packed_ok;      // packed weights accepted: both algorithms take the shape
    int max_tiles;       // upper bound of 128-pair tiles over all experts
    size_t off_y;
    size_t off_ys;       // grouped GEMM: y as fp16 at off_y, its scale bytes here
    size_t off_h;
    size_t off_xq, off_tiles;                        // grouped GEMM: x terms, tile table
    size_t ws_bytes;
};
MlpPlan plan_mlp(int T, int D, int F, int E, int k);
// algo: 0 = automatic, 1 = weight streaming (requires stream_ok), 2 = grouped
// GEMM (requires gemm_ok); packed: w13q and w2q in the mxfp4_pack layout
// (requires packed_ok)
hipError_t launch_mlp(const MlpPlan& p, int algo, bool packed, const uint16_t* x, const uint8_t* w13q,
                      const uint8_t* w13s, const uint8_t* w2q, const uint8_t* w2s,
                      const float* topk_w, const int32_t* offsets, const int32_t* sorted,
                      const int32_t* pos, uint16_t* out, void* ws, hipEvent_t* events,
                      hipStream_t stream);

// grouped-GEMM path (expert_gemm.hip)
int gemm_max_tiles(int T, int E, int k);
size_t gemm_h_bytes(int64_t P, int F);   // h term rows of the grouped GEMM, with slack
size_t gemm_term_bytes(int rows, int K);
size_t gemm_lds_bytes(int K, bool gate_up);
constexpr size_t kGemmMaxLds = 157 * 1024;    // of 160 KiB; the rest is static LDS
constexpr int kGemmMaxContraction = 8192;      // D and F limit of the grouped GEMM
hipError_t launch_mlp_gemm(const MlpPlan& p, bool packed, const uint16_t* x, const uint8_t* w13q,
                           const uint8_t* w13s, const uint8_t* w2q, const uint8_t* w2s,
                           const int32_t* offsets, const int32_t* sorted, uint16_t* y16,
                           uint8_t* ys, char* base,
                           hipEvent_t* events, hipStream_t stream);

// the streaming down kernel alone (h fp32 [P, F] in pair order -> y fp32
// [P, D] in slot order: the pair of slot j of token t at row t k + j), and
// the streaming gate/up kernel's blocks per expert (expert_mlp.hip)
hipError_t launch_stream_down(const MlpPlan& p, bool packed, const float* h, const uint8_t* w2q,
                              const uint8_t* w2s, const int32_t* offsets, const int32_t* sorted,
                              float* y, hipStream_t stream);
int stream_blocks_gate_up(const MlpPlan& p);

// out[t] = bf16(sum_j topk_w[t, j] y[pos[t k + j]]), slots in order
// (expert_mlp.hip); events, if given, are recorded as stage events 2 and 3
hipError_t launch_combine_rows(int T, int D, int k, const float* y, const float* topk_w,
                               const int32_t* pos, uint16_t* out, hipEvent_t* events,
                               hipStream_t stream);
// out[t] = bf16(sum_j topk_w[t, j] y[t k + j]), slots in order, over y in
// slot order (expert_mlp.hip); events as above
hipError_t launch_combine_slots(int T, int D, int k, const float* y, const float* topk_w,
                                uint16_t* out, hipEvent_t* events, hipStream_t stream);

// bf16-weight comparison path (expert_bf16.hip): workspace = y fp32 [P, D]
// then h fp32 [P, F]
size_t bf16_mlp_workspace_bytes(int T, int D, int F, int k);
hipError_t launch_mlp_bf16(int T, int D, int F, int E, int k, const uint16_t* x,
                           const uint16_t* w13, const uint16_t* w2, const float* topk_w,
                           const int32_t* offsets, const int32_t* sorted, const int32_t* pos,
                           uint16_t* out, void* ws, hipEvent_t* events, hipStream_t stream);

// Fused decode front (decode.hip): router and gate/up weight stream in one
// launch, then the streaming down kernel and the combine.  Workspace: a
// 256-byte control block (zeroed once by decode_init), the router's partial
// logits, then the streaming path's y and h.
struct DecodePlan {
    RoutePlan route;
    MlpPlan mlp;
    bool ok;                 // shape taken (T <= 64, T E <= 8192, streaming shapes)
    int router_blocks;       // router tiles (one per block)
    int gate_up_bpe;         // gate/up blocks per expert
    size_t off_partials, off_mlp, ws_bytes;
};
DecodePlan plan_decode(int T, int D, int F, int E, int k);
hipError_t decode_init(void* ws, hipStream_t stream);
hipError_t launch_decode(const DecodePlan& p, bool packed, const uint16_t* x, const float* wr,
                         const float* br, const uint8_t* w13q, const uint8_t* w13s,
                         const uint8_t* w2q, const uint8_t* w2s, int32_t* ids, float* w,
                         int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* pos,
                         uint16_t* out, void* ws, int spin_limit, hipEvent_t* events,
                         hipStream_t stream);
constexpr size_t kDecodeCtlBytes = 256;
constexpr int kDecodeCtlErr = 3;      // int index of the sticky error word in the control block

}  // namespace moe
