// api.hip -- the exported C ABI of libmoe_mxfp4 (declared in
// include/moe_mxfp4.h): argument validation, workspace carving, launches.
// Every check happens before anything is enqueued.
#include "moe_mxfp4.h"
#include "launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

bool route_shape_ok(int32_t T, int32_t D, int32_t E, int32_t k) {
    if (T < 1 || D < 32 || D % 32 != 0 || E < 1 || E > 256 || k < 1 || k > 8 || k > E)
        return false;
    return (int64_t)T * k < ((int64_t)1 << 31) && (int64_t)T * D < ((int64_t)1 << 40);
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "a size is out of range or not a multiple of 32";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_ENUM: return "unknown scale rule or algorithm";
        case MOE_ERR_HIP: return "kernel launch failed";
        case MOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        default: return "unknown status";
    }
}

int moe_abi_version(void) { return 1; }

moe_status_t mxfp4_quantize_ex(const uint16_t* w, int64_t rows, int64_t K, int scale_rule,
                               int rounding, uint64_t seed, uint8_t* q, uint8_t* s,
                               hipStream_t stream) {
    if (rows < 0 || K <= 0 || K % 32 != 0) return MOE_ERR_SHAPE;
    if (scale_rule != MXFP4_SCALE_FLOOR_DIV6 && scale_rule != MXFP4_SCALE_OCP &&
        scale_rule != MXFP4_SCALE_CEIL_DIV6)
        return MOE_ERR_ENUM;
    if (rounding != MXFP4_ROUND_NEAREST_EVEN && rounding != MXFP4_ROUND_STOCHASTIC)
        return MOE_ERR_ENUM;
    if (rows == 0) return MOE_OK;
    if (!w || !q || !s) return MOE_ERR_NULL;
    if (!aligned16(w) || !aligned16(q)) return MOE_ERR_ALIGN;
    return hip_status(moe::launch_quantize(w, rows, K, scale_rule, rounding, seed, q, s, stream));
}

moe_status_t mxfp4_quantize(const uint16_t* w, int64_t rows, int64_t K, int scale_rule,
                            uint8_t* q, uint8_t* s, hipStream_t stream) {
    return mxfp4_quantize_ex(w, rows, K, scale_rule, MXFP4_ROUND_NEAREST_EVEN, 0, q, s, stream);
}

moe_status_t mxfp4_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t K,
                              uint16_t* out, hipStream_t stream) {
    if (rows < 0 || K <= 0 || K % 32 != 0) return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!q || !s || !out) return MOE_ERR_NULL;
    if (!aligned16(q) || !aligned16(out)) return MOE_ERR_ALIGN;
    return hip_status(moe::launch_dequantize(q, s, rows, K, out, stream));
}

moe_status_t mxfp4_pack(const uint8_t* q, int64_t rows, int64_t K, uint8_t* out,
                        hipStream_t stream) {
    if (rows < 0 || K <= 0 || K % 64 != 0 || rows % 32 != 0) return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!q || !out) return MOE_ERR_NULL;
    if (!aligned16(q) || !aligned16(out)) return MOE_ERR_ALIGN;
    const uintptr_t a0 = (uintptr_t)q, a1 = a0 + (uintptr_t)(rows * (K / 2));
    const uintptr_t b0 = (uintptr_t)out, b1 = b0 + (uintptr_t)(rows * (K / 2));
    if (a0 < b1 && b0 < a1) return MOE_ERR_SHAPE;       // in place or overlapping
    return hip_status(moe::launch_pack(q, rows, K, out, stream));
}

size_t moe_route_workspace_size(int32_t T, int32_t D, int32_t E, int32_t k) {
    if (!route_shape_ok(T, D, E, k)) return 0;
    return moe::plan_route(T, D, E, k).ws_bytes;
}

moe_status_t moe_route(const uint16_t* x, const float* wr, const float* br, int32_t T,
                       int32_t D, int32_t E, int32_t k, int32_t* topk_ids, float* topk_w,
                       int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                       int32_t* pair_pos, float* logits_out, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    if (!route_shape_ok(T, D, E, k)) return MOE_ERR_SHAPE;
    if (!x || !wr || !topk_ids || !topk_w || !counts || !offsets || !sorted_pairs || !pair_pos)
        return MOE_ERR_NULL;
    const moe::RoutePlan plan = moe::plan_route(T, D, E, k);
    if (!ws || ws_bytes < plan.ws_bytes) return MOE_ERR_WORKSPACE;
    if (!aligned16(x) || !aligned16(wr) || !aligned16(ws)) return MOE_ERR_ALIGN;
    return hip_status(moe::launch_route(plan, x, wr, br, topk_ids, topk_w, counts, offsets,
                                        sorted_pairs, pair_pos, logits_out, ws, stream));
}

size_t moe_expert_mlp_workspace_size(int32_t T, int32_t D, int32_t F, int32_t E, int32_t k) {
    if (!route_shape_ok(T, D, E, k) || F < 32 || F % 32 != 0) return 0;
    return moe::plan_mlp(T, D, F, E, k).ws_bytes;
}

moe_status_t moe_expert_mlp(const uint16_t* x, const uint8_t* w13_q, const uint8_t* w13_s,
                            const uint8_t* w2_q, const uint8_t* w2_s, const float* topk_w,
                            const int32_t* offsets, const int32_t* sorted_pairs,
                            const int32_t* pair_pos, int32_t T, int32_t D, int32_t F,
                            int32_t E, int32_t k, uint16_t* out, void* ws, size_t ws_bytes,
                            hipEvent_t* stage_events, hipStream_t stream) {
    return moe_expert_mlp_ex(x, w13_q, w13_s, w2_q, w2_s, topk_w, offsets, sorted_pairs,
                             pair_pos, T, D, F, E, k, out, ws, ws_bytes, MOE_MLP_AUTO,
                             stage_events, stream);
}

moe_status_t moe_expert_mlp_ex(const uint16_t* x, const uint8_t* w13_q, const uint8_t* w13_s,
                               const uint8_t* w2_q, const uint8_t* w2_s, const float* topk_w,
                               const int32_t* offsets, const int32_t* sorted_pairs,
                               const int32_t* pair_pos, int32_t T, int32_t D, int32_t F,
                               int32_t E, int32_t k, uint16_t* out, void* ws, size_t ws_bytes,
                               int algo, hipEvent_t* stage_events, hipStream_t stream) {
    const bool packed = (algo & MOE_MLP_WEIGHTS_PACKED) != 0;
    const int base = algo & ~MOE_MLP_WEIGHTS_PACKED;
    if (base != MOE_MLP_AUTO && base != MOE_MLP_STREAM && base != MOE_MLP_GROUPED_GEMM)
        return MOE_ERR_ENUM;
    if (!route_shape_ok(T, D, E, k) || F < 32 || F % 32 != 0) return MOE_ERR_SHAPE;
    if (base == MOE_MLP_GROUPED_GEMM && (D % 64 != 0 || F % 64 != 0)) return MOE_ERR_SHAPE;
    if (!x || !w13_q || !w13_s || !w2_q || !w2_s || !topk_w || !offsets || !sorted_pairs ||
        !pair_pos || !out)
        return MOE_ERR_NULL;
    const moe::MlpPlan plan = moe::plan_mlp(T, D, F, E, k);
    if (base == MOE_MLP_GROUPED_GEMM && !plan.gemm_ok) return MOE_ERR_SHAPE;
    if (packed && !plan.packed_ok) return MOE_ERR_SHAPE;
    if (!ws || ws_bytes < plan.ws_bytes) return MOE_ERR_WORKSPACE;
    if (!aligned16(x) || !aligned16(w13_q) || !aligned16(w13_s) || !aligned16(w2_q) ||
        !aligned16(w2_s) || !aligned16(out) || !aligned16(ws))
        return MOE_ERR_ALIGN;
    return hip_status(moe::launch_mlp(plan, base, packed, x, w13_q, w13_s, w2_q, w2_s, topk_w,
                                      offsets, sorted_pairs, pair_pos, out, ws, stage_events,
                                      stream));
}

}  // extern "C"
