// api.hip -- the exported C ABI of libmoe_mxfp4 (declared in
// include/moe_mxfp4.h): argument validation, the device check, workspace
// carving, launches.  Every check happens before anything is enqueued.
#include <atomic>
#include <cstring>

#include "moe_mxfp4.h"
#include "launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The device a call's work would run on (the stream's, or the current one
// for the null stream) must be a gfx950.  The answer is cached per device
// id: 0 = not asked yet, 1 = gfx950, 2 = something else.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_kind[kMaxDevices];

moe_status_t check_device(hipStream_t stream) {
    int dev = -1;
    if (stream) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) return MOE_ERR_DEVICE;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return MOE_ERR_DEVICE;
    }
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
    int kind = g_device_kind[dev].load(std::memory_order_acquire);
    if (kind == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_DEVICE;
        // gcnArchName is e.g. "gfx950:sramecc+:xnack-"
        kind = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                       (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':')
                   ? 1 : 2;
        g_device_kind[dev].store(kind, std::memory_order_release);
    }
    return kind == 1 ? MOE_OK : MOE_ERR_DEVICE;
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

bool route_shape_ok(int32_t T, int32_t D, int32_t E, int32_t k) {
    if (T < 1 || D < 32 || D % 32 != 0 || E < 1 || E > 256 || k < 1 || k > 8 || k > E)
        return false;
    return (int64_t)T * k < ((int64_t)1 << 31) && (int64_t)T * D < ((int64_t)1 << 40);
}

// ---------------------------------------------------------------------------
// Workspace of moe_expert_mlp_noalloc: a fixed device array, one copy per
// GPU (each device holds its own at its own address until the process ends).
// Host code never uses the array's name as an address: the device address
// is looked up once per device with hipGetSymbolAddress (that device
// current) and kept in g_scratch.
// ---------------------------------------------------------------------------
__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch[kMaxDevices];

// Device of `stream` (the current device for the null stream), or -1.
int stream_device(hipStream_t stream) {
    int dev = -1;
    if (stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) return -1;
    return dev >= 0 && dev < kMaxDevices ? dev : -1;
}

// This device's copy of `scratch`, or nullptr if its address cannot be had.
void* scratch_on(int dev) {
    void* ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    const hipError_t er = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (er != hipSuccess) return nullptr;
    g_scratch[dev].store(ptr, std::memory_order_release);
    return ptr;
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
        case MOE_ERR_DEVICE: return "no gfx950 (MI355X) device for the stream";
        case MOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        default: return "unknown status";
    }
}

int moe_abi_version(void) { return MOE_ABI_VERSION; }

moe_status_t mxfp4_quantize_ex(const uint16_t* w, int64_t rows, int64_t K, uint8_t* q,
                               uint8_t* s, int scale_rule, int rounding, uint64_t seed,
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
    if (const moe_status_t d = check_device(stream)) return d;
    return hip_status(moe::launch_quantize(w, rows, K, scale_rule, rounding, seed, q, s, stream));
}

moe_status_t mxfp4_quantize(const uint16_t* w, int64_t rows, int64_t K, uint8_t* q, uint8_t* s,
                            int scale_rule, hipStream_t stream) {
    return mxfp4_quantize_ex(w, rows, K, q, s, scale_rule, MXFP4_ROUND_NEAREST_EVEN, 0, stream);
}

moe_status_t mxfp4_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t K,
                              uint16_t* out, hipStream_t stream) {
    if (rows < 0 || K <= 0 || K % 32 != 0) return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!q || !s || !out) return MOE_ERR_NULL;
    if (!aligned16(q) || !aligned16(out)) return MOE_ERR_ALIGN;
    if (const moe_status_t d = check_device(stream)) return d;
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
    if (const moe_status_t d = check_device(stream)) return d;
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
    if (const moe_status_t d = check_device(stream)) return d;
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
                            hipStream_t stream) {
    return moe_expert_mlp_ex(x, w13_q, w13_s, w2_q, w2_s, topk_w, offsets, sorted_pairs,
                             pair_pos, T, D, F, E, k, out, ws, ws_bytes, MOE_MLP_AUTO, nullptr,
                             stream);
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
    if (!x || !w13_q || !w13_s || !w2_q || !w2_s || !topk_w || !offsets || !sorted_pairs ||
        !pair_pos || !out)
        return MOE_ERR_NULL;
    const moe::MlpPlan plan = moe::plan_mlp(T, D, F, E, k);
    if (base == MOE_MLP_GROUPED_GEMM && !plan.gemm_ok) return MOE_ERR_SHAPE;
    if (base == MOE_MLP_STREAM && !plan.stream_ok) return MOE_ERR_SHAPE;
    if (base == MOE_MLP_AUTO && !plan.stream_ok && !plan.gemm_ok) return MOE_ERR_SHAPE;
    if (packed && !plan.packed_ok) return MOE_ERR_SHAPE;
    if (!ws || ws_bytes < plan.ws_bytes) return MOE_ERR_WORKSPACE;
    if (!aligned16(x) || !aligned16(w13_q) || !aligned16(w13_s) || !aligned16(w2_q) ||
        !aligned16(w2_s) || !aligned16(out) || !aligned16(ws))
        return MOE_ERR_ALIGN;
    if (const moe_status_t d = check_device(stream)) return d;
    return hip_status(moe::launch_mlp(plan, base, packed, x, w13_q, w13_s, w2_q, w2_s, topk_w,
                                      offsets, sorted_pairs, pair_pos, out, ws, stage_events,
                                      stream));
}

size_t moe_expert_mlp_bf16_workspace_size(int32_t T, int32_t D, int32_t F, int32_t E,
                                          int32_t k) {
    if (!route_shape_ok(T, D, E, k) || F < 32 || F % 32 != 0) return 0;
    return moe::bf16_mlp_workspace_bytes(T, D, F, k);
}

moe_status_t moe_expert_mlp_bf16_ex(const uint16_t* x, const uint16_t* w13, const uint16_t* w2,
                                    const float* topk_w, const int32_t* offsets,
                                    const int32_t* sorted_pairs, const int32_t* pair_pos,
                                    int32_t T, int32_t D, int32_t F, int32_t E, int32_t k,
                                    uint16_t* out, void* ws, size_t ws_bytes,
                                    hipEvent_t* stage_events, hipStream_t stream) {
    if (!route_shape_ok(T, D, E, k) || F < 32 || F % 32 != 0) return MOE_ERR_SHAPE;
    if (!x || !w13 || !w2 || !topk_w || !offsets || !sorted_pairs || !pair_pos || !out)
        return MOE_ERR_NULL;
    if (!ws || ws_bytes < moe::bf16_mlp_workspace_bytes(T, D, F, k)) return MOE_ERR_WORKSPACE;
    if (!aligned16(x) || !aligned16(w13) || !aligned16(w2) || !aligned16(out) || !aligned16(ws))
        return MOE_ERR_ALIGN;
    if (const moe_status_t d = check_device(stream)) return d;
    return hip_status(moe::launch_mlp_bf16(T, D, F, E, k, x, w13, w2, topk_w, offsets,
                                           sorted_pairs, pair_pos, out, ws, stage_events,
                                           stream));
}

moe_status_t moe_expert_mlp_bf16(const uint16_t* x, const uint16_t* w13, const uint16_t* w2,
                                 const float* topk_w, const int32_t* offsets,
                                 const int32_t* sorted_pairs, const int32_t* pair_pos, int32_t T,
                                 int32_t D, int32_t F, int32_t E, int32_t k, uint16_t* out,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
    return moe_expert_mlp_bf16_ex(x, w13, w2, topk_w, offsets, sorted_pairs, pair_pos, T, D, F,
                                  E, k, out, ws, ws_bytes, nullptr, stream);
}

size_t moe_layer_decode_workspace_size(int32_t T, int32_t D, int32_t F, int32_t E, int32_t k) {
    if (!route_shape_ok(T, D, E, k) || F < 32 || F % 32 != 0) return 0;
    const moe::DecodePlan p = moe::plan_decode(T, D, F, E, k);
    return p.ok ? p.ws_bytes : 0;
}

moe_status_t moe_layer_decode_init(void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!ws) return MOE_ERR_NULL;
    if (ws_bytes < moe::kDecodeCtlBytes) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    if (const moe_status_t d = check_device(stream)) return d;
    return hip_status(moe::decode_init(ws, stream));
}

moe_status_t moe_layer_decode_ex(const uint16_t* x, const float* wr, const float* br,
                                 const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                                 const uint8_t* w2_s, int32_t T, int32_t D, int32_t F, int32_t E,
                                 int32_t k, int32_t* topk_ids, float* topk_w, int32_t* counts,
                                 int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                                 uint16_t* out, void* ws, size_t ws_bytes, int flags,
                                 int32_t spin_limit, hipEvent_t* stage_events,
                                 hipStream_t stream) {
    if (flags != 0 && flags != MOE_MLP_WEIGHTS_PACKED) return MOE_ERR_ENUM;
    if (!route_shape_ok(T, D, E, k) || F < 32 || F % 32 != 0 || spin_limit < 0)
        return MOE_ERR_SHAPE;
    const moe::DecodePlan plan = moe::plan_decode(T, D, F, E, k);
    const bool packed = flags == MOE_MLP_WEIGHTS_PACKED;
    if (!plan.ok || (packed && !plan.mlp.packed_ok)) return MOE_ERR_SHAPE;
    if (!x || !wr || !w13_q || !w13_s || !w2_q || !w2_s || !topk_ids || !topk_w || !counts ||
        !offsets || !sorted_pairs || !pair_pos || !out)
        return MOE_ERR_NULL;
    if (!ws || ws_bytes < plan.ws_bytes) return MOE_ERR_WORKSPACE;
    if (!aligned16(x) || !aligned16(wr) || !aligned16(w13_q) || !aligned16(w13_s) ||
        !aligned16(w2_q) || !aligned16(w2_s) || !aligned16(out) || !aligned16(ws))
        return MOE_ERR_ALIGN;
    if (const moe_status_t d = check_device(stream)) return d;
    return hip_status(moe::launch_decode(plan, packed, x, wr, br, w13_q, w13_s, w2_q, w2_s,
                                         topk_ids, topk_w, counts, offsets, sorted_pairs,
                                         pair_pos, out, ws, spin_limit, stage_events, stream));
}

moe_status_t moe_layer_decode(const uint16_t* x, const float* wr, const float* br,
                              const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                              const uint8_t* w2_s, int32_t T, int32_t D, int32_t F, int32_t E,
                              int32_t k, int32_t* topk_ids, float* topk_w, int32_t* counts,
                              int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                              uint16_t* out, void* ws, size_t ws_bytes, int flags,
                              hipStream_t stream) {
    return moe_layer_decode_ex(x, wr, br, w13_q, w13_s, w2_q, w2_s, T, D, F, E, k, topk_ids,
                               topk_w, counts, offsets, sorted_pairs, pair_pos, out, ws, ws_bytes,
                               flags, 1 << 20, nullptr, stream);
}

moe_status_t moe_layer_decode_error(const void* ws, int32_t* error, hipStream_t stream) {
    if (!ws || !error) return MOE_ERR_NULL;
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    if (const moe_status_t d = check_device(stream)) return d;
    const int32_t* word = static_cast<const int32_t*>(ws) + moe::kDecodeCtlErr;
    hipError_t er = hipMemcpyAsync(error, word, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (er == hipSuccess) er = hipStreamSynchronize(stream);
    return hip_status(er);
}

moe_status_t moe_expert_mlp_noalloc(const uint16_t* x, const uint8_t* w13_q,
                                    const uint8_t* w13_s, const uint8_t* w2_q,
                                    const uint8_t* w2_s, const float* topk_w,
                                    const int32_t* offsets, const int32_t* sorted_pairs,
                                    const int32_t* pair_pos, int32_t T, int32_t D, int32_t F,
                                    int32_t E, int32_t k, uint16_t* out, int algo,
                                    hipStream_t stream) {
    const bool packed = (algo & MOE_MLP_WEIGHTS_PACKED) != 0;
    const int base = algo & ~MOE_MLP_WEIGHTS_PACKED;
    if (base != MOE_MLP_AUTO && base != MOE_MLP_STREAM && base != MOE_MLP_GROUPED_GEMM)
        return MOE_ERR_ENUM;
    if (!route_shape_ok(T, D, E, k) || F < 32 || F % 32 != 0) return MOE_ERR_SHAPE;
    if (!x || !w13_q || !w13_s || !w2_q || !w2_s || !topk_w || !offsets || !sorted_pairs ||
        !pair_pos || !out)
        return MOE_ERR_NULL;
    const moe::MlpPlan plan = moe::plan_mlp(T, D, F, E, k);
    if (base == MOE_MLP_GROUPED_GEMM && !plan.gemm_ok) return MOE_ERR_SHAPE;
    if (base == MOE_MLP_STREAM && !plan.stream_ok) return MOE_ERR_SHAPE;
    if (base == MOE_MLP_AUTO && !plan.stream_ok && !plan.gemm_ok) return MOE_ERR_SHAPE;
    if (packed && !plan.packed_ok) return MOE_ERR_SHAPE;
    if (plan.ws_bytes > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    if (!aligned16(x) || !aligned16(w13_q) || !aligned16(w13_s) || !aligned16(w2_q) ||
        !aligned16(w2_s) || !aligned16(out))
        return MOE_ERR_ALIGN;
    if (const moe_status_t d = check_device(stream)) return d;
    const int dev = stream_device(stream);
    void* ws = dev < 0 ? nullptr : scratch_on(dev);
    if (!ws) return MOE_ERR_HIP;
    return hip_status(moe::launch_mlp(plan, base, packed, x, w13_q, w13_s, w2_q, w2_s, topk_w,
                                      offsets, sorted_pairs, pair_pos, out, ws, nullptr, stream));
}

}  // extern "C"

