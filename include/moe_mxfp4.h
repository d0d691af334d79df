/*
 * moe_mxfp4.h -- C ABI of libmoe_mxfp4, a GPT-OSS-style mixture-of-experts
 * MLP layer with MXFP4 expert weights, written for AMD MI355X (gfx950).
 *
 * The layer (page sources by title and section):
 *  - MXFP4 storage: 4-bit E2M1 elements (1 sign, 2 exponent, 1 mantissa bit)
 *    with one shared scale per block of 32 elements.  "Tricks from OpenAI
 *    gpt-oss you can use with transformers" (pogovet.com summary) section 6;
 *    "Transformers 4.40 のパフォーマンス向上" section "MXFP4 とは"; the
 *    format is the OCP Microscaling one ("MXFP4 기반 MoE 기술 리뷰" section 1),
 *    whose shared scale is an E8M0 power of two.
 *  - Token-choice routing, top-k experts, softmax over the selected experts
 *    only, SwiGLU experts: "Welcome GPT OSS" (pogovet.com summary) section 4;
 *    k = 4 of 32 or 128 experts: the aitrends.kr talk summary, section
 *    "Architecture details: MoE and attention"; no shared expert: same page,
 *    Q&A section.
 *  - Weights stay in the 4-bit format and are widened only inside the
 *    arithmetic (GEMMs that understand blocks and scales): "Tricks" section 8;
 *    talk summary section "Hardware optimisation: Triton and Metal kernels".
 *
 * Conventions for every call:
 *  - All array pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *    tensors), row-major and contiguous, 16-byte aligned.  bf16 values are
 *    passed as their uint16_t bit patterns.  Outputs must not alias inputs.
 *  - The caller owns every buffer, including the workspace.  The library never
 *    allocates, frees or synchronises, and keeps no mutable global state; a
 *    call only enqueues kernels on `stream` and returns.  Calls that run
 *    concurrently on different streams need separate workspaces.
 *  - Argument errors are detected before anything is enqueued and returned
 *    as a status; outputs are then untouched.  A failed launch returns
 *    MOE_ERR_HIP (outputs undefined).  Device faults surface at the caller's
 *    next synchronisation, as usual in HIP.
 *  - Results are deterministic: identical inputs give bit-identical outputs.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,       /* a required pointer is NULL */
    MOE_ERR_SHAPE = 2,      /* a size is out of range or not a multiple of 32 */
    MOE_ERR_WORKSPACE = 3,  /* workspace NULL or smaller than *_workspace_size */
    MOE_ERR_ENUM = 4,       /* unknown scale rule or expert-MLP algorithm */
    MOE_ERR_HIP = 5,        /* a kernel launch failed */
    MOE_ERR_ALIGN = 6       /* a pointer is not 16-byte aligned */
} moe_status_t;

/* How a block's shared exponent s is chosen from its largest magnitude amax.
 * Both clamp s to [-127, 127]; an all-zero block gets s = -127 (byte 0). */
typedef enum {
    MXFP4_SCALE_FLOOR_DIV6 = 0, /* s = floor(log2(amax / 6)): the block maximum
                                   scales into [6, 12) and saturates to 6 */
    MXFP4_SCALE_OCP = 1,        /* s = floor(log2(amax)) - 2 (OCP MX v1.0) */
    MXFP4_SCALE_CEIL_DIV6 = 2   /* s = ceil(log2(amax / 6)): the smallest scale
                                   at which no element exceeds 6 */
} mxfp4_scale_rule_t;

/* Element rounding of mxfp4_quantize_ex. */
typedef enum {
    MXFP4_ROUND_NEAREST_EVEN = 0,
    MXFP4_ROUND_STOCHASTIC = 1  /* see mxfp4_quantize_ex */
} mxfp4_rounding_t;

/* How moe_expert_mlp_ex runs the experts (moe_expert_mlp: automatic). */
typedef enum {
    MOE_MLP_AUTO = 0,          /* grouped GEMM when it takes the shape (see
                                  MOE_MLP_GROUPED_GEMM) and T*k >= 32*E (32 pairs
                                  per expert on average), weight streaming
                                  otherwise */
    MOE_MLP_STREAM = 1,        /* weight streaming: each touched expert's weights
                                  are read once per group of 16 of its pairs */
    MOE_MLP_GROUPED_GEMM = 2,  /* tiled grouped GEMM over 128-pair tiles; needs
                                  D % 64 == 0, F % 64 == 0, D <= 8192, F <= 7232
                                  (LDS budget), and T*(D/64)*144, T*k*F*2 and
                                  E*F*D under 4 GiB (32-bit offsets), else
                                  MOE_ERR_SHAPE */
    MOE_MLP_WEIGHTS_PACKED = 0x100  /* flag, OR-ed into the algorithm: w13_q and w2_q
                                  are in the layout mxfp4_pack writes (the scales
                                  are unchanged); needs D % 64 == 0, F % 64 == 0
                                  and a shape both algorithms take (the streaming
                                  kernels' LDS budget: D <= 3840, F <= 2944),
                                  else MOE_ERR_SHAPE */
} moe_mlp_algo_t;

/* Human-readable name of a status code (static string). */
MOE_API const char *moe_status_string(int status);

/* ABI version of this header (bumped on any incompatible change). */
MOE_API int moe_abi_version(void);

/*
 * mxfp4_quantize -- bf16 rows to MXFP4.
 *   w      [rows, K] bf16 bits
 *   q      [rows, K/2] uint8: element 2i in the low nibble of byte i,
 *          element 2i+1 in the high nibble; each nibble is an E2M1 code
 *   s      [rows, K/32] uint8 E8M0 scales: byte b means 2^(b-127)
 * Per 32-element block: s from the rule; each element v becomes the E2M1
 * code nearest to v * 2^-s, ties to the even code, saturating at +-6, sign
 * kept (so -0 and small negatives give code 0x8).
 * Preconditions: finite inputs; rows >= 0; K > 0 and K % 32 == 0.
 * Errors: MOE_ERR_SHAPE, MOE_ERR_NULL (rows > 0 with a NULL pointer),
 * MOE_ERR_ENUM, MOE_ERR_ALIGN, MOE_ERR_HIP.  rows == 0 enqueues nothing.
 */
MOE_API moe_status_t mxfp4_quantize(const uint16_t *w, int64_t rows, int64_t K,
                            int scale_rule, uint8_t *q, uint8_t *s,
                            hipStream_t stream);

/*
 * mxfp4_quantize_ex -- mxfp4_quantize with the element rounding chosen.
 * MXFP4_ROUND_STOCHASTIC (the stochastic-rounding training recipe cited in
 * "MXFP4 기반 MoE (Mixture-of-Experts) 기술 리뷰", section 2; the pages give
 * no details, the reading here): element i = row * K + col, scaled to
 * y = v * 2^-s, takes the upper of its two neighbouring E2M1 values
 * lo <= |y| < hi when u < 2^24 (|y| - lo) / (hi - lo), else the lower one,
 * where u is the top 24 bits of output i + 1 of a SplitMix64 generator whose
 * state starts at `seed` (state += 0x9E3779B97F4A7C15, output = the mix64
 * finalizer of java.util.SplittableRandom); |y| >= 6 saturates; sign kept.
 * With MXFP4_SCALE_CEIL_DIV6 no element saturates, so the expected
 * dequantized value equals the input.  The same seed gives the same codes.
 * Errors as for mxfp4_quantize (MOE_ERR_ENUM also for an unknown rounding).
 */
MOE_API moe_status_t mxfp4_quantize_ex(const uint16_t *w, int64_t rows, int64_t K,
                            int scale_rule, int rounding, uint64_t seed,
                            uint8_t *q, uint8_t *s, hipStream_t stream);

/*
 * mxfp4_pack -- reorder MXFP4 codes for the expert kernels (done once, when
 * the weights are loaded).
 *   q    [rows, K/2] codes as mxfp4_quantize writes them
 *   out  [rows, K/2] bytes: for each 32-row fragment f and 64-element
 *        contraction step t, the fragment's 32 rows x 32 bytes of that step
 *        form one contiguous 1 KiB chunk, chunks in (f, t) order; inside a
 *        chunk the first 32-element half (16 bytes) of rows 0..31 comes
 *        first, then the second half of rows 0..31:
 *        out[(f*K/64 + t)*1024 + h*512 + r*16 + b] = q[(32f + r)*K/2 + 32t + 16h + b]
 *        (h in {0, 1}, r in [0, 32), b in [0, 16))
 * The expert kernels then read each matrix-core operand fragment (one
 * 16-byte piece per lane) as one contiguous 1 KiB load instead of 32 row
 * pieces.  The E8M0 scales keep their layout.  Preconditions: rows % 32 == 0, K % 64 == 0, out does not overlap q.
 * Errors: MOE_ERR_SHAPE, MOE_ERR_NULL, MOE_ERR_ALIGN, MOE_ERR_HIP.
 */
MOE_API moe_status_t mxfp4_pack(const uint8_t *q, int64_t rows, int64_t K, uint8_t *out,
                                hipStream_t stream);

/*
 * mxfp4_dequantize -- MXFP4 to bf16 (exact for every scale byte in
 * [1, 252]; the value e2m1 * 2^(b-127) is then a bf16 number).
 *   q [rows, K/2], s [rows, K/32] as produced by mxfp4_quantize
 *   out [rows, K] bf16 bits
 * Errors as for mxfp4_quantize.
 */
MOE_API moe_status_t mxfp4_dequantize(const uint8_t *q, const uint8_t *s, int64_t rows,
                              int64_t K, uint16_t *out, hipStream_t stream);

/*
 * moe_route -- router of a token-choice MoE layer.
 *   x        [T, D] bf16 bits, activations
 *   wr       [E, D] fp32 router weight
 *   br       [E] fp32 router bias, or NULL for zero bias
 * Outputs:
 *   topk_ids     [T, k] int32: the k experts with the largest logits
 *                logit = x[t] . wr[e] + br[e] (fp32), in descending logit
 *                order, equal logits ordered by lower expert id
 *   topk_w       [T, k] fp32: softmax over the k selected logits only
 *   counts       [E] int32: pairs routed to each expert
 *   offsets      [E+1] int32: exclusive prefix sum of counts (offsets[E] = T*k)
 *   sorted_pairs [T*k] int32: pair ids p = t*k + j grouped by expert, in
 *                increasing p inside each expert (stable counting sort)
 *   pair_pos     [T*k] int32: inverse permutation, sorted_pairs[pair_pos[p]] = p
 *   logits_out   [T, E] fp32, or NULL to skip
 *   ws, ws_bytes workspace of at least moe_route_workspace_size(T, D, E, k)
 * Preconditions: 1 <= T, 32 <= D, D % 32 == 0, 1 <= E <= 256,
 * 1 <= k <= min(E, 8), T*k < 2^31, finite inputs.
 * Errors: MOE_ERR_SHAPE, MOE_ERR_NULL, MOE_ERR_WORKSPACE, MOE_ERR_ALIGN,
 * MOE_ERR_HIP.
 */
MOE_API size_t moe_route_workspace_size(int32_t T, int32_t D, int32_t E, int32_t k);
MOE_API moe_status_t moe_route(const uint16_t *x, const float *wr, const float *br,
                       int32_t T, int32_t D, int32_t E, int32_t k,
                       int32_t *topk_ids, float *topk_w, int32_t *counts,
                       int32_t *offsets, int32_t *sorted_pairs,
                       int32_t *pair_pos, float *logits_out, void *ws,
                       size_t ws_bytes, hipStream_t stream);

/*
 * moe_expert_mlp -- the experts and the weighted combine.
 *   x        [T, D] bf16 bits
 *   w13_q    [E, 2F, D/2] MXFP4 codes, w13_s [E, 2F, D/32] E8M0 scales:
 *            rows 0..F-1 are the gate projection, rows F..2F-1 the up
 *            projection, blocks run along D
 *   w2_q     [E, D, F/2], w2_s [E, D, F/32]: the down projection, blocks
 *            along F
 *   topk_w, offsets, sorted_pairs, pair_pos: as written by moe_route
 *   out      [T, D] bf16 bits
 * For each routed pair p = t*k + j with expert e = the expert of p:
 *   g = Wg_e x_t, u = Wu_e x_t, h = silu(g) * u, y_p = W2_e h,
 *   out[t] = sum over j = 0..k-1 (in slot order) of topk_w[t, j] * y_p.
 * Arithmetic: the weights enter the gfx950 block-scaled matrix-core product
 * as stored (E2M1 codes, with their E8M0 block scales as the hardware scale
 * operand); the activations enter it as fp8 (E4M3) residual terms, each with
 * its own E8M0 scale per 32-element block: x as 2 terms (exact for bf16), h
 * as 3 terms (h rounded to fp16 first on the weight-streaming path, split
 * from fp32 on the grouped-GEMM path); fp32 accumulation and combine; output
 * rounded to bf16.  (With D or F above 4096 the streaming path widens the
 * weights instead: to bf16 for gate/up, exactly, and to fp16 for down, exact
 * for scale bytes in [104, 140].)
 * Preconditions: as moe_route, plus 32 <= F, F % 32 == 0, the routing arrays
 * consistent with each other (as moe_route writes them).
 * stage_events: NULL, or 4 events recorded on `stream` before the gate/up
 * kernel, after it, after the down kernel and after the combine kernel.
 * Errors: MOE_ERR_SHAPE, MOE_ERR_NULL, MOE_ERR_WORKSPACE, MOE_ERR_ALIGN,
 * MOE_ERR_HIP.  The workspace size covers both algorithms.
 * moe_expert_mlp_ex: the same with the algorithm chosen by the caller
 * (moe_mlp_algo_t); MOE_ERR_ENUM for an unknown value.
 */
MOE_API size_t moe_expert_mlp_workspace_size(int32_t T, int32_t D, int32_t F,
                                     int32_t E, int32_t k);
MOE_API moe_status_t moe_expert_mlp(const uint16_t *x, const uint8_t *w13_q,
                            const uint8_t *w13_s, const uint8_t *w2_q,
                            const uint8_t *w2_s, const float *topk_w,
                            const int32_t *offsets,
                            const int32_t *sorted_pairs,
                            const int32_t *pair_pos, int32_t T, int32_t D,
                            int32_t F, int32_t E, int32_t k, uint16_t *out,
                            void *ws, size_t ws_bytes,
                            hipEvent_t *stage_events, hipStream_t stream);
MOE_API moe_status_t moe_expert_mlp_ex(const uint16_t *x, const uint8_t *w13_q,
                            const uint8_t *w13_s, const uint8_t *w2_q,
                            const uint8_t *w2_s, const float *topk_w,
                            const int32_t *offsets,
                            const int32_t *sorted_pairs,
                            const int32_t *pair_pos, int32_t T, int32_t D,
                            int32_t F, int32_t E, int32_t k, uint16_t *out,
                            void *ws, size_t ws_bytes, int algo,
                            hipEvent_t *stage_events, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
