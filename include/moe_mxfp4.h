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
 *    allocates, frees or synchronises; a call only enqueues kernels on
 *    `stream` and returns.  Its only global state is a per-device cache of
 *    the device check below and, for moe_expert_mlp_noalloc, one fixed
 *    device array per GPU.  Calls that run concurrently on different
 *    streams need separate workspaces.
 *  - Argument errors are detected before anything is enqueued and returned
 *    as a status; outputs are then untouched.  After the arguments, every
 *    call that would enqueue work checks that the device `stream` belongs to
 *    (the current device for the null stream) is a gfx950, else returns
 *    MOE_ERR_DEVICE.  A failed launch returns MOE_ERR_HIP (outputs
 *    undefined).  Device faults surface at the caller's next
 *    synchronisation, as usual in HIP.
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

/* Version of this ABI; moe_abi_version() returns it.  Bumped on any
 * incompatible change (2: status codes and argument order of the contract,
 * stage events only in moe_expert_mlp_ex). */
#define MOE_ABI_VERSION 4

/* Size of the fixed device workspace of moe_expert_mlp_noalloc (16 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,       /* a required pointer is NULL */
    MOE_ERR_SHAPE = 2,      /* a size is out of range or not a multiple of 32,
                               or no kernel of the library takes the shape */
    MOE_ERR_WORKSPACE = 3,  /* workspace NULL or smaller than *_workspace_size */
    MOE_ERR_ENUM = 4,       /* unknown scale rule, rounding or algorithm */
    MOE_ERR_HIP = 5,        /* a HIP call or kernel launch failed */
    MOE_ERR_DEVICE = 6,     /* the stream's device is not a gfx950 (or none) */
    MOE_ERR_ALIGN = 7       /* a pointer is not 16-byte aligned */
} moe_status_t;

/* How a block's shared exponent s is chosen from its largest magnitude amax.
 * The pages give no rule ("Tricks" section 6 and "MXFP4 とは" name only the
 * shared power-of-two scale per 32 elements).  All clamp s to [-127, 127];
 * an all-zero block gets s = -127 (byte 0). */
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
    MOE_MLP_AUTO = 0,          /* grouped GEMM when it takes the shape and
                                  T*k >= 32*E (32 pairs per expert on average)
                                  or the streaming kernels cannot take it;
                                  weight streaming otherwise */
    MOE_MLP_STREAM = 1,        /* weight streaming: each touched expert's weights
                                  are read once per group of 16 of its pairs;
                                  needs D <= 3840 and F <= 2944 (LDS budget),
                                  else MOE_ERR_SHAPE */
    MOE_MLP_GROUPED_GEMM = 2,  /* tiled grouped GEMM over 128-pair tiles; needs
                                  D % 64 == 0, F % 64 == 0, D and F <= 8192,
                                  and T*(D/64)*160, T*k*(F/64)*160 and E*F*D
                                  under 4 GiB (32-bit offsets), else
                                  MOE_ERR_SHAPE */
    MOE_MLP_WEIGHTS_PACKED = 0x100  /* flag, OR-ed into the algorithm: w13_q and w2_q
                                  are in the layout mxfp4_pack writes (the scales
                                  are unchanged); needs a shape both algorithms
                                  take, else MOE_ERR_SHAPE */
} moe_mlp_algo_t;

/* Human-readable name of a status code (static string). */
MOE_API const char *moe_status_string(int status);

/* MOE_ABI_VERSION of the built library. */
MOE_API int moe_abi_version(void);

/*
 * mxfp4_quantize -- bf16 rows to MXFP4: 4-bit E2M1 codes plus one E8M0 scale
 * per 32-element block ("Tricks" section 6; "MXFP4 とは"; OCP MX per
 * "MXFP4 기반 MoE 기술 리뷰" section 1; the layer keeps its expert weights in
 * this form, "Welcome GPT OSS" section 4).
 *   w      [rows, K] bf16 bits (read only)
 *   q      [rows, K/2] uint8 (written): element 2i in the low nibble of byte
 *          i, element 2i+1 in the high nibble; each nibble an E2M1 code
 *   s      [rows, K/32] uint8 (written) E8M0 scales: byte b means 2^(b-127)
 *   scale_rule  mxfp4_scale_rule_t
 * Per 32-element block: s from the rule; each element v becomes the E2M1
 * code nearest to v * 2^-s, ties to the even code, saturating at +-6, sign
 * kept (so -0 and small negatives give code 0x8).
 * Preconditions: finite inputs; rows >= 0; K > 0 and K % 32 == 0; w and q
 * 16-byte aligned.  rows == 0 enqueues nothing and returns MOE_OK.
 * Errors: MOE_ERR_SHAPE, MOE_ERR_NULL (rows > 0 with a NULL pointer),
 * MOE_ERR_ENUM, MOE_ERR_ALIGN, MOE_ERR_DEVICE, MOE_ERR_HIP.
 */
MOE_API moe_status_t mxfp4_quantize(const uint16_t *w, int64_t rows, int64_t K,
                                    uint8_t *q, uint8_t *s, int scale_rule,
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
 * Arguments, preconditions and errors as for mxfp4_quantize (MOE_ERR_ENUM
 * also for an unknown rounding).
 */
MOE_API moe_status_t mxfp4_quantize_ex(const uint16_t *w, int64_t rows, int64_t K,
                                       uint8_t *q, uint8_t *s, int scale_rule,
                                       int rounding, uint64_t seed, hipStream_t stream);

/*
 * mxfp4_pack -- reorder MXFP4 codes for the expert kernels (done once, when
 * the weights are loaded).  Not an operation of the pages: the pages keep
 * MXFP4 blocks and scales row-major ("Tricks" section 6); this layout only
 * makes each gfx950 matrix-core operand fragment one contiguous load.
 *   q    [rows, K/2] codes as mxfp4_quantize writes them (read only)
 *   out  [rows, K/2] bytes (written): for each 32-row fragment f and
 *        64-element contraction step t, the fragment's 32 rows x 32 bytes of
 *        that step form one contiguous 1 KiB chunk, chunks in (f, t) order;
 *        inside a chunk the first 32-element half (16 bytes) of rows 0..31
 *        comes first, then the second half of rows 0..31:
 *        out[(f*K/64 + t)*1024 + h*512 + r*16 + b] = q[(32f + r)*K/2 + 32t + 16h + b]
 *        (h in {0, 1}, r in [0, 32), b in [0, 16))
 * The E8M0 scales keep their layout.  Preconditions: rows % 32 == 0,
 * K % 64 == 0, out does not overlap q, both 16-byte aligned.
 * Errors: MOE_ERR_SHAPE, MOE_ERR_NULL, MOE_ERR_ALIGN, MOE_ERR_DEVICE,
 * MOE_ERR_HIP.
 */
MOE_API moe_status_t mxfp4_pack(const uint8_t *q, int64_t rows, int64_t K, uint8_t *out,
                                hipStream_t stream);

/*
 * mxfp4_dequantize -- MXFP4 to bf16: value = e2m1(code) * 2^(b-127)
 * ("Tricks" section 6: weights are widened only when they are used; a test
 * helper here).  Exact for every scale byte in [1, 252] (the value is then a
 * bf16 number).
 *   q [rows, K/2], s [rows, K/32] as produced by mxfp4_quantize (read only)
 *   out [rows, K] bf16 bits (written)
 * Errors as for mxfp4_quantize.
 */
MOE_API moe_status_t mxfp4_dequantize(const uint8_t *q, const uint8_t *s, int64_t rows,
                                      int64_t K, uint16_t *out, hipStream_t stream);

/*
 * moe_route -- router of a token-choice MoE layer: logits, top-k, softmax
 * over the selected logits only ("Welcome GPT OSS" section 4; k = 4 per the
 * talk summary's architecture block), then the grouping of the routed
 * (token, slot) pairs by expert that the grouped expert GEMMs read (a stable
 * counting sort; the pages do not spell it out).
 *   x        [T, D] bf16 bits, activations (read only)
 *   wr       [E, D] fp32 router weight (read only)
 *   br       [E] fp32 router bias, or NULL for zero bias (read only)
 * Outputs (written):
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
 *                bytes (scratch: contents on entry do not matter)
 * Preconditions: 1 <= T, 32 <= D, D % 32 == 0, 1 <= E <= 256,
 * 1 <= k <= min(E, 8), T*k < 2^31, finite inputs; x, wr, ws 16-byte aligned.
 * Errors: MOE_ERR_SHAPE, MOE_ERR_NULL, MOE_ERR_WORKSPACE, MOE_ERR_ALIGN,
 * MOE_ERR_DEVICE, MOE_ERR_HIP.
 * moe_route_workspace_size returns 0 for shapes moe_route rejects.
 */
MOE_API size_t moe_route_workspace_size(int32_t T, int32_t D, int32_t E, int32_t k);
MOE_API moe_status_t moe_route(const uint16_t *x, const float *wr, const float *br,
                               int32_t T, int32_t D, int32_t E, int32_t k,
                               int32_t *topk_ids, float *topk_w, int32_t *counts,
                               int32_t *offsets, int32_t *sorted_pairs,
                               int32_t *pair_pos, float *logits_out, void *ws,
                               size_t ws_bytes, hipStream_t stream);

/*
 * moe_expert_mlp -- the experts and the weighted combine: SwiGLU experts on
 * MXFP4 weights, their outputs summed with the softmax-after-topk weights
 * ("Welcome GPT OSS" section 4; no shared expert, talk summary Q&A), with
 * the weights widened only inside the matrix-core products ("Tricks"
 * section 8).
 *   x        [T, D] bf16 bits (read only)
 *   w13_q    [E, 2F, D/2] MXFP4 codes, w13_s [E, 2F, D/32] E8M0 scales
 *            (read only): rows 0..F-1 are the gate projection, rows F..2F-1
 *            the up projection, blocks run along D
 *   w2_q     [E, D, F/2], w2_s [E, D, F/32] (read only): the down
 *            projection, blocks along F
 *   topk_w, offsets, sorted_pairs, pair_pos: as written by moe_route
 *   out      [T, D] bf16 bits (written)
 *   ws, ws_bytes workspace of at least moe_expert_mlp_workspace_size(T, D,
 *            F, E, k) bytes (scratch; the size covers both algorithms)
 * For each routed pair p = t*k + j with expert e = the expert of p:
 *   g = Wg_e x_t, u = Wu_e x_t, h = silu(g) * u, y_p = W2_e h,
 *   out[t] = sum over j = 0..k-1 (in slot order) of topk_w[t, j] * y_p.
 * Arithmetic: the weights enter the gfx950 block-scaled matrix-core products
 * as stored (E2M1 codes, with their E8M0 block scales as the hardware scale
 * operand); the activations enter them as residual terms with their own
 * E8M0 scale per 32-element block, so no intermediate has a range limit
 * narrower than fp32's:
 *  - weight streaming (few pairs per expert): x as 2 E4M3 terms (exact for
 *    bf16 elements within 13 binades of their block's largest magnitude,
 *    error below 2^-21 of it further down); h kept in fp32 and carried as 3
 *    E4M3 terms (relative error below 2^-12 within those 13 binades);
 *  - grouped GEMM: x and h each as 3 E2M3 (fp6) terms (error below 2^-12 of
 *    the block's largest magnitude); h goes from fp32 straight to its terms;
 *    each pair's down output y is held as fp16 with one power-of-two scale
 *    per 32 outputs that brings their largest magnitude into [2^14, 2^15)
 *    (error below 2^-11 of it, no range limit);
 * fp32 accumulation and combine; output rounded to bf16 (nearest even).
 * Preconditions: as moe_route, plus 32 <= F, F % 32 == 0, a shape one of the
 * algorithms takes (see moe_mlp_algo_t), the routing arrays consistent with
 * each other (as moe_route writes them); all pointers 16-byte aligned.
 * Errors: MOE_ERR_SHAPE, MOE_ERR_NULL, MOE_ERR_WORKSPACE, MOE_ERR_ALIGN,
 * MOE_ERR_DEVICE, MOE_ERR_HIP.
 * moe_expert_mlp_workspace_size returns 0 for shapes the layer rejects.
 *
 * moe_expert_mlp_ex -- the same with the algorithm chosen by the caller
 * (moe_mlp_algo_t; MOE_ERR_ENUM for an unknown value) and optional
 * instrumentation: stage_events is NULL, or 4 events recorded on `stream`
 * before the gate/up kernel, after it, after the down kernel and after the
 * combine kernel (for per-stage timing; a few microseconds per record).
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
                                    void *ws, size_t ws_bytes, hipStream_t stream);
MOE_API moe_status_t moe_expert_mlp_ex(const uint16_t *x, const uint8_t *w13_q,
                                       const uint8_t *w13_s, const uint8_t *w2_q,
                                       const uint8_t *w2_s, const float *topk_w,
                                       const int32_t *offsets,
                                       const int32_t *sorted_pairs,
                                       const int32_t *pair_pos, int32_t T, int32_t D,
                                       int32_t F, int32_t E, int32_t k, uint16_t *out,
                                       void *ws, size_t ws_bytes, int algo,
                                       hipEvent_t *stage_events, hipStream_t stream);

/*
 * moe_expert_mlp_bf16 -- the same layer (steps and combine as moe_expert_mlp)
 * on bf16 expert weights: the fallback the pages name for hardware without
 * MXFP4 kernels, at about four times the weight bytes ("Tricks" section 7;
 * Japanese Transformers page, "メモリ削減効果").  A comparison path: it lets
 * both weight formats run on the same layer and be measured side by side.
 *   x        [T, D] bf16 bits (read only)
 *   w13      [E, 2F, D] bf16 bits (read only): rows 0..F-1 gate, F..2F-1 up
 *   w2       [E, D, F] bf16 bits (read only)
 *   topk_w, offsets, sorted_pairs, pair_pos: as written by moe_route
 *   out      [T, D] bf16 bits (written)
 *   ws, ws_bytes workspace of at least moe_expert_mlp_bf16_workspace_size(T,
 *            D, F, E, k) bytes (scratch)
 * Arithmetic: weight streaming on bf16 matrix-core products (each expert's
 * weights are read once per group of 16 of its pairs: meant for decode-sized
 * batches); x and the weights enter exactly, products are exact and
 * accumulate in fp32; h is kept in fp32 and enters the down products as two
 * bf16 terms (error below 2^-17 of |h|); y and the combine in fp32; output
 * rounded to bf16 (nearest even).
 * Preconditions: as moe_route, plus 32 <= F, F % 32 == 0, the routing arrays
 * consistent with each other; x, w13, w2, out and ws 16-byte aligned.
 * Errors: MOE_ERR_SHAPE, MOE_ERR_NULL, MOE_ERR_WORKSPACE, MOE_ERR_ALIGN,
 * MOE_ERR_DEVICE, MOE_ERR_HIP.  moe_expert_mlp_bf16_workspace_size returns 0
 * for shapes the call rejects.
 *
 * moe_expert_mlp_bf16_ex -- the same with optional instrumentation:
 * stage_events is NULL or 4 events, recorded as for moe_expert_mlp_ex.
 */
MOE_API size_t moe_expert_mlp_bf16_workspace_size(int32_t T, int32_t D, int32_t F,
                                                  int32_t E, int32_t k);
MOE_API moe_status_t moe_expert_mlp_bf16(const uint16_t *x, const uint16_t *w13,
                                         const uint16_t *w2, const float *topk_w,
                                         const int32_t *offsets,
                                         const int32_t *sorted_pairs,
                                         const int32_t *pair_pos, int32_t T, int32_t D,
                                         int32_t F, int32_t E, int32_t k, uint16_t *out,
                                         void *ws, size_t ws_bytes, hipStream_t stream);
MOE_API moe_status_t moe_expert_mlp_bf16_ex(const uint16_t *x, const uint16_t *w13,
                                            const uint16_t *w2, const float *topk_w,
                                            const int32_t *offsets,
                                            const int32_t *sorted_pairs,
                                            const int32_t *pair_pos, int32_t T, int32_t D,
                                            int32_t F, int32_t E, int32_t k, uint16_t *out,
                                            void *ws, size_t ws_bytes,
                                            hipEvent_t *stage_events, hipStream_t stream);

/*
 * moe_layer_decode -- the whole layer for a decode-sized batch (moe_route
 * followed by moe_expert_mlp with weight streaming) with the routing fused
 * into the gate/up weight stream: one launch computes the router logits,
 * the top-k routing and the gate/up experts, its expert blocks issuing
 * their first weight loads before the routing is known and waiting for it
 * on the device; the down experts and the combine follow as two more
 * kernels.  Same layer and arithmetic as moe_route + moe_expert_mlp_ex
 * (MOE_MLP_STREAM): every output, the routing arrays included, is
 * bit-identical to theirs ("Welcome GPT OSS" section 4; "Tricks" section 4:
 * kernels measured on the real, small-batch workload).
 *   x, wr, br          as moe_route;  w13_q, w13_s, w2_q, w2_s as
 *                      moe_expert_mlp (flags: 0 or MOE_MLP_WEIGHTS_PACKED)
 *   topk_ids, topk_w, counts, offsets, sorted_pairs, pair_pos
 *                      written as moe_route writes them
 *   out                [T, D] bf16 bits (written)
 *   ws, ws_bytes       workspace of at least moe_layer_decode_workspace_size
 *                      bytes whose first 256 bytes (the control block) were
 *                      zeroed by moe_layer_decode_init; every successful call
 *                      leaves them so.  Calls that overlap on one workspace
 *                      race.
 * Preconditions: as moe_route and moe_expert_mlp, plus T <= 64,
 * T * E <= 8192 and a shape the streaming kernels take (D <= 3840 and
 * F <= 2944, their LDS budget; with packed codes also D % 64 == 0 and
 * F % 64 == 0).
 * Device-side waits are bounded: if one gives up (a launch whose blocks
 * could not all make progress), the call's outputs are invalid, an error is
 * recorded in the control block (read with moe_layer_decode_error), all
 * later kernels of the call stay in bounds, and the workspace must be
 * initialised again before the next call.
 * Errors: MOE_ERR_SHAPE, MOE_ERR_NULL, MOE_ERR_WORKSPACE, MOE_ERR_ENUM,
 * MOE_ERR_ALIGN, MOE_ERR_DEVICE, MOE_ERR_HIP.
 *
 * moe_layer_decode_init -- zero the control block (enqueued on stream).
 * moe_layer_decode_ex -- the same with spin_limit (polls per device-side
 * wait, about 0.1 us apart; moe_layer_decode uses 1 << 20) and optional
 * stage events as for moe_expert_mlp_ex (before the fused launch, after it,
 * after the down kernel, after the combine).
 * moe_layer_decode_error -- wait for `stream`, then store the control
 * block's error word in *error (0: no wait gave up since the last init).
 */
MOE_API size_t moe_layer_decode_workspace_size(int32_t T, int32_t D, int32_t F, int32_t E,
                                               int32_t k);
MOE_API moe_status_t moe_layer_decode_init(void *ws, size_t ws_bytes, hipStream_t stream);
MOE_API moe_status_t moe_layer_decode(const uint16_t *x, const float *wr, const float *br,
                                      const uint8_t *w13_q, const uint8_t *w13_s,
                                      const uint8_t *w2_q, const uint8_t *w2_s, int32_t T,
                                      int32_t D, int32_t F, int32_t E, int32_t k,
                                      int32_t *topk_ids, float *topk_w, int32_t *counts,
                                      int32_t *offsets, int32_t *sorted_pairs,
                                      int32_t *pair_pos, uint16_t *out, void *ws,
                                      size_t ws_bytes, int flags, hipStream_t stream);
MOE_API moe_status_t moe_layer_decode_ex(const uint16_t *x, const float *wr, const float *br,
                                         const uint8_t *w13_q, const uint8_t *w13_s,
                                         const uint8_t *w2_q, const uint8_t *w2_s, int32_t T,
                                         int32_t D, int32_t F, int32_t E, int32_t k,
                                         int32_t *topk_ids, float *topk_w, int32_t *counts,
                                         int32_t *offsets, int32_t *sorted_pairs,
                                         int32_t *pair_pos, uint16_t *out, void *ws,
                                         size_t ws_bytes, int flags, int32_t spin_limit,
                                         hipEvent_t *stage_events, hipStream_t stream);
MOE_API moe_status_t moe_layer_decode_error(const void *ws, int32_t *error,
                                            hipStream_t stream);

/*
 * moe_expert_mlp_noalloc -- moe_expert_mlp_ex without a workspace argument
 * and without stage events, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The workspace is instead a fixed device array of
 * MOE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends; its device address is looked up on the first call on each
 * device.  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).  Arguments, arithmetic, preconditions and results are
 * those of moe_expert_mlp_ex (bit-identical outputs), the caller still
 * passes every input and the output.
 * Limit: calls whose moe_expert_mlp_workspace_size(T, D, F, E, k) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES are refused with MOE_ERR_WORKSPACE before
 * anything is enqueued (at D = F = 2880 and k = 4: up to T = 168 tokens).
 * Every call on one GPU uses that GPU's one array, which keeps the last
 * call's contents (nothing in it needs to start at zero): calls that overlap
 * on one GPU -- on different streams, or from different threads -- race and
 * must be serialised by the caller.
 * Errors: as moe_expert_mlp_ex; MOE_ERR_HIP also if the array's address
 * cannot be obtained.
 */
MOE_API moe_status_t moe_expert_mlp_noalloc(const uint16_t *x, const uint8_t *w13_q,
                                            const uint8_t *w13_s, const uint8_t *w2_q,
                                            const uint8_t *w2_s, const float *topk_w,
                                            const int32_t *offsets,
                                            const int32_t *sorted_pairs,
                                            const int32_t *pair_pos, int32_t T, int32_t D,
                                            int32_t F, int32_t E, int32_t k, uint16_t *out,
                                            int algo, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
