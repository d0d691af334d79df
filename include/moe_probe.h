/*
 * moe_probe.h -- C ABI of libmoe_probe, achievable-peak microbenchmarks for
 * MI355X (gfx950): the measured ceilings that the MXFP4 MoE layer's kernels
 * are compared with beside the published peaks.  Not part of the layer (the
 * pages define no such measurement; they ask only that kernels be measured
 * on the real workload, "Tricks from OpenAI gpt-oss" section 4).
 *
 * All pointers are device pointers owned by the caller; calls only enqueue
 * on `stream`.  Return 0 on success, 1 for bad arguments (nothing enqueued),
 * 4 for an unknown kind, 5 if the launch failed.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_PROBE_API __attribute__((visibility("default")))
#else
#define MOE_PROBE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core product kinds of moe_probe_mfma (all 32x32 outputs, fp32
 * accumulate): block-scaled 32x32x64 with A x B operand types, or 32x32x16
 * half precision. */
enum {
    MOE_PROBE_FP4_FP4 = 0,
    MOE_PROBE_FP4_FP6 = 1,   /* fp4 (E2M1) x fp6 (E2M3) */
    MOE_PROBE_FP4_FP8 = 2,   /* fp4 x fp8 (E4M3) */
    MOE_PROBE_FP8_FP8 = 3,
    MOE_PROBE_F16 = 4,
    MOE_PROBE_BF16 = 5
};

/*
 * moe_probe_read -- read `bytes` (a multiple of 16 is used; buf 16-byte
 * aligned) once with `blocks` blocks of 256 threads, 16 bytes per load, four
 * independent loads per trip; each thread writes the XOR of what it read to
 * sink[blocks * 256] (uint32).
 */
MOE_PROBE_API int moe_probe_read(const void *buf, size_t bytes, int blocks, uint32_t *sink,
                   hipStream_t stream);

/*
 * moe_probe_read_grouped -- read blocks * 8 * chunks_per_wave KiB of buf
 * (16-byte aligned) once with `blocks` blocks of 8 wavefronts, each wavefront
 * reading chunks_per_wave 1 KiB chunks (16 bytes per lane, four independent
 * loads per trip).  Groups of `group` consecutive wavefronts interleave their
 * chunks (chunk c of member r of group q is chunk (q * chunks_per_wave + c) *
 * group + r of buf): group 1 gives every wavefront a private contiguous range,
 * group = blocks * 8 makes the grid sweep buf together.  group must divide
 * blocks * 8 (else 1, nothing enqueued).  Each thread writes the XOR of what it
 * read to sink[blocks * 512] (uint32).
 */
MOE_PROBE_API int moe_probe_read_grouped(const void *buf, int chunks_per_wave, int blocks,
                                         int group, uint32_t *sink, hipStream_t stream);

/*
 * moe_probe_mfma -- `blocks` blocks of 4 wavefronts, each wavefront issuing
 * iters x 8 independent products of `kind`; each thread writes a sum of its
 * accumulators to sink[blocks * 256] (float).  Total flops =
 * blocks * 4 * 8 * iters * moe_probe_mfma_flops(kind).
 */
MOE_PROBE_API int moe_probe_mfma(int kind, int blocks, int iters, float *sink, hipStream_t stream);

/* Flops of one product of `kind` (0 for an unknown kind). */
MOE_PROBE_API double moe_probe_mfma_flops(int kind);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
