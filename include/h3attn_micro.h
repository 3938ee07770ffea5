/*
 * h3attn_micro: microbenchmarks that measure the achievable denominators of
 * the rooflines the attention step is reported against, on the device that
 * runs it (MI355X, gfx950): the sustained bf16 matrix-core rate and the
 * shader clock under that load, the rate of the fp32 exponential the online
 * softmax issues once per score, and the bandwidth of a plain device copy.
 * They sit beside the library so that the nominal peaks (2516.6 TFLOP/s
 * bf16 dense, 8 TB/s HBM) can be read next to what the chip sustains under
 * its power limit. The work per launch is fixed by the arguments, so the
 * caller times launches with events and divides:
 *   mfma: blocks * 4 waves * iters * 8 instructions * 16384 flop
 *         (v_mfma_f32_16x16x32_bf16: 16 x 16 x 32 multiply-adds, 2 flop each);
 *   exp:  blocks * 256 lanes * iters * 8 exponentials;
 *   copy: bytes read + bytes written.
 *
 * Conventions are those of h3attn.h: caller-owned device pointers, work
 * enqueued on `stream` (a hipStream_t as void*, NULL the null stream),
 * arguments validated before anything is enqueued, status codes from
 * enum h3attn_status, gfx950 only (else H3ATTN_ERR_UNSUPPORTED_DEVICE).
 */
#ifndef H3ATTN_MICRO_H_
#define H3ATTN_MICRO_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Matrix-core rate: `blocks` workgroups of four waves; every wave issues
 * iters rounds of eight independent v_mfma_f32_16x16x32_bf16 chains.
 *   sink:   device fp32 [blocks * 256], written (keeps the results live).
 *   clocks: device uint64 [blocks * 4 * 2]: per wave, the shader clock
 *           cycles (s_memtime) and the 100 MHz reference ticks
 *           (s_memrealtime) that its loop took, so cycles / ticks * 100 MHz
 *           is the clock the chip ran at under this load.
 * blocks in [1, 65536], iters in [1, 2^24].
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_ALIGNMENT (8 bytes), ALIASING,
 * UNSUPPORTED_DEVICE, HIP.
 */
int h3micro_mfma_bf16(int32_t blocks, int32_t iters, float* sink, uint64_t* clocks, void* stream);

/*
 * Exponential rate: `blocks` workgroups of 256 lanes; every lane runs iters
 * rounds of eight independent chains x <- exp2(-x) (v_exp_f32, one
 * instruction per exponential).
 *   sink: device fp32 [blocks * 256], written.
 * blocks in [1, 65536], iters in [1, 2^24].
 * Errors: NULL_POINTER, BAD_SHAPE, UNSUPPORTED_DEVICE, HIP.
 */
int h3micro_exp(int32_t blocks, int32_t iters, float* sink, void* stream);

/*
 * Device copy dst[0, bytes) = src[0, bytes) with 16-byte accesses,
 * non-temporal (streamed past the caches), one workgroup of 256 lanes per
 * 4 KB.
 *   src, dst: device, 16-byte aligned, disjoint; bytes a multiple of 16,
 *   1 <= bytes / 16 < 2^31.
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_ALIGNMENT, ALIASING,
 * UNSUPPORTED_DEVICE, HIP.
 */
int h3micro_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* H3ATTN_MICRO_H_ */
