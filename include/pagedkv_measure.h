/*
 * Hardware ceilings that the hot path's rates are read against.
 *
 * Decode is bound by HBM bandwidth ("vLLM 引擎解剖", section
 * "预填充、解码与三个时延指标": every decode step streams the whole KV cache)
 * and chunked prefill by matrix throughput (same section: prefill is
 * compute-heavy).  Vendor peaks are one yardstick; these two kernels measure
 * what this GPU reaches with the same instruction kinds the hot path uses,
 * a second one.  Both run asynchronously on the caller's stream; time them
 * with events.  They allocate nothing.
 */
#ifndef PAGEDKV_MEASURE_H
#define PAGEDKV_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pkv_measure_hbm_read -- stream `bytes` of device memory at `buf` through
 * 16-byte non-temporal loads (the load kind the decode uses), one
 * contiguous range per workgroup over the whole GPU, and fold every 32-bit
 * word into an XOR checksum.
 *   buf       device memory, 16-byte aligned, `bytes` a positive multiple
 *             of 16 and below 2^40
 *   checksum  device uint32[1]: receives the XOR of all 32-bit words of
 *             buf (so the caller can check that every byte was read); the
 *             kernel clears it first
 * Errors: PKV_ERR_NULL, PKV_ERR_ALIGN, PKV_ERR_SHAPE, PKV_ERR_LAUNCH.
 */
pkv_status pkv_measure_hbm_read(const void* buf, int64_t bytes, uint32_t* checksum,
                                void* stream);

/*
 * pkv_measure_mfma_bf16 -- a register-only loop of independent
 * v_mfma_f32_16x16x32_bf16 (the instruction of the prefill products), two
 * waves on every SIMD.  Each wave issues `iterations` x 8 MFMAs into eight
 * accumulators (16 x 16 x 32 x 2 = 16,384 flop each); the grid has `waves`
 * waves in workgroups of eight (`waves` a positive multiple of 8; 2048 puts
 * two on each of MI355X's 1024 SIMDs).  The A operand's row m is all
 * m + 1 and the B operand all ones, so one product adds 32 (m + 1) to
 * output element (m, n).
 *   iterations  1 .. 524288 (the sums stay exact in fp32)
 *   result      device float[waves]: wave w writes element (0, 0) of its
 *               first accumulator, which must equal 32 * iterations
 * Errors: PKV_ERR_NULL, PKV_ERR_ALIGN, PKV_ERR_SHAPE, PKV_ERR_LAUNCH.
 */
pkv_status pkv_measure_mfma_bf16(int32_t iterations, int32_t waves, float* result,
                                 void* stream);

/*
 * pkv_measure_mfma_valu -- how much of the softmax's vector work the matrix
 * cores hide: the loop of pkv_measure_mfma_bf16 (8 independent MFMAs per
 * iteration) and, from the same waves, 5 chains of fp32 vector work per
 * iteration (fma, integer and, sub, add; a transcendental 2^x on 2 of the 5):
 * 3 vector instructions and 0.25 exp2 per MFMA, near the prefill tile's mix.
 *   mode  0: the MFMAs only; 1: the vector work only; 2: both, interleaved
 *   result device float[2 * waves]: wave w writes 32 * iterations to
 *          result[2w] when it ran the MFMAs (else 0), and its vector sum to
 *          result[2w + 1] (the same in every wave; 0 without vector work)
 * Time the three modes with events: (t2 - t0) / t1 is the share of the
 * vector work the MFMAs do not hide.
 * Errors: PKV_ERR_NULL, PKV_ERR_ALIGN, PKV_ERR_SHAPE, PKV_ERR_LAUNCH.
 */
pkv_status pkv_measure_mfma_valu(int32_t iterations, int32_t waves, int32_t mode,
                                 float* result, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_MEASURE_H */
