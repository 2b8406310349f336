/*
 * qgemm_peaks.h -- measurement probes of libqgemm (AMD MI355X, gfx950).
 *
 * Not part of the quantized layer: these kernels measure the two ceilings the
 * layer's kernels are held against -- a plain streaming read of HBM at the
 * decode layers' sizes and the matrix cores' rate on random operands -- and
 * the fixed cost of one launch, in the way 「LLM推理降本五要素」 §2.1 quotes
 * the W8A8 layer's weight bandwidth against the part's own peak.
 *
 * Conventions as in qgemm.h: device pointers owned by the caller, a
 * hipStream_t passed as void* (NULL = default stream), status codes from
 * qgemm.h, every argument checked on the host before anything is enqueued.
 */
#ifndef QGEMM_PEAKS_H
#define QGEMM_PEAKS_H

#include <stdint.h>

#include "qgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Number of int32 words qg_peak_stream_read writes to `sink` for a read of
 * `bytes` bytes (0 for bytes <= 0). */
int64_t qg_peak_stream_read_sink(int64_t bytes);

/*
 * Read bytes [0, bytes) of `src` once, as the best plain read measured on
 * MI355X does: at most one workgroup of 8 waves per CU (256), each workgroup
 * a contiguous stretch of whole kilobytes, each wave a contiguous part of it,
 * all of a wave's 16-byte non-temporal loads issued before any is used.
 * src:  device buffer of at least `bytes` bytes, 16-byte aligned; read only.
 * sink: qg_peak_stream_read_sink(bytes) int32 words, written (an xor of the
 *       data per wave, so the loads cannot be dropped).
 * 0 < bytes <= 2^31.  QG_ERR_NULL / QG_ERR_SHAPE / QG_ERR_ALIGN on bad
 * arguments, QG_ERR_HIP if the launch fails.
 */
qg_status_t qg_peak_stream_read(const void* src, int64_t bytes, int32_t* sink, void* stream);

/*
 * Matrix-core loop on random full-range register operands: `workgroups`
 * workgroups of 4 waves, each wave `iters` rounds of 4 independent
 * instructions of one kind:
 *   kind 0: v_mfma_i32_32x32x32_i8    (65536 ops each)
 *   kind 1: v_mfma_i32_16x16x64_i8    (32768 ops)
 *   kind 2: v_mfma_f32_32x32x16_f16   (32768 flops)
 *   kind 3: v_mfma_f32_32x32x16_bf16  (32768 flops)
 * clocks: 2 * 4 * workgroups uint64, written: per wave, the shader-clock
 *         counter (s_memtime) and the 100 MHz real-time counter
 *         (s_memrealtime) elapsed over its loop.
 * sink:   256 * workgroups int32, written (accumulator bits).
 * 1 <= iters, 1 <= workgroups <= 65535; kind in 0..3 (else QG_ERR_ARG).
 */
qg_status_t qg_peak_mfma(int kind, int64_t iters, int64_t workgroups, uint64_t* clocks,
                         int32_t* sink, void* stream);

/* Operations qg_peak_mfma(kind, iters, workgroups, ...) performs (-1 for a
 * bad argument). */
int64_t qg_peak_mfma_ops(int kind, int64_t iters, int64_t workgroups);

/* One workgroup that does nothing: the fixed cost of a launch. */
qg_status_t qg_peak_empty(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_PEAKS_H */
