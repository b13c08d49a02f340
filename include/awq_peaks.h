/*
 * awq_peaks.h -- calibration probes of libawq_mi355x.so: the measured peaks that the
 * rooflines of the AWQ kernels are judged against, taken in the same process.
 *
 * The decode GEMV is bound by HBM reads ("AWQ量化实战" §3.4: decode is memory-bound) and
 * the dequant-GEMM and the searches by the fp16 matrix cores ("AWQ量化技术Skill",
 * "主要功能和特点": a GEMM kernel for batches). These two probes measure what the chip
 * actually sustains on those two paths; they compute nothing of the method.
 *
 * Return value: 0 on success, 2 for a bad argument (nothing launched), 6 when the launch
 * failed. Both enqueue one kernel on `stream` (a hipStream_t) and never synchronize.
 */
#ifndef AWQ_MI355X_PEAKS_H
#define AWQ_MI355X_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read stream: every byte of buf (device, 16-byte aligned, bytes % 16 == 0) is loaded once
 * with 16-byte vector loads, per_thread (4, 8 or 16) of them in flight per thread, by
 * ceil(bytes / (4096 * per_thread)) blocks of 256 threads, and folded by XOR into sink
 * (device uint32, one word per wave: 4 * that many blocks; contents meaningless).
 * Bandwidth = bytes / kernel time. */
int awq_peak_read_stream(const void* buf, size_t bytes, uint32_t* sink, int32_t per_thread,
                         void* stream);

/* Matrix-core loop: `blocks` blocks of 4 waves, each wave issuing iters x 8 independent
 * v_mfma_f32_32x32x16_f16 (2 * 32 * 32 * 16 flop each) from registers; sink (device float
 * [4 * blocks]) receives one value per wave. Rate = blocks * 4 * iters * 8 * 32768 flop /
 * kernel time. */
int awq_peak_mfma(int64_t iters, float* sink, int32_t blocks, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* AWQ_MI355X_PEAKS_H */
