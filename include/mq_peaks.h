/*
 * mq_peaks.h: measured-peak probes of one gfx950 device (libmq_peaks.so).
 *
 * Not part of the product path: these kernels measure the ceilings the
 * sliced-integer products are reported against, next to the vendor figures
 * (8 TB/s HBM3E, 2.5 PFLOP/s dense bf16).  A batch-1 decode product is bound
 * by moving the weights out of HBM (the "Matryoshka Quantization" explainer,
 * §2 "Context"); a prefill product by the matrix cores.  The caller times the
 * launches (HIP events on `stream`).  Device pointers; nothing is allocated.
 * Return 0 on success, 1 on an invalid argument, 2 if the launch failed.
 */
#ifndef MQ_PEAKS_H
#define MQ_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MQP_API __attribute__((visibility("default")))
#else
#define MQP_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16, buf 16-byte aligned) with `blocks`
 * workgroups of 256 threads, 16-byte loads, 8 in flight per thread; writes
 * one word per workgroup to sink (uint32 [blocks]). */
MQP_API int mqp_stream_read(const void* buf, size_t bytes, int blocks, uint32_t* sink, void* stream);

/* `blocks` workgroups of 4 waves, each wave `iters` x 4 independent
 * v_mfma_f32_32x32x16_bf16 on register operands; out: fp32 [blocks * 256]. */
MQP_API int mqp_mfma_loop(float* out, int blocks, int iters, void* stream);

/* Flops of one mqp_mfma_loop launch (2 * 32 * 32 * 16 per product). */
MQP_API double mqp_mfma_loop_flops(int blocks, int iters);

/* One empty kernel (one 64-thread workgroup): the per-launch cadence. */
MQP_API int mqp_empty(void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MQ_PEAKS_H */
