/*
 * moe_calib.h -- counter calibration for the MoE kernels (libmoe_calib.so).
 *
 * Not part of the MoE computation.
 *
 * Byte counters. Hardware byte counters (the L2's reads
 * from and writes to memory) count requests, and how a request of a given
 * size is counted depends on the instruction that caused it. This call reads
 * a buffer of known size with exactly the instruction the grouped GEMMs use
 * to stage their operands (16-byte buffer_load_dwordx4 ... lds, each lane
 * writing its 16 bytes to LDS), so that a counter run can measure the scale
 * between the counter's reading and the bytes the GEMMs really move.
 *
 * Conventions as in moe.h: device pointer, the call only enqueues on
 * `stream` and returns a moe_status value (0 on success).
 */
#ifndef MOE_CALIB_H_
#define MOE_CALIB_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read bytes [0, bytes) of src once, in 1 KiB pieces (one load instruction
 * of a 64-lane wave each), into LDS; nothing is written to memory.
 * src: device pointer, 16-byte aligned. bytes: a multiple of 1024, at most
 * 1 GiB; bytes == 0 launches nothing. Returns 0, -1 (MOE_ERR_INVALID_ARG) on
 * a bad size or pointer, -4 (MOE_ERR_HIP) when the launch fails. */
int moe_calib_dma_read(const void* src, size_t bytes, hipStream_t stream);

/* Matrix-core rate. The engine clock the chip sustains under matrix load is
 * below the one its dense bf16 peak figure assumes; this loop measures the
 * rate that is attainable in practice. Every wave of `waves_per_simd` x 4 x
 * (compute units) waves runs `iters` rounds of 8 independent
 * v_mfma_f32_16x16x32_bf16 (16384 flop each) on register operands, with no
 * memory traffic inside the loop. *flop receives the launch's flop count
 * (host pointer). sink: device float, written only in a case that never
 * occurs (it keeps the loop from being removed). iters >= 1, waves_per_simd
 * in 1..8; else -1. */
int moe_calib_mfma_loop(int iters, int waves_per_simd, float* sink, double* flop, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_CALIB_H_ */
