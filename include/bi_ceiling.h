/*
 * bi_ceiling.h -- measurement probes beside the batch-invariant kernels
 * (libbi_ceiling.so, gfx950).
 *
 * These are not operations of the method and are not part of libbi.so's
 * interface.  They measure, on the GPU at hand and in the same process as a
 * benchmark, what a plain kernel sustains against the two limits the
 * batch-invariant kernels are priced against:
 *  - bic_stream_read: device-memory read bandwidth of a streaming kernel
 *    (16-byte non-temporal loads, every byte read once, one word written per
 *    work-group);
 *  - bic_mfma_bf16: the dense bf16 matrix-core rate with data-dependent
 *    operands (v_mfma_f32_32x32x16_bf16, 16 independent accumulators per wave,
 *    operands read once from device memory), and the shader clock while it runs.
 * The published peaks (8 TB/s, 2.5 PFLOP/s bf16) stay the reference for the
 * roofline fraction; these figures say what part of the gap a plain kernel
 * leaves too.
 *
 * Conventions: device pointers, caller-owned buffers, asynchronous on the given
 * stream (0 = null stream), nothing allocated.  Return 0 on success, 1 for a
 * null or misaligned pointer, 2 for a size outside the stated range (nothing is
 * launched then), 3 when the launch fails.
 */
#ifndef BI_CEILING_H
#define BI_CEILING_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of x (16-byte aligned; bytes a positive multiple of 16) with
 * `grid` work-groups of 256 threads (1 <= grid <= 65536): work-group g reads the g-th
 * of grid equal contiguous spans (the last one shorter) in 16-byte loads and writes the
 * XOR of every 32-bit word of its span to out[g] (out: grid words, 4-byte aligned). */
int bic_stream_read(const void* x, int64_t bytes, uint32_t* out, int grid, hipStream_t stream);

/* Dense bf16 MFMA rate probe.  src: 32768 bf16 values (64 KB, 16-byte aligned).  grid
 * work-groups of 4 waves (1 <= grid <= 65536), iters >= 1.  Lane l of wave w takes its
 * operands from src as 16-byte fragments: a[i] = fragment (64 w + l) * 8 + i and
 * b[i] = fragment (64 w + l) * 8 + 4 + i (i = 0..3, fragment index mod 4096), and runs
 * iters rounds of 16 MFMAs, acc[j] += a[j % 4] x b[j / 4] (j = 0..15), 32768 flops each.
 * out (grid * 256 floats): lane's sum of its 256 accumulator values (acc[0] .. acc[15],
 * registers 0 .. 15 each, in that order).  clk (2 values): the shader-clock cycles and
 * the 100 MHz real-time ticks that wave 0 of work-group 0 counted over its loop. */
int bic_mfma_bf16(const uint16_t* src, int grid, int iters, float* out, uint64_t* clk, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BI_CEILING_H */
