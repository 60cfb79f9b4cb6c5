/*
 * moe_peaks.h -- peak-rate microbenchmarks of the GPU the MoE layer runs on.
 *
 * They measure, on the running GPU, the two rates that bound the layer's kernels: dense
 * bf16 MFMA throughput (the grouped expert GEMMs when rows per expert are many) and HBM
 * streaming bandwidth (the expert-weight stream when they are few, and the routing,
 * grouping and combine stages).  The benchmark reports them beside the published MI355X
 * peaks; roofline fractions stay against the published figures.
 *
 * Conventions are those of moe.h: device pointers, 16-byte aligned; each call checks its
 * arguments on the host, enqueues one kernel on `stream` and returns without
 * synchronising; a failed check returns its code (and sets moe_last_error()) and
 * enqueues nothing; a failed launch returns MOE_ERR_HIP.  The caller times the kernel
 * with events around the call.
 */
#ifndef MOE_PEAKS_H
#define MOE_PEAKS_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* MFMA-only loop: `blocks` workgroups of 256 threads (four wavefronts), each wavefront
 * issuing iters x 32 v_mfma_f32_16x16x32_bf16 on register operands into 32 independent
 * accumulators (each updated once per iteration), no memory traffic in the loop.
 *   FLOPs = blocks * 4 * iters * 32 * 16384.
 * sink   (device, blocks * 256 floats): each thread's accumulator sum (keeps the work).
 * clocks (device, 2 uint64): workgroup 0's shader-clock cycles and constant-clock ticks
 *        over its loop; cycles / (ticks / wall_khz) is the shader clock under MFMA load.
 * wall_khz (host, may be NULL): receives the constant clock's rate in kHz.
 * Errors: NULL sink/clocks -> MOE_ERR_NULL; blocks outside [1, 65536] or iters < 1 ->
 * MOE_ERR_SHAPE; misaligned pointer -> MOE_ERR_ALIGN. */
moe_status moe_peak_mfma_bf16(int blocks, int iters, float* sink, uint64_t* clocks, int* wall_khz,
                              hipStream_t stream);

/* Streaming read: every 16-byte chunk of src[0, bytes) is loaded once by a grid of
 * `blocks` workgroups of 256 threads (grid-stride, four loads in flight per thread).
 * sink (device, blocks * 256 floats) receives a per-thread digest of what it read.
 * Errors: NULL pointer -> MOE_ERR_NULL; bytes not a positive multiple of 16 or blocks
 * outside [1, 65536] -> MOE_ERR_SHAPE; misaligned pointer -> MOE_ERR_ALIGN. */
moe_status moe_peak_hbm_read(const void* src, size_t bytes, int blocks, float* sink, hipStream_t stream);

/* Streaming copy of src[0, bytes) to dst (the buffers must not overlap), same grid and
 * errors as moe_peak_hbm_read.  It moves 2 * bytes through HBM. */
moe_status moe_peak_hbm_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PEAKS_H */
