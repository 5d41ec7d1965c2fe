/*
 * tpmlp_calib.h -- measurement aids for the MI355X (gfx950) shard kernels.
 * Not part of the method: these calls help read the kernels' numbers against
 * the hardware (the MFMA rate at the clock the power limit allows, the
 * streaming-read rate of HBM), for benchmarks and profiling.
 */
#ifndef TPMLP_CALIB_H
#define TPMLP_CALIB_H

#include <stdint.h>

#include "tpmlp.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Dense bf16 MFMA throughput and the shader clock it runs at, for operands of
 * a given kind.  Launches `nwg` workgroups of 4 wavefronts (one per SIMD);
 * each wavefront issues `iters` x 8 v_mfma_f32_32x32x16_bf16 (32768 flops
 * each) on four independent accumulators, with the A and B operands cycling
 * through eight register sets so that every product sees new operands.
 *   gaussian = 0: all operands zero; 1: A ~ N(0,1), B ~ N(0, 0.02^2) bf16
 *                 (the value mix of the synthetic MLP workloads).
 *   stats: device buffer of 2*nwg uint64 (caller-owned); on completion
 *          stats[2w] = shader-clock cycles (s_memtime) and stats[2w+1] = ticks
 *          of the 100 MHz constant clock (s_memrealtime) spent by workgroup w,
 *          so sum(cycles)/sum(ticks) * 100 MHz is the mean clock.
 * The caller times the launch (e.g. with events on `stream`) for the flop
 * rate: nwg * 4 * iters * 8 * 32768 flops.  Errors: TP_ERR_BAD_SHAPE for
 * nwg < 1 or iters < 1, TP_ERR_NULL_POINTER for stats = NULL, TP_ERR_HIP if the
 * launch fails; nothing is launched on an error.
 */
tp_status tp_calib_mfma_bf16(int32_t gaussian, int64_t iters, uint64_t *stats, int32_t nwg,
                             void *stream);

/*
 * Streaming-read rate of HBM: `nwg` workgroups of 256 threads read `bytes`
 * (a multiple of 16) of device memory at `buf` exactly once, each workgroup a
 * contiguous 1/nwg of it, 16 bytes per load with the nontemporal hint (as the
 * few-token kernels stream weights), and write (almost) nothing.  Timing one launch gives the per-launch read ceiling
 * of a kernel that streams that many bytes (ramp and drain included); the
 * caller rotates buffers larger than the 256 MB Infinity Cache to measure HBM.
 *   sink: device buffer of nwg uint32 (caller-owned; written only in the
 *         unlikely case that the data folds to one particular word).
 * Errors: TP_ERR_BAD_SHAPE for nwg < 1 or bytes not a non-negative multiple of
 * 16, TP_ERR_NULL_POINTER for sink = NULL or buf = NULL with bytes > 0,
 * TP_ERR_MISALIGNED for buf not 16-byte aligned, TP_ERR_HIP if the launch
 * fails; nothing is launched on an error, or when bytes = 0.
 */
tp_status tp_calib_hbm_read(const void *buf, int64_t bytes, uint32_t *sink, int32_t nwg,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TPMLP_CALIB_H */
