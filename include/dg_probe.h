/* Register-only throughput probe of the GEMM inner loop's instruction mixes
 * on gfx950 (libdg_probe.so).  A measurement tool beside libdg.so, not part
 * of the GEMM interface: it bounds what the fine-grained-scaled K loop can
 * reach on the matrix cores before any memory traffic.
 *
 * The loop it mirrors is the per-128-K-slice work of the method ("Deepseek
 * DeepGEMM technical principles", Technical background and core principles:
 * an FP8 partial product per 128-deep slice, promoted into an fp32
 * accumulator with the slice's scales; DeepGEMM project introduction,
 * Optimisations: overlapping the matrix-core products with the CUDA-core
 * promotion).  Here a "slice" is, per wave, a 128 x 64 output tile: 32
 * v_mfma_f32_16x16x128_f8f6f4 instructions, in the same register layout as
 * the GEMM's 256 x 256 tile.
 */
#ifndef DG_PROBE_H
#define DG_PROBE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Modes of dg_probe_loop. */
enum {
  /* 16 independent accumulating MFMA chains per wave (C = acc): the matrix
   * core's own rate, 16 MFMAs per iteration. */
  DG_PROBE_MFMA_CHAINS = 0,
  /* The fp32-scale promotion: per fragment row, 4 MFMAs into partials
   * (C = 0), one scale multiply, then 16 FMAs acc += P * s; 32 MFMAs,
   * 128 FMAs and 8 multiplies per iteration. */
  DG_PROBE_FP32_PROMOTION = 1,
  /* The power-of-two-scale form: 32 block-scaled MFMAs accumulating in the
   * matrix core (v_mfma_scale_f32_16x16x128_f8f6f4, C = acc), no VALU. */
  DG_PROBE_BLOCK_SCALED = 2
};

/* Runs `workgroups` workgroups of `waves_per_wg` waves (4 or 8: one or two
 * waves per SIMD), each wave `iters` iterations of the mode's loop on
 * register operands only (e4m3 codes in [0.5, 2), so every product is
 * finite).
 *   out: device, workgroups * waves_per_wg * 64 floats; each thread writes the
 *        sum of its accumulators (keeps the work observable).
 *   clk: device, workgroups * 2 uint64: per workgroup, the shader-clock
 *        cycles (s_memtime) and the 100 MHz real-time ticks (s_memrealtime)
 *        its first wave spent in the loop, from which the clock under load
 *        follows.
 * Both are written, never read; the caller owns them.  Enqueued on `stream`;
 * the host is not synchronised.
 * Returns 0, -1 for a bad argument (unknown mode, waves_per_wg not 4 or 8,
 * workgroups outside [1, 65535], iters < 1, NULL pointer) or -5 when the
 * launch fails. */
int dg_probe_loop(int mode, int waves_per_wg, int workgroups, int iters, float* out,
                  unsigned long long* clk, hipStream_t stream);

/* MFMA instructions one wave issues per iteration of `mode` (16 or 32), or
 * -1 for an unknown mode.  Each is 2 * 16 * 16 * 128 flops. */
int dg_probe_mfma_per_iter(int mode);

#ifdef __cplusplus
}
#endif

#endif /* DG_PROBE_H */
