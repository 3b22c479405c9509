// Register-only throughput probe of the GEMM inner loop's instruction mixes
// (libdg_probe.so; interface and modes in include/dg_probe.h).
//
// The fine-grained-scaled method promotes every 128-deep FP8 partial product
// into an fp32 accumulator with the slice's scales ("Deepseek DeepGEMM
// technical principles", Technical background and core principles).  On
// gfx950 that is one v_mfma_f32_16x16x128_f8f6f4 per 16 x 16 fragment and
// slice, followed by four fp32 FMAs per lane.  This probe runs exactly that
// mix, and the two bounds around it, with every operand in registers, so the
// rates it measures are ceilings for the GEMM's K loop before LDS reads,
// DMA and barriers are added.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_probe.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Tells the compiler the value may have changed, at no run-time cost, so a
// product of loop-invariant operands is not hoisted out of the loop.
__device__ __forceinline__ void opaque(v8i& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void opaque_f(float& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ v4f mfma(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// e4m3 codes 0x30 .. 0x3f: 0.5 .. 0.9375 and 1 .. 1.875, finite and nonzero.
__device__ __forceinline__ v8i codes(int lane, int salt) {
  v8i r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t b = 0x30u + (uint32_t)((lane + 3 * e + salt) & 15);
    r[e] = (int)(b * 0x01010101u);
  }
  return r;
}

template <int MODE>
__global__ __launch_bounds__(512) void probe_kernel(int iters, float* __restrict__ out,
                                                    unsigned long long* __restrict__ clk) {
  const int lane = threadIdx.x & 63;
  v8i a = codes(lane, 0);
  v8i b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = codes(lane, 5 + j);
  float total = 0.0f;
  const bool timer = threadIdx.x == 0;
  uint64_t t0 = 0, r0 = 0;
  if (timer) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  if constexpr (MODE == DG_PROBE_MFMA_CHAINS) {
    v4f acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = mfma(a, b[j & 3], acc[j]);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) total += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  } else {
    // One wave's 128 x 64 tile of the 256 x 256 GEMM tile: 8 fragment rows
    // of 4 fragments.
    v4f acc[8][4];
    float sa[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sa[i] = 0.5f + 0.0625f * (float)((lane + i) & 7);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const float sb = 0.75f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        opaque(a);  // the next fragment row's operand, as if just read
        if constexpr (MODE == DG_PROBE_FP32_PROMOTION) {
          v4f part[4];
          // The GEMM's schedule: the row's MFMAs as one block at raised wave
          // priority, then its promotion FMAs.
          __builtin_amdgcn_s_setprio(2);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < 4; ++j) part[j] = mfma(a, b[j], v4f{0.0f, 0.0f, 0.0f, 0.0f});
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_setprio(0);
          float si = sa[i];
          opaque_f(si);  // read with the fragment row, as in the GEMM
          const float sc = si * sb;
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = fmaf(part[j][e], sc, acc[i][j][e]);
        } else {
          // Exponent bytes 127 + small offsets: scales 2^-1 .. 2^1.
          const int ea = 126 + (i & 3), eb = 127;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[j], acc[i][j], 0, 0, 0, ea, 0, eb);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) total += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
  }
  if (timer) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = total;
}

}  // namespace

extern "C" int dg_probe_mfma_per_iter(int mode) {
  switch (mode) {
    case DG_PROBE_MFMA_CHAINS: return 16;
    case DG_PROBE_FP32_PROMOTION:
    case DG_PROBE_BLOCK_SCALED: return 32;
    default: return -1;
  }
}

extern "C" int dg_probe_loop(int mode, int waves_per_wg, int workgroups, int iters, float* out,
                             unsigned long long* clk, hipStream_t stream) {
  if (dg_probe_mfma_per_iter(mode) < 0 || (waves_per_wg != 4 && waves_per_wg != 8) || workgroups < 1 ||
      workgroups > 65535 || iters < 1 || out == nullptr || clk == nullptr)
    return -1;
  const dim3 grid(workgroups), block(64 * waves_per_wg);
  switch (mode) {
    case DG_PROBE_MFMA_CHAINS:
      hipLaunchKernelGGL(probe_kernel<DG_PROBE_MFMA_CHAINS>, grid, block, 0, stream, iters, out, clk);
      break;
    case DG_PROBE_FP32_PROMOTION:
      hipLaunchKernelGGL(probe_kernel<DG_PROBE_FP32_PROMOTION>, grid, block, 0, stream, iters, out, clk);
      break;
    default:
      hipLaunchKernelGGL(probe_kernel<DG_PROBE_BLOCK_SCALED>, grid, block, 0, stream, iters, out, clk);
      break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
