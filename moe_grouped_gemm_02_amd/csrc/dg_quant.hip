// Fine-grained FP8 quantisers for gfx950: 1x128 activation tiles and 128x128
// weight blocks, amax/448 fp32 scales, e4m3 codes rounded to nearest even.
//
// Source of the scale granularity: "Deepseek DeepGEMM technical principles"
// (blog.51cto.com), section "Technical background and core principles"; fp32
// scales: yfxerp.com DeepGEMM article, section 3.1; transposed (MN-major)
// activation-scale layout: DeepGEMM project introduction, section Interfaces.
//
// Both kernels are HBM-bound streams (2 bytes read, ~1.03 bytes written per
// element): loads are 16-byte vectors, one 128-element tile is owned by 16
// consecutive lanes so a wave reads 1 KB of contiguous memory per step.

#include "dg_device.h"
#include "dg_internal.h"

namespace dg {

// One 1x128 tile per 16 lanes; each lane owns 8 consecutive bf16 values.
__global__ __launch_bounds__(256) void quant_1x128_kernel(const uint16_t* __restrict__ x,
                                                          uint8_t* __restrict__ q,
                                                          float* __restrict__ sf, int rows,
                                                          int cols, int64_t ld_sf, int groups) {
  const int tiles_per_row = cols / kBlockK;
  const int64_t tiles = (int64_t)groups * rows * tiles_per_row;
  const int sub = threadIdx.x & 15;  // lane within the tile's 16-lane group
  const int64_t first = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const int64_t step = ((int64_t)gridDim.x * blockDim.x) >> 4;
  for (int64_t t = first; t < tiles; t += step) {
    const int j = (int)(t % tiles_per_row);
    const int64_t gr = t / tiles_per_row;  // g * rows + r
    const int r = (int)(gr % rows);
    const int g = (int)(gr / rows);
    const int64_t elem = gr * cols + (int64_t)j * kBlockK + sub * 8;
    const uint4 raw = *reinterpret_cast<const uint4*>(x + elem);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
      amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    const float s = amax / 448.0f;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = (s == 0.0f) ? ((__float_as_uint(v[i]) >> 24) & 0x80u)
                                     : f32_to_e4m3_rne(v[i] / s);
      if (i < 4) lo |= c << (8 * i);
      else hi |= c << (8 * (i - 4));
    }
    *reinterpret_cast<uint2*>(q + elem) = make_uint2(lo, hi);
    if (sub == 0) sf[((int64_t)g * tiles_per_row + j) * ld_sf + r] = s;
  }
  // Padding entries of the scale matrix (rows in [rows, ld_sf)) are zero.
  const int pad = (int)(ld_sf - rows);
  if (pad > 0) {
    const int64_t pads = (int64_t)groups * tiles_per_row * pad;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < pads;
         i += (int64_t)gridDim.x * blockDim.x) {
      const int64_t col = i / pad;  // g * tiles_per_row + j
      sf[col * ld_sf + rows + (i % pad)] = 0.0f;
    }
  }
}

// One 128x128 block per workgroup of 256 threads: 2048 16-byte chunks, 8 per
// thread, held in registers between the amax reduction and the encode.
__global__ __launch_bounds__(256) void quant_128x128_kernel(const uint16_t* __restrict__ w,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ sf, int rows,
                                                            int cols) {
  __shared__ float wave_max[4];
  const int kb = blockIdx.x, nb = blockIdx.y, g = blockIdx.z;
  const int kblocks = cols / kBlockK;
  const int nblocks = (rows + kBlockK - 1) / kBlockK;
  const int tid = threadIdx.x;
  const int chunk = tid & 15;  // 8-element chunk within a 128-wide row
  const int64_t base = (int64_t)g * rows * cols;
  uint4 raw[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = nb * kBlockK + (tid >> 4) + 16 * i;
    if (r < rows) {
      raw[i] = *reinterpret_cast<const uint4*>(w + base + (int64_t)r * cols + kb * kBlockK + chunk * 8);
      const uint32_t p[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(p[e] & 0xFFFFu)),
                                 fabsf(bf16_bits_to_f32(p[e] >> 16))));
    } else {
      raw[i] = make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((tid & 63) == 0) wave_max[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  const float s = amax / 448.0f;
  if (tid == 0) sf[((int64_t)g * nblocks + nb) * kblocks + kb] = s;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = nb * kBlockK + (tid >> 4) + 16 * i;
    if (r >= rows) continue;
    const uint32_t p[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t bits = (e & 1) ? (p[e >> 1] >> 16) : (p[e >> 1] & 0xFFFFu);
      const float v = bf16_bits_to_f32(bits);
      const uint32_t c = (s == 0.0f) ? ((bits >> 8) & 0x80u) : f32_to_e4m3_rne(v / s);
      if (e < 4) lo |= c << (8 * e);
      else hi |= c << (8 * (e - 4));
    }
    *reinterpret_cast<uint2*>(q + base + (int64_t)r * cols + kb * kBlockK + chunk * 8) =
        make_uint2(lo, hi);
  }
}

hipError_t launch_quant_1x128(const uint16_t* x, uint8_t* q, float* sf, int rows, int cols,
                              int64_t ld_sf, int groups, hipStream_t stream) {
  const int64_t tiles = (int64_t)groups * rows * (cols / kBlockK);
  const int64_t pads = (int64_t)groups * (cols / kBlockK) * (ld_sf - rows);
  const int64_t want = (tiles * 16 > pads ? tiles * 16 : pads);
  int64_t blocks = (want + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(quant_1x128_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, q, sf,
                     rows, cols, ld_sf, groups);
  return hipGetLastError();
}

hipError_t launch_quant_128x128(const uint16_t* w, uint8_t* q, float* sf, int rows, int cols,
                                int groups, hipStream_t stream) {
  const dim3 grid(cols / kBlockK, (rows + kBlockK - 1) / kBlockK, groups);
  hipLaunchKernelGGL(quant_128x128_kernel, grid, dim3(256), 0, stream, w, q, sf, rows, cols);
  return hipGetLastError();
}

}  // namespace dg
