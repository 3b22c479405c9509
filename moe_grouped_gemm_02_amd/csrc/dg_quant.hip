// Fine-grained FP8 quantisers for gfx950: 1x128 activation tiles and 128x128
// weight blocks, amax/448 fp32 scales, e4m3 codes rounded to nearest even.
//
// Source of the scale granularity: "Deepseek DeepGEMM technical principles"
// (blog.51cto.com), section "Technical background and core principles"; fp32
// scales: yfxerp.com DeepGEMM article, section 3.1; transposed (MN-major)
// activation-scale layout: DeepGEMM project introduction, section Interfaces.
//
// Both kernels are HBM-bound streams (2 bytes read, ~1.03 bytes written per
// element) with 16-byte vector loads and stores.

#include "dg_device.h"
#include "dg_internal.h"

namespace dg {

// 1x128 activation tiles.  Each wave owns 8 tiles of a row (8 consecutive
// lanes per tile, 16 bf16 values = 32 bytes each, so a load reads 2 KB of
// one row) and walks down the rows U at a time, issuing the loads of its U
// rows before quantising any of them.  Block (x, y) holds 4 waves: tiles
// [8 x, 8 x + 8), wave w starting at row (4 y + w) U, then every
// 4 U gridDim.y rows further down.  U trades bytes in flight against the
// serial work of a wave: 4 on tall matrices (32768 x 7168: 132 us, against
// 142 us with one row per trip), 2 on 4096-row ones, 1 on decode-sized ones,
// where four rows quantised one after another added 0.7 us to a 2.7 us call.
constexpr int kQTilesPerWave = 8;
constexpr int kQWaves = 4;

// POW2: scales are UE8M0 exponents (one byte each) instead of fp32 values;
// the scale matrices have the same [(G)][C/128][ld] shape either way.
template <bool POW2, int U>
__global__ __launch_bounds__(64 * kQWaves) void quant_1x128_kernel(const uint16_t* __restrict__ x,
                                                                   uint8_t* __restrict__ q,
                                                                   void* __restrict__ sf_out, int rows,
                                                                   int cols, int64_t ld_sf, int groups) {
  float* sf = static_cast<float*>(sf_out);
  uint8_t* sf8 = static_cast<uint8_t*>(sf_out);
  const int tiles_per_row = cols / kBlockK;
  const int total_rows = groups * rows;
  const int sub = threadIdx.x & 7;  // lane within the tile's 8-lane group
  const int j = blockIdx.x * kQTilesPerWave + ((threadIdx.x & 63) >> 3);
  const int wave = threadIdx.x >> 6;
  if (j < tiles_per_row) {
    const int step = gridDim.y * kQWaves * U;
    for (int gr0 = (blockIdx.y * kQWaves + wave) * U; gr0 < total_rows; gr0 += step) {  // gr = g * rows + r
      uint4 lo[U], hi[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // Rows past the end reload the last row; their results are dropped.
        const int64_t elem = (int64_t)min(gr0 + u, total_rows - 1) * cols + j * kBlockK + sub * 16;
        lo[u] = *reinterpret_cast<const uint4*>(x + elem);
        hi[u] = *reinterpret_cast<const uint4*>(x + elem + 8);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int gr = gr0 + u;
        const int g = gr / rows, r = gr - g * rows;
        const uint32_t w[8] = {lo[u].x, lo[u].y, lo[u].z, lo[u].w, hi[u].x, hi[u].y, hi[u].z, hi[u].w};
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(w[i] & 0xFFFFu)), fabsf(bf16_bits_to_f32(w[i] >> 16))));
#pragma unroll
        for (int off = 4; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 8));
        uint32_t out[4];
        const int64_t sf_at = ((int64_t)g * tiles_per_row + j) * ld_sf + r;
        const bool live = gr < total_rows;
        if constexpr (POW2) {
          const uint32_t e = ue8m0_exponent(amax);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            out[i] = e4m3_x4(pow2_quotient(w[2 * i] & 0xFFFFu, e), pow2_quotient(w[2 * i] >> 16, e),
                             pow2_quotient(w[2 * i + 1] & 0xFFFFu, e), pow2_quotient(w[2 * i + 1] >> 16, e));
          if (live && sub == 0) sf8[sf_at] = (uint8_t)e;
        } else {
          const float s = amax / 448.0f;
          const double rcp = tile_reciprocal(s);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            out[i] = e4m3_x4(quotient(w[2 * i] & 0xFFFFu, rcp), quotient(w[2 * i] >> 16, rcp),
                             quotient(w[2 * i + 1] & 0xFFFFu, rcp), quotient(w[2 * i + 1] >> 16, rcp));
          if (live && sub == 0) sf[sf_at] = s;
        }
        if (live)
          *reinterpret_cast<uint4*>(q + (int64_t)gr * cols + j * kBlockK + sub * 16) =
              make_uint4(out[0], out[1], out[2], out[3]);
      }
    }
  }
  // Padding entries of the scale matrix (rows in [rows, ld_sf)) are zero.
  const int pad = (int)(ld_sf - rows);
  if (pad > 0 && blockIdx.y == 0) {
    const int64_t pads = (int64_t)groups * tiles_per_row * pad;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < pads;
         i += (int64_t)gridDim.x * blockDim.x) {
      const int64_t col = i / pad;  // g * tiles_per_row + j
      if constexpr (POW2) sf8[col * ld_sf + rows + (i % pad)] = 0;
      else sf[col * ld_sf + rows + (i % pad)] = 0.0f;
    }
  }
}

// 1x128 activation tiles of an M-major matrix: x is stored [K][M] (the K
// values of logical row m are a column), and tile (kb, m) is the column
// segment x[128 kb .. 128 kb + 127][m].  The codes keep the [K][M] layout;
// the scales are [K/128][ld_sf] as for the row form, so this is
// quant_1x128 of x^T with its codes stored transposed.  A wave covers 64
// columns and 128 rows: lane l owns columns 8 (l % 8) .. + 7 of the wave's
// 64 and rows 16 (l / 8) .. + 15, held in registers between the amax and the
// encode; the 8 lanes of a column group combine their amax with shuffles.
// Block (x, y): columns [256 x, 256 x + 256), K block y; cols % 8 == 0.
// POW2: UE8M0 exponent bytes instead of fp32 scales, same [K/128][ld_sf] shape.
template <bool POW2>
__global__ __launch_bounds__(256) void quant_1x128_mn_kernel(const uint16_t* __restrict__ x,
                                                             uint8_t* __restrict__ q,
                                                             void* __restrict__ sf_out, int rows,
                                                             int cols, int64_t ld_sf) {
  float* sf = static_cast<float*>(sf_out);
  uint8_t* sf8 = static_cast<uint8_t*>(sf_out);
  const int lane = threadIdx.x & 63;
  const int col = blockIdx.x * 256 + (threadIdx.x >> 6) * 64 + (lane & 7) * 8;
  const int kb = blockIdx.y;
  const int r0 = kb * kBlockK + (lane >> 3) * 16;
  if (col < cols) {
    uint4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const uint4*>(x + (int64_t)(r0 + i) * cols + col);
    float amax[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) amax[c] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        amax[2 * h] = fmaxf(amax[2 * h], fabsf(bf16_bits_to_f32(w[h] & 0xFFFFu)));
        amax[2 * h + 1] = fmaxf(amax[2 * h + 1], fabsf(bf16_bits_to_f32(w[h] >> 16)));
      }
    }
    // The 8 lanes l, l + 8, ..., l + 56 hold the 8 row groups of a column group.
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int off = 8; off <= 32; off <<= 1) amax[c] = fmaxf(amax[c], __shfl_xor(amax[c], off, 64));
    if constexpr (POW2) {
      uint32_t e[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) e[c] = ue8m0_exponent(amax[c]);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        const uint32_t lo = e4m3_x4(pow2_quotient(w[0] & 0xFFFFu, e[0]), pow2_quotient(w[0] >> 16, e[1]),
                                    pow2_quotient(w[1] & 0xFFFFu, e[2]), pow2_quotient(w[1] >> 16, e[3]));
        const uint32_t hi = e4m3_x4(pow2_quotient(w[2] & 0xFFFFu, e[4]), pow2_quotient(w[2] >> 16, e[5]),
                                    pow2_quotient(w[3] & 0xFFFFu, e[6]), pow2_quotient(w[3] >> 16, e[7]));
        *reinterpret_cast<uint2*>(q + (int64_t)(r0 + i) * cols + col) = make_uint2(lo, hi);
      }
      if ((lane >> 3) == 0) {
        uint8_t* out = sf8 + (int64_t)kb * ld_sf + col;
#pragma unroll
        for (int c = 0; c < 8; ++c) out[c] = (uint8_t)e[c];
      }
    } else {
      double rcp[8];
      float s[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        s[c] = amax[c] / 448.0f;
        rcp[c] = tile_reciprocal(s[c]);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        const uint32_t lo = e4m3_x4(quotient(w[0] & 0xFFFFu, rcp[0]), quotient(w[0] >> 16, rcp[1]),
                                    quotient(w[1] & 0xFFFFu, rcp[2]), quotient(w[1] >> 16, rcp[3]));
        const uint32_t hi = e4m3_x4(quotient(w[2] & 0xFFFFu, rcp[4]), quotient(w[2] >> 16, rcp[5]),
                                    quotient(w[3] & 0xFFFFu, rcp[6]), quotient(w[3] >> 16, rcp[7]));
        *reinterpret_cast<uint2*>(q + (int64_t)(r0 + i) * cols + col) = make_uint2(lo, hi);
      }
      if ((lane >> 3) == 0) {
        float* out = sf + (int64_t)kb * ld_sf + col;
#pragma unroll
        for (int c = 0; c < 8; ++c) out[c] = s[c];
      }
    }
  }
  // Padding entries of the scale matrix (columns in [cols, ld_sf)) are zero.
  const int pad = (int)(ld_sf - cols);
  if (pad > 0 && blockIdx.x == 0 && (int)threadIdx.x < pad) {
    for (int i = threadIdx.x; i < pad; i += 256) {
      if constexpr (POW2) sf8[(int64_t)kb * ld_sf + cols + i] = 0;
      else sf[(int64_t)kb * ld_sf + cols + i] = 0.0f;
    }
  }
}

// One 128x128 block per workgroup of 256 threads: 2048 16-byte chunks, 8 per
// thread, held in registers between the amax reduction and the encode.
// POW2: UE8M0 exponents in an MN-major [G][K/128][ld_n] byte matrix,
// ld_n = round_up(ceil(N/128), 4), instead of fp32 [G][ceil(N/128)][K/128].
template <bool POW2>
__global__ __launch_bounds__(256) void quant_128x128_kernel(const uint16_t* __restrict__ w,
                                                            uint8_t* __restrict__ q,
                                                            void* __restrict__ sf_out, int rows,
                                                            int cols) {
  float* sf = static_cast<float*>(sf_out);
  uint8_t* sf8 = static_cast<uint8_t*>(sf_out);
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
  const double rcp = tile_reciprocal(s);
  const uint32_t e = POW2 ? ue8m0_exponent(amax) : 0u;
  if constexpr (POW2) {
    const int ld_n = (nblocks + 3) / 4 * 4;
    uint8_t* col = sf8 + ((int64_t)g * kblocks + kb) * ld_n;
    if (tid == 0) col[nb] = (uint8_t)e;
    if (nb == nblocks - 1 && tid >= 1 && tid < 4 && nb + tid < ld_n) col[nb + tid] = 0;  // pads
  } else {
    if (tid == 0) sf[((int64_t)g * nblocks + nb) * kblocks + kb] = s;
  }
  auto quo = [&](uint32_t bits) { return POW2 ? pow2_quotient(bits, e) : quotient(bits, rcp); };
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = nb * kBlockK + (tid >> 4) + 16 * i;
    if (r >= rows) continue;
    const uint32_t p[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
    const uint32_t lo = e4m3_x4(quo(p[0] & 0xFFFFu), quo(p[0] >> 16), quo(p[1] & 0xFFFFu), quo(p[1] >> 16));
    const uint32_t hi = e4m3_x4(quo(p[2] & 0xFFFFu), quo(p[2] >> 16), quo(p[3] & 0xFFFFu), quo(p[3] >> 16));
    *reinterpret_cast<uint2*>(q + base + (int64_t)r * cols + kb * kBlockK + chunk * 8) =
        make_uint2(lo, hi);
  }
}

hipError_t launch_quant_1x128(const uint16_t* x, uint8_t* q, void* sf, int rows, int cols,
                              int64_t ld_sf, int groups, bool pow2, hipStream_t stream) {
  const int tiles_per_row = cols / kBlockK;
  const int gx = (tiles_per_row + kQTilesPerWave - 1) / kQTilesPerWave;
  const int64_t total_rows = (int64_t)groups * rows;
  // Rows per trip and waves in flight by height (measured on 64 .. 32768
  // rows of 512 .. 16384 columns).
  const int u = total_rows >= 16384 ? 4 : total_rows >= 2048 ? 2 : 1;
  const int64_t waves = total_rows >= 16384 ? 16384 : 8192;
  int64_t gy = (waves / kQWaves + gx - 1) / gx;
  const int64_t need = (total_rows + (int64_t)kQWaves * u - 1) / ((int64_t)kQWaves * u);
  if (gy > need) gy = need;
  if (gy > 65535) gy = 65535;
  if (gy < 1) gy = 1;
  const dim3 grid(gx > 0 ? gx : 1, (unsigned)gy), block(64 * kQWaves);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, x, q, sf, rows, cols, ld_sf, groups);
  };
  if (pow2) {
    if (u == 4) go(quant_1x128_kernel<true, 4>);
    else if (u == 2) go(quant_1x128_kernel<true, 2>);
    else go(quant_1x128_kernel<true, 1>);
  } else {
    if (u == 4) go(quant_1x128_kernel<false, 4>);
    else if (u == 2) go(quant_1x128_kernel<false, 2>);
    else go(quant_1x128_kernel<false, 1>);
  }
  return hipGetLastError();
}

hipError_t launch_quant_1x128_mn(const uint16_t* x, uint8_t* q, void* sf, int rows, int cols,
                                 int64_t ld_sf, bool pow2, hipStream_t stream) {
  const dim3 grid(cols / 256 + (cols % 256 != 0), rows / kBlockK);
  if (pow2)
    hipLaunchKernelGGL(quant_1x128_mn_kernel<true>, grid, dim3(256), 0, stream, x, q, sf, rows, cols, ld_sf);
  else
    hipLaunchKernelGGL(quant_1x128_mn_kernel<false>, grid, dim3(256), 0, stream, x, q, sf, rows, cols, ld_sf);
  return hipGetLastError();
}

hipError_t launch_quant_128x128(const uint16_t* w, uint8_t* q, void* sf, int rows, int cols,
                                int groups, bool pow2, hipStream_t stream) {
  const dim3 grid(cols / kBlockK, (rows + kBlockK - 1) / kBlockK, groups);
  if (pow2)
    hipLaunchKernelGGL(quant_128x128_kernel<true>, grid, dim3(256), 0, stream, w, q, sf, rows, cols);
  else
    hipLaunchKernelGGL(quant_128x128_kernel<false>, grid, dim3(256), 0, stream, w, q, sf, rows, cols);
  return hipGetLastError();
}

}  // namespace dg
