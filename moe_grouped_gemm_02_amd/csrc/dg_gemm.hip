// Fine-grained-scaled FP8 GEMM kernels for gfx950 (CDNA4).
//
// Method (DeepGEMM project introduction, section Interfaces; "Deepseek
// DeepGEMM technical principles", section "Technical background and core
// principles"): for every 128-wide K slice, form the FP8 partial product on
// the matrix cores, scale it by sa*sb (1x128 activation scale times 128x128
// weight scale) and add it into an fp32 accumulator ("promotion" every
// N_C = 128).  Output bf16.
//
// gfx950 mapping: one v_mfma_f32_16x16x128_f8f6f4 covers exactly one 128-deep
// scale slice of a 16x16 output fragment, so the partial product never mixes
// two slices and needs no chained accumulation: P = mfma(a, b, 0), then
// acc += P * (sa * sb) on the VALU, per lane for its 4 rows x 1 column.
//
// Fragment layouts (64-wide wavefronts):
//   A/B operand: lane l holds 32 bytes of K for row (l % 16); lane group
//   l / 16 selects which 32 bytes.  A and B use the same K assignment, so the
//   contraction over the slice is the full 128-term dot product whatever order
//   the matrix core visits the bytes in.
//   Result: lane l holds column (l % 16), rows 4 * (l / 16) + i, i = 0..3.
//
// LDS tiles are row-major with 128-byte rows; the 16-byte chunk c of row r is
// stored at chunk position c ^ (r % 8), so that the 16 lanes reading 16
// consecutive rows at the same K offset hit distinct banks.

#include "dg_device.h"
#include "dg_internal.h"

namespace dg {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ v8i make_v8i(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

__device__ __forceinline__ v4f mfma_fp8_slice(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // Format codes 0/0 = e4m3 for both operands; no block scale (the scales here
  // are arbitrary fp32 values, applied on the VALU below).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Basic tiled kernel: one BM x BN output tile per workgroup of four waves
// (2 x 2), each wave owning a (BM/2) x (BN/2) sub-tile of 16x16 fragments.
// HBM -> registers -> LDS double buffering, one barrier per K slice.
template <int BM, int BN, int LAYOUT>
__global__ __launch_bounds__(kThreads) void gemm_tile_kernel(GemmParams p) {
  constexpr int kWavesN = 2;
  constexpr int TM = BM / 2, TN = BN / kWavesN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int LA = BM * 8 / kThreads;  // 16-byte chunks per thread per slice
  constexpr int LB = BN * 8 / kThreads;
  static_assert(FM >= 1 && FN >= 1 && LA >= 1 && LB >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kBlockK];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * kBlockK];
  __shared__ int row_group[BM];
  __shared__ int wave_group[kThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  int g = blockIdx.z;

  const uint8_t* A = p.a;
  const float* SA = p.sfa;
  uint16_t* D = p.d;
  int rows_valid = p.m;

  if (LAYOUT == kMasked) {
    int mm = p.masked_m[g];
    mm = mm < 0 ? 0 : (mm > p.m ? p.m : mm);
    if (m0 >= mm) return;  // uniform across the workgroup
    rows_valid = mm;
    A += (int64_t)g * p.a_gstride;
    SA += (int64_t)g * p.sfa_gstride;
    D += (int64_t)g * p.d_gstride;
  } else if (LAYOUT == kContiguous) {
    int id = -1;
    if (tid < BM) {
      id = p.m_indices[m0 + tid];
      if (id < 0 || id >= p.num_groups) id = -1;
      row_group[tid] = id;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) id = max(id, __shfl_xor(id, off, 64));
    if (lane == 0) wave_group[wave] = id;
    __syncthreads();
    g = wave_group[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) g = max(g, wave_group[w]);
    if (g < 0) return;  // an all-padding block: nothing to write
  }
  const uint8_t* B = p.b + (int64_t)g * p.b_gstride;
  const float* SB = p.sfb + (int64_t)g * p.sfb_gstride;

  const int nkb = p.k / kBlockK;
  const int n_blocks = (p.n + kBlockK - 1) / kBlockK;

  // Global -> register staging: chunk (tid + 256 i) is row (tid / 8 + 32 i),
  // 16-byte column (tid % 8) of the slice.
  const int ch = tid & 7;
  uint4 ra[LA], rb[LB];
  auto load_slice = [&](int kb) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = (tid >> 3) + 32 * i;
      const int gr = min(m0 + r, rows_valid - 1);
      ra[i] = *reinterpret_cast<const uint4*>(A + (int64_t)gr * p.lda + kb * kBlockK + ch * 16);
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int r = (tid >> 3) + 32 * i;
      const int gn = min(n0 + r, p.n - 1);
      rb[i] = *reinterpret_cast<const uint4*>(B + (int64_t)gn * p.ldb + kb * kBlockK + ch * 16);
    }
  };
  auto store_slice = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<uint4*>(&lds_a[buf][r * kBlockK + ((ch ^ (r & 7)) << 4)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<uint4*>(&lds_b[buf][r * kBlockK + ((ch ^ (r & 7)) << 4)]) = rb[i];
    }
  };

  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int fr = lane & 15;        // fragment row (A) / column (B) of this lane
  const int kg = lane >> 4;        // which 32 bytes of the slice
  const int c0 = (2 * kg) ^ (fr & 7), c1 = (2 * kg + 1) ^ (fr & 7);

  if (nkb > 0) {
    load_slice(0);
    store_slice(0);
  }
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load_slice(kb + 1);

    // Scales of this slice: 4 consecutive rows per fragment row-block.
    float sa[FM][4];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      int r4 = m0 + wm * TM + i * 16 + 4 * kg;
      r4 = min(r4, (int)p.ld_sfa - 4);
      const float4 s4 = *reinterpret_cast<const float4*>(SA + (int64_t)kb * p.ld_sfa + r4);
      sa[i][0] = s4.x; sa[i][1] = s4.y; sa[i][2] = s4.z; sa[i][3] = s4.w;
    }
    float sb[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int cb = min((n0 + wn * TN + j * 16) >> 7, n_blocks - 1);
      sb[j] = SB[cb * nkb + kb];
    }

    v8i af[FM], bf[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const uint8_t* rowp = &lds_a[buf][(wm * TM + i * 16 + fr) * kBlockK];
      af[i] = make_v8i(*reinterpret_cast<const uint4*>(rowp + (c0 << 4)),
                       *reinterpret_cast<const uint4*>(rowp + (c1 << 4)));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const uint8_t* rowp = &lds_b[buf][(wn * TN + j * 16 + fr) * kBlockK];
      bf[j] = make_v8i(*reinterpret_cast<const uint4*>(rowp + (c0 << 4)),
                       *reinterpret_cast<const uint4*>(rowp + (c1 << 4)));
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const v4f part = mfma_fp8_slice(af[i], bf[j]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = fmaf(part[e], sa[i][e] * sb[j], acc[i][j][e]);
      }

    if (kb + 1 < nkb) store_slice(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: bf16 (RNE) stores of the rows this layout writes.
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rl = wm * TM + i * 16 + 4 * kg + e;
      const int row = m0 + rl;
      bool ok;
      if (LAYOUT == kContiguous) ok = row_group[rl] == g;
      else ok = row < rows_valid;
      if (!ok) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * TN + j * 16 + fr;
        if (col < p.n) D[(int64_t)row * p.ldd + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][e]);
      }
    }
}

template <int BM, int BN>
hipError_t launch_tile(int layout, const GemmParams& p, hipStream_t stream) {
  const int groups = layout == kDense ? 1 : (layout == kMasked ? p.num_groups : 1);
  const dim3 grid((p.n + BN - 1) / BN, (p.m + BM - 1) / BM, groups);
  const dim3 block(kThreads);
  switch (layout) {
    case kDense:
      hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, kDense>), grid, block, 0, stream, p);
      break;
    case kContiguous:
      hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, kContiguous>), grid, block, 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, kMasked>), grid, block, 0, stream, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace

GemmConfig choose_config(int layout, int m, int n, int k, int groups, int num_cus) {
  (void)k;
  GemmConfig c{};
  c.bm = 128;
  c.bn = 128;
  c.split_k = 1;
  c.variant = 0;
  const int mt = (m + c.bm - 1) / c.bm;
  const int nt = (n + c.bn - 1) / c.bn;
  c.tiles = mt * nt * (layout == kMasked ? groups : 1);
  c.grid = c.tiles;
  (void)num_cus;
  return c;
}

size_t workspace_bytes_for(const GemmConfig& cfg, int layout, int m, int n, int groups) {
  (void)cfg; (void)layout; (void)m; (void)n; (void)groups;
  return 0;
}

hipError_t launch_gemm(int layout, const GemmParams& p, const GemmConfig& cfg,
                       hipStream_t stream) {
  (void)cfg;
  return launch_tile<128, 128>(layout, p, stream);
}

}  // namespace dg
