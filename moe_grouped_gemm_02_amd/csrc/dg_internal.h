// Internal host/device interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

enum Layout : int { kDense = 0, kContiguous = 1, kMasked = 2, kKGrouped = 3 };

// Everything a GEMM kernel needs; group strides are in elements.
struct GemmParams {
  const uint8_t* a;
  const float* sfa;
  const uint8_t* b;
  const float* sfb;
  uint16_t* d;
  const int32_t* m_indices;  // contiguous layout only
  const int32_t* masked_m;   // masked layout only
  const int32_t* k_offsets;  // K-grouped layout only: [G + 1] K offsets of the groups
  float* workspace;          // stream-K partials (fp32), may be null
  int* counters;             // stream-K arrival counters, may be null
  int m;                     // dense: M; contiguous: M_total; masked: M_max
  int n;
  int k;
  int num_groups;
  int64_t lda, ldb, ldd, ld_sfa;
  int64_t a_gstride, sfa_gstride, b_gstride, sfb_gstride, d_gstride;
  // UE8M0 scales (power-of-two exponent bytes): sfa/sfb point at bytes, the
  // weight exponents are MN-major [G][K/128][ld_sfb], and the scale group
  // strides count bytes.  K-grouped layout: sfb is fp32 [K/128][ld_sfb], one
  // scale per row of B and 128-wide K slice.
  int sf_ue8m0;
  int64_t ld_sfb;
  // Quantised copy of the output (null: none): e4m3 codes [G][rows][n] and
  // fp32 scales [G][n/128][ld_dsf] of every 1x128 tile of D, as the
  // activation quantiser would compute them from the bf16 output.
  uint8_t* dq;
  float* dsf;
  int64_t ld_dsf, dq_gstride, dsf_gstride;
  int dq_ue8m0;  // 1: dsf holds UE8M0 exponent bytes (same shape and strides in elements)
  // Operand majors (dense layout): bit 0 = A stored M-major as
  // [K][lda], bit 1 = B stored N-major as [K][ldb]; 0 = both K-major.
  int majors;
};

// Tile variants built with UE8M0 scales.
// Tile variants built for the K-grouped layout.
inline bool kgrouped_variant_built(int variant) {
  return variant == 0 || variant == 4 || variant == 5 || variant == 6;
}

// Tile variants built with MN-major operands.
inline bool majors_variant_built(int variant) {
  return variant == 0 || variant == 4 || variant == 5 || variant == 6;
}

inline bool ue8m0_variant_built(int variant) {
  return variant == 0 || variant == 1 || variant == 4 || variant == 5 || variant == 6;
}

// Stream-K workspace layout.  Offset 0 holds a region of kStreamKCounters
// int32 arrival counters (one per output tile); the fp32 partial-tile slots
// follow it.  The counters sit at the same place whatever the configuration,
// and every call leaves the counters it used at zero, so a workspace that was
// zero-filled once serves later calls of any shape or configuration.
// Configurations with more tiles than counters run without stream-K.
constexpr int kStreamKCounters = 8192;
constexpr size_t kStreamKCounterBytes = (size_t)kStreamKCounters * sizeof(int);

// Tile configuration chosen on the host (deterministically, from the shape).
struct GemmConfig {
  int variant;   // kernel instance (tile shape), index into the kernel table
  int bm;
  int bn;
  int stream_k;  // 1: K ranges of tiles divided among workgroups (stream-K)
  int sk_split;  // 0: equal runs of iterations; S >= 2: S equal parts per tile
  int sk_slots;  // fp32 partial-tile slots: one per run with S parts per tile, two per equal run
  int grid;      // workgroups launched (persistent)
  int tiles;     // output tiles over all groups (masked: worst case)
  int group_m;   // raster group height in M tiles
  int k_rotate;  // 1: each tile starts its K walk at slice (tile mod slices)
};

// What the device needs to walk the work units of one launch.
struct Schedule {
  int tiles;
  int m_tiles;       // M tiles (masked: worst-case total over groups)
  int n_tiles;
  int stream_k;
  int sk_split;
  int sk_slots;      // see GemmConfig
  int group_m;
  int k_rotate;      // see GemmConfig
};

// Whether choose_config() may be asked about this shape: the output tile
// count at the smallest tile variant (times the groups of the masked and
// K-grouped layouts) is below 2^31.  Its precondition; every caller checks.
bool plannable(int layout, int m, int n, int groups);
// expected_m (masked layout only, 0 = unknown): typical valid rows per group,
// used to pick the tile shape.
// qout: the call also quantises its output, which needs tiles whose columns
// are whole 128-column blocks.
// narrow_ok: the 256 x 160 tile (built for fp32 scales with both operands
// K-major, dense / contiguous / masked) may be chosen.
GemmConfig choose_config(int layout, int m, int n, int k, int groups, int num_cus, int expected_m = 0,
                         bool qout = false, bool narrow_ok = true);
// Whether a tile variant's columns are whole 128-column blocks.
bool variant_quantises_output(int variant);
size_t workspace_bytes_for(const GemmConfig& cfg, int layout, int m, int n, int groups);

hipError_t launch_gemm(int layout, const GemmParams& p, const GemmConfig& cfg,
                       hipStream_t stream);
// pow2: UE8M0 exponent bytes instead of fp32 scales (see dg_quant.hip).
hipError_t launch_quant_1x128(const uint16_t* x, uint8_t* q, void* sf, int rows, int cols,
                              int64_t ld_sf, int groups, bool pow2, hipStream_t stream);
// x [rows][cols] stored M-major (rows = K, a multiple of 128; cols % 8 == 0):
// 1x128 tiles along the rows, scales [rows/128][ld_sf] (fp32, or UE8M0
// exponent bytes with pow2).
hipError_t launch_quant_1x128_mn(const uint16_t* x, uint8_t* q, void* sf, int rows, int cols,
                                 int64_t ld_sf, bool pow2, hipStream_t stream);
hipError_t launch_quant_128x128(const uint16_t* w, uint8_t* q, void* sf, int rows, int cols,
                                int groups, bool pow2, hipStream_t stream);

}  // namespace dg
