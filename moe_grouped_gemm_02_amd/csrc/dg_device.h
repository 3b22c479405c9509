// Device-side helpers shared by the gfx950 kernels of libdg.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBlockK = 128;  // scale granularity along K (1x128 / 128x128)

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even.  Inputs are finite here.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Division and encoding of the 1x128 / 128x128 quantisation, shared by the
// quantiser kernels and the GEMM epilogue that quantises its own output.
//
// q = fp32(x / s) is formed as fp32((double)x * RN64(1 / (double)s)): one
// correctly rounded fp64 reciprocal per tile, then one fp64 multiply per
// element.  For a bf16 x (8 significant bits) and an fp32 s (24 bits) the
// exact quotient lies at least 2^-49 (relative) away from any fp32 rounding
// boundary, while this product is within about 2^-52 of it, so rounding it
// to fp32 gives the IEEE quotient itself (also checked exhaustively on the
// host: every s = fp32(a / 448) over the positive finite bf16 a, against every
// bf16 x with |x| <= a, 1.07e9 pairs, no difference).  A zero tile (s = 0)
// uses a zero reciprocal, which keeps each x's signed zero.
__device__ __forceinline__ double tile_reciprocal(float s) { return s == 0.0f ? 0.0 : 1.0 / (double)s; }

__device__ __forceinline__ float quotient(uint32_t bf16_bits, double rcp) {
  return (float)((double)bf16_bits_to_f32(bf16_bits) * rcp);
}

// e4m3 codes of four quotients, packed little-endian into one word, by the
// hardware fp32 -> fp8 conversion (OCP e4m3fn, round to nearest even, signed
// zero kept).  It agrees with a bit-field encoder of the same rule (nearest
// value, ties to even, magnitudes at or above 448 clamped to 448) for every
// fp32 value of magnitude below 450 (checked on gfx950 for all 2.28e9 such bit
// patterns); quotients here are at most 448 * (1 + 2^-24).
__device__ __forceinline__ uint32_t e4m3_x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Power-of-two (UE8M0) scales: E = ceil(log2(amax / 448)) + 127, clamped to
// [0, 254], 0 for an all-zero tile; the scale is 2^(E - 127).  The quotient
// amax/448 is formed in fp64: for a bf16 amax it is either exactly a power of
// two (amax = 7 * 2^j) or at least 2^-11 (relative) away from one, so the
// fp64 rounding cannot move it across a power of two.
__device__ __forceinline__ uint32_t ue8m0_exponent(float amax) {
  if (amax == 0.0f) return 0u;
  const double v = (double)amax / 448.0;
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  int e = (int)((u >> 52) & 0x7FF) - 1023;  // v is a normal fp64 number
  if (u & 0xFFFFFFFFFFFFFull) e += 1;       // not a power of two: round up
  e += 127;
  return (uint32_t)(e < 0 ? 0 : (e > 254 ? 254 : e));
}

// x / 2^(E - 127): exact in fp32 except below the normal range, where
// v_ldexp_f32 rounds to nearest even.
__device__ __forceinline__ float pow2_quotient(uint32_t bf16_bits, uint32_t e) {
  return __builtin_ldexpf(bf16_bits_to_f32(bf16_bits), 127 - (int)e);
}

}  // namespace dg
