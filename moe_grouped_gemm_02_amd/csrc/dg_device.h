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

// fp32 -> OCP e4m3fn code: nearest value, ties to even, magnitudes at or
// above 448 clamp to 448 (0x7E), sign bit kept (so -0 and values that round
// to zero keep it).  Worked out on the bit fields of the fp32 value:
//  * |v| < 2^-6 is the e4m3 subnormal range, spaced 2^-9: the code is
//    rint(|v| * 2^9), which is exact to form and rounds half to even;
//  * otherwise keep the fp32 exponent and round the 23-bit mantissa to 3 bits
//    (add 0x7FFFF plus the kept LSB, then truncate); a carry moves into the
//    exponent field, which is what rounding up to the next binade means.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __uint_as_float(bits & 0x7FFFFFFFu);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {  // 2^-6
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    uint32_t u = bits & 0x7FFFFFFFu;
    u += 0x7FFFFu + ((u >> 20) & 1u);
    code = ((u >> 20) - (120u << 3)) & 0x7Fu;  // rebias exponent 127 -> 7
  }
  return sign | code;
}

}  // namespace dg
