// E4M3 element and E8M0 shared-exponent encoding of MX blocks (OCP
// Microscaling Formats v1.0: MXFP8 E4M3, 32-element blocks), shared by the
// dispatch quantiser and the GEMM1 epilogue that re-quantises h.
#pragma once

#include "mok_common.h"

namespace mok {

// floor(log2(v)) of a positive finite fp32 value (subnormals included).
__device__ __forceinline__ int ilog2f(float v) {
  uint32_t b = __float_as_uint(v);
  int ex = (int)((b >> 23) & 0xFF);
  if (ex != 0) return ex - 127;
  uint32_t m = b & 0x7FFFFFu;
  return (31 - __clz((int)m)) - 149;
}

// Shared exponent of an MX block from its max magnitude (OCP MX v1.0: largest
// power of two <= amax, divided by 2^8, 8 = largest E4M3 exponent).
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e = ilog2f(amax) - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Nearest E4M3 (OCP "fn") code of v, ties to even, saturating at +-448.
// Normal range: round the fp32 bits to 3 mantissa bits and rebias the
// exponent (127 -> 7); below 2^-6 the code is the integer v * 2^9.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  uint32_t b = __float_as_uint(v);
  uint32_t s = (b >> 24) & 0x80u;
  float a = __uint_as_float(b & 0x7FFFFFFFu);
  if (a >= 448.0f) return s | 0x7Eu;
  uint32_t ab = b & 0x7FFFFFFFu;
  if (ab < 0x3C800000u) {  // a < 2^-6
    return s | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  uint32_t r = (ab + 0x7FFFFu + ((ab >> 20) & 1u)) >> 20;
  return s | (r - 960u);
}

}  // namespace mok
