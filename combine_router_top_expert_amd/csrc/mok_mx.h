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

// Nearest E4M3 (OCP "fn") code of v, ties to even, saturating at +-448: the
// value clamped to +-448, then gfx950's fp8 conversion (which rounds to
// nearest even and keeps E4M3 subnormals).  Over every finite fp32 value
// below 1024 in magnitude (and so every scaled block value, which stays
// below 512) this gives the codes of the bit-level rule -- the fp32 bits
// rounded to 3 mantissa bits and rebiased (127 -> 7), and v * 2^9 rounded
// below 2^-6 -- with no exception; above 448 both saturate.
__device__ __forceinline__ float e4m3_clamp(float v) {
  return __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
}
// Codes of v[0..3] * 2^-sh in bytes 0..3 (two packed conversions).
__device__ __forceinline__ uint32_t e4m3_pack4(float v0, float v1, float v2, float v3, int sh) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(__builtin_amdgcn_ldexpf(v0, -sh)),
                                          e4m3_clamp(__builtin_amdgcn_ldexpf(v1, -sh)), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(__builtin_amdgcn_ldexpf(v2, -sh)),
                                      e4m3_clamp(__builtin_amdgcn_ldexpf(v3, -sh)), w, true);
  return (uint32_t)w;
}

}  // namespace mok
