// Matrix-core rate probe: the practical ceiling the expert GEMMs are compared
// with.  Each wave keeps the engine's 4 x 4 blocks of 32 x 32 fp32
// accumulators and issues nothing but MFMAs on operands held in registers
// (no loads, no LDS), so the measured rate is what the matrix cores sustain
// under the chip's power limit for the given operand data.  kind 0:
// v_mfma_f32_32x32x16_bf16; kind 1: v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3
// codes with unit scales.  data 0: operand words from an integer hash of the
// lane (bf16 values in [2^-7, 2), E4M3 codes without NaN); data 1: every
// operand 1.0.  Each lane writes the sum of its accumulators, so with data 1
// the result is exact: 256 accumulator values x (16 or 64) x iters.
#include "mok_internal.h"

namespace mok {

namespace {

constexpr int kProbeThreads = 256;

__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* out, int64_t iters,
                                                                  int constant) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  const uint32_t t = blockIdx.x * kProbeThreads + threadIdx.x;
  i32x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t ha = probe_hash(t * 64u + i * 8u + j), hb = probe_hash(t * 64u + 32u + i * 8u + j);
      if (KIND == 0) {
        ha = constant ? 0x3F803F80u : ((ha & 0x3FFF3FFFu) | 0x3C003C00u);
        hb = constant ? 0x3F803F80u : ((hb & 0x3FFF3FFFu) | 0x3C003C00u);
      } else {
        ha = constant ? 0x38383838u : (ha & 0xF7F7F7F7u);  // exponent below all-ones: no NaN
        hb = constant ? 0x38383838u : (hb & 0xF7F7F7F7u);
      }
      a[i][j] = (int)ha;
      b[i][j] = (int)hb;
    }
  f32x16 c[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) c[i][j][e] = 0.0f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (KIND == 1) {
          c[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], c[i][j], 0, 0, 0, 127,
                                                                    0, 127);
        } else {
          bf16x8 x, y;
          __builtin_memcpy(&x, &a[i], 16);
          __builtin_memcpy(&y, &b[j], 16);
          c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, x, c[i][j], 0, 0, 0);
        }
      }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += c[i][j][e];
  out[t] = s;
}

}  // namespace

mok_status launch_mfma_probe(int kind, int constant, int64_t iters, int workgroups, float* out,
                             hipStream_t stream) {
  if (kind == 0)
    hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3((unsigned)workgroups), dim3(kProbeThreads), 0,
                       stream, out, iters, constant);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3((unsigned)workgroups), dim3(kProbeThreads), 0,
                       stream, out, iters, constant);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

}  // namespace mok
