// Streaming probe of the HBM: the ceiling that the layer's data-movement
// kernels (gather, push, combine, reverse-combine pull, SwiGLU backward) are
// held against.  Every lane moves 16-byte units with plain vector loads and
// stores, four units in flight per lane, over a grid-stride loop of one
// 256-thread workgroup per SIMD (four per CU): the access pattern those
// kernels use.  Modes: 0 = read only (the loaded words are folded into one
// value per lane, stored only if it equals a value the host never passes, so
// the loads cannot be dropped), 1 = write only, 2 = copy (read + write).
#include "mok_internal.h"

namespace mok {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kStreamThreads) void stream_kernel(int mode, uint4* dst,
                                                                const uint4* src, int64_t n,
                                                                uint32_t never) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  uint32_t fold = 0;
  const uint4 fill = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    uint4 v[kUnroll];
    if (mode != 1) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
    }
    if (mode == 0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) fold ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    } else {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) dst[i + u * stride] = mode == 1 ? fill : v[u];
    }
  }
  for (; i < n; i += stride) {
    if (mode == 0) {
      const uint4 v = src[i];
      fold ^= v.x ^ v.y ^ v.z ^ v.w;
    } else {
      dst[i] = mode == 1 ? fill : src[i];
    }
  }
  if (mode == 0 && fold == never) dst[blockIdx.x * kStreamThreads + threadIdx.x] = make_uint4(fold, 0, 0, 0);
}

}  // namespace

mok_status launch_stream(int mode, void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  const int64_t n = bytes / 16;
  if (n == 0) return MOK_OK;
  int cus = device_cus();
  if (cus <= 0) return MOK_EDEVICE;
  int64_t blocks = (int64_t)cus * 4;
  const int64_t need = (n + kStreamThreads - 1) / kStreamThreads;
  if (blocks > need) blocks = need;
  hipLaunchKernelGGL(stream_kernel, dim3((unsigned)blocks), dim3(kStreamThreads), 0, stream, mode,
                     reinterpret_cast<uint4*>(dst), reinterpret_cast<const uint4*>(src), n,
                     0xA5A5A5A5u);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

}  // namespace mok
