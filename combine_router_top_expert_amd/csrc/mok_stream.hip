// Streaming probe of the HBM: the rate that the layer's data-movement
// kernels (gather, push, combine, reverse-combine pull, SwiGLU backward) are
// compared with.  Like those kernels it moves plain 16-byte vector loads and
// stores.  A persistent grid (a few workgroups per CU) walks chunks of
// 256 lanes x kUnroll units (32 KiB) with a grid stride; every lane issues
// all kUnroll loads of a chunk before it uses any.  Modes: 0 = read only (the
// loaded words are folded into one value per lane, stored only if it equals a
// value the host never passes, so the loads cannot be dropped), 1 = write
// only, 2 = copy (read + write).
#include "mok_internal.h"

namespace mok {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kUnroll = 8;
constexpr int kStreamWgsPerCu = 8;

template <int MODE>
__global__ __launch_bounds__(kStreamThreads) void stream_kernel(uint4* dst, const uint4* src,
                                                                int64_t n, uint32_t never) {
  const int64_t per_chunk = (int64_t)kStreamThreads * kUnroll;
  const int64_t chunks = (n + per_chunk - 1) / per_chunk;
  const uint4 fill = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
  uint32_t fold = 0;
  for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
    const int64_t base = c * per_chunk + threadIdx.x;
    uint4 v[kUnroll];
    if (MODE != 1) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kStreamThreads;
        v[u] = i < n ? src[i] : make_uint4(0, 0, 0, 0);
      }
    }
    if (MODE == 0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) fold ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    } else {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kStreamThreads;
        if (i < n) dst[i] = MODE == 1 ? fill : v[u];
      }
    }
  }
  if (MODE == 0) {
    const int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    if (fold == never && i < n) dst[i] = make_uint4(fold, 0, 0, 0);
  }
}

}  // namespace

mok_status launch_stream(int mode, void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  const int64_t n = bytes / 16;
  if (n == 0) return MOK_OK;
  const int64_t per_chunk = (int64_t)kStreamThreads * kUnroll;
  const int64_t chunks = (n + per_chunk - 1) / per_chunk;
  const int cus = device_cus();
  if (cus <= 0) return MOK_EDEVICE;
  const int64_t grid = chunks < (int64_t)cus * kStreamWgsPerCu ? chunks : (int64_t)cus * kStreamWgsPerCu;
  uint4* d = reinterpret_cast<uint4*>(dst);
  const uint4* sp = reinterpret_cast<const uint4*>(src);
  const uint32_t never = 0xA5A5A5A5u;
  if (mode == 0)
    hipLaunchKernelGGL(stream_kernel<0>, dim3((unsigned)grid), dim3(kStreamThreads), 0, stream, d, sp, n, never);
  else if (mode == 1)
    hipLaunchKernelGGL(stream_kernel<1>, dim3((unsigned)grid), dim3(kStreamThreads), 0, stream, d, sp, n, never);
  else
    hipLaunchKernelGGL(stream_kernel<2>, dim3((unsigned)grid), dim3(kStreamThreads), 0, stream, d, sp, n, never);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

}  // namespace mok
