// Streaming probe of the HBM: the ceiling that the layer's data-movement
// kernels (gather, push, combine, reverse-combine pull, SwiGLU backward) are
// held against.  Like those kernels, every workgroup streams a contiguous
// span with plain 16-byte vector loads and stores: 256 lanes x kUnroll units
// (16 KiB), all loads of a lane issued before any is used, one span per
// workgroup, as many workgroups as spans.  Modes: 0 = read only (the loaded
// words are folded into one value per lane, stored only if it equals a value
// the host never passes, so the loads cannot be dropped), 1 = write only,
// 2 = copy (read + write).
#include "mok_internal.h"

namespace mok {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kStreamThreads) void stream_kernel(int mode, uint4* dst,
                                                                const uint4* src, int64_t n,
                                                                uint32_t never) {
  const int64_t base = (int64_t)blockIdx.x * kStreamThreads * kUnroll + threadIdx.x;
  uint4 v[kUnroll];
  if (mode != 1) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kStreamThreads;
      v[u] = i < n ? src[i] : make_uint4(0, 0, 0, 0);
    }
  }
  if (mode == 0) {
    uint32_t fold = 0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) fold ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    if (fold == never && base < n) dst[base] = make_uint4(fold, 0, 0, 0);
    return;
  }
  const uint4 fill = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = base + (int64_t)u * kStreamThreads;
    if (i < n) dst[i] = mode == 1 ? fill : v[u];
  }
}

}  // namespace

mok_status launch_stream(int mode, void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  const int64_t n = bytes / 16;
  if (n == 0) return MOK_OK;
  const int64_t per_block = (int64_t)kStreamThreads * kUnroll;
  const int64_t blocks = (n + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFF) return MOK_EINVAL;
  hipLaunchKernelGGL(stream_kernel, dim3((unsigned)blocks), dim3(kStreamThreads), 0, stream, mode,
                     reinterpret_cast<uint4*>(dst), reinterpret_cast<const uint4*>(src), n,
                     0xA5A5A5A5u);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

}  // namespace mok
