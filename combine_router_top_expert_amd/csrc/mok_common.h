// Shared device/host helpers of the gfx950 MoE layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mok.h"

namespace mok {

typedef uint16_t bf16_t;  // bf16 bit pattern

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;

struct SrcTable {
  const void* p[MOK_MAX_SOURCES];
};
struct DstTable {
  void* p[MOK_MAX_SOURCES];
};

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) {
  return bf16_to_f32(v);
}

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
  return f32_to_bf16(v);
}

// First device-side error wins; later ones are dropped.
__device__ __forceinline__ void latch(int32_t* st, int32_t code) {
  if (st) atomicCAS(st, 0, code);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// 16-byte vector load/store helpers.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

// Record one trace event after the kernel just launched (host side).
inline void trace_mark(mok_trace* t, const char* name, hipStream_t s) {
  if (!t || !t->events || t->count >= t->capacity) return;
  (void)hipEventRecord((hipEvent_t)t->events[t->count], s);
  if (t->names) t->names[t->count] = name;
  t->count += 1;
}

}  // namespace mok

#define MOK_HIP_CHECK(x)                         \
  do {                                           \
    hipError_t e_ = (x);                         \
    if (e_ != hipSuccess) return MOK_EDEVICE;    \
  } while (0)
