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

// fp32 -> bf16, round to nearest even: gfx950 converts in hardware
// (v_cvt_pk_bf16_f32, two values per instruction).
typedef __bf16 bf16x2_hw_t __attribute__((ext_vector_type(2)));
typedef float f32x2_hw_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}
// Two values -> one word (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  const f32x2_hw_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw_t));
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

// sigmoid(a) = 1 / (1 + e^-a) with the hardware base-2 exponential and
// reciprocal (each within 1 ulp): e^-a = 2^(-a log2 e).  a -> -inf gives
// 1/inf = 0, a -> +inf gives 1.
__device__ __forceinline__ float sigmoid_f(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * -1.4426950408889634f));
}
__device__ __forceinline__ float silu_f(float a) { return a * sigmoid_f(a); }

// Record one trace event after the kernel just launched (host side).
inline void trace_mark(mok_trace* t, const char* name, hipStream_t s) {
  if (!t || !t->events || t->count >= t->capacity) return;
  (void)hipEventRecord((hipEvent_t)t->events[t->count], s);
  if (t->names) t->names[t->count] = name;
  // the previous event on the same stream (the last two streams are kept)
  int slot = t->last_stream[0] == (void*)s ? 0 : t->last_stream[1] == (void*)s ? 1 : -1;
  if (t->from) t->from[t->count] = slot >= 0 ? t->last_idx[slot] : -1;
  if (slot < 0) {  // replace the older entry
    slot = t->last_idx[0] <= t->last_idx[1] ? 0 : 1;
    t->last_stream[slot] = (void*)s;
  }
  t->last_idx[slot] = t->count;
  t->count += 1;
}

}  // namespace mok

#define MOK_HIP_CHECK(x)                         \
  do {                                           \
    hipError_t e_ = (x);                         \
    if (e_ != hipSuccess) return MOK_EDEVICE;    \
  } while (0)
