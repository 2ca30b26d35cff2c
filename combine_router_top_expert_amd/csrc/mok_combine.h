// The final weighted combine of one token, shared by the stand-alone combine
// kernel and the persistent ring kernel's dispatch/combine side (kucoin
// article, section 03: the final weighted combine is its own step of the
// layer): out[c] = sum over the token's slots j in ascending order of
// gate_j * staging_j[c], in fp32 from 0, rounded once to the storage dtype.
// A slot whose local row was dropped beyond R_cap (dest_row >= R_cap) is left
// out; a remote slot (dest_row == -1) holds what the GPU with that expert
// pushed.  Lanes lane0, lane0 + nlanes, ... take 16-byte units of the row.
#pragma once

#include "mok_common.h"

namespace mok {

template <typename T>
__device__ __forceinline__ void combine_token(const int32_t* dest_row, const float* gate,
                                              int64_t n0, int k, int R_cap, const T* stg, T* o,
                                              int d, int lane0, int nlanes) {
  constexpr int U = 16 / sizeof(T);
  constexpr int G = 8;  // slots whose loads are in flight together
  const int units = d / U;
  for (int u = lane0; u < units; u += nlanes) {
    float acc[U];
#pragma unroll
    for (int i = 0; i < U; ++i) acc[i] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += G) {
      uint4 v[G];
#pragma unroll
      for (int q = 0; q < G; ++q)
        if (j0 + q < k) v[q] = ld16(stg + (size_t)(j0 + q) * d + u * U);
#pragma unroll
      for (int q = 0; q < G; ++q) {
        const int j = j0 + q;
        if (j >= k || dest_row[n0 + j] >= R_cap) continue;
        const float gj = gate[n0 + j];
        const T* e = reinterpret_cast<const T*>(&v[q]);
#pragma unroll
        for (int i = 0; i < U; ++i) acc[i] = __builtin_fmaf(gj, to_f32<T>(e[i]), acc[i]);
      }
    }
    uint4 outv;
    T* ov = reinterpret_cast<T*>(&outv);
#pragma unroll
    for (int i = 0; i < U; ++i) ov[i] = from_f32<T>(acc[i]);
    st16(o + u * U, outv);
  }
}

}  // namespace mok
