// Router kernel: logits on the vector ALU (fp32 chain), top-k, gates.
//
// A router picks a few experts per token (kucoin article, section 01).  The
// pages fix neither the score function nor the tie rule; this library uses:
//   z[t][e] = fp32 chain over i ascending: z = fma(x_i, w_i, z), from 0,
//             then one fp32 add of bias[e];
//   top-k   = k largest z, equal z -> lower expert id first, slot 0 largest;
//   gate_j  = exp(z_j - z_0) / sum_i exp(z_i - z_0) over the chosen slots
//             (= softmax over all experts renormalised over the chosen ones).
// Every output (t, e) keeps its own sequential chain, so the logits -- and
// hence the selection -- are reproducible bit for bit.  No matrix cores here:
// the chain order is the contract.
#include "mok_internal.h"

namespace mok {

namespace {

constexpr int kRouteThreads = 256;
constexpr int kTE = 4;      // experts per thread
constexpr int kMaxK = 16;

struct RouteArgs {
  SrcTable src;     // token buffers: token g of the launch is src.p[src_lo + g / T_src][g % T_src]
  int src_lo, T_src;
  const void* w;
  const float* bias;
  int32_t* topk_idx;  // [T, k] for the launch's tokens, in order
  float* topk_gate;
  int T, d, E, k;
  int EG, TG, TB;   // threads across experts, threads across tokens, tokens per block
  int dc;           // d-chunk staged through LDS
  int xs_pitch, ws_pitch, zs_pitch;
};

template <typename T>
struct Unit;
template <>
struct Unit<bf16_t> {
  static constexpr int n = 8;
};
template <>
struct Unit<float> {
  static constexpr int n = 4;
};

template <typename T>
__device__ __forceinline__ void unpack(uint4 u, float* out);
template <>
__device__ __forceinline__ void unpack<bf16_t>(uint4 u, float* out) {
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void unpack<float>(uint4 u, float* out) {
  out[0] = __uint_as_float(u.x);
  out[1] = __uint_as_float(u.y);
  out[2] = __uint_as_float(u.z);
  out[3] = __uint_as_float(u.w);
}

template <typename T, int TT>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
  extern __shared__ float smem[];
  float* xs = smem;                              // [dc][xs_pitch]  (token fastest)
  float* ws = xs + a.dc * a.xs_pitch;            // [dc][ws_pitch]  (expert fastest)
  float* zs = smem;                              // [TB][zs_pitch] logits, after the d loop
  constexpr int U = Unit<T>::n;
  const int UPR = a.dc / U;                      // units per row chunk

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * a.TB;
  const int eg = tid % a.EG;
  const int tg = tid / a.EG;
  const bool computes = tg < a.TG;
  const T* w = reinterpret_cast<const T*>(a.w);
  const int Epad = a.EG * kTE;

  float acc[TT][kTE];
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < kTE; ++j) acc[i][j] = 0.0f;

  for (int c0 = 0; c0 < a.d; c0 += a.dc) {
    // stage x[t0 .. t0+TB) x [c0, c0+dc) transposed
    for (int u = tid; u < a.TB * UPR; u += kRouteThreads) {
      int t = u / UPR, q = u % UPR;
      float v[U];
      if (t0 + t < a.T) {
        const int g = t0 + t;
        const T* x = reinterpret_cast<const T*>(a.src.p[a.src_lo + g / a.T_src]) +
                     (size_t)(g % a.T_src) * a.d;
        unpack<T>(ld16(x + c0 + q * U), v);
      } else {
#pragma unroll
        for (int i = 0; i < U; ++i) v[i] = 0.0f;
      }
#pragma unroll
      for (int i = 0; i < U; ++i) xs[(q * U + i) * a.xs_pitch + t] = v[i];
    }
    // stage w[0 .. Epad) x [c0, c0+dc) transposed
    for (int u = tid; u < Epad * UPR; u += kRouteThreads) {
      int e = u / UPR, q = u % UPR;
      float v[U];
      if (e < a.E) {
        unpack<T>(ld16(w + (size_t)e * a.d + c0 + q * U), v);
      } else {
#pragma unroll
        for (int i = 0; i < U; ++i) v[i] = 0.0f;
      }
#pragma unroll
      for (int i = 0; i < U; ++i) ws[(q * U + i) * a.ws_pitch + e] = v[i];
    }
    __syncthreads();
    if (computes) {
#pragma unroll 4
      for (int i = 0; i < a.dc; ++i) {
        float xv[TT], wv[kTE];
#pragma unroll
        for (int q = 0; q < TT; ++q) xv[q] = xs[i * a.xs_pitch + tg * TT + q];
#pragma unroll
        for (int q = 0; q < kTE; ++q) wv[q] = ws[i * a.ws_pitch + eg * kTE + q];
#pragma unroll
        for (int p = 0; p < TT; ++p)
#pragma unroll
          for (int q = 0; q < kTE; ++q) acc[p][q] = __builtin_fmaf(xv[p], wv[q], acc[p][q]);
      }
    }
    __syncthreads();
  }

  if (computes) {
#pragma unroll
    for (int p = 0; p < TT; ++p)
#pragma unroll
      for (int q = 0; q < kTE; ++q) {
        int e = eg * kTE + q;
        if (e < a.E) {
          float z = acc[p][q];
          if (a.bias) z = z + a.bias[e];
          zs[(tg * TT + p) * a.zs_pitch + e] = z;
        }
      }
  }
  __syncthreads();

  // selection: one wave per token
  const int lane = tid & 63, wave = tid >> 6;
  const int MPL = (a.E + 63) / 64;   // entries per lane (<= 8)
  for (int tl = wave; tl < a.TB; tl += kRouteThreads / 64) {
    const int t = t0 + tl;
    if (t >= a.T) break;
    float zv[8];
    uint32_t used = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      int e = lane + 64 * m;
      zv[m] = (m < MPL && e < a.E) ? zs[tl * a.zs_pitch + e] : -__builtin_inff();
    }
    float zsel[kMaxK];
    int esel[kMaxK];
    for (int j = 0; j < a.k; ++j) {
      float bz = -__builtin_inff();
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        int e = lane + 64 * m;
        bool ok = m < MPL && e < a.E && !((used >> m) & 1u);
        if (ok && (zv[m] > bz || (zv[m] == bz && e < be))) {
          bz = zv[m];
          be = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        float oz = __shfl_xor(bz, off, 64);
        int oe = __shfl_xor(be, off, 64);
        if (oz > bz || (oz == bz && oe < be)) {
          bz = oz;
          be = oe;
        }
      }
      if ((be & 63) == lane) used |= 1u << (be >> 6);
      zsel[j < kMaxK ? j : 0] = bz;
      esel[j < kMaxK ? j : 0] = be;
    }
    float sum = 0.0f;
    float ex[kMaxK];
    for (int j = 0; j < a.k; ++j) {
      ex[j] = expf(zsel[j] - zsel[0]);
      sum += ex[j];
    }
    for (int j = 0; j < a.k; ++j) {
      if (lane == j) {
        a.topk_idx[(size_t)t * a.k + j] = esel[j];
        a.topk_gate[(size_t)t * a.k + j] = ex[j] / sum;
      }
    }
  }
}

}  // namespace

// Block geometry for E experts: EG threads across experts (kTE each), TG across
// tokens (TT each), TB tokens per block, dc-wide d chunks.  Returns TT.
int route_geometry(int E, int T, int* EG, int* TG, int* TB, int* dc) {
  *EG = (E + kTE - 1) / kTE;
  int tg = kRouteThreads / *EG;
  *dc = E > 256 ? 16 : 32;
  // 4 tokens per thread, fewer when that leaves fewer than two workgroups per CU
  int TT = 4;
  while (TT > 1) {
    int cap = 128 / TT;
    int g = tg < cap ? tg : cap;
    if ((T + g * TT - 1) / (g * TT) >= 512) break;
    TT >>= 1;
  }
  int cap = 128 / TT;
  *TG = tg < cap ? tg : cap;
  *TB = *TG * TT;
  return TT;
}

mok_status launch_route(int prec, const SrcTable& src, int src_lo, int T_src, int T, int d,
                        int E, int k, const void* w, const float* bias, int32_t* topk_idx,
                        float* topk_gate, hipStream_t stream, mok_trace* tr) {
  if (T == 0) return MOK_OK;
  RouteArgs a;
  a.src = src;
  a.src_lo = src_lo;
  a.T_src = T_src;
  a.w = w;
  a.bias = bias;
  a.topk_idx = topk_idx;
  a.topk_gate = topk_gate;
  a.T = T;
  a.d = d;
  a.E = E;
  a.k = k;
  const int TT = route_geometry(E, T, &a.EG, &a.TG, &a.TB, &a.dc);
  a.xs_pitch = a.TB + 4;
  a.ws_pitch = a.EG * kTE + 4;
  a.zs_pitch = a.EG * kTE + 1;
  size_t smem = route_smem_bytes(E, T);
  dim3 grid((T + a.TB - 1) / a.TB);
  dim3 blk(kRouteThreads);
#define MOK_ROUTE_LAUNCH(TY, TTV) \
  hipLaunchKernelGGL((route_kernel<TY, TTV>), grid, blk, smem, stream, a)
  if (prec == MOK_F32) {
    if (TT == 4) MOK_ROUTE_LAUNCH(float, 4);
    else if (TT == 2) MOK_ROUTE_LAUNCH(float, 2);
    else MOK_ROUTE_LAUNCH(float, 1);
  } else {
    if (TT == 4) MOK_ROUTE_LAUNCH(bf16_t, 4);
    else if (TT == 2) MOK_ROUTE_LAUNCH(bf16_t, 2);
    else MOK_ROUTE_LAUNCH(bf16_t, 1);
  }
#undef MOK_ROUTE_LAUNCH
  trace_mark(tr, "route", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

size_t route_smem_bytes(int E, int T) {
  int EG, TG, TB, dc;
  route_geometry(E, T, &EG, &TG, &TB, &dc);
  size_t stage = (size_t)dc * (TB + 4) + (size_t)dc * (EG * kTE + 4);
  size_t logits = (size_t)TB * (EG * kTE + 1);
  return sizeof(float) * (stage > logits ? stage : logits);
}

}  // namespace mok
