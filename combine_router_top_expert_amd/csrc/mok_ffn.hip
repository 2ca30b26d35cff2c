// Forward expert FFN as two M-grouped GEMMs on the matrix cores.
//
// kucoin article, section 01: each expert's tokens are grouped so that a
// grouped GEMM receives ordered input; section 02 names SwiGLU in the expert
// path.  For expert e and its rows [offsets[e], offsets[e+1]):
//   GEMM1: a = x W_gate[e]^T, b = x W_up[e]^T   (one tile holds matching
//          32-column blocks of gate and up, so a and b of the same (row, i)
//          meet in one lane), epilogue h = silu(a) * b -> h, and a | b saved
//          for the backward pass;
//   GEMM2: y = h W_down[e]^T, epilogue either stores y in expert order or
//          pushes each row straight to its (source, token, slot) staging row
//          (push combine fused into the GEMM epilogue).
// Tiles are 128 x 128, a flat grid over (m-tile of the grouped rows, n-tile);
// workgroups past the routed rows exit at once (row counts stay on device).
// This engine runs the fp32 layer only; bf16 goes to the pipelined engine
// (mok_ffn2.hip), the one the layer path uses.
#include "mok_gemm.h"
#include "mok_internal.h"

namespace mok {

namespace {

struct Ffn1Args {
  const void* x;      // [R_cap, d]
  const void* wg;     // [E_local, I, d]
  const void* wu;
  const int32_t* offsets;
  void* h;            // [R_cap, I]
  void* ab;           // [R_cap, 2I] or null
  int d, I, E_local, R_cap, ntn;
};

template <typename T>
__global__ __launch_bounds__(kGemmThreads) void ffn1_kernel(Ffn1Args a) {
  __shared__ __attribute__((aligned(16))) T smem[TileSmem<T>::BYTES / sizeof(T)];
  __shared__ int s_prefix[257];
  const int mtile = blockIdx.x / a.ntn, nt = blockIdx.x % a.ntn;
  GroupTile g;
  if (!find_group_tile(a.offsets, a.E_local, a.R_cap, mtile, s_prefix, &g)) return;
  const T* x = reinterpret_cast<const T*>(a.x);
  const T* wg = reinterpret_cast<const T*>(a.wg) + (size_t)g.e * a.I * a.d;
  const T* wu = reinterpret_cast<const T*>(a.wu) + (size_t)g.e * a.I * a.d;
  KLoader<T, kBM> la;
  KLoader<T, kBN> lb;
  la.init([&](int row) -> const T* {
    const int r = g.r0 + row;
    return r < g.r1 ? x + (size_t)r * a.d : nullptr;
  });
  lb.init([&](int nr) -> const T* {
    const int blk = nr >> 5;
    const int i = nt * 64 + (blk >> 1) * 32 + (nr & 31);
    if (i >= a.I) return nullptr;
    return ((blk & 1) ? wu : wg) + (size_t)i * a.d;
  });
  Acc acc;
  gemm_mainloop<T>(a.d / MfmaT<T>::BK, la, lb, [&](int kt, uint4(&r)[KLoader<T, kBM>::NU]) { la.load(kt, r); },
                   [&](int kt, uint4(&r)[KLoader<T, kBN>::NU]) { lb.load(kt, r); }, smem, acc);
  T* h = reinterpret_cast<T*>(a.h);
  T* ab = reinterpret_cast<T*>(a.ab);
  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
  const int i = nt * 64 + wn * 32 + (lane & 31);
  if (i >= a.I) return;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = g.r0 + acc_row(mi, v);
      if (r >= g.r1) continue;
      const float av = acc.c[mi][0][v], bv = acc.c[mi][1][v];
      h[(size_t)r * a.I + i] = from_f32<T>(silu_f(av) * bv);
      if (ab) {
        ab[(size_t)r * 2 * a.I + i] = from_f32<T>(av);
        ab[(size_t)r * 2 * a.I + a.I + i] = from_f32<T>(bv);
      }
    }
}

struct Ffn2Args {
  const void* h;      // [R_cap, I]
  const void* wd;     // [E_local, d, I]
  const int32_t* offsets;
  const int32_t* row_src;
  void* y;            // [R_cap, d] when not pushing
  DstTable staging;   // push destinations [T_src*k, d]
  int push;
  int d, I, E_local, R_cap, ntn, T_src, k;
};

template <typename T>
__global__ __launch_bounds__(kGemmThreads) void ffn2_kernel(Ffn2Args a) {
  __shared__ __attribute__((aligned(16))) T smem[TileSmem<T>::BYTES / sizeof(T)];
  __shared__ int s_prefix[257];
  const int mtile = blockIdx.x / a.ntn, nt = blockIdx.x % a.ntn;
  GroupTile g;
  if (!find_group_tile(a.offsets, a.E_local, a.R_cap, mtile, s_prefix, &g)) return;
  const T* hp = reinterpret_cast<const T*>(a.h);
  const T* wd = reinterpret_cast<const T*>(a.wd) + (size_t)g.e * a.d * a.I;
  KLoader<T, kBM> la;
  KLoader<T, kBN> lb;
  la.init([&](int row) -> const T* {
    const int r = g.r0 + row;
    return r < g.r1 ? hp + (size_t)r * a.I : nullptr;
  });
  lb.init([&](int nr) -> const T* {
    const int c = nt * kBN + nr;
    return c < a.d ? wd + (size_t)c * a.I : nullptr;
  });
  Acc acc;
  gemm_mainloop<T>(a.I / MfmaT<T>::BK, la, lb, [&](int kt, uint4(&r)[KLoader<T, kBM>::NU]) { la.load(kt, r); },
                   [&](int kt, uint4(&r)[KLoader<T, kBN>::NU]) { lb.load(kt, r); }, smem, acc);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = g.r0 + acc_row(mi, v);
      if (r >= g.r1) continue;
      T* dst;
      if (a.push) {
        const int n = a.row_src[r];
        const int tok = n / a.k, j = n % a.k;
        const int s = tok / a.T_src, t = tok % a.T_src;
        dst = reinterpret_cast<T*>(a.staging.p[s]) + ((size_t)t * a.k + j) * a.d;
      } else {
        dst = reinterpret_cast<T*>(a.y) + (size_t)r * a.d;
      }
#pragma unroll
      for (int nj = 0; nj < 2; ++nj) {
        const int c = nt * kBN + acc_col(nj);
        if (c < a.d) dst[c] = from_f32<T>(acc.c[mi][nj][v]);
      }
    }
}

}  // namespace

int grouped_mtiles_bound(int R_cap, int E_local) { return (R_cap + kBM - 1) / kBM + E_local; }

mok_status launch_ffn(int prec, int d, int I, int E_local, int R_cap, const void* x,
                      const int32_t* offsets, const int32_t* row_src, const void* wg,
                      const void* wu, const void* wd, void* h, void* ab, void* y,
                      const DstTable* staging, int T_src, int k, hipStream_t stream,
                      mok_trace* tr) {
  if (R_cap == 0) return MOK_OK;
  // bf16 runs on the pipelined engine of the layer path; this engine is fp32 only
  if (prec == MOK_BF16)
    return launch_ffn_bf16(d, I, E_local, R_cap, x, nullptr, T_src, k, offsets, row_src, wg, wu,
                           wd, h, ab, y, staging, stream, tr);
  if (prec != MOK_F32) return MOK_EINVAL;
  const int mt = grouped_mtiles_bound(R_cap, E_local);
  Ffn1Args a1;
  a1.x = x;
  a1.wg = wg;
  a1.wu = wu;
  a1.offsets = offsets;
  a1.h = h;
  a1.ab = ab;
  a1.d = d;
  a1.I = I;
  a1.E_local = E_local;
  a1.R_cap = R_cap;
  a1.ntn = (I + 63) / 64;
  dim3 g1((unsigned)(mt * a1.ntn));
  Ffn2Args a2;
  a2.h = h;
  a2.wd = wd;
  a2.offsets = offsets;
  a2.row_src = row_src;
  a2.y = y;
  a2.push = staging != nullptr;
  if (staging) a2.staging = *staging;
  a2.d = d;
  a2.I = I;
  a2.E_local = E_local;
  a2.R_cap = R_cap;
  a2.ntn = (d + kBN - 1) / kBN;
  a2.T_src = T_src;
  a2.k = k;
  dim3 g2((unsigned)(mt * a2.ntn));
  hipLaunchKernelGGL(ffn1_kernel<float>, g1, dim3(kGemmThreads), 0, stream, a1);
  trace_mark(tr, "ffn1_gate_up_swiglu", stream);
  hipLaunchKernelGGL(ffn2_kernel<float>, g2, dim3(kGemmThreads), 0, stream, a2);
  trace_mark(tr, "ffn2_down", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

}  // namespace mok
