// Forward expert FFN kernels, one launch per GEMM, on the pipelined 256 x 256
// tile engine (tile code in mok_ffn_tiles.h).
//
// The A operand of GEMM1 is either the gathered rows x_perm or -- in the
// layer's forward pass -- the token rows themselves, read from the source
// buffers through row_src: the pull dispatch is then part of the GEMM's own
// loads (kucoin article, section 02: the receiver reads the tokens it needs
// from their sources and places them expert by expert).  GEMM2's epilogue
// pushes y straight to the staging rows (push combine, same section).
#include <string.h>

#include "mok_ffn_tiles.h"
#include "mok_internal.h"

namespace mok {

namespace {

using namespace g2;

// Persistent grouped-M launch: workgroup b runs tiles b, b + gridDim.x, ...
// of the (expert rows, N-tile) grid in XCD-aware grouped order (gridDim.x a
// multiple of 8, so every tile of a workgroup stays on its XCD's range); the
// per-expert tile prefix is built once per workgroup.  fn(g, nt) runs one
// tile; a barrier separates one tile's epilogue from the next tile's loads
// into the same LDS.
template <class Fn>
__device__ __forceinline__ void persistent_tiles(const int32_t* offsets, int E_local, int R_cap,
                                                 int ntn, int* s_prefix, Fn fn) {
  const int total_m = group_prefix(offsets, E_local, R_cap, s_prefix);
  const int total = total_m * ntn;
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    int mt, nt;
    grouped_order(xcd_tile(t, total), total_m, ntn, &mt, &nt);
    const GTile g = group_tile(offsets, E_local, R_cap, s_prefix, mt);
    __syncthreads();
    fn(g, nt);
  }
}

template <class C>
__global__ __launch_bounds__(kThreads, C::OCC) void ffn1_g2(F1Args a, SrcTable src) {
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int s_prefix[257];
  persistent_tiles(a.offsets, a.E_local, a.R_cap, a.ntn, s_prefix, [&](const GTile& g, int nt) {
    ffn1_tile<C>(a, smem, g, nt, [&](int row) -> const bf16_t* {
      const int r = g.r0 + row;
      if (r >= g.r1) return nullptr;
      if (a.x) return a.x + (size_t)r * a.d;
      const int tok = a.row_src[r] / a.k;
      return reinterpret_cast<const bf16_t*>(src.p[tok / a.T_src]) + (size_t)(tok % a.T_src) * a.d;
    });
  });
}

template <class C>
__global__ __launch_bounds__(kThreads, C::OCC) void ffn2_g2(F2Args a, DstTable staging) {
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int s_prefix[257];
  persistent_tiles(a.offsets, a.E_local, a.R_cap, a.ntn, s_prefix,
                   [&](const GTile& g, int nt) { ffn2_tile<C>(a, staging, smem, g, nt); });
}

// Workgroups of a persistent launch over at most `tiles` tiles: one per CU
// (OCC per CU), a multiple of 8.
static unsigned persistent_grid(int tiles, int occ) {
  const int cus = device_cus();
  int n = cus > 0 ? cus * occ : 256;
  n -= n % 8;
  if (n < 8) n = 8;
  return (unsigned)(tiles < n ? ((tiles + 7) / 8) * 8 : n);
}

// One tile per workgroup: GEMM1's epilogue keeps many addresses live, and a
// tile loop around it spills (measured slower than one tile per workgroup).
__global__ __launch_bounds__(kThreads) void ffn1_mx(F1MxArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[MxCfg::SMEM];
  __shared__ int s_prefix[257];
  const int total_m = group_prefix(a.offsets, a.E_local, a.R_cap, s_prefix);
  const int total = total_m * a.ntn;
  if ((int)blockIdx.x >= total) return;
  int mt, nt;
  grouped_order(xcd_tile(blockIdx.x, total), total_m, a.ntn, &mt, &nt);
  const GTile g = group_tile(a.offsets, a.E_local, a.R_cap, s_prefix, mt);
  const int KS = a.d / 32;
  ffn1_mx_tile(
      a, smem, g, nt,
      [&](int row) -> const bf16_t* {
        const int r = g.r0 + row;
        return r < g.r1 ? reinterpret_cast<const bf16_t*>(a.xq + (size_t)r * a.d) : nullptr;
      },
      [&](int row) -> const uint8_t* {
        const int r = g.r0 + row;
        return r < g.r1 ? a.xs + (size_t)r * KS : nullptr;
      });
}

__global__ __launch_bounds__(kThreads) void ffn2_mx(F2Args a, DstTable staging) {
  __shared__ __attribute__((aligned(16))) char smem[MxCfg::SMEM];
  __shared__ int s_prefix[257];
  persistent_tiles(a.offsets, a.E_local, a.R_cap, a.ntn, s_prefix,
                   [&](const GTile& g, int nt) { ffn2_mx_tile(a, staging, smem, g, nt); });
}

}  // namespace

mok_status launch_ffn_bf16(int d, int I, int E_local, int R_cap, const void* x,
                           const SrcTable* src, int T_src, int k, const int32_t* offsets,
                           const int32_t* row_src, const void* wg, const void* wu, const void* wd,
                           void* h, void* ab, void* y, const DstTable* staging,
                           hipStream_t stream, mok_trace* tr) {
  if (R_cap == 0) return MOK_OK;
  const int mt = (R_cap + BM - 1) / BM + E_local;
  F1Args a1;
  memset(&a1, 0, sizeof(a1));
  SrcTable stab;
  memset(&stab, 0, sizeof(stab));
  if (src) stab = *src;
  a1.x = reinterpret_cast<const bf16_t*>(x);
  a1.row_src = row_src;
  a1.wg = reinterpret_cast<const bf16_t*>(wg);
  a1.wu = reinterpret_cast<const bf16_t*>(wu);
  a1.offsets = offsets;
  a1.h = reinterpret_cast<bf16_t*>(h);
  a1.ab = reinterpret_cast<bf16_t*>(ab);
  a1.d = d;
  a1.I = I;
  a1.E_local = E_local;
  a1.R_cap = R_cap;
  a1.ntn = (I + Default::BN / 2 - 1) / (Default::BN / 2);
  a1.T_src = T_src;
  a1.k = k;
  hipLaunchKernelGGL(ffn1_g2<Default>, dim3(persistent_grid(mt * a1.ntn, Default::OCC)), dim3(kThreads),
                     0, stream, a1, stab);
  trace_mark(tr, "ffn1_gate_up_swiglu", stream);
  F2Args a2;
  memset(&a2, 0, sizeof(a2));
  a2.h = reinterpret_cast<const bf16_t*>(h);
  a2.wd = reinterpret_cast<const bf16_t*>(wd);
  a2.offsets = offsets;
  a2.row_src = row_src;
  a2.y = reinterpret_cast<bf16_t*>(y);
  a2.push = staging != nullptr;
  DstTable gtab;
  memset(&gtab, 0, sizeof(gtab));
  if (staging) gtab = *staging;
  a2.d = d;
  a2.I = I;
  a2.E_local = E_local;
  a2.R_cap = R_cap;
  a2.ntn = (d + Default::BN - 1) / Default::BN;
  a2.T_src = T_src;
  a2.k = k;
  hipLaunchKernelGGL(ffn2_g2<Default>, dim3(persistent_grid(mt * a2.ntn, Default::OCC)), dim3(kThreads),
                     0, stream, a2,
                     gtab);
  trace_mark(tr, "ffn2_down", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

mok_status launch_ffn_mx(int d, int I, int E_local, int R_cap, const uint8_t* xq,
                         const uint8_t* xs, const int32_t* offsets, const int32_t* row_src,
                         const mok_expert_weights* w, uint8_t* hq, uint8_t* hs, void* ab, void* y,
                         const DstTable* staging, int T_src, int k, hipStream_t stream,
                         mok_trace* tr) {
  if (R_cap == 0) return MOK_OK;
  if (d % MxCfg::KB != 0 || I % MxCfg::KB != 0) return MOK_EINVAL;
  const int mt = (R_cap + BM - 1) / BM + E_local;
  F1MxArgs a1;
  a1.xq = xq;
  a1.xs = xs;
  a1.wg = reinterpret_cast<const uint8_t*>(w->w_gate);
  a1.wu = reinterpret_cast<const uint8_t*>(w->w_up);
  a1.sg = w->s_gate;
  a1.su = w->s_up;
  a1.offsets = offsets;
  a1.hq = hq;
  a1.hs = hs;
  a1.ab = reinterpret_cast<bf16_t*>(ab);
  a1.d = d;
  a1.I = I;
  a1.E_local = E_local;
  a1.R_cap = R_cap;
  a1.ntn = (I + MxCfg::BN / 2 - 1) / (MxCfg::BN / 2);
  hipLaunchKernelGGL(ffn1_mx, dim3((unsigned)(mt * a1.ntn)), dim3(kThreads), 0, stream, a1);
  trace_mark(tr, "ffn1_gate_up_swiglu_mx", stream);
  F2Args a2;
  memset(&a2, 0, sizeof(a2));
  a2.h = reinterpret_cast<const bf16_t*>(hq);
  a2.wd = reinterpret_cast<const bf16_t*>(w->w_down);
  a2.hs = hs;
  a2.sd = w->s_down;
  a2.offsets = offsets;
  a2.row_src = row_src;
  a2.y = reinterpret_cast<bf16_t*>(y);
  a2.push = staging != nullptr;
  DstTable gtab;
  memset(&gtab, 0, sizeof(gtab));
  if (staging) gtab = *staging;
  a2.d = d;
  a2.I = I;
  a2.E_local = E_local;
  a2.R_cap = R_cap;
  a2.ntn = (d + MxCfg::BN - 1) / MxCfg::BN;
  a2.T_src = T_src;
  a2.k = k;
  hipLaunchKernelGGL(ffn2_mx, dim3(persistent_grid(mt * a2.ntn, 1)), dim3(kThreads), 0, stream, a2, gtab);
  trace_mark(tr, "ffn2_down_mx", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

mok_status launch_mx_rows_gemm(const uint8_t* aq, const uint8_t* as, const uint8_t* bq,
                               const uint8_t* bs, int K, int N, int E_local, int R_cap,
                               const int32_t* offsets, const int32_t* row_src, void* y, int ldy,
                               const DstTable* push, int T_src, int k, hipStream_t stream,
                               mok_trace* tr, const char* name) {
  if (R_cap == 0) return MOK_OK;
  if (K % MxCfg::KB != 0) return MOK_EINVAL;
  const int mt = (R_cap + BM - 1) / BM + E_local;
  F2Args a;
  memset(&a, 0, sizeof(a));
  a.h = reinterpret_cast<const bf16_t*>(aq);
  a.hs = as;
  a.wd = reinterpret_cast<const bf16_t*>(bq);
  a.sd = bs;
  a.offsets = offsets;
  a.row_src = row_src;
  a.y = reinterpret_cast<bf16_t*>(y);
  a.ldy = ldy;
  a.push = push != nullptr;
  DstTable tab;
  memset(&tab, 0, sizeof(tab));
  if (push) tab = *push;
  a.d = N;  // output columns (the tile's N)
  a.I = K;  // contraction
  a.E_local = E_local;
  a.R_cap = R_cap;
  a.ntn = (N + MxCfg::BN - 1) / MxCfg::BN;
  a.T_src = T_src;
  a.k = k;
  hipLaunchKernelGGL(ffn2_mx, dim3((unsigned)(mt * a.ntn)), dim3(kThreads), 0, stream, a, tab);
  trace_mark(tr, name, stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

}  // namespace mok
