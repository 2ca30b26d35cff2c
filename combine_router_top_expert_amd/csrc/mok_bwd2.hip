// Backward expert GEMMs, bf16, on the pipelined 256 x 256 tile engine.
//   dh  : dh = dy W_down[e]           A = dy (k = d contiguous), B = W_down
//         read as [d][I] (n contiguous) -> epilogue SwiGLU derivative, dab
//   dx  : dx = dab [W_gate; W_up]      A = dab (k = 2I contiguous), B = the
//         two weight matrices read as [2I][d] -> epilogue pushes dx rows to
//         their reverse-dispatch staging rows
//   wgrad (per expert, contraction over the expert's rows in ascending row
//         order; rows past the expert read zeros):
//         [dW_gate; dW_up][e] = dab^T X_e   (A = dab, B = gathered rows X)
//         dW_down[e]          = dy^T h_e    (A = dy,  B = h)
// The m/n-contiguous operands are read with the transposing LDS fragment
// loads of the engine; no operand is transposed in memory.
#include "mok_gemm2.h"
#include "mok_internal.h"

namespace mok {

namespace {

using namespace g2;

struct DhArgs {
  const bf16_t* dy;    // [R_cap, d]
  const bf16_t* wd;    // [E_local, d, I]
  const bf16_t* ab;    // [R_cap, 2I]
  bf16_t* dab;         // [R_cap, 2I]
  const int32_t* offsets;
  int d, I, E_local, R_cap, ntn;
};

template <class C>
__global__ __launch_bounds__(kThreads) void dh_g2(DhArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int s_prefix[257];
  const int total_m = group_prefix(a.offsets, a.E_local, a.R_cap, s_prefix);
  const int total = total_m * a.ntn;
  if ((int)blockIdx.x >= total) return;
  const int t = xcd_tile(blockIdx.x, total);
  const int mtile = t / a.ntn, nt = t % a.ntn;
  const GTile g = group_tile(a.offsets, a.E_local, a.R_cap, s_prefix, mtile);
  const int n0 = nt * C::BN;
  const bf16_t* wd = a.wd + (size_t)g.e * a.d * a.I + n0;
  KMajor<BM, C::BK> la;
  la.init([&](int row) -> const bf16_t* {
    const int r = g.r0 + row;
    return r < g.r1 ? a.dy + (size_t)r * a.d : nullptr;
  });
  MNMajor<C::BN, C::BK> lb;
  lb.ncols_left = a.I - n0;
  Acc<C> acc;
  mainloop<C, false, true>(a.d / C::BK, [&](int kt, unsigned l) { la.issue(kt, l); },
                        [&](int kt, unsigned l) {
                          lb.issue(kt, l, [&](int kk) -> const bf16_t* { return wd + (size_t)kk * a.I; });
                        },
                        smem, acc);
  // dh staged as fp32; the row walk reads a | b and writes da | db with
  // contiguous 8-byte pieces per lane
  __syncthreads();
  const WaveStage<C, float> st(smem);
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int pass = 0; pass < WaveStage<C, float>::PASSES; ++pass) {
    st.put(acc, pass);
    wave_lds_fence();
    st.for_chunks(pass, [&](int trow, int srow, int c) {
      const int r = g.r0 + (wave >> 1) * 128 + trow;
      const int i = n0 + (wave & 1) * (C::BN / 2) + c * 4;
      if (r >= g.r1 || i >= a.I) return;
      float dh[4];
      st.get(srow, c, dh);
      const bf16_t* abr = a.ab + (size_t)r * 2 * a.I;
      bf16_t* dabr = a.dab + (size_t)r * 2 * a.I;
      const uint2 av4 = *reinterpret_cast<const uint2*>(abr + i);
      const uint2 bv4 = *reinterpret_cast<const uint2*>(abr + a.I + i);
      const uint32_t aw[2] = {av4.x, av4.y}, bw[2] = {bv4.x, bv4.y};
      float da[4], db[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float av = __uint_as_float(e & 1 ? aw[e >> 1] & 0xFFFF0000u : aw[e >> 1] << 16);
        const float bv = __uint_as_float(e & 1 ? bw[e >> 1] & 0xFFFF0000u : bw[e >> 1] << 16);
        const float sg = 1.0f / (1.0f + __expf(-av));
        da[e] = dh[e] * bv * sg * (1.0f + av * (1.0f - sg));
        db[e] = dh[e] * av * sg;
      }
      *reinterpret_cast<uint2*>(dabr + i) = pack4_bf16(da[0], da[1], da[2], da[3]);
      *reinterpret_cast<uint2*>(dabr + a.I + i) = pack4_bf16(db[0], db[1], db[2], db[3]);
    });
    wave_lds_fence();
  }
}

struct DxArgs {
  const bf16_t* dab;   // [R_cap, 2I]
  const bf16_t* wg;    // [E_local, I, d]
  const bf16_t* wu;
  const int32_t* offsets;
  const int32_t* row_src;
  DstTable dx_stage;
  int d, I, E_local, R_cap, ntn, T_src, k;
};

template <class C>
__global__ __launch_bounds__(kThreads) void dx_g2(DxArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int s_prefix[257];
  const int total_m = group_prefix(a.offsets, a.E_local, a.R_cap, s_prefix);
  const int total = total_m * a.ntn;
  if ((int)blockIdx.x >= total) return;
  const int t = xcd_tile(blockIdx.x, total);
  const int mtile = t / a.ntn, nt = t % a.ntn;
  const GTile g = group_tile(a.offsets, a.E_local, a.R_cap, s_prefix, mtile);
  const int n0 = nt * C::BN;
  const bf16_t* wg = a.wg + (size_t)g.e * a.I * a.d + n0;
  const bf16_t* wu = a.wu + (size_t)g.e * a.I * a.d + n0;
  KMajor<BM, C::BK> la;
  la.init([&](int row) -> const bf16_t* {
    const int r = g.r0 + row;
    return r < g.r1 ? a.dab + (size_t)r * 2 * a.I : nullptr;
  });
  MNMajor<C::BN, C::BK> lb;
  lb.ncols_left = a.d - n0;
  Acc<C> acc;
  mainloop<C, false, true>(2 * a.I / C::BK, [&](int kt, unsigned l) { la.issue(kt, l); },
                        [&](int kt, unsigned l) {
                          lb.issue(kt, l, [&](int kk) -> const bf16_t* {
                            return kk < a.I ? wg + (size_t)kk * a.d : wu + (size_t)(kk - a.I) * a.d;
                          });
                        },
                        smem, acc);
  __syncthreads();
  const WaveStage<C, bf16_t> st(smem);
  st.put(acc, 0);
  wave_lds_fence();
  const int wave = threadIdx.x >> 6;
  st.for_chunks(0, [&](int trow, int srow, int c) {
    const int r = g.r0 + (wave >> 1) * 128 + trow;
    const int col = n0 + (wave & 1) * (C::BN / 2) + c * 8;
    if (r >= g.r1 || col >= a.d) return;
    const int n = a.row_src[r];
    const int tok = n / a.k, j = n % a.k;
    bf16_t* dst = reinterpret_cast<bf16_t*>(a.dx_stage.p[tok / a.T_src]) +
                  ((size_t)(tok % a.T_src) * a.k + j) * a.d;
    *reinterpret_cast<uint4*>(dst + col) = st.raw(srow, c);
  });
}

// MODE 0: M = 2I (dab columns), N = d (gathered token rows); MODE 1: M = d (dy), N = I (h)
struct WgArgs {
  const bf16_t* A;     // [R_cap, lda] rows of the expert
  const bf16_t* B;     // [R_cap, ldb]
  float* out0;         // MODE 0: dW_gate [E_local, I, d]; MODE 1: dW_down [E_local, d, I]
  float* out1;         // MODE 0: dW_up
  const int32_t* offsets;
  int lda, ldb, M, N, I, E_local, R_cap, mtn, ntn;
};

template <class C, int MODE>
__global__ __launch_bounds__(kThreads) void wgrad_g2(WgArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  const int per = a.mtn * a.ntn;
  const int total = a.E_local * per;
  const int t = xcd_tile(blockIdx.x, total);
  const int e = t / per;
  const int mt = (t % per) / a.ntn, nt = t % a.ntn;
  const int off = min(a.offsets[e], a.R_cap);
  const int end = min(a.offsets[e + 1], a.R_cap);
  const int cnt = end > off ? end - off : 0;
  const int m0 = mt * BM, n0 = nt * C::BN;
  MNMajor<BM, C::BK> la;
  MNMajor<C::BN, C::BK> lb;
  la.ncols_left = a.M - m0;
  lb.ncols_left = a.N - n0;
  const bf16_t* Ab = a.A + (size_t)off * a.lda + m0;
  const bf16_t* Bb = a.B + (size_t)off * a.ldb + n0;
  Acc<C> acc;
  mainloop<C, true, true>((cnt + C::BK - 1) / C::BK,
                       [&](int kt, unsigned l) {
                         la.issue(kt, l, [&](int kk) -> const bf16_t* {
                           return kk < cnt ? Ab + (size_t)kk * a.lda : nullptr;
                         });
                       },
                       [&](int kt, unsigned l) {
                         lb.issue(kt, l, [&](int kk) -> const bf16_t* {
                           return kk < cnt ? Bb + (size_t)kk * a.ldb : nullptr;
                         });
                       },
                       smem, acc);
  __syncthreads();
  const WaveStage<C, float> st(smem);
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int pass = 0; pass < WaveStage<C, float>::PASSES; ++pass) {
    st.put(acc, pass);
    wave_lds_fence();
    st.for_chunks(pass, [&](int trow, int srow, int c) {
      const int m = m0 + (wave >> 1) * 128 + trow;
      const int col = n0 + (wave & 1) * (C::BN / 2) + c * 4;
      if (m >= a.M || col >= a.N) return;
      float* dst;
      if (MODE == 0)
        dst = m < a.I ? a.out0 + ((size_t)e * a.I + m) * a.N : a.out1 + ((size_t)e * a.I + (m - a.I)) * a.N;
      else
        dst = a.out0 + ((size_t)e * a.M + m) * a.N;
      *reinterpret_cast<uint4*>(dst + col) = st.raw(srow, c);
    });
    wave_lds_fence();
  }
}

}  // namespace

mok_status launch_bwd_gemms_bf16(const BwdPlan& p, const void* x_perm, hipStream_t stream) {
  const int mt = (p.R_cap + BM - 1) / BM + p.E_local;
  if (p.R_cap > 0) {
    DhArgs d;
    d.dy = reinterpret_cast<const bf16_t*>(p.dy);
    d.wd = reinterpret_cast<const bf16_t*>(p.wd);
    d.ab = reinterpret_cast<const bf16_t*>(p.ab);
    d.dab = reinterpret_cast<bf16_t*>(p.dab);
    d.offsets = p.offsets;
    d.d = p.d;
    d.I = p.I;
    d.E_local = p.E_local;
    d.R_cap = p.R_cap;
    d.ntn = (p.I + Default::BN - 1) / Default::BN;
    hipLaunchKernelGGL(dh_g2<Default>, dim3((unsigned)(mt * d.ntn)), dim3(kThreads), 0, stream, d);
    trace_mark(p.tr, "bwd_dh_swiglu", stream);
    DxArgs x;
    x.dab = reinterpret_cast<const bf16_t*>(p.dab);
    x.wg = reinterpret_cast<const bf16_t*>(p.wg);
    x.wu = reinterpret_cast<const bf16_t*>(p.wu);
    x.offsets = p.offsets;
    x.row_src = p.row_src;
    x.dx_stage = p.dx_stage;
    x.d = p.d;
    x.I = p.I;
    x.E_local = p.E_local;
    x.R_cap = p.R_cap;
    x.ntn = (p.d + Default::BN - 1) / Default::BN;
    x.T_src = p.T_src;
    x.k = p.k;
    hipLaunchKernelGGL(dx_g2<Default>, dim3((unsigned)(mt * x.ntn)), dim3(kThreads), 0, stream, x);
    trace_mark(p.tr, "bwd_dx_push", stream);
  }
  WgArgs w;
  w.A = reinterpret_cast<const bf16_t*>(p.dab);
  w.B = reinterpret_cast<const bf16_t*>(x_perm);
  w.out0 = p.dw_gate;
  w.out1 = p.dw_up;
  w.offsets = p.offsets;
  w.lda = 2 * p.I;
  w.ldb = p.d;
  w.M = 2 * p.I;
  w.N = p.d;
  w.I = p.I;
  w.E_local = p.E_local;
  w.R_cap = p.R_cap;
  w.mtn = (w.M + BM - 1) / BM;
  w.ntn = (w.N + Default::BN - 1) / Default::BN;
  hipLaunchKernelGGL((wgrad_g2<Default, 0>), dim3((unsigned)(p.E_local * w.mtn * w.ntn)), dim3(kThreads), 0,
                     stream, w);
  trace_mark(p.tr, "bwd_wgrad_gate_up", stream);
  w.A = reinterpret_cast<const bf16_t*>(p.dy);
  w.B = reinterpret_cast<const bf16_t*>(p.h);
  w.out0 = p.dw_down;
  w.out1 = nullptr;
  w.lda = p.d;
  w.ldb = p.I;
  w.M = p.d;
  w.N = p.I;
  w.mtn = (w.M + BM - 1) / BM;
  w.ntn = (w.N + Default::BN - 1) / Default::BN;
  hipLaunchKernelGGL((wgrad_g2<Default, 1>), dim3((unsigned)(p.E_local * w.mtn * w.ntn)), dim3(kThreads), 0,
                     stream, w);
  trace_mark(p.tr, "bwd_wgrad_down", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

}  // namespace mok
