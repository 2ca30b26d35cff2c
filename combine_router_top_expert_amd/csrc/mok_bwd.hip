// Backward pass of the MoE layer.
//
// kucoin article, section 01: the backward pass runs two more rounds of
// communication in the reverse direction; section 02: pull reverse-combine
// and push reverse-dispatch.  Steps (float32 accumulation everywhere, every
// reduction in a fixed order, no floating-point atomics):
//   1. reverse-combine pull: for every routed row r <- item n = (s, t, j):
//        dy[r] = g_n * dout_s[t]                                  (bf16 rows)
//        d_gate[n] = dout_s[t] . y_n   (y_n = the row the forward pushed)
//   2. dgrad through W_down with the SwiGLU derivative in the epilogue:
//        dh = dy W_down[e];  s = sigmoid(a);
//        da = dh b s (1 + a (1 - s)),  db = dh a s   -> dab[r] = da | db
//   3. dgrad to the tokens:  dx = dab [W_gate[e]; W_up[e]], pushed to the
//      item's reverse-dispatch staging row dx_stage_s[t*k + j];
//   4. weight gradients per expert, contraction over the expert's rows in
//      ascending row order (one workgroup owns each output tile):
//        [dW_gate; dW_up][e] = dab^T X_e,   dW_down[e] = dy^T h_e
//      with X_e the expert's token rows gathered again through row_src;
//   5. per own token: dz_j = g_j (dg_j - sum_i g_i dg_i) over the chosen
//      experts (router through the renormalised softmax; selection is
//      piecewise constant), d_x = sum_j dx_stage_j + sum_j dz_j w_router[e_j],
//      over every slot but local rows dropped beyond R_cap (a remote slot's
//      dg and dx_stage row are written by the GPU holding that expert);
//   6. dW_router[e] = sum_t dz_{t,e} x_t: partial sums over fixed token
//      chunks, then a fixed-order sum of the chunks.
#include "mok_gemm.h"
#include "mok_internal.h"

namespace mok {

namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------------ 1. pull
// Token-major: a workgroup takes kPullTok consecutive tokens (s, t) of the
// item order; its lanes read the tokens' k row indices at once and list the
// tokens that have a row computed here.  For each listed token it reads the
// upstream gradient row once into registers (lane l keeps units l, l + 256,
// ... of the row) and serves every slot whose row is here: the dot product
// with the pushed y row gives d_gate, and g * dout is the slot's dy row.
// Per slot, the dot product is summed per lane in unit order, then over the
// wave's lanes by a butterfly and over the waves in order.  UMAX = units of
// the row a lane keeps (0: re-read per slot).
constexpr int kPullTok = 16;

template <typename T, int UMAX>
__global__ __launch_bounds__(kThreads) void rc_pull_kernel(BwdPlan p) {
  __shared__ float red[kThreads / 64][16];
  __shared__ uint32_t s_loc[kPullTok];
  __shared__ int s_list[kPullTok];
  __shared__ int s_nlist;
  constexpr int U = 16 / sizeof(T);
  const int units = p.d / U;
  const int64_t n_tok = (int64_t)p.S * p.T_src;
  const int64_t tok0 = (int64_t)blockIdx.x * kPullTok;
  if (threadIdx.x < kPullTok) s_loc[threadIdx.x] = 0;
  __syncthreads();
  // slots with a row here (a dropped row, >= R_cap, is skipped); through the
  // ring, rows of the current window [lo, hi) only, their dy at r - lo
  const int lo = p.win ? p.win[0] : 0;
  const int hi = p.win ? p.win[1] : p.R_cap;
  for (int i = threadIdx.x; i < kPullTok * p.k; i += kThreads) {
    const int64_t tok = tok0 + i / p.k;
    if (tok >= n_tok) break;
    const int r = p.dest_row[tok * p.k + i % p.k];
    if (r >= lo && r < hi) atomicOr(&s_loc[i / p.k], 1u << (i % p.k));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    for (int q = 0; q < kPullTok; ++q)
      if (s_loc[q]) s_list[n++] = q;
    s_nlist = n;
  }
  __syncthreads();
  const int nlist = s_nlist;
  for (int li = 0; li < nlist; ++li) {
    const int q = s_list[li];
    const uint32_t loc = s_loc[q];
    const int64_t tok = tok0 + q;
    const int64_t n0 = tok * p.k;
    const int s = (int)(tok / p.T_src), t = (int)(tok % p.T_src);
    const T* dout = reinterpret_cast<const T*>(p.d_out.p[s]) + (size_t)t * p.d;
    const T* ybase = reinterpret_cast<const T*>(p.staging.p[s]) + (size_t)t * p.k * p.d;
    uint4 dv[UMAX > 0 ? UMAX : 1];
    if constexpr (UMAX > 0) {
#pragma unroll
      for (int i = 0; i < UMAX; ++i) {
        const int u = threadIdx.x + i * kThreads;
        if (u < units) dv[i] = ld16(dout + u * U);
      }
    }
    for (int j = 0; j < p.k; ++j) {
      if (!((loc >> j) & 1u)) continue;
      const int r = p.dest_row[n0 + j];
      const float g = p.topk_gate[n0 + j];
      const T* y = ybase + (size_t)j * p.d;
      T* dy = reinterpret_cast<T*>(p.dy) + (size_t)(r - lo) * p.d;
      float part = 0.0f;
      auto unit = [&](int u, const uint4& dvu) {
        const uint4 yv = ld16(y + u * U);
        const T* de = reinterpret_cast<const T*>(&dvu);
        const T* ye = reinterpret_cast<const T*>(&yv);
        uint4 ov;
        T* oe = reinterpret_cast<T*>(&ov);
#pragma unroll
        for (int i = 0; i < U; ++i) {
          const float dvf = to_f32<T>(de[i]);
          part = __builtin_fmaf(dvf, to_f32<T>(ye[i]), part);
          oe[i] = from_f32<T>(g * dvf);
        }
        st16(dy + u * U, ov);
      };
      if constexpr (UMAX > 0) {
#pragma unroll
        for (int i = 0; i < UMAX; ++i) {
          const int u = threadIdx.x + i * kThreads;
          if (u < units) unit(u, dv[i]);
        }
      } else {
        for (int u = threadIdx.x; u < units; u += kThreads) unit(u, ld16(dout + u * U));
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6][j] = part;
    }
    __syncthreads();
    if (threadIdx.x < 16 && threadIdx.x < p.k && ((loc >> threadIdx.x) & 1u)) {
      float tot = 0.0f;
      for (int w = 0; w < kThreads / 64; ++w) tot += red[w][threadIdx.x];
      p.d_gate[n0 + threadIdx.x] = tot;
    }
    __syncthreads();  // red is read before the next token's slots write it
  }
}

// Through the ring: the rows of the current window [lo, hi), row-major (a
// workgroup per row: the window's rows are few, and a scan of every token
// per window would cost more than re-reading a token's upstream gradient
// for each of its rows).  Same sums in the same order as above.
template <typename T>
__global__ __launch_bounds__(kThreads) void rc_pull_rows_kernel(BwdPlan p) {
  __shared__ float red[kThreads / 64];
  constexpr int U = 16 / sizeof(T);
  const int lo = p.win[0], hi = p.win[1];
  for (int r = lo + blockIdx.x; r < hi; r += gridDim.x) {
    const int n = p.row_src[r];
    const int tok = n / p.k, j = n % p.k;
    const int s = tok / p.T_src, t = tok % p.T_src;
    const float g = p.topk_gate[n];
    const T* dout = reinterpret_cast<const T*>(p.d_out.p[s]) + (size_t)t * p.d;
    const T* y = reinterpret_cast<const T*>(p.staging.p[s]) + ((size_t)t * p.k + j) * p.d;
    T* dy = reinterpret_cast<T*>(p.dy) + (size_t)(r - lo) * p.d;
    float part = 0.0f;
    for (int u = threadIdx.x; u < p.d / U; u += kThreads) {
      const uint4 dv = ld16(dout + u * U), yv = ld16(y + u * U);
      const T* de = reinterpret_cast<const T*>(&dv);
      const T* ye = reinterpret_cast<const T*>(&yv);
      uint4 ov;
      T* oe = reinterpret_cast<T*>(&ov);
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const float dvf = to_f32<T>(de[i]);
        part = __builtin_fmaf(dvf, to_f32<T>(ye[i]), part);
        oe[i] = from_f32<T>(g * dvf);
      }
      st16(dy + u * U, ov);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
    __syncthreads();
    if (threadIdx.x == 0) {
      float tot = 0.0f;
      for (int w = 0; w < kThreads / 64; ++w) tot += red[w];
      p.d_gate[n] = tot;
    }
    __syncthreads();  // red is read before the next row writes it
  }
}

template <typename T>
mok_status launch_rc_pull(const BwdPlan& p, hipStream_t stream) {
  if (p.win) {
    if (p.R_cap == 0) return MOK_OK;
    const int cus = device_cus();
    int blocks = (cus > 0 ? cus : 256) * 8;
    if (blocks > p.win_rows) blocks = p.win_rows;
    hipLaunchKernelGGL(rc_pull_rows_kernel<T>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
    trace_mark(p.tr, "bwd_reverse_combine_pull", stream);
    return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
  }
  const int64_t n_tok = (int64_t)p.S * p.T_src;
  if (n_tok == 0 || p.R_cap == 0) return MOK_OK;
  const int64_t blocks = (n_tok + kPullTok - 1) / kPullTok;
  const int units = p.d / (16 / (int)sizeof(T));
  const int per_lane = (units + kThreads - 1) / kThreads;
  dim3 g((unsigned)blocks), b(kThreads);
  if (per_lane <= 1)
    hipLaunchKernelGGL((rc_pull_kernel<T, 1>), g, b, 0, stream, p);
  else if (per_lane <= 2)
    hipLaunchKernelGGL((rc_pull_kernel<T, 2>), g, b, 0, stream, p);
  else if (per_lane <= 4)
    hipLaunchKernelGGL((rc_pull_kernel<T, 4>), g, b, 0, stream, p);
  else if (per_lane <= 8)
    hipLaunchKernelGGL((rc_pull_kernel<T, 8>), g, b, 0, stream, p);
  else
    hipLaunchKernelGGL((rc_pull_kernel<T, 0>), g, b, 0, stream, p);
  trace_mark(p.tr, "bwd_reverse_combine_pull", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

// ------------------------------------------------------------------ 2. dh + SwiGLU'
template <typename T>
__global__ __launch_bounds__(kGemmThreads) void dh_kernel(BwdPlan p, int ntn) {
  __shared__ __attribute__((aligned(16))) T smem[TileSmem<T>::BYTES / sizeof(T)];
  __shared__ int s_prefix[257];
  const int mtile = blockIdx.x / ntn, nt = blockIdx.x % ntn;
  GroupTile g;
  if (!find_group_tile(p.offsets, p.E_local, p.R_cap, mtile, s_prefix, &g)) return;
  const T* dy = reinterpret_cast<const T*>(p.dy);
  const int n0 = nt * kBN;
  const T* wd = reinterpret_cast<const T*>(p.wd) + (size_t)g.e * p.d * p.I + n0;
  KLoader<T, kBM> la;
  la.init([&](int row) -> const T* {
    const int r = g.r0 + row;
    return r < g.r1 ? dy + (size_t)r * p.d : nullptr;
  });
  MNLoader<T, kBN> lb;
  lb.init(p.I - n0);
  auto kptr = [&](int kk) -> const T* { return wd + (size_t)kk * p.I; };
  Acc acc;
  gemm_mainloop<T>(p.d / MfmaT<T>::BK, la, lb,
                   [&](int kt, uint4(&r)[KLoader<T, kBM>::NU]) { la.load(kt, r); },
                   [&](int kt, uint4(&r)[MNLoader<T, kBN>::NU]) { lb.load(kt, kptr, r); }, smem,
                   acc);
  const T* ab = reinterpret_cast<const T*>(p.ab);
  T* dab = reinterpret_cast<T*>(p.dab);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = g.r0 + acc_row(mi, v);
      if (r >= g.r1) continue;
#pragma unroll
      for (int nj = 0; nj < 2; ++nj) {
        const int i = n0 + acc_col(nj);
        if (i >= p.I) continue;
        const float dh = acc.c[mi][nj][v];
        const float av = to_f32<T>(ab[(size_t)r * 2 * p.I + i]);
        const float bv = to_f32<T>(ab[(size_t)r * 2 * p.I + p.I + i]);
        const float sg = sigmoid_f(av);
        dab[(size_t)r * 2 * p.I + i] = from_f32<T>(dh * bv * sg * (1.0f + av * (1.0f - sg)));
        dab[(size_t)r * 2 * p.I + p.I + i] = from_f32<T>(dh * av * sg);
      }
    }
}

// ------------------------------------------------------------------ 3. dx + push
template <typename T>
__global__ __launch_bounds__(kGemmThreads) void dx_kernel(BwdPlan p, int ntn) {
  __shared__ __attribute__((aligned(16))) T smem[TileSmem<T>::BYTES / sizeof(T)];
  __shared__ int s_prefix[257];
  const int mtile = blockIdx.x / ntn, nt = blockIdx.x % ntn;
  GroupTile g;
  if (!find_group_tile(p.offsets, p.E_local, p.R_cap, mtile, s_prefix, &g)) return;
  const T* dab = reinterpret_cast<const T*>(p.dab);
  const int n0 = nt * kBN;
  const T* wg = reinterpret_cast<const T*>(p.wg) + (size_t)g.e * p.I * p.d + n0;
  const T* wu = reinterpret_cast<const T*>(p.wu) + (size_t)g.e * p.I * p.d + n0;
  KLoader<T, kBM> la;
  la.init([&](int row) -> const T* {
    const int r = g.r0 + row;
    return r < g.r1 ? dab + (size_t)r * 2 * p.I : nullptr;
  });
  MNLoader<T, kBN> lb;
  lb.init(p.d - n0);
  auto kptr = [&](int kk) -> const T* {
    return kk < p.I ? wg + (size_t)kk * p.d : wu + (size_t)(kk - p.I) * p.d;
  };
  Acc acc;
  gemm_mainloop<T>(2 * p.I / MfmaT<T>::BK, la, lb,
                   [&](int kt, uint4(&r)[KLoader<T, kBM>::NU]) { la.load(kt, r); },
                   [&](int kt, uint4(&r)[MNLoader<T, kBN>::NU]) { lb.load(kt, kptr, r); }, smem,
                   acc);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = g.r0 + acc_row(mi, v);
      if (r >= g.r1) continue;
      const int n = p.row_src[r];
      const int tok = n / p.k, j = n % p.k;
      const int s = tok / p.T_src, t = tok % p.T_src;
      T* dst = reinterpret_cast<T*>(p.dx_stage.p[s]) + ((size_t)t * p.k + j) * p.d;
#pragma unroll
      for (int nj = 0; nj < 2; ++nj) {
        const int c = n0 + acc_col(nj);
        if (c < p.d) dst[c] = from_f32<T>(acc.c[mi][nj][v]);
      }
    }
}

// ------------------------------------------------------------------ 4. wgrad
// mode 0: [dW_gate; dW_up][e] (M = 2I, N = d) = dab^T X_e
// mode 1: dW_down[e]          (M = d,  N = I) = dy^T h_e
template <typename T, int MODE>
__global__ __launch_bounds__(kGemmThreads) void wgrad_kernel(BwdPlan p, int mtn, int ntn) {
  __shared__ __attribute__((aligned(16))) T smem[TileSmem<T>::BYTES / sizeof(T)];
  const int per = mtn * ntn;
  const int e = blockIdx.x / per;
  const int mt = (blockIdx.x % per) / ntn, nt = blockIdx.x % ntn;
  int off = p.offsets[e], end = p.offsets[e + 1];
  if (off > p.R_cap) off = p.R_cap;
  if (end > p.R_cap) end = p.R_cap;
  const int cnt = end > off ? end - off : 0;
  const int M = MODE == 0 ? 2 * p.I : p.d;
  const int N = MODE == 0 ? p.d : p.I;
  const int m0 = mt * kBM, n0 = nt * kBN;
  MNLoader<T, kBM> la;
  MNLoader<T, kBN> lb;
  la.init(M - m0);
  lb.init(N - n0);
  const T* Abase = reinterpret_cast<const T*>(MODE == 0 ? p.dab : p.dy);
  const int lda = MODE == 0 ? 2 * p.I : p.d;
  auto aptr = [&](int kk) -> const T* {
    return kk < cnt ? Abase + (size_t)(off + kk) * lda + m0 : nullptr;
  };
  auto bptr = [&](int kk) -> const T* {
    if (kk >= cnt) return nullptr;
    if (MODE == 0) {
      const int n = p.row_src[off + kk];
      const int tok = n / p.k;
      const int s = tok / p.T_src, t = tok % p.T_src;
      return reinterpret_cast<const T*>(p.src_x.p[s]) + (size_t)t * p.d + n0;
    } else {
      return reinterpret_cast<const T*>(p.h) + (size_t)(off + kk) * p.I + n0;
    }
  };
  const int BK = MfmaT<T>::BK;
  Acc acc;
  gemm_mainloop<T>((cnt + BK - 1) / BK, la, lb,
                   [&](int kt, uint4(&r)[MNLoader<T, kBM>::NU]) { la.load(kt, aptr, r); },
                   [&](int kt, uint4(&r)[MNLoader<T, kBN>::NU]) { lb.load(kt, bptr, r); }, smem,
                   acc);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + acc_row(mi, v);
      if (m >= M) continue;
      float* dst;
      if (MODE == 0)
        dst = m < p.I ? p.dw_gate + ((size_t)e * p.I + m) * p.d
                      : p.dw_up + ((size_t)e * p.I + (m - p.I)) * p.d;
      else
        dst = p.dw_down + ((size_t)e * p.d + m) * p.I;
#pragma unroll
      for (int nj = 0; nj < 2; ++nj) {
        const int c = n0 + acc_col(nj);
        if (c < N) dst[c] = acc.c[mi][nj][v];
      }
    }
}

// ------------------------------------------------------------------ 5. d_x
// Two own tokens per workgroup.  Lanes 16q + j of wave 0 read slot j of
// token q in parallel and each group forms its token's dz in the order
// written out -- m = sum_j g_j dg_j by fma in slot order (the slot values
// gathered with lane shuffles), dz_j = g_j (dg_j - m) -- for the whole
// workgroup through LDS.
constexpr int kDxTokPerBlock = 2;

template <typename T>
__global__ __launch_bounds__(kThreads) void dx_final_kernel(BwdPlan p) {
  __shared__ float s_dz[kDxTokPerBlock][16];
  __shared__ int s_e[kDxTokPerBlock][16];
  __shared__ int s_loc[kDxTokPerBlock][16];
  const int64_t n_tok = (int64_t)p.own_n * p.T_src;
  // workgroups stride over the token pairs (the grid may be capped so that
  // the sum runs thin beside a GEMM on another stream)
  for (int64_t g0 = (int64_t)blockIdx.x * kDxTokPerBlock; g0 < n_tok;
       g0 += (int64_t)gridDim.x * kDxTokPerBlock) {
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x, q = lane >> 4, j = lane & 15;
      const int64_t gt = g0 + q;
      const bool valid = q < kDxTokPerBlock && gt < n_tok && j < p.k;
      float g = 0.0f, dg = 0.0f;
      int e = 0, loc = 0;
      if (valid) {
        const int s = p.own_lo + (int)(gt / p.T_src);
        const int t = (int)(gt % p.T_src);
        const int64_t n = ((int64_t)s * p.T_src + t) * p.k + j;
        // present: a local row, or a remote slot whose gate gradient and dx row
        // the GPU holding that expert wrote here; absent: dropped beyond R_cap
        loc = p.dest_row[n] < p.R_cap;
        dg = loc ? p.d_gate[n] : 0.0f;
        g = p.topk_gate[n];
        e = p.topk_idx[n];
      }
      float m = 0.0f;
      for (int i = 0; i < p.k; ++i)
        m = __builtin_fmaf(__shfl(g, (lane & ~15) + i, 64), __shfl(dg, (lane & ~15) + i, 64), m);
      if (valid) {
        const float dz = g * (dg - m);
        // an id outside [0, E) has no router row: latched, and its router
        // term left out (the router only writes valid ids)
        const bool ok_e = e >= 0 && e < p.E;
        if (!ok_e) latch(p.status, MOK_EROUTE);
        s_dz[q][j] = ok_e ? dz : 0.0f;
        s_e[q][j] = ok_e ? e : 0;
        s_loc[q][j] = loc;
        p.dz[gt * p.k + j] = ok_e ? dz : 0.0f;
      }
    }
    __syncthreads();
    constexpr int U = 16 / sizeof(T);
    const T* wr = reinterpret_cast<const T*>(p.w_router);
    for (int q = 0; q < kDxTokPerBlock; ++q) {
      const int64_t gt = g0 + q;
      if (gt >= n_tok) break;
      const int s = p.own_lo + (int)(gt / p.T_src);
      const int t = (int)(gt % p.T_src);
      const T* stg = reinterpret_cast<const T*>(p.dx_stage.p[s]) + (size_t)t * p.k * p.d;
      T* o = reinterpret_cast<T*>(p.d_x.p[s]) + (size_t)t * p.d;
      for (int u = threadIdx.x; u < p.d / U; u += kThreads) {
        float acc[U];
#pragma unroll
        for (int i = 0; i < U; ++i) acc[i] = 0.0f;
        for (int j = 0; j < p.k; ++j) {
          if (!s_loc[q][j]) continue;
          uint4 v = ld16(stg + (size_t)j * p.d + u * U);
          const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
          for (int i = 0; i < U; ++i) acc[i] += to_f32<T>(e[i]);
        }
        for (int j = 0; j < p.k; ++j) {
          const float dz = s_dz[q][j];
          uint4 v = ld16(wr + (size_t)s_e[q][j] * p.d + u * U);
          const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
          for (int i = 0; i < U; ++i) acc[i] = __builtin_fmaf(dz, to_f32<T>(e[i]), acc[i]);
        }
        uint4 ov;
        T* oe = reinterpret_cast<T*>(&ov);
#pragma unroll
        for (int i = 0; i < U; ++i) oe[i] = from_f32<T>(acc[i]);
        st16(o + u * U, ov);
      }
    }
    __syncthreads();  // the slot values of this pair are read before the next pair's
  }
}

// ------------------------------------------------------------------ 6. dW_router
// The own tokens' items are grouped by expert (the same stable counting-sort
// layout as the forward pass, over all E experts); the rows of every expert
// are cut into chunks of kRChunk rows.  One workgroup sums one chunk in row
// order (partial[chunk][d]); a second kernel sums each expert's chunks in
// chunk order.
constexpr int kRChunk = 64;

__global__ void iota_kernel(int32_t* v, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) v[i] = i;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void dwr_part_kernel(BwdPlan p, int N_own) {
  __shared__ int s_prefix[257];
  __shared__ int s_tok[kRChunk];
  __shared__ float s_dz[kRChunk];
  // chunk -> (expert, rows): same prefix search as the grouped GEMM tiles
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int loc[4], run = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      int c = 0;
      if (e < p.E) {
        const int lo = p.r_offsets[e], hi = p.r_offsets[e + 1];
        c = (hi - lo + kRChunk - 1) / kRChunk;
      }
      loc[q] = c;
      run += c;
    }
    int incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    int excl = incl - run;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s_prefix[lane * 4 + q] = excl;
      excl += loc[q];
    }
    if (lane == 63) s_prefix[256] = incl;
  }
  __syncthreads();
  const int total = s_prefix[p.E];
  // workgroups stride over the chunks (the grid may be capped so that the
  // partial sums run thin beside a GEMM on another stream)
  for (int chunk = blockIdx.x; chunk < total; chunk += gridDim.x) {
    int lo = 0, hi = p.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_prefix[mid] <= chunk) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int r0 = p.r_offsets[e] + (chunk - s_prefix[e]) * kRChunk;
    const int r1 = min(r0 + kRChunk, p.r_offsets[e + 1]);
    const int nr = r1 - r0;
    if (threadIdx.x < nr) {
      const int n = p.r_row_src[r0 + threadIdx.x];  // item index among the own items
      s_tok[threadIdx.x] = n / p.k;
      s_dz[threadIdx.x] = p.dz[n];
    }
    __syncthreads();
    constexpr int U = 16 / sizeof(T);
    float* out = p.dwr_part + (size_t)chunk * p.d;
    for (int u = threadIdx.x; u < p.d / U; u += kThreads) {
      float acc[U];
#pragma unroll
      for (int i = 0; i < U; ++i) acc[i] = 0.0f;
      for (int r = 0; r < nr; ++r) {
        const int gt = s_tok[r];
        const int s = p.own_lo + gt / p.T_src, t = gt % p.T_src;
        uint4 v = ld16(reinterpret_cast<const T*>(p.src_x.p[s]) + (size_t)t * p.d + u * U);
        const T* xe = reinterpret_cast<const T*>(&v);
        const float z = s_dz[r];
#pragma unroll
        for (int i = 0; i < U; ++i) acc[i] = __builtin_fmaf(z, to_f32<T>(xe[i]), acc[i]);
      }
#pragma unroll
      for (int i = 0; i < U; ++i) out[u * U + i] = acc[i];
    }
    __syncthreads();  // s_tok / s_dz are read before the next chunk's rows
  }
}

// dW_router[e][c] = sum over e's chunks in order; grid (column blocks, E)
__global__ __launch_bounds__(kThreads) void dwr_reduce_kernel(BwdPlan p) {
  const int e = blockIdx.y;
  const int c = blockIdx.x * kThreads + threadIdx.x;
  if (c >= p.d) return;
  int c0 = 0;
  for (int q = 0; q < e; ++q)
    c0 += (p.r_offsets[q + 1] - p.r_offsets[q] + kRChunk - 1) / kRChunk;
  const int nc = (p.r_offsets[e + 1] - p.r_offsets[e] + kRChunk - 1) / kRChunk;
  float acc = 0.0f;
  for (int q = 0; q < nc; ++q) acc += p.dwr_part[(size_t)(c0 + q) * p.d + c];
  p.dw_router[(size_t)e * p.d + c] = acc;
}

// bf16 backward over two streams.  The call's stream runs the chain that
// feeds the next GEMM (reverse-combine pull, dh, SwiGLU backward, dx with the
// reverse-dispatch push, the weight gradients); the second stream runs what
// only a later step reads, beside it: the transposed re-gather of the token
// rows (read by the gate/up weight gradient) and the router-gradient layout
// (read by the router weight gradient) once the reverse-combine pull is
// done, then -- once dx has been pushed -- the per-token dx sum and the
// router weight gradient.
// Every buffer is written on one stream and read after an event the reader
// waits for; no kernel changes, so results are bit-identical to one stream.
template <typename T>
mok_status run_bwd_two_streams(const BwdPlan& p, hipStream_t stream) {
  hipStream_t aux = p.aux;
  hipEvent_t fork = p.aux_ev[0], gx_ready = p.aux_ev[1], dx_pushed = p.aux_ev[2];
  // the pull is HBM-bound like the side work: fork after it, so the side
  // work meets the dh GEMM instead
  {
    mok_status rc = launch_rc_pull<T>(p, stream);
    if (rc != MOK_OK) return rc;
  }
  MOK_HIP_CHECK(hipEventRecord(fork, stream));
  MOK_HIP_CHECK(hipStreamWaitEvent(aux, fork, 0));
  trace_mark(p.tr, "start", aux);
  const int64_t n_own = (int64_t)p.own_n * p.T_src;
  const int N_own = (int)(n_own * p.k);
  const int cus = device_cus();
  if (p.R_cap > 0) {
    // one workgroup per CU: the copy runs thin beside dh (mid-size layer: dh
    // 870 -> 800 us, step 7.31 -> 7.27 ms; half that made it outlast dx)
    mok_status rc = launch_gather_t(p, p.x_perm, aux, cus);
    if (rc != MOK_OK) return rc;
    if (p.hT) rc = launch_gather_t(p, p.hT, aux, cus, p.h, p.I);
    if (rc != MOK_OK) return rc;
    trace_mark(p.tr, p.hT ? "bwd_transpose_x_h" : "bwd_regather_x", aux);
  }
  MOK_HIP_CHECK(hipEventRecord(gx_ready, aux));
  if (p.dw_router) {
    hipLaunchKernelGGL(iota_kernel, dim3((p.E + 255) / 256), dim3(256), 0, aux, p.r_ident, p.E);
    mok_status rc = launch_layout(N_own, p.E, p.E, N_own, p.topk_idx + (int64_t)p.own_lo * p.T_src * p.k,
                                  p.r_ident, p.r_counts, p.r_offsets, p.r_row_src, p.r_dest_row,
                                  p.r_scratch, nullptr, aux, nullptr);
    if (rc != MOK_OK) return rc;
    trace_mark(p.tr, "bwd_router_layout", aux);
  }
  mok_status rc = launch_bwd_gemms_bf16(p, p.x_perm, stream, gx_ready, dx_pushed);
  if (rc != MOK_OK) return rc;
  MOK_HIP_CHECK(hipStreamWaitEvent(aux, dx_pushed, 0));
  trace_mark(p.tr, "start", aux);  // the wait is not the dx sum's time
  if (n_own > 0) {
    // one workgroup per CU, striding over the tokens: the sum runs thin
    // beside the gate/up weight gradient instead of in a burst (mid-size
    // layer: that GEMM 1.54 -> 1.51 ms, step 7.17 -> 7.15 ms; 64 workgroups
    // made the sum outlast the GEMM)
    int64_t blocks = (n_own + kDxTokPerBlock - 1) / kDxTokPerBlock;
    if (cus > 0 && blocks > cus) blocks = cus;
    hipLaunchKernelGGL(dx_final_kernel<T>, dim3((unsigned)blocks), dim3(kThreads), 0, aux, p);
    trace_mark(p.tr, "bwd_dx_sum_router", aux);
  }
  if (p.dw_router) {
    const int nchunk = N_own / kRChunk + p.E;
    // one workgroup per CU, as the dx sum (mid-size layer: the gate/up
    // weight gradient beside it 1.56 -> 1.51 ms, step 7.24 -> 7.21 ms)
    const int gx = cus > 0 && nchunk > cus ? cus : nchunk;
    hipLaunchKernelGGL(dwr_part_kernel<T>, dim3(gx), dim3(kThreads), 0, aux, p, N_own);
    trace_mark(p.tr, "bwd_dw_router_part", aux);
    dim3 g((p.d + kThreads - 1) / kThreads, p.E);
    hipLaunchKernelGGL(dwr_reduce_kernel, g, dim3(kThreads), 0, aux, p);
    trace_mark(p.tr, "bwd_dw_router_reduce", aux);
  }
  MOK_HIP_CHECK(hipEventRecord(fork, aux));  // re-recorded as the join
  MOK_HIP_CHECK(hipStreamWaitEvent(stream, fork, 0));
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

// The per-token part of the backward on one stream, once every dx row is
// pushed: the dx sum with the router path, then the router weight gradient.
template <typename T>
mok_status run_bwd_tail(const BwdPlan& p, hipStream_t stream) {
  const int64_t n_own = (int64_t)p.own_n * p.T_src;
  if (n_own > 0) {
    hipLaunchKernelGGL(dx_final_kernel<T>, dim3((unsigned)((n_own + kDxTokPerBlock - 1) / kDxTokPerBlock)),
                       dim3(kThreads), 0, stream, p);
    trace_mark(p.tr, "bwd_dx_sum_router", stream);
  }
  if (p.dw_router) {
    const int N_own = (int)(n_own * p.k);
    hipLaunchKernelGGL(iota_kernel, dim3((p.E + 255) / 256), dim3(256), 0, stream, p.r_ident, p.E);
    mok_status rc = launch_layout(N_own, p.E, p.E, N_own, p.topk_idx + (int64_t)p.own_lo * p.T_src * p.k,
                                  p.r_ident, p.r_counts, p.r_offsets, p.r_row_src, p.r_dest_row,
                                  p.r_scratch, nullptr, stream, nullptr);
    if (rc != MOK_OK) return rc;
    trace_mark(p.tr, "bwd_router_layout", stream);
    const int nchunk = N_own / kRChunk + p.E;
    hipLaunchKernelGGL(dwr_part_kernel<T>, dim3(nchunk), dim3(kThreads), 0, stream, p, N_own);
    trace_mark(p.tr, "bwd_dw_router_part", stream);
    dim3 g((p.d + kThreads - 1) / kThreads, p.E);
    hipLaunchKernelGGL(dwr_reduce_kernel, g, dim3(kThreads), 0, stream, p);
    trace_mark(p.tr, "bwd_dw_router_reduce", stream);
  }
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

// bf16 backward through the ring: window by window (dy, da | db and the
// transposed token rows of a window in the ring's slots, reused by the next
// window), the weight gradients carried over from window to window; then the
// split-K reduction and the per-token and router parts, as in one launch.
template <typename T>
mok_status run_bwd_ring(const BwdPlan& p, hipStream_t stream) {
  mok_status rc = MOK_OK;
  if (p.R_cap > 0) {
    for (int w = 0; w < p.n_win; ++w) {
      rc = launch_bwd_window(p, w, stream);
      if (rc != MOK_OK) return rc;
      rc = launch_rc_pull<T>(p, stream);
      if (rc != MOK_OK) return rc;
      rc = launch_gather_t(p, p.x_perm, stream);
      if (rc != MOK_OK) return rc;
      trace_mark(p.tr, "bwd_regather_x", stream);
      rc = launch_bwd_dgrad(p, stream);
      if (rc != MOK_OK) return rc;
      // (the first window also orders the experts for the spread schedule,
      // from the routed counts of all windows)
      rc = launch_bwd_wgrad(p, p.x_perm, stream, w == 0, false);
      if (rc != MOK_OK) return rc;
    }
    rc = launch_bwd_reduce(p, stream);
    if (rc != MOK_OK) return rc;
  }
  return run_bwd_tail<T>(p, stream);
}

template <typename T>
mok_status run_bwd(const BwdPlan& p, hipStream_t stream) {
  if constexpr (sizeof(T) == 2) {
    if (p.win) return run_bwd_ring<T>(p, stream);
    if (p.aux) return run_bwd_two_streams<T>(p, stream);
    if (p.R_cap > 0) {
      mok_status rc = launch_rc_pull<T>(p, stream);
      if (rc != MOK_OK) return rc;
      rc = launch_gather_t(p, p.x_perm, stream);
      if (rc != MOK_OK) return rc;
      if (p.hT) rc = launch_gather_t(p, p.hT, stream, 0, p.h, p.I);
      if (rc != MOK_OK) return rc;
      trace_mark(p.tr, p.hT ? "bwd_transpose_x_h" : "bwd_regather_x", stream);
    }
    mok_status rc = launch_bwd_gemms_bf16(p, p.x_perm, stream);
    if (rc != MOK_OK) return rc;
  } else {
  if (p.R_cap > 0) {
    const int mt = grouped_mtiles_bound(p.R_cap, p.E_local);
    mok_status rc = launch_rc_pull<T>(p, stream);
    if (rc != MOK_OK) return rc;
    int ntn = (p.I + kBN - 1) / kBN;
    hipLaunchKernelGGL(dh_kernel<T>, dim3(mt * ntn), dim3(kGemmThreads), 0, stream, p, ntn);
    trace_mark(p.tr, "bwd_dh_swiglu", stream);
    ntn = (p.d + kBN - 1) / kBN;
    hipLaunchKernelGGL(dx_kernel<T>, dim3(mt * ntn), dim3(kGemmThreads), 0, stream, p, ntn);
    trace_mark(p.tr, "bwd_dx_push", stream);
  }
  {
    int mtn = (2 * p.I + kBM - 1) / kBM, ntn = (p.d + kBN - 1) / kBN;
    hipLaunchKernelGGL((wgrad_kernel<T, 0>), dim3(p.E_local * mtn * ntn), dim3(kGemmThreads), 0,
                       stream, p, mtn, ntn);
    trace_mark(p.tr, "bwd_wgrad_gate_up", stream);
    mtn = (p.d + kBM - 1) / kBM;
    ntn = (p.I + kBN - 1) / kBN;
    hipLaunchKernelGGL((wgrad_kernel<T, 1>), dim3(p.E_local * mtn * ntn), dim3(kGemmThreads), 0,
                       stream, p, mtn, ntn);
    trace_mark(p.tr, "bwd_wgrad_down", stream);
  }
  }
  return run_bwd_tail<T>(p, stream);
}

// MXFP8 backward: the bf16 reverse-combine pull, the four expert GEMMs on
// the scaled matrix cores, then the per-token part as for bf16.
mok_status run_bwd_mx(const BwdPlan& p, hipStream_t stream) {
  if (p.R_cap > 0) {
    const mok_status rc = launch_rc_pull<bf16_t>(p, stream);
    if (rc != MOK_OK) return rc;
  }
  const mok_status rc = launch_bwd_mx_gemms(p, stream);
  if (rc != MOK_OK) return rc;
  return run_bwd_tail<bf16_t>(p, stream);
}

}  // namespace

mok_status launch_bwd(const BwdPlan& p, hipStream_t stream) {
  if (p.prec == MOK_MXFP8) return run_bwd_mx(p, stream);
  return p.prec == MOK_F32 ? run_bwd<float>(p, stream) : run_bwd<bf16_t>(p, stream);
}

}  // namespace mok
