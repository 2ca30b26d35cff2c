// Backward expert GEMMs, bf16, on the pipelined 256 x 256 tile engine.
//   dh  : dh = dy W_down[e]           A = dy (k = d contiguous), B = W_down
//         read as [d][I] (n contiguous), or W_down^T [I][d] (k contiguous)
//         when the caller prepared it -> bf16 dh, then the SwiGLU
//         derivative pass turns it into dab
//   dx  : dx = dab [W_gate; W_up]      A = dab (k = 2I contiguous), B = the
//         two weight matrices read as [2I][d], or [W_gate; W_up]^T [d][2I]
//         when prepared -> epilogue pushes dx rows to their reverse-dispatch
//         staging rows
// The transposed weights give the MFMAs the same fragments (lane l: column
// n0 + l % 32, k = 16 s + 8 (l / 32) + 0..7 either way), so dh and dx are
// bit-identical with and without them; they spare the transposing LDS reads.
//   wgrad (per expert, contraction over the expert's rows in ascending row
//         order, split into chunks of 4096 rows whose partial sums are
//         added in chunk order; rows past a chunk read zeros):
//         [dW_gate; dW_up][e] = dab^T X_e   (A = dab, B = gathered rows X)
//         dW_down[e]          = dy^T h_e    (A = dy,  B = h)
// The m/n-contiguous operands are read with the transposing LDS fragment
// loads of the engine; no operand is transposed in memory.
//
// Ring windows.  Through the ring, the backward runs in windows of whole
// minibatches (consecutive rows [lo, hi) of the expert order, cut at
// minibatch boundaries): dy, dab and the transposed token rows of the
// window's rows live in the ring at rows r - lo.  `win` (device memory)
// holds lo, hi, the window's index and the expert pieces clipped to the
// window, woff[e] = clamp(offsets[e], lo, hi); the GEMMs tile the pieces.
// A weight-gradient tile sums its chunk's rows inside the window and, when
// the chunk began in an earlier window, continues from the partial sum that
// window stored (fp32, reloaded exactly into the accumulators): the MFMAs
// then run on the same operands in the same order as in one launch, because
// window cuts fall on minibatch boundaries (multiples of 64 rows from the
// expert's first row), so the results are bit-identical to the one-launch
// backward.  win == null: one launch over all rows.
#include <string.h>

#include "mok_gemm2.h"
#include "mok_internal.h"

namespace mok {

namespace {

using namespace g2;

struct DhArgs {
  const bf16_t* dy;    // [R_cap, d] (ring window: [rows, d] at r - lo)
  const bf16_t* wd;    // [E_local, d, I]
  const bf16_t* wt;    // [E_local, I, d] = W_down^T, or null
  const bf16_t* ab;    // [R_cap, 2I]
  bf16_t* dab;         // [R_cap, 2I] (ring window: at r - lo)
  const int32_t* offsets;  // expert rows (ring window: the pieces woff)
  const int32_t* win;      // ring window descriptor or null
  int d, I, E_local, R_cap, ntn;
};

__device__ __forceinline__ int win_lo(const int32_t* win) { return win ? win[0] : 0; }

template <class C, bool BT>
__global__ __launch_bounds__(kThreads, C::OCC) void dh_g2(DhArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int s_prefix[257];
  const int total_m = group_prefix(a.offsets, a.E_local, a.R_cap, s_prefix);
  const int total = total_m * a.ntn;
  if ((int)blockIdx.x >= total) return;
  int mtile, nt;
  grouped_order(xcd_tile(blockIdx.x, total), total_m, a.ntn, &mtile, &nt);
  const GTile g = group_tile(a.offsets, a.E_local, a.R_cap, s_prefix, mtile);
  const int lo = win_lo(a.win);
  const int n0 = nt * C::BN;
  const bf16_t* wd = a.wd + (size_t)g.e * a.d * a.I + n0;
  KMajor<BM, C::BK> la;
  la.init([&](int row) -> const bf16_t* {
    const int r = g.r0 + row;
    return r < g.r1 ? a.dy + (size_t)(r - lo) * a.d : nullptr;
  });
  Acc<C> acc;
  if constexpr (BT) {
    const bf16_t* wt = a.wt + (size_t)g.e * a.I * a.d;
    KMajor<C::BN, C::BK> lb;
    lb.init([&](int nr) -> const bf16_t* {
      const int n = n0 + nr;
      return n < a.I ? wt + (size_t)n * a.d : nullptr;
    });
    mainloop<C, false, false>(a.d / C::BK, [&](int kt, unsigned l, auto pt) { la.issue(kt, l, pt); },
                              [&](int kt, unsigned l, auto pt) { lb.issue(kt, l, pt); }, smem, acc);
  } else {
    MNMajor<C::BN, C::BK> lb;
    lb.ncols_left = a.I - n0;
    mainloop<C, false, true>(a.d / C::BK, [&](int kt, unsigned l, auto pt) { la.issue(kt, l, pt); },
                             [&](int kt, unsigned l, auto pt) {
                               lb.issue(kt, l, [&](int kk) -> const bf16_t* { return wd + (size_t)kk * a.I; }, pt);
                             },
                             smem, acc);
  }
  // dh (bf16) goes to the first half of its dab row; swiglu_bwd_kernel then
  // turns it into da | db in place with the saved a | b, as a separate pass
  // that runs at full memory bandwidth (as an epilogue, every workgroup would
  // stall on its a | b loads at the same time while the matrix cores idle).
  __syncthreads();
  const WaveStage<C, bf16_t> st(smem);
  static_assert(WaveStage<C, bf16_t>::PASSES == 1, "one staging pass");
  st.put(acc, 0);
  wave_lds_fence();
  const int wave = threadIdx.x >> 6;
  st.for_chunks(0, [&](int trow, int srow, int c) {
    const int r = g.r0 + (wave >> 1) * 128 + trow;
    const int col = n0 + (wave & 1) * (C::BN / 2) + c * 8;
    if (r >= g.r1 || col >= a.I) return;
    *reinterpret_cast<uint4*>(a.dab + (size_t)(r - lo) * 2 * a.I + col) = st.raw(srow, c);
  });
}

// SwiGLU backward of every routed row, in place: dab[r] = da | db from
// dh = dab[r][0, I) and the saved a | b:  s = sigmoid(a),
// da = dh * b * s * (1 + a (1 - s)),  db = dh * a * s.  One 8-column piece
// per thread; rows beyond R are skipped.
__global__ __launch_bounds__(kThreads) void swiglu_bwd_kernel(const bf16_t* ab, bf16_t* dab,
                                                              const int32_t* offsets, int E_local,
                                                              int R_cap, int I,
                                                              const int32_t* win) {
  // rows [lo, hi): all routed rows, or a ring window's (dab at r - lo)
  const int lo = win_lo(win);
  const int hi = win ? win[1] : min(offsets[E_local], R_cap);
  const int per_row = I / 8;
  const size_t u = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const int r = lo + (int)(u / per_row), c = (int)(u % per_row) * 8;
  if (r >= hi) return;
  const bf16_t* abr = ab + (size_t)r * 2 * I;
  bf16_t* dabr = dab + (size_t)(r - lo) * 2 * I;
  const uint4 hv = *reinterpret_cast<const uint4*>(dabr + c);
  const uint4 av = *reinterpret_cast<const uint4*>(abr + c);
  const uint4 bv = *reinterpret_cast<const uint4*>(abr + I + c);
  const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w}, aw[4] = {av.x, av.y, av.z, av.w},
                 bw[4] = {bv.x, bv.y, bv.z, bv.w};
  float da[8], db[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int w = e >> 1;
    const float dh = __uint_as_float(e & 1 ? hw[w] & 0xFFFF0000u : hw[w] << 16);
    const float x = __uint_as_float(e & 1 ? aw[w] & 0xFFFF0000u : aw[w] << 16);
    const float y = __uint_as_float(e & 1 ? bw[w] & 0xFFFF0000u : bw[w] << 16);
    const float sg = sigmoid_f(x);
    da[e] = dh * y * sg * (1.0f + x * (1.0f - sg));
    db[e] = dh * x * sg;
  }
  const uint2 d0 = pack4_bf16(da[0], da[1], da[2], da[3]), d1 = pack4_bf16(da[4], da[5], da[6], da[7]);
  const uint2 e0 = pack4_bf16(db[0], db[1], db[2], db[3]), e1 = pack4_bf16(db[4], db[5], db[6], db[7]);
  *reinterpret_cast<uint4*>(dabr + c) = make_uint4(d0.x, d0.y, d1.x, d1.y);
  *reinterpret_cast<uint4*>(dabr + I + c) = make_uint4(e0.x, e0.y, e1.x, e1.y);
}

struct DxArgs {
  const bf16_t* dab;   // [R_cap, 2I] (ring window: at r - lo)
  const int32_t* win;  // ring window descriptor or null (offsets: the pieces woff)
  const bf16_t* wg;    // [E_local, I, d]
  const bf16_t* wu;
  const bf16_t* wt;    // [E_local, d, 2I] = [W_gate; W_up]^T, or null
  const int32_t* offsets;
  const int32_t* row_src;
  DstTable dx_stage;
  int d, I, E_local, R_cap, ntn, T_src, k;
};

template <class C, bool BT>
__global__ __launch_bounds__(kThreads, C::OCC) void dx_g2(DxArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int s_prefix[257];
  const int total_m = group_prefix(a.offsets, a.E_local, a.R_cap, s_prefix);
  const int total = total_m * a.ntn;
  if ((int)blockIdx.x >= total) return;
  int mtile, nt;
  grouped_order(xcd_tile(blockIdx.x, total), total_m, a.ntn, &mtile, &nt);
  const GTile g = group_tile(a.offsets, a.E_local, a.R_cap, s_prefix, mtile);
  const int lo = win_lo(a.win);
  const int n0 = nt * C::BN;
  const bf16_t* wg = a.wg + (size_t)g.e * a.I * a.d + n0;
  const bf16_t* wu = a.wu + (size_t)g.e * a.I * a.d + n0;
  KMajor<BM, C::BK> la;
  la.init([&](int row) -> const bf16_t* {
    const int r = g.r0 + row;
    return r < g.r1 ? a.dab + (size_t)(r - lo) * 2 * a.I : nullptr;
  });
  Acc<C> acc;
  if constexpr (BT) {
    const bf16_t* wt = a.wt + (size_t)g.e * a.d * 2 * a.I;
    KMajor<C::BN, C::BK> lb;
    lb.init([&](int nr) -> const bf16_t* {
      const int n = n0 + nr;
      return n < a.d ? wt + (size_t)n * 2 * a.I : nullptr;
    });
    mainloop<C, false, false>(2 * a.I / C::BK, [&](int kt, unsigned l, auto pt) { la.issue(kt, l, pt); },
                              [&](int kt, unsigned l, auto pt) { lb.issue(kt, l, pt); }, smem, acc);
  } else {
    MNMajor<C::BN, C::BK> lb;
    lb.ncols_left = a.d - n0;
    mainloop<C, false, true>(2 * a.I / C::BK, [&](int kt, unsigned l, auto pt) { la.issue(kt, l, pt); },
                             [&](int kt, unsigned l, auto pt) {
                               lb.issue(kt, l, [&](int kk) -> const bf16_t* {
                                 return kk < a.I ? wg + (size_t)kk * a.d : wu + (size_t)(kk - a.I) * a.d;
                               }, pt);
                             },
                             smem, acc);
  }
  __shared__ bf16_t* s_dst[BM];
  stage_dst_rows(s_dst, a.row_src, g, a.dx_stage, a.k, a.T_src, a.d);
  __syncthreads();
  const WaveStage<C, bf16_t> st(smem);
  static_assert(WaveStage<C, bf16_t>::PASSES == 1, "one staging pass");
  st.put(acc, 0);
  wave_lds_fence();
  const int wave = threadIdx.x >> 6;
  st.for_chunks(0, [&](int trow, int srow, int c) {
    const int r = g.r0 + (wave >> 1) * 128 + trow;
    const int col = n0 + (wave & 1) * (C::BN / 2) + c * 8;
    if (r >= g.r1 || col >= a.d) return;
    *reinterpret_cast<uint4*>(s_dst[r - g.r0] + col) = st.raw(srow, c);
  });
}

// MODE 0: M = 2I (dab columns), N = d (gathered token rows); MODE 1: M = d (dy), N = I (h)
struct WgArgs {
  const bf16_t* A;     // [R_cap, lda] rows of the expert
  const bf16_t* B;     // [R_cap, ldb]
  float* out0;         // MODE 0: dW_gate [E_local, I, d]; MODE 1: dW_down [E_local, d, I]
  float* out1;         // MODE 0: dW_up
  float* part;         // [extra chunks, M, N] partial sums of chunks 1, 2, ... of an expert
  const bf16_t* BT;    // MODE 0: the expert rows' tokens transposed, [N, ldt] (gather_t_kernel)
  int64_t ldt;
  const int32_t* offsets;
  int lda, ldb, M, N, I, E_local, R_cap, mtn, ntn;
  const int32_t* order;  // [E_local] local experts by routed rows, descending (spread mode)
  const int32_t* win;    // ring window descriptor or null; A (ring) rows at r - lo
};

// Split-K of the weight gradients.  An expert's rows are cut into chunks of
// kWgChunk rows (contraction length of one tile), so that a heavily routed
// expert spreads over as many tiles as its rows need instead of one long
// tile per output block.  Chunk 0 writes dW; chunk c >= 1 writes a partial
// block, and wgrad_reduce adds the partials to dW in chunk order (a fixed
// order: the result is run-to-run identical).
constexpr int kWgChunk = 4096;
// Tiles per expert from which the weight gradients may run in spread mode.
constexpr int kSpreadTiles = 32;

// Wave 0 scans the per-expert chunk counts: s_cp[e] = chunks of the experts
// before e, s_xp[e] = their chunks beyond the first (partial slots), s_tp[e]
// = their 64-row tiles (the expert's first column in the transposed token
// rows is 64 s_tp[e]); index 256 holds the totals.
__device__ __forceinline__ void wg_chunk_prefix(const int32_t* offsets, int E_local, int R_cap,
                                                int* s_cp, int* s_xp, int* s_tp, int* s_rows) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int ch[4], tl[4], run_c = 0, run_x = 0, run_t = 0, rmax = 0, rtot = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      int c = 0, t = 0;
      if (e < E_local) {
        const int lo = min(offsets[e], R_cap), hi = min(offsets[e + 1], R_cap);
        // an expert without rows keeps one empty chunk: its tiles write zeros
        c = hi > lo ? (hi - lo + kWgChunk - 1) / kWgChunk : 1;
        t = hi > lo ? (hi - lo + 63) / 64 : 0;
        rmax = max(rmax, hi - lo);
        rtot += hi - lo;
      }
      ch[q] = c;
      tl[q] = t;
      run_c += c;
      run_x += c > 1 ? c - 1 : 0;
      run_t += t;
    }
    int inc_c = run_c, inc_x = run_x, inc_t = run_t;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int oc = __shfl_up(inc_c, off, 64), ox = __shfl_up(inc_x, off, 64),
                ot = __shfl_up(inc_t, off, 64);
      if (lane >= off) {
        inc_c += oc;
        inc_x += ox;
        inc_t += ot;
      }
    }
    int ec = inc_c - run_c, ex = inc_x - run_x, et = inc_t - run_t;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s_cp[lane * 4 + q] = ec;
      s_xp[lane * 4 + q] = ex;
      s_tp[lane * 4 + q] = et;
      ec += ch[q];
      ex += ch[q] > 1 ? ch[q] - 1 : 0;
      et += tl[q];
    }
    if (lane == 63) {
      s_cp[256] = inc_c;
      s_xp[256] = inc_x;
      s_tp[256] = inc_t;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      rmax = max(rmax, __shfl_xor(rmax, off, 64));
      rtot += __shfl_xor(rtot, off, 64);
    }
    if (lane == 0) {
      s_rows[0] = rmax;
      s_rows[1] = rtot;
    }
  }
  __syncthreads();
}

// Spread mode (whole experts, no split-K, tiles of every expert over all
// XCDs, most routed expert first) when an expert's output tiles fill an
// eighth of the chip and no expert's single tile -- the whole expert's rows
// -- is longer than a CU's average share of the work (rows_max <= per * R /
// 256, so the longest-first order keeps the CUs balanced); otherwise the
// experts are cut into kWgChunk-row chunks whose partial sums are added in
// chunk order.  Decided on the device, identically by every workgroup of
// both kernels, from the routed counts.
__device__ __forceinline__ bool wg_spread(int per, const int* s_rows) {
  return per >= kSpreadTiles && (int64_t)s_rows[0] * 256 <= (int64_t)per * s_rows[1];
}

// Token rows of the local experts gathered again for the gate/up weight
// gradients, transposed: xT[c][col] = x_token(r)[c] for routed row r of
// expert e at column col = 64 P(e) + (r - offsets[e]), P(e) = 64-row tiles of
// the experts before e; the columns up to the next multiple of 64 hold zeros.
// The weight-gradient GEMM then reads this operand k-contiguous, in whole
// 64-k stages, instead of through transposing LDS reads.  A workgroup covers
// 4 consecutive 64-row tiles (256 columns of xT) x 64 columns of d: thread
// (rg, cb) loads 16 bytes (8 columns of d) of each of its 8 rows, transposes
// the 8 x 8 block in registers and stores 16 bytes (8 rows) into each of its
// 8 columns of d.  A wave instruction reads 8 rows x 128 bytes; a workgroup
// writes 512 contiguous bytes of each of its 64 rows of xT.  Workgroups
// stride over the tile groups so the per-expert tile prefix is computed once
// per workgroup.
struct GatherTArgs {
  SrcTable src;
  const bf16_t* rows;  // a row-major [R_cap, d] matrix to transpose instead of the token rows
  const int32_t* row_src;
  const int32_t* offsets;
  bf16_t* xT;      // [d, ldt]
  int64_t ldt;
  int d, E_local, R_cap, T_src, k;
};

__global__ __launch_bounds__(kThreads) void gather_t_kernel(GatherTArgs a) {
  __shared__ int s_prefix[257];
  __shared__ const bf16_t* s_src[4][64];  // each wave's 64 tile rows (null past the expert)
  const int total = group_prefix(a.offsets, a.E_local, a.R_cap, s_prefix, 64);
  const int cb = threadIdx.x & 7, rg = (threadIdx.x >> 3) & 7, sub = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int c0 = blockIdx.y * 64 + 8 * cb;
  for (int grp = blockIdx.x; 4 * grp < total; grp += gridDim.x) {
    const int mt = 4 * grp + sub;  // this wave's 64-row tile
    if (mt >= total) continue;
    const GTile g = group_tile(a.offsets, a.E_local, a.R_cap, s_prefix, mt, 64);
    {
      // lane l looks up row l of the tile once (the 8 lanes that read a row
      // share it), so no lane divides per load
      const int r = g.r0 + lane;
      const bf16_t* p = nullptr;
      if (r < g.r1) {
        if (a.rows) {
          p = a.rows + (size_t)r * a.d;
        } else {
          const int tok = a.row_src[r] / a.k;
          p = reinterpret_cast<const bf16_t*>(a.src.p[tok / a.T_src]) + (size_t)(tok % a.T_src) * a.d;
        }
      }
      s_src[sub][lane] = p;
      wave_lds_fence();
    }
    uint32_t v[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16_t* p = s_src[sub][8 * rg + i];
      uint4 u = make_uint4(0, 0, 0, 0);
      if (p) u = *reinterpret_cast<const uint4*>(p + c0);
      v[i][0] = u.x;
      v[i][1] = u.y;
      v[i][2] = u.z;
      v[i][3] = u.w;
    }
    bf16_t* dst = a.xT + (size_t)c0 * a.ldt + 64 * mt + 8 * rg;
#pragma unroll
    for (int jc = 0; jc < 8; ++jc) {
      const int w = jc >> 1;
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = (jc & 1) ? (v[2 * q][w] >> 16) | (v[2 * q + 1][w] & 0xFFFF0000u)
                        : (v[2 * q][w] & 0xFFFFu) | (v[2 * q + 1][w] << 16);
      *reinterpret_cast<uint4*>(dst + (size_t)jc * a.ldt) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

// WIN: launched for one window of the backward through the ring (a.win set);
// a one-launch kernel (WIN false) has none of the window code, so its
// accumulators have one definition and stay in registers.
// HT (MODE 1, one launch): B = h transposed per expert like the token rows
// (a.BT, [I, ldt]), k-contiguous, instead of h read n-contiguous.
template <class C, int MODE, bool WIN, bool HT = false>
__global__ __launch_bounds__(kThreads, C::OCC) void wgrad_g2(WgArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int s_cp[257], s_xp[257], s_tp[257], s_rows[2], s_tpw[257];
  wg_chunk_prefix(a.offsets, a.E_local, a.R_cap, s_cp, s_xp, s_tp, s_rows);
  // ring window: 64-row tiles of the window's pieces before each expert (the
  // expert's first column in the window's transposed rows is 64 s_tpw[e])
  if (MODE == 0 && WIN) group_prefix(a.win + 3, a.E_local, a.R_cap, s_tpw, 64);
  const int per = a.mtn * a.ntn;
  const bool spread = wg_spread(per, s_rows);
  int e, c, mt, nt;
  if (spread) {
    // Spread mode: expert order(j) owns workgroups [j per, (j+1) per), the
    // most routed expert first so its long tiles start first; within an
    // expert each XCD gets a contiguous range of tiles in grouped order, so
    // tiles sharing operand panels share an L2.
    const int j = blockIdx.x / per;
    if (j >= a.E_local) return;
    e = a.order[j];
    c = 0;
    grouped_order(xcd_tile(blockIdx.x % per, per), a.mtn, a.ntn, &mt, &nt);
  } else {
    // Chunks are dealt round-robin to the 8 XCDs (workgroup b runs on XCD
    // b % 8) and a chunk's tiles stay on one XCD: chunks of a heavily routed
    // expert spread over all XCDs while the tiles that share a chunk's
    // operand rows share an L2.  The grid holds a multiple of 8 chunk slots.
    const int TC = s_cp[a.E_local < 256 ? a.E_local : 256];
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int q = xcd + 8 * (slot / per);
    if (q >= TC) return;
    const int tile = slot % per;
    mt = tile / a.ntn;
    nt = tile % a.ntn;
    e = 0;
    int hi = a.E_local - 1;
    while (e < hi) {
      const int mid = (e + hi + 1) >> 1;
      if (s_cp[mid] <= q) e = mid; else hi = mid - 1;
    }
    c = q - s_cp[e];
  }
  const int e_lo = min(a.offsets[e], a.R_cap), e_hi = min(a.offsets[e + 1], a.R_cap);
  const int cs = e_lo + c * kWgChunk;                       // the chunk's rows [cs, ce)
  const int ce = spread ? e_hi : min(cs + kWgChunk, e_hi);
  int off = cs, cnt = ce - cs, lo = 0, xcol = 0;
  bool keep = false;
  if constexpr (WIN) {
    // the chunk's rows inside the window; an expert without rows writes its
    // zero gradient in the first window
    lo = a.win[0];
    const int ws = a.win[3 + e], we = a.win[3 + e + 1];
    const int ks = max(cs, ws), ke = min(ce, we);
    if (ke <= ks && !(e_hi == e_lo && a.win[2] == 0)) return;
    off = ke > ks ? ks : cs;
    cnt = ke > ks ? ke - ks : 0;
    keep = off > cs;  // the chunk began in an earlier window
    xcol = off - ws;  // column of the row in the window's transposed rows
  }
  const int m0 = mt * BM, n0 = nt * C::BN;
  float* part = c > 0 ? a.part + (size_t)(s_xp[e] + c - 1) * a.M * a.N : nullptr;
  auto out_row_ptr = [&](int m) -> float* {
    if (part) return part + (size_t)m * a.N;
    if (MODE == 0)
      return m < a.I ? a.out0 + ((size_t)e * a.I + m) * a.N
                     : a.out1 + ((size_t)e * a.I + (m - a.I)) * a.N;
    return a.out0 + ((size_t)e * a.M + m) * a.N;
  };
  Acc<C> acc;
  // through the ring: the partial sum of the chunk's earlier rows as the
  // last window left it, else zeros -- one unconditional definition of every
  // accumulator, right before the main loop continues from it (earlier, the
  // accumulators would be live across the loaders' set-up and spill)
  // (branch-free: every lane loads, from the zero page where there is nothing
  // to carry, so the loads stay in one block)
  auto preload = [&]() {
    if constexpr (WIN) {
      const float* rowp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + out_row(i);
        rowp[i] = keep && m < a.M ? out_row_ptr(m) : nullptr;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < C::WNB; ++j)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int col = n0 + out_col<C>(j, g4);
            const float* src = rowp[i] && col < a.N ? rowp[i] + col
                                                    : reinterpret_cast<const float*>(g_zero);
            const float4 v = *reinterpret_cast<const float4*>(src);
            acc.c[i][j][4 * g4] = v.x;
            acc.c[i][j][4 * g4 + 1] = v.y;
            acc.c[i][j][4 * g4 + 2] = v.z;
            acc.c[i][j][4 * g4 + 3] = v.w;
          }
    }
  };
  MNMajor<BM, C::BK> la;
  la.ncols_left = a.M - m0;
  const bf16_t* Ab = a.A + (size_t)(off - lo) * a.lda + m0;
  auto issue_a = [&](int kt, unsigned l, auto pt) {
    la.issue(kt, l, [&](int kk) -> const bf16_t* { return kk < cnt ? Ab + (size_t)kk * a.lda : nullptr; }, pt);
  };
  if constexpr (MODE == 0 || HT) {
    // B = the chunk's token rows (MODE 0) or h rows (MODE 1) from the
    // transposed copy: row n of the tile is column n0 + n of d (of I),
    // k-contiguous from the chunk's first column; the last stage runs into
    // the expert's zero padding
    static_assert(64 % C::BK == 0, "the transposed rows are padded to 64");
    KMajor<C::BN, C::BK> lb;
    const bf16_t* Bt = WIN ? a.BT + (size_t)64 * s_tpw[e] + xcol
                           : a.BT + (size_t)64 * s_tp[e] + (size_t)c * kWgChunk;
    lb.init([&](int nr) -> const bf16_t* {
      const int n = n0 + nr;
      return n < a.N ? Bt + (size_t)n * a.ldt : nullptr;
    });
    preload();
    mainloop<C, true, false>((cnt + C::BK - 1) / C::BK, issue_a,
                             [&](int kt, unsigned l, auto pt) { lb.issue(kt, l, pt); }, smem, acc, WIN);
  } else {
    MNMajor<C::BN, C::BK> lb;
    lb.ncols_left = a.N - n0;
    const bf16_t* Bb = a.B + (size_t)off * a.ldb + n0;
    preload();
    mainloop<C, true, true>((cnt + C::BK - 1) / C::BK, issue_a,
                            [&](int kt, unsigned l, auto pt) {
                              lb.issue(kt, l, [&](int kk) -> const bf16_t* {
                                return kk < cnt ? Bb + (size_t)kk * a.ldb : nullptr;
                              }, pt);
                            },
                            smem, acc, WIN);
  }
  __syncthreads();
  const WaveStage<C, float> st(smem);
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int pass = 0; pass < WaveStage<C, float>::PASSES; ++pass) {
    st.put(acc, pass);
    wave_lds_fence();
    st.for_chunks(pass, [&](int trow, int srow, int cc) {
      const int m = m0 + (wave >> 1) * 128 + trow;
      const int col = n0 + (wave & 1) * (C::BN / 2) + cc * 4;
      if (m >= a.M || col >= a.N) return;
      *reinterpret_cast<uint4*>(out_row_ptr(m) + col) = st.raw(srow, cc);
    });
    wave_lds_fence();
  }
}

// dW[e] += partial chunks 1, 2, ... of expert e, in chunk order; grid
// (blocks per expert, E_local), experts with one chunk return at once.
template <int MODE>
__global__ __launch_bounds__(kThreads) void wgrad_reduce(WgArgs a) {
  __shared__ int s_cp[257], s_xp[257], s_tp[257], s_rows[2];
  const int e = blockIdx.y;
  const int lo = min(a.offsets[e], a.R_cap), hi = min(a.offsets[e + 1], a.R_cap);
  const int ch = hi > lo ? (hi - lo + kWgChunk - 1) / kWgChunk : 0;
  if (ch <= 1) return;
  wg_chunk_prefix(a.offsets, a.E_local, a.R_cap, s_cp, s_xp, s_tp, s_rows);
  if (wg_spread(a.mtn * a.ntn, s_rows)) return;  // no partial sums were written
  const int xp = s_xp[e];
  const int n4 = a.N / 4;
  const size_t units = (size_t)a.M * n4;
  for (size_t u = (size_t)blockIdx.x * kThreads + threadIdx.x; u < units;
       u += (size_t)gridDim.x * kThreads) {
    const int m = (int)(u / n4), c4 = (int)(u % n4);
    float* dst;
    if (MODE == 0)
      dst = m < a.I ? a.out0 + ((size_t)e * a.I + m) * a.N : a.out1 + ((size_t)e * a.I + (m - a.I)) * a.N;
    else
      dst = a.out0 + ((size_t)e * a.M + m) * a.N;
    float4 v = *reinterpret_cast<const float4*>(dst + c4 * 4);
    for (int c = 1; c < ch; ++c) {
      const float4 p = *reinterpret_cast<const float4*>(a.part + (size_t)(xp + c - 1) * a.M * a.N +
                                                        (size_t)m * a.N + c4 * 4);
      v.x += p.x;
      v.y += p.y;
      v.z += p.z;
      v.w += p.w;
    }
    *reinterpret_cast<float4*>(dst + c4 * 4) = v;
  }
}

}  // namespace

size_t wgrad_partial_bytes(int R_cap, int d, int I) {
  return (size_t)(R_cap / kWgChunk) * 2 * (size_t)I * d * sizeof(float);
}

// Local experts by routed rows (clipped to R_cap), descending; equal counts
// keep the lower id first.  One workgroup of 256 threads, thread e ranks
// expert e against all others.
__global__ __launch_bounds__(kThreads) void expert_order_kernel(const int32_t* offsets, int E_local,
                                                                int R_cap, int32_t* order) {
  __shared__ int s_cnt[kThreads];
  const int e = threadIdx.x;
  int c = -1;
  if (e < E_local) c = min(offsets[e + 1], R_cap) - min(offsets[e], R_cap);
  s_cnt[e] = c;
  __syncthreads();
  if (e < E_local) {
    int rank = 0;
    for (int f = 0; f < E_local; ++f) {
      const int cf = s_cnt[f];
      rank += (cf > c || (cf == c && f < e)) ? 1 : 0;
    }
    order[rank] = e;
  }
}

// Rows of a launch: all routed rows, or one ring window's (at most win_rows).
static int launch_rows(const BwdPlan& p) { return p.win ? p.win_rows : p.R_cap; }

bool bwd_ring_geometry(int64_t ring_bytes, int d, int I, int E_local, int mb, int R_cap,
                       int* slots, int* rows, int64_t* cols, int* n_win) {
  if (mb < 64 || mb % 64 != 0) return false;  // windows cut at multiples of 64 rows
  const int64_t slot = (int64_t)mb * (2 * (int64_t)d + 2 * (int64_t)I) * 2;
  const int64_t fixed = (64 * (int64_t)E_local + 64) * d * 2 + 3 * 256;
  if (ring_bytes < fixed + slot) return false;
  int64_t ns = (ring_bytes - fixed) / slot;
  const int64_t m_max = ((int64_t)R_cap + mb - 1) / mb + E_local;  // minibatches, at most
  if (ns > m_max) ns = m_max;
  if (ns < 1) ns = 1;
  *slots = (int)ns;
  *rows = (int)(ns * mb);
  *cols = ((int64_t)*rows + 64 * (int64_t)E_local + 63) / 64 * 64;
  *n_win = (int)((m_max + ns - 1) / ns);
  return true;
}

mok_status launch_gather_t(const BwdPlan& p, void* xT, hipStream_t stream, int max_blocks,
                           const void* rows, int width) {
  if (p.R_cap == 0) return MOK_OK;
  GatherTArgs g;
  g.src = p.src_x;
  g.rows = reinterpret_cast<const bf16_t*>(rows);
  g.row_src = p.row_src;
  // a ring window's pieces: columns 64 P(e) + (r - woff[e]) of the window's rows
  g.offsets = p.win ? p.win + 3 : p.offsets;
  g.xT = reinterpret_cast<bf16_t*>(xT);
  g.ldt = p.win ? p.win_cols : xt_ld(p.R_cap, p.E_local);
  g.d = rows ? width : p.d;
  g.E_local = p.E_local;
  g.R_cap = p.R_cap;
  g.T_src = p.T_src;
  g.k = p.k;
  const int tiles = (launch_rows(p) + 63) / 64 + p.E_local;  // bound of the 64-row tiles
  const int groups = (tiles + 3) / 4;
  int gx = groups < 256 ? groups : 256;
  // a cap on the workgroups (the copy then runs thin beside a GEMM on
  // another stream); workgroups stride over the tile groups either way
  if (max_blocks > 0) {
    const int cap = max_blocks / (g.d / 64) > 0 ? max_blocks / (g.d / 64) : 1;
    if (gx > cap) gx = cap;
  }
  hipLaunchKernelGGL(gather_t_kernel, dim3((unsigned)gx, (unsigned)(g.d / 64)), dim3(kThreads), 0,
                     stream, g);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

// W^T of the expert weights, bf16, for dh and dx: out[e][n][k] for k < K0
// from src0[e][k][n], for K0 <= k < K0 + K1 from src1[e][k - K0][n].  A
// workgroup moves 128 k x 64 n through LDS; K0 + K1 and N are multiples of
// 128 and 64 (d % 128 == 0, I % 64 == 0).
__global__ __launch_bounds__(kThreads) void transpose_weights_kernel(const bf16_t* src0,
                                                                    const bf16_t* src1,
                                                                    int64_t estride, int K0,
                                                                    int K1, int N, bf16_t* out) {
  __shared__ bf16_t tile[128][64 + 8];
  const int e = blockIdx.z, n0 = blockIdx.y * 64, K = K0 + K1;
  const int k0 = blockIdx.x * 128;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int row = pass * 32 + threadIdx.x / 8, c = threadIdx.x % 8;
    const int k = k0 + row;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (k < K) {
      const bf16_t* src = k < K0 ? src0 + (size_t)e * estride + (size_t)k * N
                                 : src1 + (size_t)e * estride + (size_t)(k - K0) * N;
      v = ld16(src + n0 + c * 8);
    }
    *reinterpret_cast<uint4*>(&tile[row][c * 8]) = v;
  }
  __syncthreads();
  // 64 rows n x 16 chunks of 8 k; lanes take consecutive n (conflict-free LDS)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = threadIdx.x + kThreads * j, n = q % 64, kc = q / 64;
    if (k0 + kc * 8 >= K) continue;
    uint32_t w[4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
      w[h] = (uint32_t)tile[kc * 8 + 2 * h][n] | ((uint32_t)tile[kc * 8 + 2 * h + 1][n] << 16);
    *reinterpret_cast<uint4*>(out + ((size_t)e * N + n0 + n) * K + k0 + kc * 8) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

mok_status launch_swiglu_bwd(const BwdPlan& p, hipStream_t stream) {
  const size_t pieces = (size_t)launch_rows(p) * (p.I / 8);
  if (pieces == 0) return MOK_OK;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)((pieces + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, reinterpret_cast<const bf16_t*>(p.ab),
                     reinterpret_cast<bf16_t*>(p.dab), p.offsets, p.E_local, p.R_cap, p.I, p.win);
  trace_mark(p.tr, "bwd_swiglu", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

mok_status launch_prepare_bwd_bf16(int E_local, int d, int I, const void* w_gate, const void* w_up,
                                   const void* w_down, void* wt_down, void* wt_gu,
                                   hipStream_t stream) {
  // W_down^T [E_local, I, d] from W_down [E_local, d, I]
  hipLaunchKernelGGL(transpose_weights_kernel, dim3((unsigned)((d + 127) / 128), (unsigned)(I / 64),
                                                    (unsigned)E_local),
                     dim3(kThreads), 0, stream, reinterpret_cast<const bf16_t*>(w_down),
                     (const bf16_t*)nullptr, (int64_t)d * I, d, 0, I,
                     reinterpret_cast<bf16_t*>(wt_down));
  // [W_gate; W_up]^T [E_local, d, 2I] from W_gate, W_up [E_local, I, d]
  hipLaunchKernelGGL(transpose_weights_kernel, dim3((unsigned)((2 * I + 127) / 128),
                                                    (unsigned)(d / 64), (unsigned)E_local),
                     dim3(kThreads), 0, stream, reinterpret_cast<const bf16_t*>(w_gate),
                     reinterpret_cast<const bf16_t*>(w_up), (int64_t)I * d, I, I, d,
                     reinterpret_cast<bf16_t*>(wt_gu));
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

mok_status launch_bwd_dgrad(const BwdPlan& p, hipStream_t stream) {
  if (p.R_cap == 0) return MOK_OK;
  const int rows = launch_rows(p);
  const int mt = (rows + BM - 1) / BM + p.E_local;
  const int32_t* offs = p.win ? p.win + 3 : p.offsets;
  DhArgs d;
  d.dy = reinterpret_cast<const bf16_t*>(p.dy);
  d.wd = reinterpret_cast<const bf16_t*>(p.wd);
  d.ab = reinterpret_cast<const bf16_t*>(p.ab);
  d.dab = reinterpret_cast<bf16_t*>(p.dab);
  d.offsets = offs;
  d.win = p.win;
  d.d = p.d;
  d.I = p.I;
  d.E_local = p.E_local;
  d.R_cap = p.R_cap;
  d.ntn = (p.I + Default::BN - 1) / Default::BN;
  d.wt = reinterpret_cast<const bf16_t*>(p.wt_down);
  if (d.wt)
    hipLaunchKernelGGL((dh_g2<Default, true>), dim3((unsigned)(mt * d.ntn)), dim3(kThreads), 0, stream, d);
  else
    hipLaunchKernelGGL((dh_g2<Default, false>), dim3((unsigned)(mt * d.ntn)), dim3(kThreads), 0, stream, d);
  trace_mark(p.tr, "bwd_dh", stream);
  const mok_status rc = launch_swiglu_bwd(p, stream);
  if (rc != MOK_OK) return rc;
  DxArgs x;
  x.dab = reinterpret_cast<const bf16_t*>(p.dab);
  x.win = p.win;
  x.wg = reinterpret_cast<const bf16_t*>(p.wg);
  x.wu = reinterpret_cast<const bf16_t*>(p.wu);
  x.offsets = offs;
  x.row_src = p.row_src;
  x.dx_stage = p.dx_stage;
  x.d = p.d;
  x.I = p.I;
  x.E_local = p.E_local;
  x.R_cap = p.R_cap;
  x.ntn = (p.d + Default::BN - 1) / Default::BN;
  x.T_src = p.T_src;
  x.k = p.k;
  x.wt = reinterpret_cast<const bf16_t*>(p.wt_gu);
  if (x.wt)
    hipLaunchKernelGGL((dx_g2<Default, true>), dim3((unsigned)(mt * x.ntn)), dim3(kThreads), 0, stream, x);
  else
    hipLaunchKernelGGL((dx_g2<Default, false>), dim3((unsigned)(mt * x.ntn)), dim3(kThreads), 0, stream, x);
  trace_mark(p.tr, "bwd_dx_push", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

static WgArgs wgrad_args(const BwdPlan& p, const void* x_perm, int mode) {
  WgArgs w;
  memset(&w, 0, sizeof(w));
  w.order = p.wg_order;
  w.part = p.wg_part;
  w.offsets = p.offsets;
  w.win = p.win;
  w.I = p.I;
  w.E_local = p.E_local;
  w.R_cap = p.R_cap;
  if (mode == 0) {
    w.A = reinterpret_cast<const bf16_t*>(p.dab);
    w.BT = reinterpret_cast<const bf16_t*>(x_perm);
    w.ldt = p.win ? p.win_cols : xt_ld(p.R_cap, p.E_local);
    w.out0 = p.dw_gate;
    w.out1 = p.dw_up;
    w.lda = 2 * p.I;
    w.ldb = p.d;
    w.M = 2 * p.I;
    w.N = p.d;
    w.mtn = (w.M + BM - 1) / BM;
    w.ntn = (w.N + Default::BN - 1) / Default::BN;
  } else {
    w.part = p.wd_part ? p.wd_part : p.wg_part;
    w.A = reinterpret_cast<const bf16_t*>(p.dy);
    w.B = reinterpret_cast<const bf16_t*>(p.h);
    w.out0 = p.dw_down;
    w.lda = p.d;
    w.ldb = p.I;
    w.M = p.d;
    w.N = p.I;
    w.mtn = (w.M + BM - 1) / BM;
    w.ntn = (w.N + Narrow::BN - 1) / Narrow::BN;
  }
  return w;
}

mok_status launch_bwd_wgrad(const BwdPlan& p, const void* x_perm, hipStream_t stream,
                            bool order, bool reduce) {
  // grid bound of the split-K tiles: every expert's chunks, at most
  // R_cap / kWgChunk + E_local of them, rounded up to a multiple of 8.  The
  // grid covers both schedules (max_chunks >= E_local); the kernels pick one
  // from the routed counts (wg_spread) and surplus workgroups return.
  const int max_chunks = (p.R_cap / kWgChunk + p.E_local + 7) / 8 * 8;
  if (order)
    hipLaunchKernelGGL(expert_order_kernel, dim3(1), dim3(kThreads), 0, stream, p.offsets,
                       p.E_local, p.R_cap, p.wg_order);
  WgArgs w = wgrad_args(p, x_perm, 0);
  const dim3 grid0((unsigned)(max_chunks * w.mtn * w.ntn));
  if (p.win)
    hipLaunchKernelGGL((wgrad_g2<Default, 0, true>), grid0, dim3(kThreads), 0, stream, w);
  else
    hipLaunchKernelGGL((wgrad_g2<Default, 0, false>), grid0, dim3(kThreads), 0, stream, w);
  trace_mark(p.tr, "bwd_wgrad_gate_up", stream);
  if (reduce) {
    hipLaunchKernelGGL((wgrad_reduce<0>), dim3(512, (unsigned)p.E_local), dim3(kThreads), 0, stream,
                       w);
    trace_mark(p.tr, "bwd_wgrad_gate_up_reduce", stream);
  }
  w = wgrad_args(p, x_perm, 1);
  if (!p.win && p.hT) {
    // h transposed per expert (k-contiguous B): the 256 x 256 tile
    w.B = nullptr;
    w.BT = reinterpret_cast<const bf16_t*>(p.hT);
    w.ldt = xt_ld(p.R_cap, p.E_local);
    w.ntn = (w.N + Default::BN - 1) / Default::BN;
    hipLaunchKernelGGL((wgrad_g2<Default, 1, false, true>),
                       dim3((unsigned)(max_chunks * w.mtn * w.ntn)), dim3(kThreads), 0, stream, w);
  } else {
    const dim3 grid1((unsigned)(max_chunks * w.mtn * w.ntn));
    if (p.win)
      hipLaunchKernelGGL((wgrad_g2<Narrow, 1, true>), grid1, dim3(kThreads), 0, stream, w);
    else
      hipLaunchKernelGGL((wgrad_g2<Narrow, 1, false>), grid1, dim3(kThreads), 0, stream, w);
  }
  trace_mark(p.tr, "bwd_wgrad_down", stream);
  if (reduce) {
    hipLaunchKernelGGL((wgrad_reduce<1>), dim3(512, (unsigned)p.E_local), dim3(kThreads), 0, stream,
                       w);
    trace_mark(p.tr, "bwd_wgrad_down_reduce", stream);
  }
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

mok_status launch_bwd_reduce(const BwdPlan& p, hipStream_t stream) {
  WgArgs w = wgrad_args(p, nullptr, 0);
  w.win = nullptr;
  hipLaunchKernelGGL((wgrad_reduce<0>), dim3(512, (unsigned)p.E_local), dim3(kThreads), 0, stream, w);
  trace_mark(p.tr, "bwd_wgrad_gate_up_reduce", stream);
  w = wgrad_args(p, nullptr, 1);
  w.win = nullptr;
  hipLaunchKernelGGL((wgrad_reduce<1>), dim3(512, (unsigned)p.E_local), dim3(kThreads), 0, stream, w);
  trace_mark(p.tr, "bwd_wgrad_down_reduce", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

mok_status launch_bwd_gemms_bf16(const BwdPlan& p, const void* x_perm, hipStream_t stream,
                                 hipEvent_t before_wgrad, hipEvent_t after_dx) {
  mok_status rc = launch_bwd_dgrad(p, stream);
  if (rc != MOK_OK) return rc;
  if (after_dx) MOK_HIP_CHECK(hipEventRecord(after_dx, stream));
  if (before_wgrad) MOK_HIP_CHECK(hipStreamWaitEvent(stream, before_wgrad, 0));
  return launch_bwd_wgrad(p, x_perm, stream, true, true);
}

// The window descriptor of ring window w: minibatches [w nslot, (w+1) nslot)
// of mb rows of one expert each, in expert order -> rows [lo, hi) and the
// expert pieces clipped to them.  A window past the last minibatch is empty
// (lo = hi = R).
__global__ __launch_bounds__(kThreads) void bwd_window_kernel(const int32_t* offsets, int E_local,
                                                              int R_cap, int mb, int nslot, int w,
                                                              int32_t* win) {
  __shared__ int s_mbp[257];
  const int M = group_prefix(offsets, E_local, R_cap, s_mbp, mb);
  const int R = min(offsets[E_local], R_cap);
  const int64_t first = (int64_t)w * nslot;
  int lo = R, hi = R;
  if (first < M) {
    const int last = (int)min<int64_t>(M, first + nslot) - 1;
    lo = group_tile(offsets, E_local, R_cap, s_mbp, (int)first, mb).r0;
    hi = group_tile(offsets, E_local, R_cap, s_mbp, last, mb).r1;
  }
  if (threadIdx.x == 0) {
    win[0] = lo;
    win[1] = hi;
    win[2] = w;
  }
  for (int e = threadIdx.x; e <= E_local; e += kThreads)
    win[3 + e] = min(max(min(offsets[e], R_cap), lo), hi);
}

mok_status launch_bwd_window(const BwdPlan& p, int w, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_window_kernel, dim3(1), dim3(kThreads), 0, stream, p.offsets, p.E_local,
                     p.R_cap, p.win_mb, p.win_slots, w, p.win);
  trace_mark(p.tr, "bwd_ring_window", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

}  // namespace mok
