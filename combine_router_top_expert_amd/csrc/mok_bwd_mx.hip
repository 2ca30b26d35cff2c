// MXFP8 backward of the expert FFN (kucoin article, section 03: the layer's
// backward in MXFP8).  Every backward GEMM runs on the scaled matrix cores
// with both operands E4M3 + one E8M0 scale per 32 along its contraction
// axis, quantised from the stored bf16 values:
//   dh = dy W_down:         dy rows quantised along d; W_down^T [I, d] along d
//   dx = [da|db] W_gu:      [da|db] rows along 2I; [W_gate; W_up]^T [d, 2I] along 2I
//   dW_gate|up = [da|db]^T X, dW_down = dy^T h: both operands transposed,
//                           each column quantised along the expert's rows in
//                           blocks of 32 (the expert's rows padded to 128)
// The transposed weights are prepared once (mok_mx_prepare_bwd); the
// transposed activations are written by one kernel that stages a block of
// 128 rows x 64 channels through LDS and quantises each channel's 32-row
// blocks.  The weight gradients contract over a whole expert per output
// tile (a fixed order; the results are run-to-run identical).
#include <string.h>

#include "mok_gemm_mx.h"
#include "mok_internal.h"
#include "mok_mx.h"

namespace mok {

namespace {

using namespace g2;

constexpr int kTqRows = 128;  // rows of a transposed block (one MX stage of k)
constexpr int kTqCh = 64;     // channels of a block

// Transposes and quantises one block: rows k = 0..127 (rowp(k): a bf16
// pointer at channel ch0 of row k, or null for a zero row) x channels
// ch0 .. ch0 + 63: codes[ch][col0 + k] E4M3 and scales[ch][(col0 + k) / 32]
// E8M0, each channel quantised in four blocks of 32 rows.
template <class RowPtr>
__device__ __forceinline__ void tq_block(RowPtr rowp, uint8_t* codes, uint8_t* scales,
                                         int64_t ldc, int64_t col0) {
  __shared__ bf16_t tile[kTqRows][kTqCh + 8];
  const int tid = threadIdx.x;
#pragma unroll
  for (int pass = 0; pass < kTqRows / 32; ++pass) {
    const int row = pass * 32 + tid / 8, chunk = tid % 8;
    const bf16_t* p = rowp(row);
    const uint4 v = p ? ld16(p + chunk * 8) : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(&tile[row][chunk * 8]) = v;
  }
  __syncthreads();
  const int ch = tid & 63, blk = tid >> 6;  // 64 channels x 4 blocks of 32 rows
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = bf16_to_f32(tile[blk * 32 + i][ch]);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const int sh = mx_shared_exp(amax);
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) word |= e4m3_code(__builtin_amdgcn_ldexpf(v[4 * q + e], -sh)) << (8 * e);
    w[q] = word;
  }
  uint8_t* out = codes + (size_t)ch * ldc + col0 + blk * 32;
  *reinterpret_cast<uint4*>(out) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint4*>(out + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  scales[(size_t)ch * (ldc / 32) + (col0 / 32) + blk] = (uint8_t)(sh + 127);
}

// Activations: the rows of every local expert, 128-row tiles of the grouped
// layout (tile t of the layout is column block t of the output); rows past
// an expert's end are zeros.  KIND 0: bf16 rows src + r * ld; KIND 1: the
// token rows of the items, from the source buffers through row_src.
struct TqArgs {
  const bf16_t* src;
  int64_t ld;
  SrcTable tok;
  const int32_t* row_src;
  const int32_t* offsets;
  uint8_t* codes;      // [channels, ldc]
  uint8_t* scales;     // [channels, ldc / 32]
  int64_t ldc;
  int E_local, R_cap, T_src, k;
};

template <int KIND>
__global__ __launch_bounds__(kThreads) void tq_rows_kernel(TqArgs a) {
  __shared__ int s_prefix[257];
  const int total = group_prefix(a.offsets, a.E_local, a.R_cap, s_prefix, kTqRows);
  const int ch0 = blockIdx.y * kTqCh;
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    const GTile g = group_tile(a.offsets, a.E_local, a.R_cap, s_prefix, t, kTqRows);
    tq_block(
        [&](int row) -> const bf16_t* {
          const int r = g.r0 + row;
          if (r >= g.r1) return nullptr;
          if (KIND == 0) return a.src + (size_t)r * a.ld + ch0;
          const int tok = a.row_src[r] / a.k;
          return reinterpret_cast<const bf16_t*>(a.tok.p[tok / a.T_src]) +
                 (size_t)(tok % a.T_src) * a.ld + ch0;
        },
        a.codes + (size_t)ch0 * a.ldc, a.scales + (size_t)ch0 * (a.ldc / 32), a.ldc,
        (int64_t)t * kTqRows);
    __syncthreads();  // the tile is read before the next block's loads overwrite it
  }
}

// Weights, per expert e: out[e][n][k] for k < K0 from src0[e][k][n] and for
// K0 <= k < K0 + K1 from src1[e][k - K0][n] (row-major [K, N] sources).
struct TqWArgs {
  const bf16_t* src0;
  const bf16_t* src1;
  int64_t estride;     // elements per expert of each source
  int K0, K1, N;
  uint8_t* codes;      // [E_local, N, K0 + K1]
  uint8_t* scales;     // [E_local, N, (K0 + K1) / 32]
};

__global__ __launch_bounds__(kThreads) void tq_weights_kernel(TqWArgs a) {
  const int e = blockIdx.z, ch0 = blockIdx.y * kTqCh;
  const int K = a.K0 + a.K1;
  const int64_t k0 = (int64_t)blockIdx.x * kTqRows;
  tq_block(
      [&](int row) -> const bf16_t* {
        const int64_t kk = k0 + row;
        if (kk >= K) return nullptr;
        return kk < a.K0 ? a.src0 + (size_t)e * a.estride + (size_t)kk * a.N + ch0
                         : a.src1 + (size_t)e * a.estride + (size_t)(kk - a.K0) * a.N + ch0;
      },
      a.codes + (size_t)e * a.N * K + (size_t)ch0 * K,
      a.scales + (size_t)e * a.N * (K / 32) + (size_t)ch0 * (K / 32), K, k0);
}

// h as GEMM2 used it: E4M3 codes and their scales -> bf16 (exact: three
// mantissa bits and an E8M0 exponent fit bf16).
__global__ __launch_bounds__(kThreads) void mx_dequant_kernel(const uint8_t* codes,
                                                              const uint8_t* scales, bf16_t* out,
                                                              int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const uint32_t c = codes[i];
  const int sh = (int)scales[i / 32] - 127;
  const uint32_t mag = c & 0x7Fu, ex = mag >> 3, man = mag & 7u;
  float v = ex ? __builtin_amdgcn_ldexpf((float)(8u + man), (int)ex - 10)
               : __builtin_amdgcn_ldexpf((float)man, -9);
  v = __builtin_amdgcn_ldexpf(v, sh);
  out[i] = f32_to_bf16((c & 0x80u) ? -v : v);
}

// Weight gradient of one local expert's output tile, contraction over its
// rows (the transposed operands' columns [128 P(e), 128 P(e) + 128 KT)).
// MODE 0: M = 2I rows of [da|db]^T, N = d; MODE 1: M = d rows of dy^T, N = I.
struct WgMxArgs {
  const uint8_t *A, *As, *B, *Bs;  // [M or N, ldc] codes, [.., ldc / 32] scales
  int64_t ldc;
  const int32_t* offsets;
  float* out0;   // MODE 0: dW_gate [E_local, I, d]; MODE 1: dW_down [E_local, d, I]
  float* out1;   // MODE 0: dW_up
  int M, N, I, E_local, R_cap, mtn, ntn;
};

template <int MODE>
__global__ __launch_bounds__(kThreads) void wgrad_mx_kernel(WgMxArgs a) {
  typedef MxCfg C;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int s_prefix[257];
  group_prefix(a.offsets, a.E_local, a.R_cap, s_prefix, kTqRows);
  const int per = a.mtn * a.ntn;
  const int e = blockIdx.x / per;
  if (e >= a.E_local) return;
  int mt, nt;
  grouped_order(xcd_tile(blockIdx.x % per, per), a.mtn, a.ntn, &mt, &nt);
  const int c0 = s_prefix[e];
  const int KT = s_prefix[e + 1] - c0;  // 128-row stages of the expert (an expert without rows: 0)
  const int m0 = mt * BM, n0 = nt * C::BN;
  const int KS = (int)(a.ldc / 32);
  KMajor<BM, C::BK> la;
  KMajor<C::BN, C::BK> lb;
  ScaleRows<BM> sa;
  ScaleRows<C::BN> sb;
  la.init([&](int row) -> const bf16_t* {
    const int m = m0 + row;
    return m < a.M ? reinterpret_cast<const bf16_t*>(a.A + (size_t)m * a.ldc + (size_t)c0 * kTqRows)
                   : nullptr;
  });
  sa.init([&](int row) -> const uint8_t* {
    const int m = m0 + row;
    return m < a.M ? a.As + (size_t)m * KS + (size_t)c0 * (kTqRows / 32) : nullptr;
  });
  lb.init([&](int row) -> const bf16_t* {
    const int n = n0 + row;
    return n < a.N ? reinterpret_cast<const bf16_t*>(a.B + (size_t)n * a.ldc + (size_t)c0 * kTqRows)
                   : nullptr;
  });
  sb.init([&](int row) -> const uint8_t* {
    const int n = n0 + row;
    return n < a.N ? a.Bs + (size_t)n * KS + (size_t)c0 * (kTqRows / 32) : nullptr;
  });
  Acc<C> acc;
  mx_mainloop(KT, la, lb, sa, sb, smem, acc);
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
      float* dst;
      if (MODE == 0)
        dst = m < a.I ? a.out0 + ((size_t)e * a.I + m) * a.N
                      : a.out1 + ((size_t)e * a.I + (m - a.I)) * a.N;
      else
        dst = a.out0 + ((size_t)e * a.M + m) * a.N;
      *reinterpret_cast<uint4*>(dst + col) = st.raw(srow, cc);
    });
    wave_lds_fence();
  }
}

}  // namespace

int64_t bwd_mx_cols(int R_cap, int E_local) {
  return ((int64_t)(R_cap + kTqRows - 1) / kTqRows + E_local) * kTqRows;
}

mok_status launch_mx_prepare_bwd(int E_local, int d, int I, const void* w_gate, const void* w_up,
                                 const void* w_down, uint8_t* wt_down, uint8_t* st_down,
                                 uint8_t* wt_gu, uint8_t* st_gu, hipStream_t stream) {
  // W_down^T: out[e][i][c] = W_down[e][c][i], quantised along c (K = d)
  TqWArgs a;
  a.src0 = reinterpret_cast<const bf16_t*>(w_down);
  a.src1 = nullptr;
  a.estride = (int64_t)d * I;
  a.K0 = d;
  a.K1 = 0;
  a.N = I;
  a.codes = wt_down;
  a.scales = st_down;
  hipLaunchKernelGGL(tq_weights_kernel, dim3((unsigned)((d + kTqRows - 1) / kTqRows),
                                             (unsigned)(I / kTqCh), (unsigned)E_local),
                     dim3(kThreads), 0, stream, a);
  // [W_gate; W_up]^T: out[e][c][k] = W_gate[e][k][c] (k < I), W_up[e][k - I][c]
  a.src0 = reinterpret_cast<const bf16_t*>(w_gate);
  a.src1 = reinterpret_cast<const bf16_t*>(w_up);
  a.estride = (int64_t)I * d;
  a.K0 = I;
  a.K1 = I;
  a.N = d;
  a.codes = wt_gu;
  a.scales = st_gu;
  hipLaunchKernelGGL(tq_weights_kernel, dim3((unsigned)((2 * I + kTqRows - 1) / kTqRows),
                                             (unsigned)(d / kTqCh), (unsigned)E_local),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

static mok_status launch_tq(const BwdPlan& p, int kind, const void* src, int64_t ld, int channels,
                            uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  TqArgs a;
  memset(&a, 0, sizeof(a));
  a.src = reinterpret_cast<const bf16_t*>(src);
  a.ld = ld;
  a.tok = p.src_x;
  a.row_src = p.row_src;
  a.offsets = p.offsets;
  a.codes = codes;
  a.scales = scales;
  a.ldc = p.mx_cols;
  a.E_local = p.E_local;
  a.R_cap = p.R_cap;
  a.T_src = p.T_src;
  a.k = p.k;
  const int tiles = (int)(p.mx_cols / kTqRows);
  const int gx = tiles < 512 ? tiles : 512;
  dim3 g((unsigned)gx, (unsigned)(channels / kTqCh));
  if (kind == 0)
    hipLaunchKernelGGL(tq_rows_kernel<0>, g, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(tq_rows_kernel<1>, g, dim3(kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

// [dW_gate; dW_up] = MX([da|db]^T) MX(X^T) and dW_down = MX(dy^T) MX(h^T),
// one output tile per workgroup, over the expert's rows.
static mok_status launch_bwd_mx_wgrad(const BwdPlan& p, hipStream_t stream) {
  WgMxArgs w;
  memset(&w, 0, sizeof(w));
  w.ldc = p.mx_cols;
  w.offsets = p.offsets;
  w.I = p.I;
  w.E_local = p.E_local;
  w.R_cap = p.R_cap;
  // [dW_gate; dW_up] = [da|db]^T X
  w.A = p.mx_dabT;
  w.As = p.mx_dabTs;
  w.B = p.mx_xT;
  w.Bs = p.mx_xTs;
  w.out0 = p.dw_gate;
  w.out1 = p.dw_up;
  w.M = 2 * p.I;
  w.N = p.d;
  w.mtn = (w.M + BM - 1) / BM;
  w.ntn = (w.N + MxCfg::BN - 1) / MxCfg::BN;
  hipLaunchKernelGGL(wgrad_mx_kernel<0>, dim3((unsigned)(p.E_local * w.mtn * w.ntn)),
                     dim3(kThreads), 0, stream, w);
  trace_mark(p.tr, "bwd_wgrad_gate_up_mx", stream);
  // dW_down = dy^T h
  w.A = p.mx_dyT;
  w.As = p.mx_dyTs;
  w.B = p.mx_hT;
  w.Bs = p.mx_hTs;
  w.out0 = p.dw_down;
  w.out1 = nullptr;
  w.M = p.d;
  w.N = p.I;
  w.mtn = (w.M + BM - 1) / BM;
  w.ntn = (w.N + MxCfg::BN - 1) / MxCfg::BN;
  hipLaunchKernelGGL(wgrad_mx_kernel<1>, dim3((unsigned)(p.E_local * w.mtn * w.ntn)),
                     dim3(kThreads), 0, stream, w);
  trace_mark(p.tr, "bwd_wgrad_down_mx", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

mok_status launch_bwd_mx_gemms(const BwdPlan& p, hipStream_t stream) {
  // (no rows: every expert's tile contracts over nothing and stores zeros)
  if (p.R_cap == 0) return launch_bwd_mx_wgrad(p, stream);
  const int d = p.d, I = p.I;
  // dh = dy W_down: dy quantised along d, into the first half of each dab row
  mok_status rc = launch_mx_quantize(p.R_cap, d, p.dy, p.mx_dyq, p.mx_dys, stream);
  if (rc != MOK_OK) return rc;
  trace_mark(p.tr, "bwd_quantise_dy_mx", stream);
  rc = launch_mx_rows_gemm(p.mx_dyq, p.mx_dys, p.mx_wt_down, p.mx_st_down, d, I, p.E_local,
                           p.R_cap, p.offsets, p.row_src, p.dab, 2 * I, nullptr, p.T_src, p.k,
                           stream, p.tr, "bwd_dh_mx");
  if (rc != MOK_OK) return rc;
  rc = launch_swiglu_bwd(p, stream);
  if (rc != MOK_OK) return rc;
  // dx = [da|db] [W_gate; W_up]: quantised along 2I, pushed to the dx rows
  rc = launch_mx_quantize(p.R_cap, 2 * I, p.dab, p.mx_dabq, p.mx_dabs, stream);
  if (rc != MOK_OK) return rc;
  trace_mark(p.tr, "bwd_quantise_dab_mx", stream);
  rc = launch_mx_rows_gemm(p.mx_dabq, p.mx_dabs, p.mx_wt_gu, p.mx_st_gu, 2 * I, d, p.E_local,
                           p.R_cap, p.offsets, p.row_src, nullptr, 0, &p.dx_stage, p.T_src, p.k,
                           stream, p.tr, "bwd_dx_push_mx");
  if (rc != MOK_OK) return rc;
  // the weight gradients' operands, transposed and quantised along the rows
  const int64_t nh = (int64_t)p.R_cap * I;
  hipLaunchKernelGGL(mx_dequant_kernel, dim3((unsigned)((nh + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, reinterpret_cast<const uint8_t*>(p.h), p.mx_hs,
                     reinterpret_cast<bf16_t*>(p.mx_hdeq), nh);
  if ((rc = launch_tq(p, 0, p.dab, 2 * I, 2 * I, p.mx_dabT, p.mx_dabTs, stream)) != MOK_OK) return rc;
  if ((rc = launch_tq(p, 1, nullptr, d, d, p.mx_xT, p.mx_xTs, stream)) != MOK_OK) return rc;
  if ((rc = launch_tq(p, 0, p.dy, d, d, p.mx_dyT, p.mx_dyTs, stream)) != MOK_OK) return rc;
  if ((rc = launch_tq(p, 0, p.mx_hdeq, I, I, p.mx_hT, p.mx_hTs, stream)) != MOK_OK) return rc;
  trace_mark(p.tr, "bwd_transpose_quantise_mx", stream);
  return launch_bwd_mx_wgrad(p, stream);
}

}  // namespace mok
