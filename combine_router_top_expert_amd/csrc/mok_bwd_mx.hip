// MXFP8 backward of the expert FFN (kucoin article, section 03: the layer's
// backward in MXFP8).  Every backward GEMM runs on the scaled matrix cores
// with both operands E4M3 + one E8M0 scale per 32 along its contraction
// axis, quantised from the stored bf16 values:
//   dh = dy W_down:         dy rows quantised along d; W_down^T [I, d] along d
//   dx = [da|db] W_gu:      [da|db] rows along 2I; [W_gate; W_up]^T [d, 2I] along 2I
//   dW_gate|up = [da|db]^T X, dW_down = dy^T h: both operands transposed,
//                           each column quantised along the expert's rows in
//                           blocks of 32 (the expert's rows padded to 128)
// The transposed weights are prepared once (mok_prepare_bwd).  The
// activations are packed by one kernel per operand that stages 128 rows (one
// MX stage of an expert's rows) x 64 channels through LDS and writes both
// quantisations from that one copy: along the row (32 channels a block, for
// dh and dx) and along the rows (32 rows a block, transposed, for the weight
// gradients).  The SwiGLU backward runs inside the [da|db] pack, and h's
// codes are decoded inside its pack, so no bf16 [da|db] or h is written.
// The weight gradients contract over a whole expert per output tile (a fixed
// order; the results are run-to-run identical).
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
    w[q] = e4m3_pack4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], sh);
  }
  uint8_t* out = codes + (size_t)ch * ldc + col0 + blk * 32;
  *reinterpret_cast<uint4*>(out) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint4*>(out + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  scales[(size_t)ch * (ldc / 32) + (col0 / 32) + blk] = (uint8_t)(sh + 127);
}

// ---------------------------------------------------------------- packs
// One tile of 128 rows x 64 channels in LDS, bf16.  Row r's elements sit at
// r * kPitch + (r / 32) * 8 + c: the 32-row blocks are shifted against each
// other by 16 bytes, so the lanes of a column read (4 blocks of one channel)
// fall in different banks, and 16-byte row chunks stay aligned.
constexpr int kPitch = kTqCh + 8;
constexpr int kTileElems = kTqRows * kPitch + 32;
__device__ __forceinline__ int tix(int r, int c) { return r * kPitch + (r >> 5) * 8 + c; }

// Both quantisations read the LDS tile twice (the block's largest
// magnitude, then the codes) rather than hold 32 values in registers: the
// packs are HBM-bound, and the registers saved let twice the workgroups
// overlap their loads with each other's quantisation.

// 8 bf16 of a 16-byte LDS chunk as floats.
__device__ __forceinline__ void unpack8(uint4 u, float* v) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
}

// Quantise tile rows [0, nrows) along the row: row r's two 32-channel blocks
// -> codes[(r0 + r) ldq + ch0 + ..], scales[(r0 + r) ldq / 32 + ch0 / 32 + ..].
__device__ __forceinline__ void pack_rows(const bf16_t* t, int nrows, uint8_t* codes,
                                          uint8_t* scales, int64_t ldq, int64_t r0, int ch0) {
  const int r = threadIdx.x >> 1, blk = threadIdx.x & 1;
  if (r >= nrows) return;
  const bf16_t* row = t + tix(r, blk * 32);
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v[8];
    unpack8(*reinterpret_cast<const uint4*>(row + q * 8), v);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  }
  const int sh = mx_shared_exp(amax);
  uint32_t wq[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v[8];
    unpack8(*reinterpret_cast<const uint4*>(row + q * 8), v);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      wq[2 * q + h] = e4m3_pack4(v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3], sh);
    }
  }
  uint8_t* out = codes + (r0 + r) * ldq + ch0 + blk * 32;
  *reinterpret_cast<uint4*>(out) = make_uint4(wq[0], wq[1], wq[2], wq[3]);
  *reinterpret_cast<uint4*>(out + 16) = make_uint4(wq[4], wq[5], wq[6], wq[7]);
  scales[(r0 + r) * (ldq / 32) + ch0 / 32 + blk] = (uint8_t)(sh + 127);
}

// Quantise the tile's channels along its 128 rows (rows past the expert's
// end are zeros): codes[(ch0 + ch) ldc + col0 + ..] and the scales of its four
// 32-row blocks.  Four consecutive lanes write one channel's 128 codes.
__device__ __forceinline__ void pack_cols(const bf16_t* t, uint8_t* codes, uint8_t* scales,
                                          int64_t ldc, int64_t col0, int ch0) {
  const int ch = threadIdx.x >> 2, blk = threadIdx.x & 3;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(bf16_to_f32(t[tix(blk * 32 + i, ch)])));
  const int sh = mx_shared_exp(amax);
  uint32_t wq[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    wq[q] = e4m3_pack4(bf16_to_f32(t[tix(blk * 32 + 4 * q, ch)]), bf16_to_f32(t[tix(blk * 32 + 4 * q + 1, ch)]),
                       bf16_to_f32(t[tix(blk * 32 + 4 * q + 2, ch)]), bf16_to_f32(t[tix(blk * 32 + 4 * q + 3, ch)]),
                       sh);
  }
  uint8_t* out = codes + (int64_t)(ch0 + ch) * ldc + col0 + blk * 32;
  *reinterpret_cast<uint4*>(out) = make_uint4(wq[0], wq[1], wq[2], wq[3]);
  *reinterpret_cast<uint4*>(out + 16) = make_uint4(wq[4], wq[5], wq[6], wq[7]);
  scales[(int64_t)(ch0 + ch) * (ldc / 32) + col0 / 32 + blk] = (uint8_t)(sh + 127);
}

// What a pack reads and writes.  KIND 0: dy rows (bf16 [R_cap, ld]) -> both
// quantisations.  KIND 1: the SwiGLU backward of the tile's 64 columns of I
// from dh (bf16 [R_cap, ld]) and the saved a | b: da -> channels ch0, db ->
// channels I + ch0, both quantisations of each.  KIND 2: h's E4M3 codes and
// scales decoded (exact in bf16) -> the transposed quantisation only.
// KIND 3: the token rows of the items, from the sources through row_src ->
// the transposed quantisation only.
struct PackArgs {
  const bf16_t* src;       // KIND 0: dy; 1: dh
  int64_t ld;              // leading dimension of src (elements)
  const bf16_t* ab;        // KIND 1: [R_cap, 2I]
  const uint8_t* hq;       // KIND 2: [R_cap, I] codes
  const uint8_t* hs;       // KIND 2: [R_cap, I / 32] scales
  SrcTable tok;            // KIND 3
  const int32_t* row_src;
  const int32_t* offsets;
  uint8_t *rq, *rs;        // along the row: codes [R_cap, ldq], scales
  int64_t ldq;
  uint8_t *cq, *cs;        // transposed: codes [channels, ldc], scales
  int64_t ldc;
  int E_local, R_cap, T_src, k, I;
};

__device__ __forceinline__ void swiglu_bwd8(const uint4 hv, const uint4 av, const uint4 bv,
                                            uint4* da_out, uint4* db_out) {
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
  *da_out = make_uint4(d0.x, d0.y, d1.x, d1.y);
  *db_out = make_uint4(e0.x, e0.y, e1.x, e1.y);
}

// One E4M3 code times 2^sh, as bf16 (exact: 4 significant bits).
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t c, int sh) {
  const uint32_t mag = c & 0x7Fu, ex = mag >> 3, man = mag & 7u;
  float v = ex ? __builtin_amdgcn_ldexpf((float)(8u + man), (int)ex - 10)
               : __builtin_amdgcn_ldexpf((float)man, -9);
  v = __builtin_amdgcn_ldexpf(v, sh);
  return f32_to_bf16((c & 0x80u) ? -v : v);
}

// A tile's raw loads, one 16-byte chunk per thread and pass (KIND 1: dh, a,
// b; KIND 2: 8 codes and their scale).  Issued for the next tile before the
// current one is quantised, so the loads are in flight during that work.
struct PackRaw {
  uint4 v[4][3];
  int sh[4];
};

template <int KIND>
__device__ __forceinline__ void pack_fetch(const PackArgs& a, const GTile& g, int ch0,
                                           PackRaw& raw) {
  const int nrows = g.r1 - g.r0, cc = threadIdx.x % 8;
#pragma unroll
  for (int pass = 0; pass < kTqRows / 32; ++pass) {
    const int row = pass * 32 + threadIdx.x / 8;
    const int r = g.r0 + row;
    const uint4 z = make_uint4(0, 0, 0, 0);
    raw.v[pass][0] = raw.v[pass][1] = raw.v[pass][2] = z;
    raw.sh[pass] = 0;
    if (row >= nrows) continue;
    if (KIND == 0) {
      raw.v[pass][0] = ld16(a.src + (size_t)r * a.ld + ch0 + cc * 8);
    } else if (KIND == 1) {
      const bf16_t* abr = a.ab + (size_t)r * 2 * a.I + ch0 + cc * 8;
      raw.v[pass][0] = ld16(a.src + (size_t)r * a.ld + ch0 + cc * 8);
      raw.v[pass][1] = ld16(abr);
      raw.v[pass][2] = ld16(abr + a.I);
    } else if (KIND == 2) {
      const uint2 c8 = *reinterpret_cast<const uint2*>(a.hq + (size_t)r * a.I + ch0 + cc * 8);
      raw.v[pass][0] = make_uint4(c8.x, c8.y, 0, 0);
      raw.sh[pass] = (int)a.hs[(size_t)r * (a.I / 32) + (ch0 + cc * 8) / 32] - 127;
    } else {
      const int tok = a.row_src[r] / a.k;
      raw.v[pass][0] = ld16(reinterpret_cast<const bf16_t*>(a.tok.p[tok / a.T_src]) +
                            (size_t)(tok % a.T_src) * a.ld + ch0 + cc * 8);
    }
  }
}

// The raw loads -> the LDS tile(s) (KIND 1: the SwiGLU backward here; rows
// past the expert's end hold zeros either way).
template <int KIND>
__device__ __forceinline__ void pack_stash(const PackRaw& raw, const GTile& g, bf16_t* t0,
                                           bf16_t* t1) {
  const int nrows = g.r1 - g.r0, cc = threadIdx.x % 8;
#pragma unroll
  for (int pass = 0; pass < kTqRows / 32; ++pass) {
    const int row = pass * 32 + threadIdx.x / 8;
    uint4 v0 = raw.v[pass][0], v1 = make_uint4(0, 0, 0, 0);
    if (KIND == 1 && row < nrows) swiglu_bwd8(raw.v[pass][0], raw.v[pass][1], raw.v[pass][2], &v0, &v1);
    if (KIND == 2) {
      const uint32_t cw[2] = {v0.x, v0.y};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = e4m3_to_bf16_bits((cw[q >> 1] >> (16 * (q & 1))) & 0xFFu, raw.sh[pass]);
        const uint32_t hi = e4m3_to_bf16_bits((cw[q >> 1] >> (16 * (q & 1) + 8)) & 0xFFu, raw.sh[pass]);
        o[q] = lo | (hi << 16);
      }
      v0 = make_uint4(o[0], o[1], o[2], o[3]);
    }
    *reinterpret_cast<uint4*>(t0 + tix(row, cc * 8)) = v0;
    if (KIND == 1) *reinterpret_cast<uint4*>(t1 + tix(row, cc * 8)) = v1;
  }
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void mx_pack_kernel(PackArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[KIND == 1 ? 2 : 1][kTileElems];
  __shared__ int s_prefix[257];
  const int total = group_prefix(a.offsets, a.E_local, a.R_cap, s_prefix, kTqRows);
  const int ch0 = blockIdx.y * kTqCh;
  int t = blockIdx.x;
  if (t >= total) return;
  GTile g = group_tile(a.offsets, a.E_local, a.R_cap, s_prefix, t, kTqRows);
  PackRaw raw;
  pack_fetch<KIND>(a, g, ch0, raw);
  for (; t < total; t += gridDim.x) {
    const GTile cur = g;
    pack_stash<KIND>(raw, cur, tile[0], tile[KIND == 1 ? 1 : 0]);
    __syncthreads();
    const int tn = t + gridDim.x;
    if (tn < total) {
      g = group_tile(a.offsets, a.E_local, a.R_cap, s_prefix, tn, kTqRows);
      pack_fetch<KIND>(a, g, ch0, raw);
    }
    const int nrows = cur.r1 - cur.r0;
    const int64_t col0 = (int64_t)t * kTqRows;
#pragma unroll
    for (int h = 0; h < (KIND == 1 ? 2 : 1); ++h) {
      const int ch = ch0 + h * a.I;  // KIND 1: da at ch0, db at I + ch0
      if (KIND <= 1) pack_rows(tile[h], nrows, a.rq, a.rs, a.ldq, cur.r0, ch);
      pack_cols(tile[h], a.cq, a.cs, a.ldc, col0, ch);
    }
    __syncthreads();  // the tile is read before the next one is stored over it
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

template <int KIND>
static mok_status launch_pack(const BwdPlan& p, const PackArgs& a, int channels,
                              hipStream_t stream) {
  // about four tiles per workgroup, so each one's loads overlap the
  // quantisation of the one before
  const int tiles = (int)(p.mx_cols / kTqRows);
  const int gx = tiles / 4 > 0 ? tiles / 4 : 1;
  hipLaunchKernelGGL(mx_pack_kernel<KIND>, dim3((unsigned)gx, (unsigned)(channels / kTqCh)),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

static PackArgs pack_args(const BwdPlan& p) {
  PackArgs a;
  memset(&a, 0, sizeof(a));
  a.tok = p.src_x;
  a.row_src = p.row_src;
  a.offsets = p.offsets;
  a.ldc = p.mx_cols;
  a.E_local = p.E_local;
  a.R_cap = p.R_cap;
  a.T_src = p.T_src;
  a.k = p.k;
  a.I = p.I;
  return a;
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
  // dy: along d for dh, along the rows for dW_down
  PackArgs a = pack_args(p);
  a.src = reinterpret_cast<const bf16_t*>(p.dy);
  a.ld = d;
  a.rq = p.mx_dyq;
  a.rs = p.mx_dys;
  a.ldq = d;
  a.cq = p.mx_dyT;
  a.cs = p.mx_dyTs;
  mok_status rc = launch_pack<0>(p, a, d, stream);
  if (rc != MOK_OK) return rc;
  trace_mark(p.tr, "bwd_pack_dy_mx", stream);
  // dh = dy W_down -> bf16 [R_cap, I] (the first R_cap I elements of dab)
  rc = launch_mx_rows_gemm(p.mx_dyq, p.mx_dys, reinterpret_cast<const uint8_t*>(p.wt_down), p.mx_st_down, d, I, p.E_local,
                           p.R_cap, p.offsets, p.row_src, p.dab, I, nullptr, p.T_src, p.k,
                           stream, p.tr, "bwd_dh_mx");
  if (rc != MOK_OK) return rc;
  // the SwiGLU backward -> [da|db] along 2I for dx, along the rows for dW
  a = pack_args(p);
  a.src = reinterpret_cast<const bf16_t*>(p.dab);
  a.ld = I;
  a.ab = reinterpret_cast<const bf16_t*>(p.ab);
  a.rq = p.mx_dabq;
  a.rs = p.mx_dabs;
  a.ldq = 2 * I;
  a.cq = p.mx_dabT;
  a.cs = p.mx_dabTs;
  if ((rc = launch_pack<1>(p, a, I, stream)) != MOK_OK) return rc;
  trace_mark(p.tr, "bwd_swiglu_pack_mx", stream);
  // dx = [da|db] [W_gate; W_up], pushed to the dx rows
  rc = launch_mx_rows_gemm(p.mx_dabq, p.mx_dabs, reinterpret_cast<const uint8_t*>(p.wt_gu), p.mx_st_gu, 2 * I, d, p.E_local,
                           p.R_cap, p.offsets, p.row_src, nullptr, 0, &p.dx_stage, p.T_src, p.k,
                           stream, p.tr, "bwd_dx_push_mx");
  if (rc != MOK_OK) return rc;
  // h (as GEMM2 read it) and the token rows, along the rows
  a = pack_args(p);
  a.hq = reinterpret_cast<const uint8_t*>(p.h);
  a.hs = p.mx_hs;
  a.cq = p.mx_hT;
  a.cs = p.mx_hTs;
  if ((rc = launch_pack<2>(p, a, I, stream)) != MOK_OK) return rc;
  a = pack_args(p);
  a.ld = d;
  a.cq = p.mx_xT;
  a.cs = p.mx_xTs;
  if ((rc = launch_pack<3>(p, a, d, stream)) != MOK_OK) return rc;
  trace_mark(p.tr, "bwd_pack_h_x_mx", stream);
  return launch_bwd_mx_wgrad(p, stream);
}

}  // namespace mok
