// MFMA tile engine for the expert grouped GEMMs (gfx950).
//
// One workgroup = 4 waves computes a BM x BN tile of C = sum_k A[m][k] B[n][k]
// with fp32 accumulation.  Waves are arranged 2 x 2, each owning a 64 x 64
// sub-tile made of 2 x 2 blocks of the 32 x 32 MFMA:
//   bf16: v_mfma_f32_32x32x16_bf16 (lane l holds 8 consecutive k of row l%32,
//         k-half l/32; same for B with column l%32),
//   fp32: v_mfma_f32_32x32x2_f32   (lane l holds k = l/32 of row l%32).
// Accumulator element v of lane l is C[8*(v/4) + 4*(l/32) + v%4][l%32].
//
// Operand tiles are staged through LDS as [rows][BK] with the contraction
// dimension innermost (padded by 16 bytes per row so that the 16-byte
// fragment reads of 16 lanes fall in distinct banks), double buffered: global
// loads of the next K tile are in flight while the MFMAs consume this one.
// Two loaders fill a tile:
//   KLoader  - operand stored with k contiguous (forward operands): 16-byte
//              units along k, copied straight into LDS;
//   MNLoader - operand stored with m (or n) contiguous and k strided (the
//              backward's weight and wgrad operands): 16-byte units along m,
//              written into LDS transposed.
// Rows / k-rows are resolved through per-kernel functors, which is how the
// row gathers (token rows via row_src) and the grouped layouts are expressed.
#pragma once

#include "mok_common.h"

namespace mok {

constexpr int kGemmThreads = 256;
constexpr int kBM = 128;
constexpr int kBN = 128;

template <typename T>
struct MfmaT;

template <>
struct MfmaT<bf16_t> {
  static constexpr int BK = 32;   // k per LDS stage
  static constexpr int KI = 16;   // k per MFMA
  static constexpr int KPL = 8;   // k elements per lane per MFMA
  static constexpr int U = 8;     // elements per 16-byte unit
  static constexpr int PITCH = BK + 8;
  typedef bf16x8_t frag_t;
  static __device__ __forceinline__ frag_t read(const bf16_t* p) {
    return *reinterpret_cast<const frag_t*>(p);
  }
  static __device__ __forceinline__ f32x16_t mma(frag_t a, frag_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct MfmaT<float> {
  static constexpr int BK = 16;
  static constexpr int KI = 2;
  static constexpr int KPL = 1;
  static constexpr int U = 4;
  static constexpr int PITCH = BK + 4;
  typedef float frag_t;
  static __device__ __forceinline__ frag_t read(const float* p) { return *p; }
  static __device__ __forceinline__ f32x16_t mma(frag_t a, frag_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

template <typename T>
struct TileSmem {
  static constexpr int A_ELEMS = kBM * MfmaT<T>::PITCH;
  static constexpr int B_ELEMS = kBN * MfmaT<T>::PITCH;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int BYTES = 2 * STAGE * (int)sizeof(T);
};

// Operand with k contiguous.  rowptr(row) gives the start of row `row` of the
// tile (element k = 0 of the whole contraction), or nullptr for a padding row.
template <typename T, int ROWS>
struct KLoader {
  static constexpr int U = MfmaT<T>::U;
  static constexpr int BK = MfmaT<T>::BK;
  static constexpr int UPR = BK / U;                         // units per row
  static constexpr int NU = ROWS * UPR / kGemmThreads;       // units per thread
  const T* ptr[NU];
  int lds_off[NU];

  template <class RowPtr>
  __device__ __forceinline__ void init(RowPtr rowptr) {
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = threadIdx.x + i * kGemmThreads;
      const int row = u / UPR, kc = u % UPR;
      const T* p = rowptr(row);
      ptr[i] = p ? p + kc * U : nullptr;
      lds_off[i] = row * MfmaT<T>::PITCH + kc * U;
    }
  }
  __device__ __forceinline__ void load(int kt, uint4 (&r)[NU]) const {
#pragma unroll
    for (int i = 0; i < NU; ++i) r[i] = ptr[i] ? ld16(ptr[i] + (size_t)kt * BK) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void store(const uint4 (&r)[NU], T* lds) const {
#pragma unroll
    for (int i = 0; i < NU; ++i) st16(lds + lds_off[i], r[i]);
  }
};

// Operand with m contiguous and k strided: element (k, m) = kptr(k)[m].
// kptr(k) returns nullptr for k outside the contraction (zero fill);
// columns m >= ncols are zero.  Written into LDS transposed ([m][k]).
//   bf16: thread t covers k-rows 2*(t%16), 2*(t%16)+1 of column chunk t/16
//         and writes packed k-pairs (one dword per column);
//   fp32: thread t covers k-row t%16 of column chunks t/16 and t/16 + 16.
// Per wave, global loads touch 16 k-rows x 64 contiguous bytes, and the LDS
// writes of each half-wave land in distinct banks.
template <typename T, int COLS>
struct MNLoader;

template <int COLS>
struct MNLoader<bf16_t, COLS> {
  static_assert(COLS == 128, "tile width");
  static constexpr int NU = 2;
  int kp, mc, ncols;
  __device__ __forceinline__ void init(int ncols_) {
    ncols = ncols_;
    kp = threadIdx.x & 15;
    mc = threadIdx.x >> 4;
  }
  template <class KPtr>
  __device__ __forceinline__ void load(int kt, KPtr kptr, uint4 (&r)[NU]) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bf16_t* p = kptr(kt * 32 + 2 * kp + i);
      r[i] = (p && mc * 8 < ncols) ? ld16(p + mc * 8) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(const uint4 (&r)[NU], bf16_t* lds) const {
    const uint32_t a[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
    const uint32_t b[4] = {r[1].x, r[1].y, r[1].z, r[1].w};
    uint32_t* l32 = reinterpret_cast<uint32_t*>(lds);
    constexpr int P2 = MfmaT<bf16_t>::PITCH / 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // column mc*8 + 2q takes the low halves, column mc*8 + 2q + 1 the high halves
      l32[(mc * 8 + 2 * q) * P2 + kp] = (a[q] & 0xFFFFu) | (b[q] << 16);
      l32[(mc * 8 + 2 * q + 1) * P2 + kp] = (a[q] >> 16) | (b[q] & 0xFFFF0000u);
    }
  }
};

template <int COLS>
struct MNLoader<float, COLS> {
  static_assert(COLS == 128, "tile width");
  static constexpr int NU = 2;
  int kr, mc, ncols;
  __device__ __forceinline__ void init(int ncols_) {
    ncols = ncols_;
    kr = threadIdx.x & 15;
    mc = threadIdx.x >> 4;
  }
  template <class KPtr>
  __device__ __forceinline__ void load(int kt, KPtr kptr, uint4 (&r)[NU]) const {
    const float* p = kptr(kt * 16 + kr);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = (mc + 16 * i) * 4;
      r[i] = (p && c < ncols) ? ld16(p + c) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(const uint4 (&r)[NU], float* lds) const {
    constexpr int P = MfmaT<float>::PITCH;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float* v = reinterpret_cast<const float*>(&r[i]);
#pragma unroll
      for (int q = 0; q < 4; ++q) lds[((mc + 16 * i) * 4 + q) * P + kr] = v[q];
    }
  }
};

// Accumulators of one wave: 2 x 2 MFMA blocks.
struct Acc {
  f32x16_t c[2][2];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) c[i][j][v] = 0.0f;
  }
};

// MFMAs over one LDS stage.
template <typename T>
__device__ __forceinline__ void tile_mma(const T* As, const T* Bs, Acc& acc) {
  typedef MfmaT<T> M;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const T* a0 = As + (wm * 64 + (lane & 31)) * M::PITCH + (lane >> 5) * M::KPL;
  const T* b0 = Bs + (wn * 64 + (lane & 31)) * M::PITCH + (lane >> 5) * M::KPL;
#pragma unroll
  for (int kk = 0; kk < M::BK; kk += M::KI) {
    typename M::frag_t fa[2], fb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) fa[i] = M::read(a0 + i * 32 * M::PITCH + kk);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = M::read(b0 + j * 32 * M::PITCH + kk);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc.c[i][j] = M::mma(fa[i], fb[j], acc.c[i][j]);
  }
}

// Row / column of accumulator element v of block (i, j) inside the tile.
__device__ __forceinline__ int acc_row(int i, int v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave >> 1) * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
__device__ __forceinline__ int acc_col(int j) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave & 1) * 64 + j * 32 + (lane & 31);
}

// Main loop over KT stages.  LA / LB are loader objects; loadA(kt, regs) and
// loadB(kt, regs) issue the global loads of stage kt.
template <typename T, class LA, class LB, class FA, class FB>
__device__ __forceinline__ void gemm_mainloop(int KT, LA& la, LB& lb, FA loadA, FB loadB,
                                              T* smem, Acc& acc) {
  typedef TileSmem<T> S;
  uint4 ra[LA::NU], rb[LB::NU];
  acc.zero();
  if (KT <= 0) return;
  loadA(0, ra);
  loadB(0, rb);
  la.store(ra, smem);
  lb.store(rb, smem + S::A_ELEMS);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    T* cur = smem + (kt & 1) * S::STAGE;
    T* nxt = smem + ((kt + 1) & 1) * S::STAGE;
    const bool more = kt + 1 < KT;
    if (more) {
      loadA(kt + 1, ra);
      loadB(kt + 1, rb);
    }
    tile_mma<T>(cur, cur + S::A_ELEMS, acc);
    if (more) {
      la.store(ra, nxt);
      lb.store(rb, nxt + S::A_ELEMS);
    }
    __syncthreads();
  }
}

// Map a flat m-tile index of an M-grouped GEMM (rows of expert e are
// [offsets[e], offsets[e+1]), tiled by kBM) to (expert, first row, end row).
// Uses one wave-wide scan of per-expert tile counts held in LDS.
struct GroupTile {
  int e, r0, r1;
};
__device__ __forceinline__ bool find_group_tile(const int32_t* offsets, int E_local, int R_cap,
                                                int mtile, int* s_prefix, GroupTile* out) {
  // s_prefix: LDS [257]; computed by wave 0.
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int loc[4];
    int run = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      int c = 0;
      if (e < E_local) {
        int lo = offsets[e], hi = offsets[e + 1];
        if (lo > R_cap) lo = R_cap;
        if (hi > R_cap) hi = R_cap;
        c = hi > lo ? (hi - lo + kBM - 1) / kBM : 0;
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
      const int e = lane * 4 + q;
      if (e <= 256) s_prefix[e] = excl;
      excl += loc[q];
    }
    if (lane == 63) s_prefix[256] = incl;
  }
  __syncthreads();
  const int total = s_prefix[E_local < 256 ? E_local : 256];
  if (mtile >= total) return false;
  // largest e with prefix[e] <= mtile (among experts with tiles)
  int lo = 0, hi = E_local - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_prefix[mid] <= mtile)
      lo = mid;
    else
      hi = mid - 1;
  }
  out->e = lo;
  int base = offsets[lo];
  int end = offsets[lo + 1];
  if (end > R_cap) end = R_cap;
  out->r0 = base + (mtile - s_prefix[lo]) * kBM;
  out->r1 = out->r0 + kBM < end ? out->r0 + kBM : end;
  return true;
}

}  // namespace mok
