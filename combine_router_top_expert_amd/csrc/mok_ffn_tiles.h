// One output tile of each forward expert GEMM, as device functions shared by
// the one-launch-per-GEMM kernels and the persistent ring kernel (which must
// give bit-identical results: the same tile code runs in both).
//
// GEMM1 + SwiGLU: a = x W_gate[e]^T, b = x W_up[e]^T, h = silu(a) * b.  A
// B-tile of 256 weight rows holds 128 columns i of both matrices as
// alternating 32-row blocks (gate, up, gate, up, ...), so the gate and up
// accumulators of the same (row, i) live in the same lane.
// GEMM2: y = h W_down[e]^T, pushed straight to the (source, token, slot)
// staging rows or stored in expert order.
// MXFP8 (E4M3 codes with one E8M0 scale per 32 along k, the contraction
// dimension): the same tiles on the scaled matrix cores; GEMM1's epilogue
// quantises h along I in blocks of 32 before it is stored (kucoin article,
// section 02: MXFP8 conversion is fused into the kernels rather than run as
// separate passes).
#pragma once

#include "mok_gemm2.h"
#include "mok_gemm_mx.h"

namespace mok {
namespace g2 {

// Argument blocks of the tiles: pointers and sizes only.  The per-source
// pointer tables (source buffers, staging buffers) travel separately: in the
// kernel arguments of the one-launch-per-GEMM kernels, in device memory for
// the ring kernel's calls.
struct F1Args {
  const bf16_t* x;     // [R_cap, d] gathered rows, or null when gathering from the sources
  const int32_t* row_src;
  const bf16_t* wg;    // [E_local, I, d]
  const bf16_t* wu;
  const int32_t* offsets;
  bf16_t* h;           // [R_cap, I]
  bf16_t* ab;          // [R_cap, 2I] or null
  int d, I, E_local, R_cap, ntn, T_src, k;
};

struct F2Args {
  const bf16_t* h;     // [R_cap, I] (MX: E4M3 codes)
  const bf16_t* wd;    // [E_local, d, I] (MX: E4M3 codes)
  const uint8_t* hs;   // MX: [R_cap, I/32] scales of h
  const uint8_t* sd;   // MX: [E_local, d, I/32] scales of W_down
  const int32_t* offsets;
  const int32_t* row_src;
  bf16_t* y;           // [R_cap, d] when not pushing (row stride ldy, 0 = d)
  int ldy;
  int push;            // 1: push each row to its staging row (table given to the tile)
  int d, I, E_local, R_cap, ntn, T_src, k;
};

struct F1MxArgs {
  const uint8_t* xq;   // [R_cap, d] E4M3 codes of the gathered rows
  const uint8_t* xs;   // [R_cap, d/32]
  const uint8_t* wg;   // [E_local, I, d] codes
  const uint8_t* wu;
  const uint8_t* sg;   // [E_local, I, d/32] scales
  const uint8_t* su;
  const int32_t* offsets;
  uint8_t* hq;         // [R_cap, I] codes of h
  uint8_t* hs;         // [R_cap, I/32] scales of h
  bf16_t* ab;          // [R_cap, 2I] a | b kept for the backward pass, or null
  int d, I, E_local, R_cap, ntn;
};

// B-tile row nr of GEMM1 (32-row blocks alternating gate, up): weight row i
// and whether it is an up row.
template <int BN>
__device__ __forceinline__ int gu_row(int nt, int nr, int* i_out) {
  const int blk = nr >> 5;
  *i_out = nt * (BN / 2) + (blk >> 1) * 32 + (nr & 31);
  return blk & 1;
}

// ---------------------------------------------------------------- bf16
// GEMM1 tile (rows [g.r0, g.r1) of expert g.e, weight columns of N-tile nt).
// arow(row) gives the x row of tile row `row` (0..255), or nullptr past g.r1.
template <class C, class ARow>
__device__ __forceinline__ void ffn1_tile(const F1Args& a, char* smem, const GTile& g, int nt,
                                          ARow arow) {
  const bf16_t* wg = a.wg + (size_t)g.e * a.I * a.d;
  const bf16_t* wu = a.wu + (size_t)g.e * a.I * a.d;
  KMajor<BM, C::BK> la;
  KMajor<C::BN, C::BK> lb;
  la.init(arow);
  lb.init([&](int nr) -> const bf16_t* {
    int i;
    const int up = gu_row<C::BN>(nt, nr, &i);
    if (i >= a.I) return nullptr;
    return (up ? wu : wg) + (size_t)i * a.d;
  });
  Acc<C> acc;
  mainloop<C, false, false>(a.d / C::BK, [&](int kt, unsigned l, auto pt) { la.issue(kt, l, pt); },
                            [&](int kt, unsigned l, auto pt) { lb.issue(kt, l, pt); }, smem, acc);
  // Wave column wn holds B-tile columns [wn*BN/2, (wn+1)*BN/2): 32-wide blocks
  // alternating gate, up, so i = nt*BN/2 + wn*BN/4 + 32*(block/2) + (col % 32).
  // Staged as fp32 so that h is formed from the unrounded a and b.
  __syncthreads();
  const WaveStage<C, float> st(smem);
  const int wave = threadIdx.x >> 6, wn = wave & 1;
  const int ib = nt * (C::BN / 2) + wn * (C::BN / 4);
#pragma unroll
  for (int pass = 0; pass < WaveStage<C, float>::PASSES; ++pass) {
    st.put(acc, pass);
    wave_lds_fence();
    // one lane per 4 gate columns (chunk in a gate block) and its up partner
    const int lane = threadIdx.x & 63;
    constexpr int GC = C::BN / 16;                // gate chunks per wave row
    constexpr int RPI = 64 / GC;                  // rows per instruction
#pragma unroll 2
    for (int r0 = 0; r0 < WaveStage<C, float>::ROWS; r0 += RPI) {
      const int srow = r0 + lane / GC;
      const int trow = pass * WaveStage<C, float>::ROWS + srow;
      const int gc = lane % GC;                   // gate chunk index
      const int blkpair = gc / 8, within = gc % 8;
      const int cg = blkpair * 16 + within;       // chunk of the gate block (8 chunks of 4 columns)
      const int cu = cg + 8;                      // chunk of the up block
      const int r = g.r0 + (wave >> 1) * 128 + trow;
      const int i = ib + blkpair * 32 + within * 4;
      if (r < g.r1 && i < a.I) {
        float av[4], bv[4], hv[4];
        st.get(srow, cg, av);
        st.get(srow, cu, bv);
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = silu_f(av[e]) * bv[e];
        *reinterpret_cast<uint2*>(a.h + (size_t)r * a.I + i) = pack4_bf16(hv[0], hv[1], hv[2], hv[3]);
        if (a.ab) {
          bf16_t* abr = a.ab + (size_t)r * 2 * a.I;
          *reinterpret_cast<uint2*>(abr + i) = pack4_bf16(av[0], av[1], av[2], av[3]);
          *reinterpret_cast<uint2*>(abr + a.I + i) = pack4_bf16(bv[0], bv[1], bv[2], bv[3]);
        }
      }
    }
    wave_lds_fence();
  }
}

// y tile -> bf16, staged through LDS, then whole 16-byte row chunks pushed to
// the staging row of each routed row (or stored at its expert-order row).
template <class C, class AccT>
__device__ __forceinline__ void ffn2_store(const AccT& acc, char* smem, const GTile& g, int nt,
                                           const F2Args& a, const DstTable& staging) {
  __shared__ bf16_t* s_dst[BM];
  if (a.push) stage_dst_rows(s_dst, a.row_src, g, staging, a.k, a.T_src, a.d);
  __syncthreads();
  const WaveStage<C, bf16_t> st(smem);
  static_assert(WaveStage<C, bf16_t>::PASSES == 1, "one staging pass");
  st.put(acc, 0);
  wave_lds_fence();
  const int wave = threadIdx.x >> 6;
  st.for_chunks(0, [&](int trow, int srow, int c) {
    const int r = g.r0 + (wave >> 1) * 128 + trow;
    const int col = nt * C::BN + (wave & 1) * (C::BN / 2) + c * 8;
    if (r >= g.r1 || col >= a.d) return;
    bf16_t* dst;
    if (a.push) {
      dst = s_dst[r - g.r0];
    } else {
      dst = a.y + (size_t)r * (a.ldy ? a.ldy : a.d);
    }
    *reinterpret_cast<uint4*>(dst + col) = st.raw(srow, c);
  });
}

// GEMM2 tile: y rows [g.r0, g.r1) x columns of N-tile nt, from h.
template <class C>
__device__ __forceinline__ void ffn2_tile(const F2Args& a, const DstTable& staging, char* smem,
                                          const GTile& g, int nt) {
  const bf16_t* wd = a.wd + (size_t)g.e * a.d * a.I;
  KMajor<BM, C::BK> la;
  KMajor<C::BN, C::BK> lb;
  la.init([&](int row) -> const bf16_t* {
    const int r = g.r0 + row;
    return r < g.r1 ? a.h + (size_t)r * a.I : nullptr;
  });
  lb.init([&](int nr) -> const bf16_t* {
    const int c = nt * C::BN + nr;
    return c < a.d ? wd + (size_t)c * a.I : nullptr;
  });
  Acc<C> acc;
  mainloop<C, false, false>(a.I / C::BK, [&](int kt, unsigned l, auto pt) { la.issue(kt, l, pt); },
                            [&](int kt, unsigned l, auto pt) { lb.issue(kt, l, pt); }, smem, acc);
  ffn2_store<C>(acc, smem, g, nt, a, staging);
}

// ---------------------------------------------------------------- MXFP8
// GEMM1 tile on E4M3 codes.  arow(row) / ascale(row): the code row and the
// scale row (k-block 0) of tile row `row`, or nullptr past g.r1.
template <class ARow, class AScale>
__device__ __forceinline__ void ffn1_mx_tile(const F1MxArgs& a, char* smem, const GTile& g,
                                             int nt, ARow arow, AScale ascale) {
  typedef MxCfg C;
  const size_t wofs = (size_t)g.e * a.I * a.d;
  const int KS = a.d / 32;  // scale bytes per row
  KMajor<BM, C::BK> la;
  KMajor<C::BN, C::BK> lb;
  ScaleRows<BM> sa;
  ScaleRows<C::BN> sb;
  la.init(arow);
  sa.init(ascale);
  lb.init([&](int nr) -> const bf16_t* {
    int i;
    const int up = gu_row<C::BN>(nt, nr, &i);
    if (i >= a.I) return nullptr;
    return reinterpret_cast<const bf16_t*>((up ? a.wu : a.wg) + wofs + (size_t)i * a.d);
  });
  sb.init([&](int nr) -> const uint8_t* {
    int i;
    const int up = gu_row<C::BN>(nt, nr, &i);
    if (i >= a.I) return nullptr;
    return (up ? a.su : a.sg) + (size_t)g.e * a.I * KS + (size_t)i * KS;
  });
  Acc<C> acc;
  mx_mainloop(a.d / C::KB, la, lb, sa, sb, smem, acc);
  // h = silu(a) * b in fp32, then MX-quantised along I: a 32-column block of
  // h is 8 lanes x 4 columns, reduced for its max magnitude by lane shuffles.
  __syncthreads();
  const WaveStage<C, float> st(smem);
  const int wave = threadIdx.x >> 6, wn = wave & 1;
  const int ib = nt * (C::BN / 2) + wn * (C::BN / 4);
  const int lane = threadIdx.x & 63;
  constexpr int GC = C::BN / 16;
  constexpr int RPI = 64 / GC;
#pragma unroll
  for (int pass = 0; pass < WaveStage<C, float>::PASSES; ++pass) {
    st.put(acc, pass);
    wave_lds_fence();
#pragma unroll 2
    for (int r0 = 0; r0 < WaveStage<C, float>::ROWS; r0 += RPI) {
      const int srow = r0 + lane / GC;
      const int trow = pass * WaveStage<C, float>::ROWS + srow;
      const int gc = lane % GC;
      const int blkpair = gc / 8, within = gc % 8;
      const int cg = blkpair * 16 + within;
      const int r = g.r0 + (wave >> 1) * 128 + trow;
      const int i = ib + blkpair * 32 + within * 4;
      const bool ok = r < g.r1 && i < a.I;  // uniform over each 8-lane block (I % 128 == 0)
      float hv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (ok) {
        float av[4], bv[4];
        st.get(srow, cg, av);
        st.get(srow, cg + 8, bv);
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = silu_f(av[e]) * bv[e];
        if (a.ab) {  // a | b for the backward pass, bf16 from the fp32 accumulators
          bf16_t* abr = a.ab + (size_t)r * 2 * a.I;
          *reinterpret_cast<uint2*>(abr + i) = pack4_bf16(av[0], av[1], av[2], av[3]);
          *reinterpret_cast<uint2*>(abr + a.I + i) = pack4_bf16(bv[0], bv[1], bv[2], bv[3]);
        }
      }
      float amax = fmaxf(fmaxf(fabsf(hv[0]), fabsf(hv[1])), fmaxf(fabsf(hv[2]), fabsf(hv[3])));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
      if (ok) {
        const int sh = mx_shared_exp(amax);
        *reinterpret_cast<uint32_t*>(a.hq + (size_t)r * a.I + i) = e4m3_pack4(hv[0], hv[1], hv[2], hv[3], sh);
        if (within == 0) a.hs[(size_t)r * (a.I / 32) + i / 32] = (uint8_t)(sh + 127);
      }
    }
    wave_lds_fence();
  }
}

// GEMM2 tile on E4M3 codes of h and W_down.
__device__ __forceinline__ void ffn2_mx_tile(const F2Args& a, const DstTable& staging, char* smem,
                                             const GTile& g, int nt) {
  typedef MxCfg C;
  const uint8_t* hq = reinterpret_cast<const uint8_t*>(a.h);
  const uint8_t* wd = reinterpret_cast<const uint8_t*>(a.wd) + (size_t)g.e * a.d * a.I;
  const int KS = a.I / 32;
  const uint8_t* sd = a.sd + (size_t)g.e * a.d * KS;
  KMajor<BM, C::BK> la;
  KMajor<C::BN, C::BK> lb;
  ScaleRows<BM> sa;
  ScaleRows<C::BN> sb;
  la.init([&](int row) -> const bf16_t* {
    const int r = g.r0 + row;
    return r < g.r1 ? reinterpret_cast<const bf16_t*>(hq + (size_t)r * a.I) : nullptr;
  });
  sa.init([&](int row) -> const uint8_t* {
    const int r = g.r0 + row;
    return r < g.r1 ? a.hs + (size_t)r * KS : nullptr;
  });
  lb.init([&](int nr) -> const bf16_t* {
    const int c = nt * C::BN + nr;
    return c < a.d ? reinterpret_cast<const bf16_t*>(wd + (size_t)c * a.I) : nullptr;
  });
  sb.init([&](int nr) -> const uint8_t* {
    const int c = nt * C::BN + nr;
    return c < a.d ? sd + (size_t)c * KS : nullptr;
  });
  Acc<C> acc;
  mx_mainloop(a.I / C::KB, la, lb, sa, sb, smem, acc);
  ffn2_store<C>(acc, smem, g, nt, a, staging);
}

}  // namespace g2
}  // namespace mok
