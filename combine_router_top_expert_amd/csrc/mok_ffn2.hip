// Forward expert FFN, bf16, on the pipelined 256 x 256 tile engine.
//
// GEMM1 + SwiGLU: a = x W_gate[e]^T, b = x W_up[e]^T, h = silu(a) * b.  A
// B-tile of 256 weight rows holds 128 columns i of both matrices as
// alternating 32-row blocks (gate, up, gate, up, ...), so the gate and up
// accumulators of the same (row, i) live in the same lane.  The A operand
// is either the gathered rows x_perm or -- in the layer's forward pass --
// the token rows themselves, read from the source buffers through row_src:
// the pull dispatch is then part of the GEMM's own loads (kucoin article,
// section 02: the receiver reads the tokens it needs from their sources and
// places them expert by expert).
// GEMM2: y = h W_down[e]^T, pushed straight to the (source, token, slot)
// staging rows or stored in expert order.
// MXFP8 (E4M3 codes with one E8M0 scale per 32 along k, the contraction
// dimension): the same tiles on the scaled matrix cores; GEMM1's epilogue
// quantises h along I in blocks of 32 before it is stored (kucoin article,
// section 02: MXFP8 conversion is fused into the kernels rather than run as
// separate passes).
#include <string.h>

#include "mok_gemm2.h"
#include "mok_gemm_mx.h"
#include "mok_internal.h"

namespace mok {

namespace {

using namespace g2;

struct F1Args {
  const bf16_t* x;     // [R_cap, d] gathered rows, or null when gathering from src
  SrcTable src;        // source buffers (used when x == null)
  const int32_t* row_src;
  const bf16_t* wg;    // [E_local, I, d]
  const bf16_t* wu;
  const int32_t* offsets;
  bf16_t* h;           // [R_cap, I]
  bf16_t* ab;          // [R_cap, 2I] or null
  int d, I, E_local, R_cap, ntn, T_src, k;
};

template <class C>
__global__ __launch_bounds__(kThreads) void ffn1_g2(F1Args a) {
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int s_prefix[257];
  const int total_m = group_prefix(a.offsets, a.E_local, a.R_cap, s_prefix);
  const int total = total_m * a.ntn;
  if ((int)blockIdx.x >= total) return;
  const int t = xcd_tile(blockIdx.x, total);
  const int mtile = t / a.ntn, nt = t % a.ntn;
  const GTile g = group_tile(a.offsets, a.E_local, a.R_cap, s_prefix, mtile);
  const bf16_t* wg = a.wg + (size_t)g.e * a.I * a.d;
  const bf16_t* wu = a.wu + (size_t)g.e * a.I * a.d;
  KMajor<BM, C::BK> la;
  KMajor<C::BN, C::BK> lb;
  la.init([&](int row) -> const bf16_t* {
    const int r = g.r0 + row;
    if (r >= g.r1) return nullptr;
    if (a.x) return a.x + (size_t)r * a.d;
    const int tok = a.row_src[r] / a.k;
    return reinterpret_cast<const bf16_t*>(a.src.p[tok / a.T_src]) + (size_t)(tok % a.T_src) * a.d;
  });
  lb.init([&](int nr) -> const bf16_t* {
    const int blk = nr >> 5;
    const int i = nt * (C::BN / 2) + (blk >> 1) * 32 + (nr & 31);
    if (i >= a.I) return nullptr;
    return ((blk & 1) ? wu : wg) + (size_t)i * a.d;
  });
  Acc<C> acc;
  mainloop<C, false, false>(a.d / C::BK, [&](int kt, unsigned l) { la.issue(kt, l); },
                            [&](int kt, unsigned l) { lb.issue(kt, l); }, smem, acc);
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

struct F2Args {
  const bf16_t* h;     // [R_cap, I] (MX: E4M3 codes)
  const bf16_t* wd;    // [E_local, d, I] (MX: E4M3 codes)
  const uint8_t* hs;   // MX: [R_cap, I/32] scales of h
  const uint8_t* sd;   // MX: [E_local, d, I/32] scales of W_down
  const int32_t* offsets;
  const int32_t* row_src;
  bf16_t* y;           // [R_cap, d] when not pushing
  DstTable staging;
  int push;
  int d, I, E_local, R_cap, ntn, T_src, k;
};

// y tile -> bf16, staged through LDS, then whole 16-byte row chunks pushed to
// the staging row of each routed row (or stored at its expert-order row).
template <class C, class AccT>
__device__ __forceinline__ void ffn2_store(const AccT& acc, char* smem, const GTile& g, int nt,
                                           const F2Args& a) {
  __syncthreads();
  const WaveStage<C, bf16_t> st(smem);
  st.put(acc, 0);
  wave_lds_fence();
  const int wave = threadIdx.x >> 6;
  st.for_chunks(0, [&](int trow, int srow, int c) {
    const int r = g.r0 + (wave >> 1) * 128 + trow;
    const int col = nt * C::BN + (wave & 1) * (C::BN / 2) + c * 8;
    if (r >= g.r1 || col >= a.d) return;
    bf16_t* dst;
    if (a.push) {
      const int n = a.row_src[r];
      const int tok = n / a.k, j = n % a.k;
      dst = reinterpret_cast<bf16_t*>(a.staging.p[tok / a.T_src]) +
            ((size_t)(tok % a.T_src) * a.k + j) * a.d;
    } else {
      dst = a.y + (size_t)r * a.d;
    }
    *reinterpret_cast<uint4*>(dst + col) = st.raw(srow, c);
  });
}

template <class C>
__global__ __launch_bounds__(kThreads) void ffn2_g2(F2Args a) {
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int s_prefix[257];
  const int total_m = group_prefix(a.offsets, a.E_local, a.R_cap, s_prefix);
  const int total = total_m * a.ntn;
  if ((int)blockIdx.x >= total) return;
  const int t = xcd_tile(blockIdx.x, total);
  const int mtile = t / a.ntn, nt = t % a.ntn;
  const GTile g = group_tile(a.offsets, a.E_local, a.R_cap, s_prefix, mtile);
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
  mainloop<C, false, false>(a.I / C::BK, [&](int kt, unsigned l) { la.issue(kt, l); },
                            [&](int kt, unsigned l) { lb.issue(kt, l); }, smem, acc);
  ffn2_store<C>(acc, smem, g, nt, a);
}

// ---------------------------------------------------------------- MXFP8
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
  int d, I, E_local, R_cap, ntn;
};

__global__ __launch_bounds__(kThreads) void ffn1_mx(F1MxArgs a) {
  typedef MxCfg C;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int s_prefix[257];
  const int total_m = group_prefix(a.offsets, a.E_local, a.R_cap, s_prefix);
  const int total = total_m * a.ntn;
  if ((int)blockIdx.x >= total) return;
  const int t = xcd_tile(blockIdx.x, total);
  const int mtile = t / a.ntn, nt = t % a.ntn;
  const GTile g = group_tile(a.offsets, a.E_local, a.R_cap, s_prefix, mtile);
  const size_t wofs = (size_t)g.e * a.I * a.d;
  const int KS = a.d / 32;  // scale bytes per row
  KMajor<BM, C::BK> la;
  KMajor<C::BN, C::BK> lb;
  ScaleRows<BM> sa;
  ScaleRows<C::BN> sb;
  la.init([&](int row) -> const bf16_t* {
    const int r = g.r0 + row;
    return r < g.r1 ? reinterpret_cast<const bf16_t*>(a.xq + (size_t)r * a.d) : nullptr;
  });
  sa.init([&](int row) -> const uint8_t* {
    const int r = g.r0 + row;
    return r < g.r1 ? a.xs + (size_t)r * KS : nullptr;
  });
  // B rows: 32-row blocks alternating gate, up (as in the bf16 kernel)
  auto wrow = [&](int nr, int* i_out) {
    const int blk = nr >> 5;
    *i_out = nt * (C::BN / 2) + (blk >> 1) * 32 + (nr & 31);
    return blk & 1;
  };
  lb.init([&](int nr) -> const bf16_t* {
    int i;
    const int up = wrow(nr, &i);
    if (i >= a.I) return nullptr;
    return reinterpret_cast<const bf16_t*>((up ? a.wu : a.wg) + wofs + (size_t)i * a.d);
  });
  sb.init([&](int nr) -> const uint8_t* {
    int i;
    const int up = wrow(nr, &i);
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
      }
      float amax = fmaxf(fmaxf(fabsf(hv[0]), fabsf(hv[1])), fmaxf(fabsf(hv[2]), fabsf(hv[3])));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
      if (ok) {
        const int sh = mx_shared_exp(amax);
        uint32_t code = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) code |= e4m3_code(__builtin_amdgcn_ldexpf(hv[e], -sh)) << (8 * e);
        *reinterpret_cast<uint32_t*>(a.hq + (size_t)r * a.I + i) = code;
        if (within == 0) a.hs[(size_t)r * (a.I / 32) + i / 32] = (uint8_t)(sh + 127);
      }
    }
    wave_lds_fence();
  }
}

__global__ __launch_bounds__(kThreads) void ffn2_mx(F2Args a) {
  typedef MxCfg C;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int s_prefix[257];
  const int total_m = group_prefix(a.offsets, a.E_local, a.R_cap, s_prefix);
  const int total = total_m * a.ntn;
  if ((int)blockIdx.x >= total) return;
  const int t = xcd_tile(blockIdx.x, total);
  const int mtile = t / a.ntn, nt = t % a.ntn;
  const GTile g = group_tile(a.offsets, a.E_local, a.R_cap, s_prefix, mtile);
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
  ffn2_store<C>(acc, smem, g, nt, a);
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
  a1.x = reinterpret_cast<const bf16_t*>(x);
  if (src) a1.src = *src;
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
  hipLaunchKernelGGL(ffn1_g2<Default>, dim3((unsigned)(mt * a1.ntn)), dim3(kThreads), 0, stream, a1);
  trace_mark(tr, "ffn1_gate_up_swiglu", stream);
  F2Args a2;
  memset(&a2, 0, sizeof(a2));
  a2.h = reinterpret_cast<const bf16_t*>(h);
  a2.wd = reinterpret_cast<const bf16_t*>(wd);
  a2.offsets = offsets;
  a2.row_src = row_src;
  a2.y = reinterpret_cast<bf16_t*>(y);
  a2.push = staging != nullptr;
  if (staging) a2.staging = *staging;
  a2.d = d;
  a2.I = I;
  a2.E_local = E_local;
  a2.R_cap = R_cap;
  a2.ntn = (d + Default::BN - 1) / Default::BN;
  a2.T_src = T_src;
  a2.k = k;
  hipLaunchKernelGGL(ffn2_g2<Default>, dim3((unsigned)(mt * a2.ntn)), dim3(kThreads), 0, stream, a2);
  trace_mark(tr, "ffn2_down", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

}  // namespace mok

namespace mok {

mok_status launch_ffn_mx(int d, int I, int E_local, int R_cap, const uint8_t* xq,
                         const uint8_t* xs, const int32_t* offsets, const int32_t* row_src,
                         const mok_expert_weights* w, uint8_t* hq, uint8_t* hs, void* ab, void* y,
                         const DstTable* staging, int T_src, int k, hipStream_t stream,
                         mok_trace* tr) {
  (void)ab;  // the MXFP8 layer keeps no pre-activations (it has no backward pass)
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
  if (staging) a2.staging = *staging;
  a2.d = d;
  a2.I = I;
  a2.E_local = E_local;
  a2.R_cap = R_cap;
  a2.ntn = (d + MxCfg::BN - 1) / MxCfg::BN;
  a2.T_src = T_src;
  a2.k = k;
  hipLaunchKernelGGL(ffn2_mx, dim3((unsigned)(mt * a2.ntn)), dim3(kThreads), 0, stream, a2);
  trace_mark(tr, "ffn2_down_mx", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

}  // namespace mok
