// MXFP8 variant of the pipelined tile engine (gfx950 scaled matrix cores).
//
// Operands are E4M3 codes, K-major, with one E8M0 scale byte per 32 k
// (OCP Microscaling v1.0).  A stage holds 128 k: 128 code bytes per row of
// A (256 rows) and B (BN rows) -- the same 16-byte chunk layout and swizzle
// as a 64-wide bf16 stage -- plus the 4 scale bytes of every row, copied to
// LDS with global_load_lds_dword.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3): lane l supplies row l % 32
// of its operand, 32 code bytes: bytes 0..15 are k = 16 (l / 32) + 0..15
// and bytes 16..31 are k = 32 + 16 (l / 32) + 0..15 of the 64-k step.  The
// scale of k-block 0 comes from lane l % 32 and that of k-block 1 from lane
// 32 + l % 32, each from the byte of the lane's scale register that the
// instruction's opsel names.  So a lane's operand for step t of a stage is
// the two bf16-engine fragments 2t and 2t + 1 of its row, and its scale
// register is the row's 4 stage scale bytes shifted right by 8 (l / 32):
// byte 2t then holds the scale of block 2t + l / 32.
#pragma once

#include <type_traits>

#include "mok_gemm2.h"
#include "mok_mx.h"

namespace mok {
namespace g2 {

struct MxCfg {
  static constexpr int BN = 256, NS = 2;
  static constexpr int BK = 64;                // stage width in the bf16 loader's 2-byte units
  static constexpr int KB = 128;               // k (code bytes) per stage
  static constexpr int WNB = BN / 64;
  static constexpr int A_BYTES = BM * KB;
  static constexpr int B_BYTES = BN * KB;
  static constexpr int AS_BYTES = BM * 4;      // 4 scale bytes per row per stage
  static constexpr int BS_BYTES = BN * 4;
  static constexpr int STAGE = A_BYTES + B_BYTES + AS_BYTES + BS_BYTES;
  static constexpr int SMEM = NS * STAGE;
  static constexpr int LOADS = (A_BYTES + B_BYTES) / 1024 / 4 + (AS_BYTES + BS_BYTES) / 256 / 4;
  static_assert(SMEM >= 4 * 32768, "epilogue staging reuses the ring");
};

// Scale rows of a stage: LDS [ROWS] dwords, dword r = scale bytes of k-blocks
// 4kt .. 4kt+3 of tile row r.  rowptr(row) gives the row's scale byte of
// k-block 0, or nullptr for a padding row (reads zeros).
template <int ROWS>
struct ScaleRows {
  static constexpr int NI = ROWS / 64 / 4;     // dword loads per wave per stage
  static_assert(NI >= 1, "rows");
  const char* p[NI];
  int adv[NI];
  template <class RowPtr>
  __device__ __forceinline__ void init(RowPtr rowptr) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int row = 64 * (w * NI + j) + lane;
      const uint8_t* rp = rowptr(row);
      p[j] = rp ? reinterpret_cast<const char*>(rp) : reinterpret_cast<const char*>(g_zero);
      adv[j] = rp ? 4 : 0;
    }
  }
  __device__ __forceinline__ void issue(int kt, unsigned lds) const {
    const unsigned w = wave_id();
#pragma unroll
    for (int j = 0; j < NI; ++j) load_lds4(p[j] + (size_t)kt * adv[j], lds + (w * NI + j) * 256);
  }
  __device__ __forceinline__ static uint32_t get(const char* lds, int row) {
    return *reinterpret_cast<const uint32_t*>(lds + row * 4);
  }
};

struct MxFrags {
  i32x8_t a[4], b[MxCfg::WNB];
  __device__ __forceinline__ static i32x8_t join(bf16x8_t lo, bf16x8_t hi) {
    i32x4_t l, h;
    __builtin_memcpy(&l, &lo, 16);
    __builtin_memcpy(&h, &hi, 16);
    i32x8_t o;
    o[0] = l[0]; o[1] = l[1]; o[2] = l[2]; o[3] = l[3];
    o[4] = h[0]; o[5] = h[1]; o[6] = h[2]; o[7] = h[3];
    return o;
  }
  // Fragments of 64-k step t, in the order the step's first MFMAs use them
  // (A block 0, every B block, then A blocks 1..3).
  __device__ __forceinline__ void load(const char* As, const char* Bs, int t) {
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    typedef KMajor<BM, MxCfg::BK> LA;
    typedef KMajor<MxCfg::BN, MxCfg::BK> LB;
    a[0] = join(LA::frag(As, wm * 128, 2 * t), LA::frag(As, wm * 128, 2 * t + 1));
#pragma unroll
    for (int j = 0; j < MxCfg::WNB; ++j) {
      const int n0 = wn * (MxCfg::BN / 2) + j * 32;
      b[j] = join(LB::frag(Bs, n0, 2 * t), LB::frag(Bs, n0, 2 * t + 1));
    }
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      const int r0 = wm * 128 + i * 32;
      a[i] = join(LA::frag(As, r0, 2 * t), LA::frag(As, r0, 2 * t + 1));
    }
  }
};

// MFMAs of 64-k step T (opsel picks scale byte 2T) for row blocks [I0, I1)
// of the wave tile; transposed blocks as in the bf16 engine (B in the
// instruction's first operand).
template <int T, int I0, int I1>
__device__ __forceinline__ void mx_rows(const MxFrags& f, const int* sa, const int* sb,
                                        Acc<MxCfg>& acc) {
#pragma unroll
  for (int i = I0; i < I1; ++i)
#pragma unroll
    for (int j = 0; j < MxCfg::WNB; ++j)
      acc.c[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          f.b[j], f.a[i], acc.c[i][j], 0, 0, 2 * T, sb[j], 2 * T, sa[i]);
}

// The scale words of a landed stage (codes A | codes B | scales A | scales B)
// that this lane's MFMAs use: row scale bytes shifted so that byte 2t holds
// the scale of k-block 2t + lane / 32.
__device__ __forceinline__ void mx_scales(const char* st, int* sa, int* sb) {
  const char* Asc = st + MxCfg::A_BYTES + MxCfg::B_BYTES;
  const char* Bsc = Asc + MxCfg::AS_BYTES;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int sh = 8 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    sa[i] = (int)(ScaleRows<BM>::get(Asc, wm * 128 + i * 32 + (lane & 31)) >> sh);
#pragma unroll
  for (int j = 0; j < MxCfg::WNB; ++j)
    sb[j] = (int)(ScaleRows<MxCfg::BN>::get(Bsc, wn * (MxCfg::BN / 2) + j * 32 + (lane & 31)) >> sh);
}

// Main loop over K / 128 stages, pipelined across stages like the bf16
// engine's: step 1's fragments are read between step 0's MFMAs; the
// hand-over to stage kt+1 (this wave's loads of kt+1 landed and its reads of
// kt done, then the workgroup barrier) comes before step 1, whose MFMAs then
// cover the loads of stage kt+2 into the freed slot and the reads of stage
// kt+1's scale words and step-0 fragments.  la/lb: code loaders (KMajor over
// 128-byte rows), sa/sb: scale loaders.  The accumulation order (64-k steps
// ascending) is that of a stage-at-a-time loop.
template <class LA, class LB, class SA, class SB>
__device__ __forceinline__ void mx_mainloop(int KT, const LA& la, const LB& lb, const SA& sa,
                                            const SB& sb, char* smem, Acc<MxCfg>& acc) {
  typedef MxCfg C;
  constexpr int NS = C::NS;
  acc.zero();
  if (KT <= 0) return;
  const unsigned lds0 = lds_addr_of(smem);
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < KT) {
      const unsigned st = lds0 + s * C::STAGE;
      la.issue(s, st);
      lb.issue(s, st + C::A_BYTES);
      sa.issue(s, st + C::A_BYTES + C::B_BYTES);
      sb.issue(s, st + C::A_BYTES + C::B_BYTES + C::AS_BYTES);
    }
  wait_stages_lgkm0<C::LOADS, NS - 1>(min(KT, NS) - 1);  // stage 0 landed
  __builtin_amdgcn_s_barrier();
  MxFrags f0, f1;
  int sca[4], scb[C::WNB];
  mx_scales(smem, sca, scb);
  f0.load(smem, smem + C::A_BYTES, 0);
  // One stage.  LOADS: issue the loads of stage kt + NS into the freed slot.
  // The stages with loads and the last NS stages without run as two loops,
  // so neither body branches: a branch around the loads would let the
  // compiler sink step 0's MFMAs below the hand-over.  (After the last
  // stage the hand-over reads a slot that holds no stage; harmless.)
  typedef KMajor<BM, C::BK> LdA;
  typedef KMajor<C::BN, C::BK> LdB;
  static_assert(LA::NI == 8 && LB::NI == 8, "eight code loads per operand per wave");
  auto stage = [&](int kt, auto loads) {
    constexpr bool L = decltype(loads)::value;
    const char* cur = smem + (kt % NS) * C::STAGE;
    f1.load(cur, cur + C::A_BYTES, 1);
    mx_rows<0, 0, 4>(f0, sca, scb, acc);
    interleave_reads<4 * C::WNB, 8 + 2 * C::WNB>();
    __builtin_amdgcn_sched_barrier(0);
    wait_stages_lgkm0<C::LOADS, NS - 2>(min(KT - 1, kt + NS - 1) - (kt + 1));
    __builtin_amdgcn_s_barrier();
    const unsigned slot = lds0 + (kt % NS) * C::STAGE;
    const char* nxt = smem + ((kt + 1) % NS) * C::STAGE;
    const char* nA = nxt;
    const char* nB = nxt + C::A_BYTES;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    auto rdA = [&](int i) {
      f0.a[i] = MxFrags::join(LdA::frag(nA, wm * 128 + i * 32, 0), LdA::frag(nA, wm * 128 + i * 32, 1));
    };
    auto rdB = [&](int j) {
      const int n0 = wn * (C::BN / 2) + j * 32;
      f0.b[j] = MxFrags::join(LdB::frag(nB, n0, 0), LdB::frag(nB, n0, 1));
    };
    int nsa[4], nsb[C::WNB];
    // Step 1's MFMAs, one row block (4 MFMAs) per region, with the loads of
    // stage kt + NS and the reads of stage kt + 1 spread over them: a wave
    // that issued all its loads at once would stall on the memory pipeline
    // with its matrix work queued behind them.
    if constexpr (L) la.template issue_range<0, 4>(kt + NS, slot);
    mx_scales(nxt, nsa, nsb);
    rdA(0);
    rdB(0);
    rdB(1);
    mx_rows<1, 0, 1>(f1, sca, scb, acc);
    interleave_reads<4, 11, 0, 3>();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (L) la.template issue_range<4, 8>(kt + NS, slot);
    rdB(2);
    rdB(3);
    rdA(1);
    rdA(2);
    mx_rows<1, 1, 2>(f1, sca, scb, acc);
    interleave_reads<4, 8>();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (L) lb.template issue_range<0, 4>(kt + NS, slot + C::A_BYTES);
    rdA(3);
    mx_rows<1, 2, 3>(f1, sca, scb, acc);
    interleave_reads<4, 2>();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (L) {
      lb.template issue_range<4, 8>(kt + NS, slot + C::A_BYTES);
      sa.issue(kt + NS, slot + C::A_BYTES + C::B_BYTES);
      sb.issue(kt + NS, slot + C::A_BYTES + C::B_BYTES + C::AS_BYTES);
    }
    mx_rows<1, 3, 4>(f1, sca, scb, acc);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) sca[i] = nsa[i];
#pragma unroll
    for (int j = 0; j < C::WNB; ++j) scb[j] = nsb[j];
  };
  int kt = 0;
  for (; kt + NS < KT; ++kt) stage(kt, std::true_type());
  for (; kt < KT; ++kt) stage(kt, std::false_type());
}

}  // namespace g2
}  // namespace mok
