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
  __device__ __forceinline__ void load(const char* As, const char* Bs, int t) {
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    typedef KMajor<BM, MxCfg::BK> LA;
    typedef KMajor<MxCfg::BN, MxCfg::BK> LB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r0 = wm * 128 + i * 32;
      a[i] = join(LA::frag(As, r0, 2 * t), LA::frag(As, r0, 2 * t + 1));
    }
#pragma unroll
    for (int j = 0; j < MxCfg::WNB; ++j) {
      const int n0 = wn * (MxCfg::BN / 2) + j * 32;
      b[j] = join(LB::frag(Bs, n0, 2 * t), LB::frag(Bs, n0, 2 * t + 1));
    }
  }
};

// MFMAs of 64-k step T (opsel picks scale byte 2T); transposed blocks as in
// the bf16 engine (B in the instruction's first operand).
template <int T>
__device__ __forceinline__ void mx_step(const MxFrags& f, const int* sa, const int* sb,
                                        Acc<MxCfg>& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < MxCfg::WNB; ++j)
      acc.c[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          f.b[j], f.a[i], acc.c[i][j], 0, 0, 2 * T, sb[j], 2 * T, sa[i]);
}

// One landed stage: codes A | codes B | scales A | scales B.
__device__ __forceinline__ void mx_stage_mma(const char* st, Acc<MxCfg>& acc) {
  const char* As = st;
  const char* Bs = st + MxCfg::A_BYTES;
  const char* Asc = Bs + MxCfg::B_BYTES;
  const char* Bsc = Asc + MxCfg::AS_BYTES;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int sh = 8 * (lane >> 5);
  int sa[4], sb[MxCfg::WNB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    sa[i] = (int)(ScaleRows<BM>::get(Asc, wm * 128 + i * 32 + (lane & 31)) >> sh);
#pragma unroll
  for (int j = 0; j < MxCfg::WNB; ++j)
    sb[j] = (int)(ScaleRows<MxCfg::BN>::get(Bsc, wn * (MxCfg::BN / 2) + j * 32 + (lane & 31)) >> sh);
  MxFrags f0, f1;
  f0.load(As, Bs, 0);
  f1.load(As, Bs, 1);
  mx_step<0>(f0, sa, sb, acc);
  mx_step<1>(f1, sa, sb, acc);
  __builtin_amdgcn_iglp_opt(0);
}

// Main loop over K / 128 stages.  la/lb: code loaders (KMajor over 128-byte
// rows), sa/sb: scale loaders.
template <class LA, class LB, class SA, class SB>
__device__ __forceinline__ void mx_mainloop(int KT, const LA& la, const LB& lb, const SA& sa,
                                            const SB& sb, char* smem, Acc<MxCfg>& acc) {
  acc.zero();
  pipeline<MxCfg>(
      KT,
      [&](int kt, unsigned st) {
        la.issue(kt, st);
        lb.issue(kt, st + MxCfg::A_BYTES);
        sa.issue(kt, st + MxCfg::A_BYTES + MxCfg::B_BYTES);
        sb.issue(kt, st + MxCfg::A_BYTES + MxCfg::B_BYTES + MxCfg::AS_BYTES);
      },
      [&](const char* cur) { mx_stage_mma(cur, acc); }, smem);
}

}  // namespace g2
}  // namespace mok
