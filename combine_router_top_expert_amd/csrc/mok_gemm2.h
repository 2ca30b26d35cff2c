// Pipelined bf16 tile engine for the expert grouped GEMMs (gfx950).
//
// One workgroup (4 waves, 2 x 2) computes a 256 x BN tile of
// C[m][n] = sum_k A(m, k) B(n, k) in fp32; each wave owns 128 x BN/2 as
// 32 x 32 blocks of v_mfma_f32_32x32x16_bf16.
//
// Operand tiles of BK k are staged through a ring of NS LDS stages.  Global memory is copied straight into LDS by
// global_load_lds_dwordx4 (lane i of an instruction fills bytes 16i..16i+15
// of a 1 KiB block), so no registers hold staged data and three stages are
// in flight while the matrix cores consume the fourth.  Every lane picks the
// global address of the 16 bytes its LDS slot must hold, which is how the
// layouts below are swizzled:
//   K-major operand (k contiguous in memory): LDS [rows][2 BK bytes] with
//     the 16-byte chunks of a row XOR-swizzled by row, so the 16-lane phases
//     of a ds_read_b128 fragment read hit 16 distinct bank groups.
//   MN-major operand (m or n contiguous, k strided): LDS [BK k-rows][2 BN
//     bytes]; chunk c of k-row r sits at c ^ (4 * (r & 3)).  Fragments are
//     read with ds_read_b64_tr_b16: in each 16-lane group lane a points at
//     (k0 + a/4, n0 + 4*(a%4)) and lane i receives k0..k0+3 of column n0 + i,
//     i.e. the k-consecutive fragment the MFMA wants, without a transpose in
//     registers.
// Rows or k-rows outside the problem read a page of zeros, so contraction
// tails contribute nothing and no address leaves its buffer.
#pragma once

#include <type_traits>
#include "mok_common.h"

namespace mok {
namespace g2 {

constexpr int kThreads = 256;
constexpr int BM = 256;

// Zeros read by lanes whose rows, k-rows or columns fall outside a problem.
static __device__ const uint4 g_zero[64] = {};

// Part P of NP of a wave's direct loads of one stage: the main loop spreads a
// stage's loads over the MFMAs of its hand-over instead of issuing them in
// one burst, which would stall the wave on the memory pipeline with its
// matrix work queued behind them.
template <int P, int NP>
struct Part {};

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// One global_load_lds_dwordx4: lane i's 16 bytes from g land at LDS byte
// lds_addr + 16 i.  Issued from inline assembly so that the compiler does not
// treat it as a pending LDS write (it would otherwise wait for every load in
// flight before each LDS read); the main loop orders it explicitly with
// s_waitcnt vmcnt and barriers.  lds_addr must be wave-uniform.
__device__ __forceinline__ void load_lds16(const void* g, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_addr)
               : "memory", "m0");
}

// One global_load_lds_dword: lane i's 4 bytes from g land at lds_addr + 4 i.
__device__ __forceinline__ void load_lds4(const void* g, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(lds_addr)
               : "memory", "m0");
}

// LDS byte address of a __shared__ location, made wave-uniform.
__device__ __forceinline__ unsigned lds_addr_of(const char* p) {
  return __builtin_amdgcn_readfirstlane((unsigned)(size_t)(__attribute__((address_space(3))) const char*)p);
}

__device__ __forceinline__ unsigned wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// s_waitcnt on vmcnt only (expcnt, lgkmcnt at their maxima = no wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// ---------------------------------------------------------------- operands
// K-major operand tile: ROWS rows x BK k (k contiguous in memory).  LDS
// [ROWS][2*BK bytes]; 16-byte chunk c of row r sits at c ^ ((r / RS) % CPR)
// (CPR chunks per row, RS = 16 / CPR), which puts the 16 lanes of each
// ds_read_b128 phase into 16 distinct bank groups.  rowptr(row) returns the
// address of element k = 0 of the row, or nullptr for a padding row.
template <int ROWS, int BK>
struct KMajor {
  static constexpr int CPR = BK / 8;            // chunks per row
  static constexpr int RPI = 1024 / (2 * BK);   // rows per 1 KiB load
  static constexpr int NI = ROWS / RPI / 4;     // loads per wave per stage
  static constexpr int RS = 16 / CPR;
  static constexpr int BYTES = ROWS * BK * 2;
  const char* p[NI];
  int adv[NI];
  template <class RowPtr>
  __device__ __forceinline__ void init(RowPtr rowptr) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int I = w * NI + j;
      const int row = RPI * I + lane / CPR;
      const int c = (lane % CPR) ^ ((row / RS) % CPR);
      const bf16_t* rp = rowptr(row);
      if (rp) {
        p[j] = reinterpret_cast<const char*>(rp) + c * 16;
        adv[j] = BK * 2;
      } else {
        p[j] = reinterpret_cast<const char*>(g_zero);
        adv[j] = 0;
      }
    }
  }
  __device__ __forceinline__ void issue(int kt, unsigned lds_op) const { issue_range<0, NI>(kt, lds_op); }
  template <int P, int NP>
  __device__ __forceinline__ void issue(int kt, unsigned lds_op, Part<P, NP>) const {
    issue_range<P * NI / NP, (P + 1) * NI / NP>(kt, lds_op);
  }
  // loads [J0, J1) of this wave's NI loads of stage kt
  template <int J0, int J1>
  __device__ __forceinline__ void issue_range(int kt, unsigned lds_op) const {
    const unsigned w = wave_id();
#pragma unroll
    for (int j = J0; j < J1; ++j) load_lds16(p[j] + (size_t)kt * adv[j], lds_op + (w * NI + j) * 1024);
  }
  // fragment of rows [r0, r0+32), k16 step s: lane l reads row r0 + l%32
  __device__ __forceinline__ static bf16x8_t frag(const char* lds_op, int r0, int s) {
    const int lane = threadIdx.x & 63;
    const int row = r0 + (lane & 31);
    const int c = (2 * s + (lane >> 5)) ^ ((row / RS) % CPR);
    return *reinterpret_cast<const bf16x8_t*>(lds_op + row * (2 * BK) + c * 16);
  }
};

// MN-major operand tile: BK k-rows x COLS (m or n contiguous in memory,
// k strided).  LDS [BK][2*COLS bytes]; chunk c of k-row r sits at
// c ^ (4 * (r & 3)).  Fragments are read with ds_read_b64_tr_b16: in each
// 16-lane group lane a points at (k0 + a/4, n0 + 4*(a%4)) and lane i
// receives k0..k0+3 of column n0 + i -- the k-consecutive fragment the MFMA
// wants, without a transpose in registers.  kptr(k) gives the address of
// element (k, 0) of the tile or nullptr outside the contraction; columns
// >= ncols_left read zeros.
template <int COLS, int BK>
struct MNMajor {
  static constexpr int RB = 2 * COLS;           // bytes per k-row
  static constexpr int KPI = 1024 / RB;         // k-rows per 1 KiB load
  static constexpr int CPK = COLS / 8;          // chunks per k-row
  static constexpr int NI = BK / KPI / 4;       // loads per wave per stage
  static constexpr int BYTES = BK * RB;
  static_assert(CPK >= 16, "swizzle needs 16 chunks per k-row");
  int ncols_left;
  template <class KPtr>
  __device__ __forceinline__ void issue(int kt, unsigned lds_op, KPtr kptr) const {
    issue(kt, lds_op, kptr, Part<0, 1>());
  }
  template <class KPtr, int P, int NP>
  __device__ __forceinline__ void issue(int kt, unsigned lds_op, KPtr kptr, Part<P, NP>) const {
    const int lane = threadIdx.x & 63;
    const unsigned w = wave_id();
#pragma unroll
    for (int j = P * NI / NP; j < (P + 1) * NI / NP; ++j) {
      const int I = w * NI + j;
      const int krow = KPI * I + lane / CPK;
      const int c = (lane % CPK) ^ (4 * (krow & 3));
      const bf16_t* kp = kptr(kt * BK + krow);
      const void* src = (kp && c * 8 < ncols_left) ? (const void*)(kp + c * 8) : (const void*)g_zero;
      load_lds16(src, lds_op + I * 1024);
    }
  }
  __device__ __forceinline__ static bf16x8_t frag(const char* lds_op, int n0, int s) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, li = lane & 15;
    const int n = n0 + 16 * (g & 1) + 4 * (li & 3);
    const int kb = 16 * s + 8 * (g >> 1) + (li >> 2);
    v4s lo, hi;
    {
      const int kr = kb;
      const int c = (n >> 3) ^ (4 * (kr & 3));
      lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(lds_op + kr * RB + c * 16 + (n & 7) * 2));
    }
    {
      const int kr = kb + 4;
      const int c = (n >> 3) ^ (4 * (kr & 3));
      hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(lds_op + kr * RB + c * 16 + (n & 7) * 2));
    }
    bf16x8_t out;
    short* o = reinterpret_cast<short*>(&out);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[q] = lo[q];
      o[4 + q] = hi[q];
    }
    return out;
  }
};

// ---------------------------------------------------------------- tile config
// BM = 256 rows x BN columns per workgroup (4 waves, 2 x 2, each 128 x BN/2),
// BK-wide k stages, NS stages in the LDS ring, OCC workgroups resident per CU
// (the kernels ask the compiler for a register budget that allows OCC).
template <int BN_, int BK_, int NS_, int OCC_ = 1>
struct Cfg {
  static constexpr int BN = BN_, BK = BK_, NS = NS_, OCC = OCC_;
  static constexpr int WNB = BN / 64;  // 32-column MFMA blocks per wave
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int SMEM = NS * STAGE;
  static constexpr int LOADS = STAGE / 1024 / 4;  // per wave per stage
  static_assert(NS >= 2 && NS <= 8 && (NS - 1) * LOADS < 64, "vmcnt range");
  static_assert(OCC * (SMEM + 4096) <= 160 * 1024, "LDS of OCC workgroups per CU");
};

// The default configuration of the expert GEMMs: 256 x 256 tiles, two 64-k
// stages, one workgroup per CU.  (A four-deep ring of 32-k stages measured
// about 2 % slower on the layer's GEMMs: operand latency is not what bounds
// them.)
typedef Cfg<256, 64, 2> Default;
// 256 x 128 tiles, three 32-k stages (72 KiB of LDS), two workgroups per CU:
// while one workgroup stores its tile or waits at a stage barrier, the other
// keeps the CU's matrix cores busy.  It pays only where both operands are
// MN-major (the down-projection weight gradient); with a K-major operand the
// extra operand traffic of the narrower tile costs more than it hides.
typedef Cfg<128, 32, 3, 2> Narrow;

template <class C>
struct Acc {
  f32x16_t c[4][C::WNB];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < C::WNB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) c[i][j][v] = 0.0f;
  }
};

// The MFMAs compute transposed 32 x 32 blocks (the B fragment goes in the
// instruction's first operand), so lane l holds, for block (i, j), row
// out_row(i) of the tile and the four consecutive columns
// out_col(j, g) .. out_col(j, g) + 3 in accumulators 4g .. 4g+3: outputs
// leave as 8- or 16-byte vectors, one row per lane.
__device__ __forceinline__ int out_row(int i) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave >> 1) * 128 + i * 32 + (lane & 31);
}
template <class C>
__device__ __forceinline__ int out_col(int j, int g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave & 1) * (C::BN / 2) + j * 32 + 8 * g + 4 * (lane >> 5);
}

// Four fp32 -> four bf16 packed in 8 bytes.
__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  return make_uint2(pack2_bf16(a, b), pack2_bf16(c, d));
}

// Fragments of one k16 step for a wave: 4 row blocks of A, WNB column blocks of B.
template <class C, bool A_MN, bool B_MN>
struct Frags {
  bf16x8_t a[4], b[C::WNB];
  __device__ __forceinline__ void load(const char* As, const char* Bs, int s) {
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = A_MN ? MNMajor<BM, C::BK>::frag(As, wm * 128 + i * 32, s)
                  : KMajor<BM, C::BK>::frag(As, wm * 128 + i * 32, s);
#pragma unroll
    for (int j = 0; j < C::WNB; ++j)
      b[j] = B_MN ? MNMajor<C::BN, C::BK>::frag(Bs, wn * (C::BN / 2) + j * 32, s)
                  : KMajor<C::BN, C::BK>::frag(Bs, wn * (C::BN / 2) + j * 32, s);
  }
};

// MFMAs of one k16 step for row blocks [I0, I1) of the wave tile.
template <class C, bool A_MN, bool B_MN, int I0, int I1>
__device__ __forceinline__ void mma_rows(const Frags<C, A_MN, B_MN>& f, Acc<C>& acc) {
#pragma unroll
  for (int i = I0; i < I1; ++i)
#pragma unroll
    for (int j = 0; j < C::WNB; ++j)
      acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc.c[i][j], 0, 0, 0);
}

// Instruction order of one k16 step: NMFMA MFMAs, with the NREAD LDS reads of
// the next step two behind each of the first MFMAs, so the reads' latency
// runs under matrix work.  Left alone, the scheduler sinks each read to just
// before its first use, and every k16 step waits on LDS latency with the
// matrix cores idle.  (Two reads per MFMA measured 1 % faster than one, all
// of them ahead of the first MFMA 1 % slower.  Scheduling hints only: they
// reorder instructions, never the MFMAs of one accumulator, so results do
// not change.)
template <int NMFMA, int NREAD, int I = 0, int PMIN = 2>
__device__ __forceinline__ void interleave_reads() {
  // reads per MFMA: PMIN, or as many as the step needs to place them all
  constexpr int P = (NREAD + NMFMA - 1) / NMFMA > PMIN ? (NREAD + NMFMA - 1) / NMFMA : PMIN;
  if constexpr (I < NMFMA) {
    constexpr int r = NREAD - P * I >= P ? P : (NREAD - P * I > 0 ? NREAD - P * I : 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // r LDS reads
    interleave_reads<NMFMA, NREAD, I + 1, PMIN>();
  }
}

// LDS reads of one k16 step's fragments (one per K-major fragment, two per
// MN-major one).
template <class C, bool A_MN, bool B_MN>
constexpr int frag_reads() {
  return (A_MN ? 8 : 4) + (B_MN ? 2 : 1) * C::WNB;
}

// s_waitcnt: vmcnt <= N and lgkmcnt == 0 (expcnt at its maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}
// As wait_stages, with this wave's LDS reads also complete.
template <int N, int MAXA>
__device__ __forceinline__ void wait_stages_lgkm0(int after) {
  if constexpr (MAXA > 0) {
    if (after >= MAXA) {
      wait_vmcnt_lgkm0<MAXA * N>();
      return;
    }
    wait_stages_lgkm0<N, MAXA - 1>(after);
  } else {
    wait_vmcnt_lgkm0<0>();
  }
}

// Issue part P of NP of a stage's loads through a loader callback that takes
// a Part; a callback without one issues the whole stage in part 0.
template <int P, int NP, class F>
__device__ __forceinline__ void issue_part(F& f, int kt, unsigned lds) {
  if constexpr (std::is_invocable_v<F&, int, unsigned, Part<P, NP>>)
    f(kt, lds, Part<P, NP>());
  else if constexpr (P == 0)
    f(kt, lds);
}

// bf16 main loop over KT stages of BK k in an NS-deep LDS ring, pipelined
// across stages.  issueA(kt, lds[, Part]) / issueB(kt, lds[, Part]) issue
// this wave's direct loads of one stage, or part P of NP of them (lds = LDS
// byte address of the operand's tile in the stage).  All NS slots are filled
// up front.  The hand-over to stage kt+1 (wait for this wave's loads of
// kt+1 -- the loads of up to NS-2 later stages stay in flight -- and for its
// LDS reads of kt, then the workgroup barrier) comes once the rest of stage
// kt's fragments are in registers: before step 2 of four with a K-major A
// operand, before the last step otherwise.  The loads of stage kt+NS into
// the slot just freed go out in parts between the remaining MFMAs (for a
// transposing A operand, B's part in step 0 of the next stage), and the
// first fragment reads of stage kt+1 between the last ones, so neither the
// loads' issue nor the reads' latency stands in front of matrix work.  The
// accumulation order (k16 steps ascending) does not depend on NS, BK or the
// hand-over.
// keep_acc: continue from the accumulators' values (a partial sum carried
// over exactly from an earlier launch) instead of starting from zero.
template <class C, bool A_MN, bool B_MN, class IA, class IB>
__device__ __forceinline__ void mainloop(int KT, IA issueA, IB issueB, char* smem, Acc<C>& acc,
                                         bool keep_acc = false) {
  constexpr int S = C::BK / 16, NS = C::NS;
  static_assert(S >= 2, "at least two k16 steps per stage");
  typedef Frags<C, A_MN, B_MN> F;
  if (!keep_acc) acc.zero();
  if (KT <= 0) return;
  const unsigned lds0 = lds_addr_of(smem);
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < KT) {
      issue_part<0, 1>(issueA, s, lds0 + s * C::STAGE);
      issue_part<0, 1>(issueB, s, lds0 + s * C::STAGE + C::A_BYTES);
    }
  wait_stages_lgkm0<C::LOADS, NS - 1>(min(KT, NS) - 1);  // stage 0 landed
  __builtin_amdgcn_s_barrier();
  if constexpr (S == 4 && !A_MN) {
    // Four k16 steps per stage: the hand-over comes before step 2, so that
    // the stage's loads spread over the 32 MFMAs of steps 2 and 3 (a wave's
    // 16 direct loads take the CU's memory pipeline about as long as 32
    // MFMAs); steps 2 and 3 are both read during step 1.  (With a
    // transposing A operand, twice a step's reads in one step cost more than
    // the spread gains: the weight gradients keep the later hand-over.)
    constexpr int R = frag_reads<C, A_MN, B_MN>();
    F fa, fb, fc;
    fa.load(smem, smem + C::A_BYTES, 0);
    for (int kt = 0; kt < KT; ++kt) {
      const char* cur = smem + (kt % NS) * C::STAGE;
      fb.load(cur, cur + C::A_BYTES, 1);
      mma_rows<C, A_MN, B_MN, 0, 4>(fa, acc);
      interleave_reads<4 * C::WNB, R>();
      fc.load(cur, cur + C::A_BYTES, 2);
      fa.load(cur, cur + C::A_BYTES, 3);
      mma_rows<C, A_MN, B_MN, 0, 4>(fb, acc);
      interleave_reads<4 * C::WNB, 2 * R>();
      __builtin_amdgcn_sched_barrier(0);
      wait_stages_lgkm0<C::LOADS, NS - 2>(min(KT - 1, kt + NS - 1) - (kt + 1));
      __builtin_amdgcn_s_barrier();
      const unsigned slot = lds0 + (kt % NS) * C::STAGE;
      const bool more = kt + NS < KT;
      // step 2 (fc) and step 3 (fa), a quarter of the operand loads before
      // each row block; the next stage's step 0 is read into fb during step 3
      if (more) issue_part<0, 4>(issueA, kt + NS, slot);
      mma_rows<C, A_MN, B_MN, 0, 1>(fc, acc);
      if (more) issue_part<1, 4>(issueA, kt + NS, slot);
      mma_rows<C, A_MN, B_MN, 1, 2>(fc, acc);
      if (more) issue_part<2, 4>(issueA, kt + NS, slot);
      mma_rows<C, A_MN, B_MN, 2, 3>(fc, acc);
      if (more) issue_part<3, 4>(issueA, kt + NS, slot);
      mma_rows<C, A_MN, B_MN, 3, 4>(fc, acc);
      if (more) issue_part<0, 4>(issueB, kt + NS, slot + C::A_BYTES);
      const char* nxt = smem + ((kt + 1) % NS) * C::STAGE;
      fb.load(nxt, nxt + C::A_BYTES, 0);
      mma_rows<C, A_MN, B_MN, 0, 1>(fa, acc);
      interleave_reads<C::WNB, R, 0, (R + C::WNB - 1) / C::WNB>();
      if (more) issue_part<1, 4>(issueB, kt + NS, slot + C::A_BYTES);
      mma_rows<C, A_MN, B_MN, 1, 2>(fa, acc);
      if (more) issue_part<2, 4>(issueB, kt + NS, slot + C::A_BYTES);
      mma_rows<C, A_MN, B_MN, 2, 3>(fa, acc);
      if (more) issue_part<3, 4>(issueB, kt + NS, slot + C::A_BYTES);
      mma_rows<C, A_MN, B_MN, 3, 4>(fa, acc);
      // the next stage's step 0 is in fb: rotate the roles
      F t = fa;
      fa = fb;
      fb = t;
    }
    return;
  }
  if constexpr (S == 4 && A_MN) {
    // Four k16 steps, a transposing A operand: the hand-over stays before the
    // last step (reading two steps in one costs these GEMMs more than it
    // gains), and the freed slot's loads are split: A during the last step
    // of stage kt, B during step 0 of stage kt + 1, which still leaves the B
    // loads three steps to land before the next hand-over.  Loads go out in
    // stage order, so the vmcnt arithmetic of whole stages holds.  The
    // steady-state stages run in a loop of their own whose body has no
    // branch (a branch around the loads lets the compiler sink MFMAs below
    // the hand-over).
    constexpr int R = frag_reads<C, A_MN, B_MN>();
    F f[2];
    f[0].load(smem, smem + C::A_BYTES, 0);
    auto stage = [&](int kt, auto steady, bool pmore, bool more) {
      constexpr bool ST = decltype(steady)::value;
      const char* cur = smem + (kt % NS) * C::STAGE;
      const unsigned pslot = lds0 + ((kt + NS - 1) % NS) * C::STAGE + C::A_BYTES;
      // step 0, with the B loads of stage kt - 1 + NS
      f[1].load(cur, cur + C::A_BYTES, 1);
      // (scheduling barriers keep each quarter of the loads in its place)
      if (ST || pmore) issue_part<0, 4>(issueB, kt - 1 + NS, pslot);
      mma_rows<C, A_MN, B_MN, 0, 1>(f[0], acc);
      interleave_reads<C::WNB, R, 0, (R + C::WNB - 1) / C::WNB>();
      __builtin_amdgcn_sched_barrier(0);
      if (ST || pmore) issue_part<1, 4>(issueB, kt - 1 + NS, pslot);
      mma_rows<C, A_MN, B_MN, 1, 2>(f[0], acc);
      __builtin_amdgcn_sched_barrier(0);
      if (ST || pmore) issue_part<2, 4>(issueB, kt - 1 + NS, pslot);
      mma_rows<C, A_MN, B_MN, 2, 3>(f[0], acc);
      __builtin_amdgcn_sched_barrier(0);
      if (ST || pmore) issue_part<3, 4>(issueB, kt - 1 + NS, pslot);
      mma_rows<C, A_MN, B_MN, 3, 4>(f[0], acc);
      __builtin_amdgcn_sched_barrier(0);
      // steps 1 .. S-2
#pragma unroll
      for (int st = 1; st + 1 < S; ++st) {
        f[(st + 1) & 1].load(cur, cur + C::A_BYTES, st + 1);
        mma_rows<C, A_MN, B_MN, 0, 4>(f[st & 1], acc);
        interleave_reads<4 * C::WNB, R>();
      }
      const F& last = f[(S - 1) & 1];
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (ST)
        wait_vmcnt_lgkm0<(NS - 2) * C::LOADS>();
      else
        wait_stages_lgkm0<C::LOADS, NS - 2>(min(KT - 1, kt + NS - 1) - (kt + 1));
      __builtin_amdgcn_s_barrier();
      // the last step, with the A loads of stage kt + NS
      const unsigned slot = lds0 + (kt % NS) * C::STAGE;
      if (ST || more) issue_part<0, 4>(issueA, kt + NS, slot);
      mma_rows<C, A_MN, B_MN, 0, 1>(last, acc);
      __builtin_amdgcn_sched_barrier(0);
      if (ST || more) issue_part<1, 4>(issueA, kt + NS, slot);
      mma_rows<C, A_MN, B_MN, 1, 2>(last, acc);
      __builtin_amdgcn_sched_barrier(0);
      if (ST || more) issue_part<2, 4>(issueA, kt + NS, slot);
      const char* nxt = smem + ((kt + 1) % NS) * C::STAGE;
      f[S & 1].load(nxt, nxt + C::A_BYTES, 0);
      mma_rows<C, A_MN, B_MN, 2, 3>(last, acc);
      interleave_reads<C::WNB, R, 0, (R + C::WNB - 1) / C::WNB>();
      __builtin_amdgcn_sched_barrier(0);
      if (ST || more) issue_part<3, 4>(issueA, kt + NS, slot);
      mma_rows<C, A_MN, B_MN, 3, 4>(last, acc);
    };
    int kt = 0;
    if (KT > 0) stage(kt++, std::false_type(), false, NS < KT);
    for (; kt + NS < KT; ++kt) stage(kt, std::true_type(), true, true);
    for (; kt < KT; ++kt) stage(kt, std::false_type(), kt - 1 + NS < KT, false);
    return;
  }
  F f[2];
  f[0].load(smem, smem + C::A_BYTES, 0);
  for (int kt = 0; kt < KT; ++kt) {
    const char* cur = smem + (kt % NS) * C::STAGE;
#pragma unroll
    for (int s = 0; s + 1 < S; ++s) {
      f[(s + 1) & 1].load(cur, cur + C::A_BYTES, s + 1);
      mma_rows<C, A_MN, B_MN, 0, 4>(f[s & 1], acc);
      interleave_reads<4 * C::WNB, frag_reads<C, A_MN, B_MN>()>();
    }
    // (the hand-over also runs after the last stage, where it is harmless:
    // every MFMA stays outside branches, so the accumulators keep one
    // register assignment through the loop)
    const F& last = f[(S - 1) & 1];
    // the MFMAs above stay above the wait (they cover the last reads' latency)
    __builtin_amdgcn_sched_barrier(0);
    wait_stages_lgkm0<C::LOADS, NS - 2>(min(KT - 1, kt + NS - 1) - (kt + 1));
    __builtin_amdgcn_s_barrier();
    const unsigned slot = lds0 + (kt % NS) * C::STAGE;
    const bool more = kt + NS < KT;
    if (more) issue_part<0, 2>(issueA, kt + NS, slot);
    mma_rows<C, A_MN, B_MN, 0, 1>(last, acc);
    if (more) issue_part<1, 2>(issueA, kt + NS, slot);
    mma_rows<C, A_MN, B_MN, 1, 2>(last, acc);
    if (more) issue_part<0, 2>(issueB, kt + NS, slot + C::A_BYTES);
    const char* nxt = smem + ((kt + 1) % NS) * C::STAGE;
    f[S & 1].load(nxt, nxt + C::A_BYTES, 0);
    mma_rows<C, A_MN, B_MN, 2, 3>(last, acc);
    interleave_reads<C::WNB, frag_reads<C, A_MN, B_MN>()>();
    if (more) issue_part<1, 2>(issueB, kt + NS, slot + C::A_BYTES);
    mma_rows<C, A_MN, B_MN, 3, 4>(last, acc);
  }
}

// ---------------------------------------------------------------- epilogue staging
// After the main loop every wave copies its 128 x BN/2 accumulator tile (as T =
// float or bf16) into a private LDS region (a quarter of the operand ring, at
// most 32 KiB), then walks it row by row:
// each lane takes one 16-byte chunk of a row, so the global stores (and the
// loads of an epilogue's extra operands) of a wave instruction cover whole
// rows instead of one 8-byte piece of 32 different rows.  Rows of a region
// are XOR-swizzled by 16-byte chunk to keep both phases free of systematic
// bank conflicts.  fp32 tiles of 256 bytes per row and more are staged in
// several passes of ROWS rows.
template <class C, typename T>
struct WaveStage {
  static constexpr int WCOLS = C::BN / 2;
  static constexpr int PITCH = WCOLS * (int)sizeof(T);       // bytes per row
  static constexpr int CPR = PITCH / 16;                      // chunks per row
  static constexpr int EPC = 16 / (int)sizeof(T);             // elements per chunk
  static constexpr int REGION = C::SMEM >= 4 * 32768 ? 32768 : C::SMEM >= 4 * 16384 ? 16384 : 8192;
  static constexpr int ROWS = REGION / PITCH < 128 ? REGION / PITCH : 128;  // rows per pass
  static constexpr int PASSES = 128 / ROWS;
  static constexpr int SW = CPR < 32 ? CPR : 32;              // swizzle period
  static_assert(C::SMEM >= 4 * REGION, "the four waves' staging regions reuse the operand ring");
  static_assert(ROWS >= 32 && 128 % ROWS == 0, "whole 32-row blocks per pass");
  char* base;
  __device__ __forceinline__ explicit WaveStage(char* smem) : base(smem + (threadIdx.x >> 6) * REGION) {}
  __device__ __forceinline__ char* chunk_addr(int row, int c) const {
    return base + row * PITCH + ((c ^ (row % SW)) * 16);
  }
  // copy accumulator rows [pass*ROWS, (pass+1)*ROWS) of the wave tile into the region
  __device__ __forceinline__ void put(const Acc<C>& acc, int pass) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if (mi * 32 < pass * ROWS || mi * 32 >= (pass + 1) * ROWS) continue;
      const int row = mi * 32 + (lane & 31) - pass * ROWS;
#pragma unroll
      for (int nj = 0; nj < C::WNB; ++nj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = nj * 32 + 8 * q + 4 * (lane >> 5);  // first of 4 columns
          const f32x16_t& a = acc.c[mi][nj];
          char* p = chunk_addr(row, col / EPC) + (col % EPC) * (int)sizeof(T);
          if constexpr (sizeof(T) == 4)
            *reinterpret_cast<float4*>(p) = make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
          else
            *reinterpret_cast<uint2*>(p) = pack4_bf16(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
        }
    }
  }
  __device__ __forceinline__ uint4 raw(int row, int c) const {
    return *reinterpret_cast<const uint4*>(chunk_addr(row, c));
  }
  // the EPC values of chunk c of staged row `row` as floats
  __device__ __forceinline__ void get(int row, int c, float* v) const {
    const uint4 u = *reinterpret_cast<const uint4*>(chunk_addr(row, c));
    if constexpr (sizeof(T) == 4) {
      v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
      v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
    } else {
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  }
  // visit every chunk of the staged pass: fn(row_in_wave_tile, chunk) with
  // CPR consecutive lanes per row
  template <class Fn>
  __device__ __forceinline__ void for_chunks(int pass, Fn fn) const {
    const int lane = threadIdx.x & 63;
    constexpr int RPI = 64 / CPR > 0 ? 64 / CPR : 1;  // rows per wave instruction
    if constexpr (CPR <= 64) {
#pragma unroll 4
      for (int r0 = 0; r0 < ROWS; r0 += RPI) {
        const int row = r0 + lane / CPR;
        fn(pass * ROWS + row, row, lane % CPR);
      }
    }
  }
};

// Wave-local ordering of LDS stores before LDS loads of the same wave.
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// XCD-aware order: workgroup b is dispatched to XCD b % 8; give each XCD a
// contiguous range of the `total` logical tiles so that neighbouring tiles
// (which share operand panels) meet in the same L2.
__device__ __forceinline__ int xcd_tile(int b, int total) {
  const int per = total / 8;
  if (b >= per * 8) return b;
  return (b % 8) * per + b / 8;
}

// Logical tile t of an mtn x ntn tile grid -> (m-tile, n-tile), walking groups
// of kGroupM consecutive m-tiles with n outer and m inner.  Together with
// xcd_tile, the 32 tiles an XCD runs at once cover about 8 m-tiles x 4
// n-tiles, whose A and B panels stay in that XCD's L2 while the tiles move
// through k together (measured on a 98304 x 2816 x 2048 GEMM: 2.7 -> 2.1 GB
// fetched, +9 % throughput over n-fastest order).  A bijection: every tile is
// computed exactly once, by the same code, whatever the order.
constexpr int kGroupM = 8;
__device__ __forceinline__ void grouped_order(int t, int mtn, int ntn, int* mt, int* nt) {
  const int grp = t / (kGroupM * ntn), w = t % (kGroupM * ntn);
  const int g0 = grp * kGroupM, gs = min(kGroupM, mtn - g0);
  *mt = g0 + w % gs;
  *nt = w / gs;
}

// Grouped-M tiles (rows of expert e are [offsets[e], offsets[e+1]), tiles of
// tile_rows rows): per-expert tile counts, exclusive-scanned by wave 0 into
// s_prefix; returns the total.
__device__ __forceinline__ int group_prefix(const int32_t* offsets, int E_local, int R_cap,
                                            int* s_prefix, int tile_rows = BM) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int loc[4];
    int run = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      int c = 0;
      if (e < E_local) {
        int lo = min(offsets[e], R_cap), hi = min(offsets[e + 1], R_cap);
        c = hi > lo ? (hi - lo + tile_rows - 1) / tile_rows : 0;
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
  return s_prefix[E_local < 256 ? E_local : 256];
}

struct GTile {
  int e, r0, r1;
};
__device__ __forceinline__ GTile group_tile(const int32_t* offsets, int E_local, int R_cap,
                                            const int* s_prefix, int mtile, int tile_rows = BM) {
  int lo = 0, hi = E_local - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_prefix[mid] <= mtile) lo = mid; else hi = mid - 1;
  }
  GTile t;
  t.e = lo;
  const int end = min(offsets[lo + 1], R_cap);
  t.r0 = offsets[lo] + (mtile - s_prefix[lo]) * tile_rows;
  t.r1 = min(t.r0 + tile_rows, end);
  return t;
}

// Destination row of every tile row for an epilogue that pushes rows into
// per-source buffers: routed row r holds item n = row_src[r] (token n / k,
// slot n % k), whose row is row (tok % T_src) * k + slot of source
// tok / T_src's buffer.  One row per thread, so the stores of the row chunks
// need no integer divisions (a barrier must follow before they are read).
__device__ __forceinline__ void stage_dst_rows(bf16_t** s_dst, const int32_t* row_src, const GTile& g,
                                               const DstTable& tab, int k, int T_src, int d) {
  static_assert(kThreads == BM, "one thread per tile row");
  const int r = g.r0 + (int)threadIdx.x;
  bf16_t* p = nullptr;
  if (r < g.r1) {
    const int n = row_src[r];
    const int tok = n / k, j = n % k;
    p = reinterpret_cast<bf16_t*>(tab.p[tok / T_src]) + ((size_t)(tok % T_src) * k + j) * d;
  }
  s_dst[threadIdx.x] = p;
}

}  // namespace g2
}  // namespace mok
