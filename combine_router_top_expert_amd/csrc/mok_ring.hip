// Persistent ring kernel of the layer's forward pass (kucoin article,
// section 02: the GPU's SMs are split into a side that dispatches, combines
// and keeps state and a side that runs the expert FFN; the two hand work over
// through local counters, a fixed-size ring token buffer whose space is reused
// once the experts are done with it, and a minibatch size; the combine of the
// previous macrobatch runs while the next one is dispatched).
//
// One launch of comm_wgs + gemm_wgs workgroups, all resident at once (one per
// CU).  comm_wgs of them, spread evenly over the XCDs, take the
// dispatch/combine role, the rest the grouped-GEMM role.  The launch serves n_calls layer calls
// (macrobatches) in a row; each call has its own sources, routing, layout,
// staging rows and outputs, and all share the weights and the ring.
//
// Work units.  Every local expert's rows [offsets[e], offsets[e+1]) of a call
// are cut into minibatches of at most MB rows, numbered in expert order, and
// the calls' minibatches are numbered on: minibatch G (over all calls) lives
// in ring slot G % nslot (MB token rows; MXFP8: their E4M3 codes and E8M0
// scales).
//   fill (G, c)   dispatch side: pull rows [32c, 32c+32) of minibatch G from
//                 their source buffers into the slot (quantising for MXFP8);
//                 waits until GEMM1 is done with the slot's previous
//                 minibatch G - nslot; then x_ready[G] += 1.
//   G1 (G, tile)  GEMM side: one 256 x BN tile of GEMM1 + SwiGLU over the
//                 slot; waits for x_ready[G] == fill chunks of G; writes h
//                 (and a | b) at the rows' positions; then g1_done[G] += 1.
//   G2 (G, tile)  GEMM side: one tile of GEMM2 over h, pushed to the staging
//                 rows (push combine); waits for g1_done[G] == GEMM1 tiles;
//                 then g2_done[call] += 1.
//   combine (call, q)  dispatch/combine side: the final weighted combine of
//                 own tokens [32q, 32q+32) of the call; waits for g2_done of
//                 the call == all its GEMM2 tiles.  Every call but the last:
//                 the last call's combine has nothing left to overlap and runs
//                 as the stand-alone combine launch after this kernel.
// Tickets, in a fixed order per queue.  Dispatch/combine (one queue): the
// fills of call 0, the fills of call 1, the combine of call 0, the fills of
// call 2, the combine of call 1, ..., the combine of the last call -- so the
// combine of one call overlaps the pull of the next.  GEMM: per call, steps
// u = 0, 1, ... each holding the GEMM1 tiles of minibatch u followed by the
// GEMM2 tiles of minibatch u - lag, until the call's last GEMM2 tiles; then
// the next call.  The lag covers the steps that run at once (GEMM workgroups
// / tiles per step, plus one), so that a GEMM2 tile's GEMM1 tiles were taken
// a full round of the GEMM side earlier and are normally done.  Every step's
// tiles are split into one share per XCD, each its own ticket queue served by
// that XCD's GEMM workgroups only: a share spans a few n-tiles and all
// m-tiles of the minibatch, so a panel of tokens or weights is fetched into
// few L2s instead of into every one.
// Every wait of a unit is on units of an earlier step (of any queue) or on
// the other side's units that precede, in that side's order, every unit the
// waiter's side still needs: a fill waits on GEMM1 of an earlier minibatch,
// GEMM1 on the fills of its own minibatch, GEMM2 on GEMM1 of its minibatch,
// and the combine of call i -- ticketed after every fill of call i + 1 --
// on GEMM2 of call i, whose tickets precede every GEMM ticket of call i + 1.
// Each queue's tickets are taken in order by its own running workgroups
// (every queue with tiles has at least one), so the unfinished unit of the
// earliest step can always proceed: the units ahead of it in its queue are
// of earlier steps, hence done, or of its own step, whose waits are met.  Every wait is also bounded in time: on
// expiry the kernel latches MOK_ETIMEOUT, raises an abort flag that every
// other wait checks, and all workgroups return.
//
// Ordering: a producer's lanes wait for their stores, the workgroup meets at
// a barrier, and one lane increments the counter with release semantics at
// agent scope (writing back the XCD's L2).  A consumer's lane acquires the
// counter at agent scope (invalidating stale L2 and L1 lines) before the
// workgroup's barrier, and only then issues its loads.
//
// The arithmetic of each tile is the same device code as the one-launch-per-
// GEMM path (mok_ffn_tiles.h), the combine is the stand-alone combine's
// (mok_combine.h), and every output element is produced by exactly one unit,
// so the two paths give bit-identical results for any ring size, minibatch
// size, split and number of calls.
#include <string.h>

#include "mok_combine.h"
#include "mok_ffn_tiles.h"
#include "mok_internal.h"
#include "mok_mx.h"

namespace mok {

namespace {

using namespace g2;

constexpr int kFillRows = 32;  // rows per fill unit
constexpr int kCombTok = 32;   // own tokens per combine unit
// GEMM tile queues: one per XCD (workgroup b runs on XCD b % 8, the order in
// which the dispatcher hands workgroups to the XCDs)
constexpr int kQueues = 8;
// counters: the fill ticket, the abort flag, then one GEMM ticket per queue
constexpr int kFillTicket = 0, kAbort = 1, kGemmTicket = 2;
constexpr int kCtr = kGemmTicket + kQueues;

struct RingArgs {
  const RingCall* calls;   // [n_calls] in device memory
  int n_calls;
  int d, I, E_local, R_cap, T_src, k;
  int mb, nslot, cpm, nmt, ntn1, ntn2, M_max;  // M_max: minibatches of one call, at most
  int comm_wgs;
  int nq;              // GEMM queues: kQueues, or 1 when an XCD class has no GEMM workgroup
  int lag;             // GEMM2 of minibatch u runs in step u + lag (>= 1)
  char* ring;
  int64_t slot_bytes;
  int32_t* ctr;        // [kCtr + 2 * n_calls * M_max + 2 * n_calls]: tickets, abort,
                       // x_ready[], g1_done[] (by minibatch over all calls), g2_done[call],
                       // combine unit tickets[call]
  int32_t* status;
  uint64_t wait_ticks;  // bound of one wait in s_memrealtime ticks (100 MHz)
  F1Args f1;            // weights and sizes; the per-call pointers are set per unit
  F1MxArgs f1m;
  F2Args f2;
};

// Minibatch layout of every call, built by each workgroup at its start.
struct CallsLds {
  int mbp[kRingMaxCalls][257];  // per call: prefix of minibatches over the experts
  int M[kRingMaxCalls];         // minibatches of the call
  int base[kRingMaxCalls + 1];  // first minibatch of the call over all calls
};

__global__ void ring_init_kernel(int32_t* ctr, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) ctr[i] = 0;
}

// Control flow of the role loops.  Every value that steers a loop containing
// a barrier is wave-uniform in the compiler's eyes (read back through
// readfirstlane), and the single-thread steps (take a ticket, wait on a
// counter, publish) run on all 64 lanes of wave 0 under a wave-uniform
// branch rather than under `threadIdx.x == 0`.  With a lane-divergent branch
// at the end of one iteration and the start of the next, the compiler
// restructures the loop into nested loops whose exit masks send lanes 1..63
// around the back edge to the next barrier before lane 0 has taken the next
// ticket; the workgroup then never leaves the loop.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ bool wave0() { return uniform((int)(threadIdx.x >> 6)) == 0; }

// Wave 0 waits until *p >= target: relaxed polls of the counter, then one
// acquire fence at agent scope.  False if the wait ran out (MOK_ETIMEOUT
// latched, abort raised) or another wait already did.
__device__ bool ring_wait(int32_t* p, int target, const RingArgs& a) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    if (uniform(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) >= target) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return true;
    }
    if (uniform(__hip_atomic_load(a.ctr + kAbort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0)
      return false;
    if (__builtin_amdgcn_s_memrealtime() - t0 > a.wait_ticks) {
      latch(a.status, MOK_ETIMEOUT);
      __hip_atomic_store(a.ctr + kAbort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Workgroup-wide wait: wave 0 waits, the result is broadcast through LDS.
__device__ bool wg_wait(int32_t* p, int target, const RingArgs& a, int* s_flag) {
  if (wave0()) *s_flag = ring_wait(p, target, a) ? 1 : 0;
  __syncthreads();
  return uniform(*s_flag) != 0;
}

// Publish this workgroup's stores: every lane waits for its own stores, the
// workgroup meets, then wave 0 adds 1 (lane 0 adds 1, the others 0) after a
// release fence at agent scope.
__device__ void wg_publish(int32_t* p) {
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), expcnt(7), lgkmcnt(0)
  __syncthreads();
  if (wave0()) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(p, (threadIdx.x & 63) == 0 ? 1 : 0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Next ticket of a counter for the workgroup (lane 0 of wave 0 adds 1, the
// other lanes 0; lane 0's pre-value is the ticket).
__device__ int wg_ticket(int32_t* p, int* s_val) {
  if (wave0()) {
    const int old = __hip_atomic_fetch_add(p, (threadIdx.x & 63) == 0 ? 1 : 0, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    *s_val = __builtin_amdgcn_readlane(old, 0);
  }
  __syncthreads();
  return uniform(*s_val);
}

// Minibatch m of call c -> (expert, rows [r0, r1)).
__device__ __forceinline__ GTile minibatch(const RingArgs& a, const CallsLds& L, int c, int m) {
  GTile t = group_tile(a.calls[c].offsets, a.E_local, a.R_cap, L.mbp[c], m, a.mb);
  t.e = uniform(t.e);
  t.r0 = uniform(t.r0);
  t.r1 = uniform(t.r1);
  return t;
}

// ---------------------------------------------------------------- dispatch side
// Rows [q0, q0 + nr) of minibatch mbt into its slot.  The rows' source
// addresses are looked up once into LDS; then every thread issues kBatch
// independent 16-byte loads before their stores, so a fill costs about one
// memory round trip per kBatch units instead of two dependent ones per unit.
// nr is uniform over the workgroup (it holds a barrier).
constexpr int kBatch = 8;

template <bool MX>
__device__ void fill_rows(const RingArgs& a, const RingCall& call, char* slot, const GTile& mbt,
                          int q0, int nr) {
  __shared__ const bf16_t* s_src[kFillRows];
  if ((int)threadIdx.x < nr) {
    const int tok = call.row_src[mbt.r0 + q0 + threadIdx.x] / a.k;
    s_src[threadIdx.x] = reinterpret_cast<const bf16_t*>(call.src.p[tok / a.T_src]) +
                         (size_t)(tok % a.T_src) * a.d;
  }
  __syncthreads();
  const int upr = a.d / 8;  // 16-byte units (8 bf16) per row
  const int total = nr * upr;
  if constexpr (!MX) {
    for (int u0 = threadIdx.x; u0 < total; u0 += kThreads * kBatch) {
      uint4 v[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int u = u0 + b * kThreads;
        if (u < total) v[b] = ld16(s_src[u / upr] + (u % upr) * 8);
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int u = u0 + b * kThreads;
        if (u < total)
          st16(reinterpret_cast<bf16_t*>(slot) + (size_t)(q0 + u / upr) * a.d + (u % upr) * 8, v[b]);
      }
    }
    return;
  }
  for (int u0 = threadIdx.x; u0 < total; u0 += kThreads * kBatch) {
    // a 32-element MX block is 4 consecutive units (4 lanes); upr % 4 == 0
    // and kThreads % 4 == 0, so a lane group is all in or all out of a batch
    // entry, and the lanes of a group take part in the same shuffles
    uint4 vb[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int u = u0 + b * kThreads;
      if (u < total) vb[b] = ld16(s_src[u / upr] + (u % upr) * 8);
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
    const int u = u0 + b * kThreads;
    if (u >= total) break;
    const int row = u / upr, c = u % upr;
    const int q = q0 + row;  // row within the minibatch
    const uint4 v = vb[b];
    {
      float f[8];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      {
        const int sh = mx_shared_exp(amax);
        const uint32_t lo = e4m3_pack4(f[0], f[1], f[2], f[3], sh);
        const uint32_t hi = e4m3_pack4(f[4], f[5], f[6], f[7], sh);
        uint8_t* codes = reinterpret_cast<uint8_t*>(slot) + (size_t)q * a.d;
        *reinterpret_cast<uint2*>(codes + c * 8) = make_uint2(lo, hi);
        if ((c & 3) == 0) {
          uint8_t* scales = reinterpret_cast<uint8_t*>(slot) + (size_t)a.mb * a.d + (size_t)q * (a.d / 32);
          scales[c >> 2] = (uint8_t)(sh + 127);
        }
      }
    }
    }
  }
}

// Combine units of a call: own tokens in groups of kCombTok.  The last call's
// combine has no later pull to overlap and runs as its own launch after this
// kernel, where many workgroups per CU hide its memory latency; the earlier
// calls' combines run here.
__device__ __forceinline__ int combine_units(const RingArgs& a, int c) {
  if (c >= a.n_calls - 1) return 0;
  return (int)(((int64_t)a.calls[c].own_n * a.T_src + kCombTok - 1) / kCombTok);
}

// Dispatch/combine ticket f -> (kind, call, index): the fills of call 0, then
// for c = 1 .. n_calls - 1 the fills of call c followed by the combine of
// call c - 1, and last the combine of the last call.  kind 0 = fill, 1 =
// combine, -1 = no more work.
__device__ int comm_unit(const RingArgs& a, const CallsLds& L, int f, int* call, int* idx) {
  for (int i = 0; i <= a.n_calls; ++i) {
    if (i < a.n_calls) {  // fills of call i
      const int nf = L.M[i] * a.cpm;
      if (f < nf) {
        *call = i;
        *idx = f;
        return 0;
      }
      f -= nf;
    }
    if (i >= 1) {  // combine of call i - 1
      const int nc = combine_units(a, i - 1);
      if (f < nc) {
        *call = i - 1;
        *idx = f;
        return 1;
      }
      f -= nc;
    }
  }
  return -1;
}

// Combine units of call c, taken from the call's combine ticket until none
// is left: the final weighted combine of own tokens [32q, 32q + 32), once
// every GEMM2 tile of the call has pushed its rows.  False if a wait failed.
__device__ bool drain_combine(const RingArgs& a, const CallsLds& L, int c, int* s_val) {
  int32_t* g2_done = a.ctr + kCtr + 2 * a.n_calls * a.M_max;
  int32_t* ctick = g2_done + a.n_calls;
  const RingCall& call = a.calls[c];
  const int nu = combine_units(a, c);
  bool waited = false;
  for (;;) {
    const int q = wg_ticket(ctick + c, s_val);
    if (q >= nu) return true;
    if (!waited) {
      if (!wg_wait(g2_done + c, L.M[c] * a.nmt * a.ntn2, a, s_val + 1)) return false;
      waited = true;
    }
    const int64_t n_tok = (int64_t)call.own_n * a.T_src;
    const int64_t g0 = (int64_t)q * kCombTok;
    for (int i = 0; i < kCombTok && g0 + i < n_tok; ++i) {
      const int64_t g = g0 + i;
      const int s = call.own_lo + (int)(g / a.T_src);
      const int t = (int)(g % a.T_src);
      const int64_t n0 = ((int64_t)s * a.T_src + t) * a.k;
      const bf16_t* stg =
          reinterpret_cast<const bf16_t*>(call.staging.p[s]) + (size_t)t * a.k * a.d;
      bf16_t* o = reinterpret_cast<bf16_t*>(call.out.p[s]) + (size_t)t * a.d;
      combine_token<bf16_t>(call.dest_row, call.gate, n0, a.k, a.R_cap, stg, o, a.d, threadIdx.x,
                            kThreads);
    }
  }
}

template <bool MX>
__device__ void dispatch_role(const RingArgs& a, const CallsLds& L, int* s_val) {
  int32_t* x_ready = a.ctr + kCtr;
  int32_t* g1_done = x_ready + a.n_calls * a.M_max;
  for (;;) {
    const int f = wg_ticket(a.ctr + kFillTicket, s_val);
    int c = 0, idx = 0;
    const int kind = uniform(comm_unit(a, L, f, &c, &idx));
    c = uniform(c);
    idx = uniform(idx);
    if (kind < 0) break;
    const RingCall& call = a.calls[c];
    if (kind == 0) {
      const int m = idx / a.cpm, ch = idx % a.cpm;
      const int G = L.base[c] + m;
      const GTile mbt = minibatch(a, L, c, m);
      if (G >= a.nslot && !wg_wait(g1_done + (G - a.nslot), a.nmt * a.ntn1, a, s_val + 1)) return;
      const int q0 = ch * kFillRows;
      const int nr = min(kFillRows, (mbt.r1 - mbt.r0) - q0);
      if (nr > 0)
        fill_rows<MX>(a, call, a.ring + (size_t)(G % a.nslot) * a.slot_bytes, mbt, q0, nr);
      wg_publish(x_ready + G);
    } else if (!drain_combine(a, L, c, s_val)) {
      // a combine ticket: help with the call's combine units until none is left
      return;
    }
  }
}

// ---------------------------------------------------------------- GEMM side
// Queue q's share of a step: the tiles [q n / nq, (q + 1) n / nq) of each
// GEMM in the step's order, n-tile outer and m-tile inner, so that the share
// spans few n-tiles (weight panels) and every m-tile of the minibatch (its
// token panels), and the tiles that read one panel run in one L2.
__device__ __forceinline__ void queue_share(int n, int q, int nq, int* off, int* cnt) {
  const int lo = (int)((int64_t)q * n / nq), hi = (int)((int64_t)(q + 1) * n / nq);
  *off = lo;
  *cnt = hi - lo;
}

template <class C, bool MX>
__device__ void gemm_role(const RingArgs& a, const CallsLds& L, int* s_val, char* smem, int q) {
  int32_t* x_ready = a.ctr + kCtr;
  int32_t* g1_done = x_ready + a.n_calls * a.M_max;
  int32_t* g2_done = g1_done + a.n_calls * a.M_max;
  const int n1 = a.nmt * a.ntn1;
  int o1, s1, o2, s2;
  queue_share(n1, q, a.nq, &o1, &s1);
  queue_share(a.nmt * a.ntn2, q, a.nq, &o2, &s2);
  const int per = s1 + s2;  // this queue's tiles per step
  for (;;) {
    __syncthreads();  // the previous unit is done with LDS and the broadcast slots
    int t = wg_ticket(a.ctr + kGemmTicket + q, s_val);
    int c = 0;
    for (; c < a.n_calls; ++c) {  // the call of ticket t (its steps: M + lag)
      const int nt_call = (L.M[c] + a.lag) * per;
      if (t < nt_call) break;
      t -= nt_call;
    }
    c = uniform(c);
    t = uniform(t);
    if (c >= a.n_calls) {
      // no GEMM work left (every GEMM tile is taken): help with the combines
      for (int cc = 0; cc < a.n_calls; ++cc)
        if (!drain_combine(a, L, cc, s_val)) return;
      return;
    }
    const RingCall& call = a.calls[c];
    const int M = L.M[c];
    const int u = t / per;
    const int o = t % per;
    if (o < s1) {
      const int m = u;
      if (m >= M) continue;
      const int G = L.base[c] + m;
      const int i = o1 + o;
      const int mt = i % a.nmt, nt = i / a.nmt;
      const GTile mbt = minibatch(a, L, c, m);
      GTile g;
      g.e = mbt.e;
      g.r0 = mbt.r0 + mt * BM;
      g.r1 = min(mbt.r1, g.r0 + BM);
      if (g.r0 < g.r1) {
        if (!wg_wait(x_ready + G, a.cpm, a, s_val + 1)) return;
        const char* slot = a.ring + (size_t)(G % a.nslot) * a.slot_bytes;
        if constexpr (!MX) {
          F1Args f1 = a.f1;
          f1.row_src = call.row_src;
          f1.offsets = call.offsets;
          f1.h = reinterpret_cast<bf16_t*>(call.h);
          f1.ab = reinterpret_cast<bf16_t*>(call.ab);
          ffn1_tile<C>(f1, smem, g, nt, [&](int row) -> const bf16_t* {
            const int r = g.r0 + row;
            return r < g.r1 ? reinterpret_cast<const bf16_t*>(slot) + (size_t)(r - mbt.r0) * a.d
                            : nullptr;
          });
        } else {
          F1MxArgs f1 = a.f1m;
          f1.offsets = call.offsets;
          f1.hq = reinterpret_cast<uint8_t*>(call.h);
          f1.hs = call.h_scale;
          f1.ab = reinterpret_cast<bf16_t*>(call.ab);
          ffn1_mx_tile(
              f1, smem, g, nt,
              [&](int row) -> const bf16_t* {
                const int r = g.r0 + row;
                return r < g.r1 ? reinterpret_cast<const bf16_t*>(slot + (size_t)(r - mbt.r0) * a.d)
                                : nullptr;
              },
              [&](int row) -> const uint8_t* {
                const int r = g.r0 + row;
                return r < g.r1 ? reinterpret_cast<const uint8_t*>(slot) + (size_t)a.mb * a.d +
                                      (size_t)(r - mbt.r0) * (a.d / 32)
                                : nullptr;
              });
        }
      }
      wg_publish(g1_done + G);
    } else {
      const int m = u - a.lag;
      if (m < 0) continue;
      const int G = L.base[c] + m;
      const int i = o2 + (o - s1);
      const int mt = i % a.nmt, nt = i / a.nmt;
      const GTile mbt = minibatch(a, L, c, m);
      GTile g;
      g.e = mbt.e;
      g.r0 = mbt.r0 + mt * BM;
      g.r1 = min(mbt.r1, g.r0 + BM);
      if (g.r0 < g.r1) {
        if (!wg_wait(g1_done + G, n1, a, s_val + 1)) return;
        F2Args f2 = a.f2;
        f2.h = reinterpret_cast<const bf16_t*>(call.h);
        f2.hs = call.h_scale;
        f2.offsets = call.offsets;
        f2.row_src = call.row_src;
        if constexpr (!MX)
          ffn2_tile<C>(f2, call.staging, smem, g, nt);
        else
          ffn2_mx_tile(f2, call.staging, smem, g, nt);
      }
      // every GEMM2 ticket of the call counts (the combine waits for all)
      wg_publish(g2_done + c);
    }
  }
}

template <class C, bool MX>
__global__ __launch_bounds__(kThreads) void ring_kernel(RingArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ CallsLds L;
  __shared__ int s_val[2];
  int base = 0;
  for (int c = 0; c < a.n_calls; ++c) {
    const int M = uniform(group_prefix(a.calls[c].offsets, a.E_local, a.R_cap, L.mbp[c], a.mb));
    if (threadIdx.x == 0) {
      L.M[c] = M;
      L.base[c] = base;
    }
    base += M;
  }
  if (threadIdx.x == 0) L.base[a.n_calls] = base;
  __syncthreads();
  // roles by workgroup index: of the workgroups of XCD x (b % 8 == x, in the
  // order j = b / 8) the first comm_wgs / 8 (one more for x < comm_wgs % 8)
  // dispatch, so both sides spread evenly over the XCDs; the others serve
  // the XCD's GEMM queue
  const int b = (int)blockIdx.x, x = b % kQueues, j = b / kQueues;
  const int cx = a.comm_wgs / kQueues + (x < a.comm_wgs % kQueues ? 1 : 0);
  if (j < cx)
    dispatch_role<MX>(a, L, s_val);
  else
    gemm_role<C, MX>(a, L, s_val, smem, a.nq == kQueues ? x : 0);
}

// Copies one call's descriptor into device memory (tables travel as kernel
// arguments, which are too large for the ring kernel to carry for every call).
__global__ void ring_call_kernel(RingCall c, RingCall* dst) {
  static_assert(sizeof(RingCall) % 8 == 0, "descriptor copied in 8-byte words");
  const uint64_t* from = reinterpret_cast<const uint64_t*>(&c);
  uint64_t* to = reinterpret_cast<uint64_t*>(dst);
  for (int i = threadIdx.x; i < (int)(sizeof(RingCall) / 8); i += blockDim.x) to[i] = from[i];
}

}  // namespace

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

// GEMM queues of a split: one per XCD class (workgroups b with b % 8 == x)
// when every class keeps at least one GEMM workgroup after its dispatch
// share, else a single queue.  Every queue with tiles needs a workgroup for
// the ring to make progress.
static int ring_gemm_queues(int comm, int gemm) {
  const int grid = comm + gemm;
  for (int x = 0; x < kQueues; ++x) {
    const int nx = grid / kQueues + (x < grid % kQueues ? 1 : 0);
    const int cx = comm / kQueues + (x < comm % kQueues ? 1 : 0);
    if (nx - cx < 1) return 1;
  }
  return kQueues;
}

int64_t ring_slot_bytes(int prec, int d, int mb) {
  const int64_t b = prec == MOK_MXFP8 ? (int64_t)mb * d + (int64_t)mb * (d / 32) : (int64_t)mb * d * 2;
  return (b + 255) & ~(int64_t)255;
}

int ring_max_minibatches(int R_cap, int E_local, int mb) {
  return (R_cap + mb - 1) / mb + E_local;
}

// Counters (tickets, abort flag, x_ready and g1_done per minibatch of every
// call, g2_done per call), then the call descriptors.
static size_t ring_counter_ints(int R_cap, int E_local, int mb) {
  return (size_t)kCtr + 2 * (size_t)kRingMaxCalls * ring_max_minibatches(R_cap, E_local, mb) +
         2 * kRingMaxCalls;
}

size_t ring_meta_bytes(int R_cap, int E_local, int mb) {
  const size_t ctr = (ring_counter_ints(R_cap, E_local, mb) * sizeof(int32_t) + 255) & ~(size_t)255;
  return ctr + kRingMaxCalls * sizeof(RingCall);
}

mok_status ring_check(int prec, int d, int I, int mb, int64_t ring_bytes, int comm_wgs,
                      int gemm_wgs, int* comm_out, int* gemm_out) {
  if (prec != MOK_BF16 && prec != MOK_MXFP8) return MOK_EINVAL;
  if (mb < 1) return MOK_EINVAL;
  if (prec == MOK_MXFP8 && (d % MxCfg::KB != 0 || I % MxCfg::KB != 0)) return MOK_ESHAPE;
  if (ring_bytes / ring_slot_bytes(prec, d, mb) < 1) return MOK_EINVAL;  // one minibatch at least
  const int cus = device_cus();
  if (cus <= 0) return MOK_EDEVICE;
  // default split: 1/8 of the CUs pull bf16 rows; MXFP8 dispatch also
  // quantises every row and needs 1/4 (measured by mok_tune_fwd on the
  // mid-size layer: 3.70 ms with 32 dispatch workgroups, 2.62 ms with 64)
  const int comm = comm_wgs > 0 ? comm_wgs
                                : (cus >= 64 ? (prec == MOK_MXFP8 ? cus / 4 : cus / 8) : 1);
  const int gemm = gemm_wgs > 0 ? gemm_wgs : cus - comm;
  if (comm < 1 || gemm < 1 || comm + gemm > cus) return MOK_EINVAL;  // all resident: one per CU
  if (comm_out) *comm_out = comm;
  if (gemm_out) *gemm_out = gemm;
  return MOK_OK;
}

mok_status launch_ring_fwd(const RingPlan& p, hipStream_t stream, mok_trace* tr) {
  int comm = 0, gemm = 0;
  const mok_status ok = ring_check(p.prec, p.d, p.I, p.mb, p.ring_bytes, p.comm_wgs, p.gemm_wgs,
                                   &comm, &gemm);
  if (ok != MOK_OK) return ok;
  if (p.n_calls < 1 || p.n_calls > kRingMaxCalls) return MOK_EINVAL;
  const int64_t slot = ring_slot_bytes(p.prec, p.d, p.mb);
  const int64_t nslot = p.ring_bytes / slot;
  if (p.R_cap == 0) return MOK_OK;
  RingArgs a;
  memset(&a, 0, sizeof(a));
  a.n_calls = p.n_calls;
  a.d = p.d;
  a.I = p.I;
  a.E_local = p.E_local;
  a.R_cap = p.R_cap;
  a.T_src = p.T_src;
  a.k = p.k;
  a.mb = p.mb;
  a.nslot = nslot > (1 << 30) ? (1 << 30) : (int)nslot;
  a.cpm = (p.mb + kFillRows - 1) / kFillRows;
  a.nmt = (p.mb + BM - 1) / BM;
  a.M_max = ring_max_minibatches(p.R_cap, p.E_local, p.mb);
  a.comm_wgs = comm;
  a.ring = reinterpret_cast<char*>(p.ring);
  a.slot_bytes = slot;
  char* meta = reinterpret_cast<char*>(p.meta);
  a.ctr = reinterpret_cast<int32_t*>(meta);
  const size_t ctr_bytes =
      (ring_counter_ints(p.R_cap, p.E_local, p.mb) * sizeof(int32_t) + 255) & ~(size_t)255;
  RingCall* calls = reinterpret_cast<RingCall*>(meta + ctr_bytes);
  a.calls = calls;
  a.status = p.status;
  const uint64_t us = p.wait_limit_us > 0 ? (uint64_t)p.wait_limit_us : 2000000ull;
  a.wait_ticks = us * 100;  // s_memrealtime runs at 100 MHz
  if (p.prec == MOK_BF16) {
    a.ntn1 = (p.I + Default::BN / 2 - 1) / (Default::BN / 2);
    a.ntn2 = (p.d + Default::BN - 1) / Default::BN;
    F1Args& f1 = a.f1;
    f1.wg = reinterpret_cast<const bf16_t*>(p.w->w_gate);
    f1.wu = reinterpret_cast<const bf16_t*>(p.w->w_up);
    f1.d = p.d;
    f1.I = p.I;
    f1.E_local = p.E_local;
    f1.R_cap = p.R_cap;
    f1.ntn = a.ntn1;
    f1.T_src = p.T_src;
    f1.k = p.k;
  } else {
    a.ntn1 = (p.I + MxCfg::BN / 2 - 1) / (MxCfg::BN / 2);
    a.ntn2 = (p.d + MxCfg::BN - 1) / MxCfg::BN;
    F1MxArgs& f1 = a.f1m;
    f1.wg = reinterpret_cast<const uint8_t*>(p.w->w_gate);
    f1.wu = reinterpret_cast<const uint8_t*>(p.w->w_up);
    f1.sg = p.w->s_gate;
    f1.su = p.w->s_up;
    f1.d = p.d;
    f1.I = p.I;
    f1.E_local = p.E_local;
    f1.R_cap = p.R_cap;
    f1.ntn = a.ntn1;
  }
  F2Args& f2 = a.f2;
  f2.wd = reinterpret_cast<const bf16_t*>(p.w->w_down);
  f2.sd = p.w->s_down;
  f2.push = 1;
  f2.d = p.d;
  f2.I = p.I;
  f2.E_local = p.E_local;
  f2.R_cap = p.R_cap;
  f2.ntn = a.ntn2;
  f2.T_src = p.T_src;
  f2.k = p.k;
  {
    const int per_step = a.nmt * (a.ntn1 + a.ntn2);
    a.lag = (gemm + per_step - 1) / per_step + 1;
  }
  a.nq = ring_gemm_queues(comm, gemm);
  for (int c = 0; c < p.n_calls; ++c)
    hipLaunchKernelGGL(ring_call_kernel, dim3(1), dim3(64), 0, stream, p.calls[c], calls + c);
  const int nctr = kCtr + 2 * p.n_calls * a.M_max + 2 * p.n_calls;
  hipLaunchKernelGGL(ring_init_kernel, dim3((nctr + 255) / 256), dim3(256), 0, stream, a.ctr, nctr);
  trace_mark(tr, "ring_init", stream);
  if (p.prec == MOK_BF16)
    hipLaunchKernelGGL((ring_kernel<Default, false>), dim3(comm + gemm), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((ring_kernel<MxCfg, true>), dim3(comm + gemm), dim3(kThreads), 0, stream, a);
  trace_mark(tr, "ring_fused_ffn", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

}  // namespace mok
