// Router kernel: logits on the vector ALU (fp32 chain), top-k, gates.
//
// A router picks a few experts per token (kucoin article, section 01).  The
// pages fix neither the score function nor the tie rule; this library uses:
//   z[t][e] = fp32 chain over i ascending: z = fma(x_i, w_i, z), from 0,
//             then one fp32 add of bias[e];
//   top-k   = k largest z, equal z -> lower expert id first, slot 0 largest;
//   gate_j  = exp(z_j - z_0) / sum_i exp(z_i - z_0) over the chosen slots
//             (= softmax over all experts renormalised over the chosen ones).
// Every output (t, e) keeps its own sequential chain (one lane, d ascending),
// so the logits -- and hence the selection -- are reproducible bit for bit.
// No matrix cores here: the chain order is the contract.
#include "mok_internal.h"

namespace mok {

namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteMinBlocks = 256;  // one block per CU before blocks shrink

struct RouteArgs {
  SrcTable src;     // token buffers: token g of the launch is src.p[src_lo + g / T_src][g % T_src]
  int src_lo, T_src;
  const void* w;
  const float* bias;
  int32_t* topk_idx;  // [T, k] for the launch's tokens, in order
  float* topk_gate;
  int T, d, E, k;
  int EL;           // expert lanes per wave (each lane: 4 experts)
  int ESETS;        // sets of 4 * EL experts
  int TB;           // tokens per block
  int dc;           // d-chunk staged through LDS
};

template <typename T>
struct Unit;
template <>
struct Unit<bf16_t> {
  static constexpr int n = 8;
};
template <>
struct Unit<float> {
  static constexpr int n = 4;
};

template <typename T>
__device__ __forceinline__ void unpack(uint4 u, float* out);
template <>
__device__ __forceinline__ void unpack<bf16_t>(uint4 u, float* out) {
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void unpack<float>(uint4 u, float* out) {
  out[0] = __uint_as_float(u.x);
  out[1] = __uint_as_float(u.y);
  out[2] = __uint_as_float(u.z);
  out[3] = __uint_as_float(u.w);
}

// Selection order of two (logit, expert) entries: the larger logit first,
// the lower expert id first on equal logits.  A NaN logit ranks after every
// number, -inf included, and NaNs rank among themselves by id, so a token
// whose logits are NaN still gets k distinct valid experts.
__device__ __forceinline__ bool ranks_before(float a, int ea, float b, int eb) {
  const bool na = __builtin_isnan(a), nb = __builtin_isnan(b);
  if (na || nb) return nb && (!na || ea < eb);
  return a > b || (a == b && ea < eb);
}

// Top-k and gates of a block's tokens from the logits zs[TB][zp].  LP = 2^LPS
// lanes per token (the power of two covering E, at most 64), 64 / LP tokens
// per wave at a time; lane li of a token's group holds experts li, li + LP,
// ...  The butterfly stays inside the group, so the reduction takes LPS
// steps.  Lanes of a token past the block's end run the same steps on -inf
// and write nothing.
template <int LPS>
__device__ __forceinline__ void select_topk(const RouteArgs& a, const float* zs, int zp, int t0,
                                            int TB, int wave, int lane) {
  constexpr int LP = 1 << LPS, TPI = 64 >> LPS;
  const int MPL = (a.E + LP - 1) >> LPS;  // entries per lane (<= 8)
  const int grp = lane >> LPS, li = lane & (LP - 1);
  for (int tb0 = wave * TPI; tb0 < TB && t0 + tb0 < a.T; tb0 += (kRouteThreads / 64) * TPI) {
    const int tl = tb0 + grp;
    const int t = t0 + tl;
    const bool live = tl < TB && t < a.T;
    float zv[8];
    uint32_t used = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      int e = li + LP * m;
      zv[m] = (live && m < MPL && e < a.E) ? zs[tl * zp + e] : -__builtin_inff();
    }
    // round j picks slot j; lane li == j keeps that slot (k <= E <= LP, so
    // every slot has a lane); the exponentials are summed in slot order
    float z0 = 0.0f, sum = 0.0f, my_ex = 0.0f;
    int my_e = 0;
    for (int j = 0; j < a.k; ++j) {
      // no candidate yet: a NaN with the largest id, which every entry beats
      float bz = __builtin_nanf("");
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        int e = li + LP * m;
        bool ok = m < MPL && e < a.E && !((used >> m) & 1u);
        if (ok && ranks_before(zv[m], e, bz, be)) {
          bz = zv[m];
          be = e;
        }
      }
#pragma unroll
      for (int off = LP >> 1; off >= 1; off >>= 1) {
        float oz = __shfl_xor(bz, off, 64);
        int oe = __shfl_xor(be, off, 64);
        if (ranks_before(oz, oe, bz, be)) {
          bz = oz;
          be = oe;
        }
      }
      if (live && (be & (LP - 1)) == li) used |= 1u << (be >> LPS);
      if (j == 0) z0 = bz;
      const float exj = expf(bz - z0);
      sum += exj;
      if (li == j) {
        my_ex = exj;
        my_e = be;
      }
    }
    if (live && li < a.k) {
      a.topk_idx[(size_t)t * a.k + li] = my_e;
      a.topk_gate[(size_t)t * a.k + li] = my_ex / sum;
    }
  }
}

// A block routes TB tokens against all E experts.  A lane keeps 16 logit
// chains: 4 consecutive experts x 4 consecutive tokens; per d step it reads
// the 4 weights and the 4 token values as one 16-byte LDS read each (lanes of
// the same tokens share the address) and issues 16 fmaf.  A wave unit is EL
// expert lanes x (64 / EL) token lanes; the block's units (expert set, token
// group) are its four waves.  Chunks of dc along d are staged
// through two LDS buffers as fp32 -- [dc][TB] tokens, [dc][Epad + 4]
// weights -- with the global loads of chunk c + 1 in flight (in registers)
// while chunk c is computed.
template <typename T, int DC, int PT>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
  extern __shared__ float smem[];
  constexpr int dc = DC;
  const int TB = a.TB, EL = a.EL;
  const int Epad = a.ESETS * 4 * EL;
  const int wpitch = Epad + 4;
  const int buf = dc * TB + dc * wpitch;         // floats per staging buffer
  constexpr int U = Unit<T>::n;
  constexpr int UPR = dc / U;                    // 16-byte units per row chunk
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int el = lane % EL, tl = lane / EL;
  const int TPU = (64 / EL) * 4;                 // tokens per unit
  const int units = a.ESETS * (TB / TPU);
  const int t0 = blockIdx.x * TB;
  const T* w = reinterpret_cast<const T*>(a.w);
  const int nx = TB * UPR, nw = Epad * UPR;      // staging units per chunk

  // This thread's staging units (up to PT per operand): global source of
  // chunk 0 (null = zeros) and LDS offset of the unit's first value.
  const T* gx[PT];
  const T* gw[PT];
  int lx[PT], lw[PT];
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    const int u = tid + j * kRouteThreads;
    const int t = u / UPR, q = u % UPR;
    gx[j] = nullptr;
    lx[j] = -1;
    if (u < nx) {
      lx[j] = (q * U) * TB + t;
      if (t0 + t < a.T) {
        const int g = t0 + t;
        gx[j] = reinterpret_cast<const T*>(a.src.p[a.src_lo + g / a.T_src]) +
                (size_t)(g % a.T_src) * a.d + q * U;
      }
    }
    gw[j] = nullptr;
    lw[j] = -1;
    if (u < nw) {
      lw[j] = (q * U) * wpitch + t;  // t = expert here
      if (t < a.E) gw[j] = w + (size_t)t * a.d + q * U;
    }
  }
  uint4 rx[PT], rw[PT];
  auto fetch = [&](int c0) {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      rx[j] = gx[j] ? ld16(gx[j] + c0) : make_uint4(0, 0, 0, 0);
      rw[j] = gw[j] ? ld16(gw[j] + c0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto deposit = [&](float* xs, float* ws) {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      float v[U];
      if (lx[j] >= 0) {
        unpack<T>(rx[j], v);
#pragma unroll
        for (int i = 0; i < U; ++i) xs[lx[j] + i * TB] = v[i];
      }
      if (lw[j] >= 0) {
        unpack<T>(rw[j], v);
#pragma unroll
        for (int i = 0; i < U; ++i) ws[lw[j] + i * wpitch] = v[i];
      }
    }
  };

  float acc[4][4];  // [token][expert]
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[p][q] = 0.0f;
  const bool active = wave < units;
  const int es = wave % a.ESETS, tg = wave / a.ESETS;

  fetch(0);
  for (int c0 = 0, b = 0; c0 < a.d; c0 += dc, b ^= 1) {
    float* xs = smem + b * buf;
    float* ws = xs + dc * TB;
    // buffer b was last read by the chunk before the previous one, which
    // every wave finished before the previous barrier
    deposit(xs, ws);
    __syncthreads();
    if (c0 + dc < a.d) fetch(c0 + dc);
    if (active) {
      const float* wr = ws + es * 4 * EL + 4 * el;
      const float* xr = xs + tg * TPU + 4 * tl;
      // the LDS reads of the next kG d steps are issued before the fmaf of
      // the current kG: with one wave per SIMD nothing else hides their
      // latency (the chains still advance one d step at a time, ascending)
      constexpr int kG = 4;
      static_assert(dc % kG == 0, "d chunk of whole groups");
      float4 wv[2][kG], xv[2][kG];
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        wv[0][g] = *reinterpret_cast<const float4*>(wr + g * wpitch);
        xv[0][g] = *reinterpret_cast<const float4*>(xr + g * TB);
      }
#pragma unroll
      for (int i0 = 0; i0 < dc; i0 += kG) {
        const int cur = (i0 / kG) & 1;
        if (i0 + kG < dc) {
#pragma unroll
          for (int g = 0; g < kG; ++g) {
            wv[cur ^ 1][g] = *reinterpret_cast<const float4*>(wr + (i0 + kG + g) * wpitch);
            xv[cur ^ 1][g] = *reinterpret_cast<const float4*>(xr + (i0 + kG + g) * TB);
          }
        }
#pragma unroll
        for (int g = 0; g < kG; ++g) {
          const float xa[4] = {xv[cur][g].x, xv[cur][g].y, xv[cur][g].z, xv[cur][g].w};
          const float wa[4] = {wv[cur][g].x, wv[cur][g].y, wv[cur][g].z, wv[cur][g].w};
#pragma unroll
          for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[p][q] = __builtin_fmaf(xa[p], wa[q], acc[p][q]);
        }
      }
    }
  }
  __syncthreads();

  // logits [TB][Epad + 1] (aliasing the staging area), then top-k per token
  const int zp = Epad + 1;
  float* zs = smem;
  if (active) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = es * 4 * EL + 4 * el + q;
      const float b = (a.bias && e < a.E) ? a.bias[e] : 0.0f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float z = acc[p][q];
        if (a.bias) z = z + b;
        zs[(tg * TPU + 4 * tl + p) * zp + e] = z;
      }
    }
  }
  __syncthreads();

  // selection: LP lanes per token (the power of two covering E, at most 64)
  const int LPS = a.E >= 64 ? 6 : (a.E <= 1 ? 0 : 32 - __builtin_clz(a.E - 1));  // log2 LP
  switch (LPS) {
    case 6: select_topk<6>(a, zs, zp, t0, TB, wave, lane); break;
    case 5: select_topk<5>(a, zs, zp, t0, TB, wave, lane); break;
    case 4: select_topk<4>(a, zs, zp, t0, TB, wave, lane); break;
    case 3: select_topk<3>(a, zs, zp, t0, TB, wave, lane); break;
    case 2: select_topk<2>(a, zs, zp, t0, TB, wave, lane); break;
    case 1: select_topk<1>(a, zs, zp, t0, TB, wave, lane); break;
    default: select_topk<0>(a, zs, zp, t0, TB, wave, lane); break;
  }
}

}  // namespace

// Block geometry: EL expert lanes per wave (4 experts each; a power of two up
// to 64), ESETS sets of 4 EL experts, TB tokens per block (four wave units
// when the expert sets allow, fewer while the T tokens would leave CUs
// without a block), dc-wide d chunks (smaller when a block holds many tokens
// or experts).  Returns the units per wave.
int route_geometry(int E, int T, int* EL, int* ESETS, int* TB, int* dc) {
  int el = 1;
  while (el < 64 && 4 * el < E) el <<= 1;
  *EL = el;
  *ESETS = (E + 4 * el - 1) / (4 * el);
  const int tpu = (64 / el) * 4;
  *TB = *ESETS >= 4 ? tpu : tpu * (4 / *ESETS);
  while (*TB > tpu && (T + *TB - 1) / *TB < kRouteMinBlocks) *TB >>= 1;
  int c = 32;
  while (c > 8 && (size_t)c * (*TB + *ESETS * 4 * el + 4) > 12288) c >>= 1;
  *dc = c;
  const int units = *ESETS * (*TB / tpu);
  return (units + 3) / 4;
}

size_t route_smem_bytes(int E, int T) {
  int EL, ES, TB, dc;
  route_geometry(E, T, &EL, &ES, &TB, &dc);
  const size_t Epad = (size_t)ES * 4 * EL;
  const size_t stage = 2 * ((size_t)dc * TB + (size_t)dc * (Epad + 4));
  const size_t logits = (size_t)TB * (Epad + 1);
  return sizeof(float) * (stage > logits ? stage : logits);
}

mok_status launch_route(int prec, const SrcTable& src, int src_lo, int T_src, int T, int d,
                        int E, int k, const void* w, const float* bias, int32_t* topk_idx,
                        float* topk_gate, hipStream_t stream, mok_trace* tr) {
  if (T == 0) return MOK_OK;
  RouteArgs a;
  a.src = src;
  a.src_lo = src_lo;
  a.T_src = T_src;
  a.w = w;
  a.bias = bias;
  a.topk_idx = topk_idx;
  a.topk_gate = topk_gate;
  a.T = T;
  a.d = d;
  a.E = E;
  a.k = k;
  const int upw = route_geometry(E, T, &a.EL, &a.ESETS, &a.TB, &a.dc);
  if (d % a.dc != 0 || upw != 1) return MOK_ESHAPE;
  // staging units per thread (both operands) must fit the kernel's slots
  const int U = prec == MOK_F32 ? 4 : 8;
  const int per = (a.ESETS * 4 * a.EL * (a.dc / U) + kRouteThreads - 1) / kRouteThreads;
  const int perx = (a.TB * (a.dc / U) + kRouteThreads - 1) / kRouteThreads;
  const int need = per > perx ? per : perx;
  const int pt = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
  if (need > 8) return MOK_ESHAPE;
  const size_t smem = route_smem_bytes(E, T);
  dim3 grid((T + a.TB - 1) / a.TB);
  dim3 blk(kRouteThreads);
#define MOK_ROUTE_LAUNCH(TY, DCV, PTV) \
  hipLaunchKernelGGL((route_kernel<TY, DCV, PTV>), grid, blk, smem, stream, a)
#define MOK_ROUTE_PT(TY, DCV)                          \
  do {                                                 \
    if (pt == 1) MOK_ROUTE_LAUNCH(TY, DCV, 1);         \
    else if (pt == 2) MOK_ROUTE_LAUNCH(TY, DCV, 2);    \
    else if (pt == 4) MOK_ROUTE_LAUNCH(TY, DCV, 4);    \
    else MOK_ROUTE_LAUNCH(TY, DCV, 8);                 \
  } while (0)
#define MOK_ROUTE_DC(TY)                               \
  do {                                                 \
    if (a.dc == 32) MOK_ROUTE_PT(TY, 32);              \
    else if (a.dc == 16) MOK_ROUTE_PT(TY, 16);         \
    else MOK_ROUTE_PT(TY, 8);                          \
  } while (0)
  if (prec == MOK_F32) MOK_ROUTE_DC(float);
  else MOK_ROUTE_DC(bf16_t);
#undef MOK_ROUTE_DC
#undef MOK_ROUTE_PT
#undef MOK_ROUTE_LAUNCH
  trace_mark(tr, "route", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

}  // namespace mok
