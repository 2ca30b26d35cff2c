// Data movement kernels: pull dispatch (gather, optionally MX-quantising),
// push combine, final weighted combine, and the E4M3/E8M0 row quantiser.
//
// All of them stream rows with 16-byte vector loads and stores; consecutive
// lanes touch consecutive 16-byte units of one row, so every wave moves whole
// 1 KiB spans of HBM.  They are bound by HBM bandwidth.
#include "mok_combine.h"
#include "mok_internal.h"
#include "mok_mx.h"

namespace mok {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- dispatch
struct GatherArgs {
  SrcTable src;          // S pointers [T_src, d]
  const int32_t* row_src;
  const int32_t* offsets;
  void* dst;             // [R_cap, d] (activation dtype or E4M3 codes)
  uint8_t* dst_scale;    // [R_cap, d/32] for MX
  int T_src, d, k, E_local, R_cap;
  int rows_per_block;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void gather_kernel(GatherArgs a) {
  int R = a.offsets[a.E_local];
  if (R > a.R_cap) R = a.R_cap;
  constexpr int U = 16 / sizeof(T);
  const int units = a.d / U;
  const int r0 = blockIdx.x * a.rows_per_block;
  for (int rr = 0; rr < a.rows_per_block; ++rr) {
    const int r = r0 + rr;
    if (r >= R) return;
    const int n = a.row_src[r];
    const int tok = n / a.k;
    const int s = tok / a.T_src, t = tok % a.T_src;
    const T* src = reinterpret_cast<const T*>(a.src.p[s]) + (size_t)t * a.d;
    T* dst = reinterpret_cast<T*>(a.dst) + (size_t)r * a.d;
    for (int u = threadIdx.x; u < units; u += kThreads) st16(dst + u * U, ld16(src + u * U));
  }
}

// MX gather: a 32-element block is 4 consecutive 16-byte units (4 lanes).
// The block's rows (kGatherRows) are loaded together before any is
// quantised, so that many 16-byte loads per lane are in flight at once.
constexpr int kGatherRows = 4;
// workgroups per CU of the persistent combine (C2: 108 / 94 / 92 µs with
// 4 / 8 / 16; one workgroup per token pair had taken 97 µs)
constexpr int kCombineWgsPerCu = 16;

__device__ __forceinline__ void mx_encode_unit(const uint4& q, bool have, uint8_t* dst,
                                               uint8_t* dsc, int u) {
  float v[8];
  float amax = 0.0f;
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  if (!have) amax = 0.0f;
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  if (have) {
    const int sh = mx_shared_exp(amax);
    const uint32_t lo = e4m3_pack4(v[0], v[1], v[2], v[3], sh);
    const uint32_t hi = e4m3_pack4(v[4], v[5], v[6], v[7], sh);
    *reinterpret_cast<uint2*>(dst + u * 8) = make_uint2(lo, hi);
    if ((u & 3) == 0) dsc[u >> 2] = (uint8_t)(sh + 127);
  }
}

// (row groups walked with the grid's stride; the launch covers them all)
__global__ __launch_bounds__(kThreads) void gather_mx_kernel(GatherArgs a) {
  int R = a.offsets[a.E_local];
  if (R > a.R_cap) R = a.R_cap;
  const int units = a.d / 8;
  for (int r0 = blockIdx.x * kGatherRows; r0 < R; r0 += gridDim.x * kGatherRows) {
  const int nr = min(kGatherRows, R - r0);
  const bf16_t* src[kGatherRows];
#pragma unroll
  for (int rr = 0; rr < kGatherRows; ++rr) {
    const int n = a.row_src[r0 + min(rr, nr - 1)];
    const int tok = n / a.k;
    const int s = tok / a.T_src, t = tok % a.T_src;
    src[rr] = reinterpret_cast<const bf16_t*>(a.src.p[s]) + (size_t)t * a.d;
  }
  for (int u0 = 0; u0 < units; u0 += kThreads) {
    const int u = u0 + threadIdx.x;
    const bool have = u < units;  // units % 4 == 0: a 4-lane group is all in or all out
    uint4 q[kGatherRows];
#pragma unroll
    for (int rr = 0; rr < kGatherRows; ++rr)
      q[rr] = (have && rr < nr) ? ld16(src[rr] + u * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int rr = 0; rr < kGatherRows; ++rr) {
      if (rr >= nr) break;  // uniform over the block
      const int r = r0 + rr;
      mx_encode_unit(q[rr], have, reinterpret_cast<uint8_t*>(a.dst) + (size_t)r * a.d,
                     a.dst_scale + (size_t)r * (a.d / 32), u);
    }
  }
  }
}

// ---------------------------------------------------------------- push combine
// Item-indexed: every item n with a local row pushes y[dest_row[n]] to its
// (source, token, slot) staging row.
struct PushArgs {
  const void* y;           // [R_cap, d] rows in expert order
  const int32_t* dest_row; // [N]
  DstTable staging;        // S pointers [T_src*k, d]
  int64_t N;
  int T_src, d, k, R_cap;
  int items_per_block;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void push_kernel(PushArgs a) {
  constexpr int U = 16 / sizeof(T);
  const int units = a.d / U;
  for (int q = 0; q < a.items_per_block; ++q) {
    const int64_t n = (int64_t)blockIdx.x * a.items_per_block + q;
    if (n >= a.N) return;
    const int r = a.dest_row[n];
    if (r < 0 || r >= a.R_cap) continue;
    const int64_t tok = n / a.k;
    const int j = (int)(n % a.k);
    const int s = (int)(tok / a.T_src), t = (int)(tok % a.T_src);
    const T* src = reinterpret_cast<const T*>(a.y) + (size_t)r * a.d;
    T* dst = reinterpret_cast<T*>(a.staging.p[s]) + ((size_t)t * a.k + j) * a.d;
    for (int u = threadIdx.x; u < units; u += kThreads) st16(dst + u * U, ld16(src + u * U));
  }
}

// ---------------------------------------------------------------- final combine
struct CombineArgs {
  const int32_t* dest_row;  // [S*T_src*k]
  const float* gate;        // [S*T_src*k]
  DstTable staging;         // S pointers [T_src*k, d]
  DstTable out;             // S pointers [T_src, d]
  int T_src, d, k, own_lo, R_cap;
  int64_t n_tok;            // own tokens
};

// A token's k slot units are loaded together before any is summed (K known
// at compile time for the common top-k values, so the k 16-byte loads per
// lane go out back to back); a slot that is not summed -- a local row
// dropped beyond R_cap -- is loaded from its staging row (which exists) and
// left out of the sum, which keeps the sum's order and rounding.  K = 0:
// any k, one slot at a time.
template <typename T, int K>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  constexpr int U = 16 / sizeof(T);
  const int units = a.d / U;
  // a persistent grid walks the tokens with a stride of the grid: no
  // workgroup launch per token, and every CU keeps its slot loads coming
  for (int64_t g = blockIdx.x; g < a.n_tok; g += gridDim.x) {
    const int s = a.own_lo + (int)(g / a.T_src);
    const int t = (int)(g % a.T_src);
    const int64_t n0 = ((int64_t)s * a.T_src + t) * a.k;
    const T* stg = reinterpret_cast<const T*>(a.staging.p[s]) + (size_t)t * a.k * a.d;
    T* o = reinterpret_cast<T*>(a.out.p[s]) + (size_t)t * a.d;
    if constexpr (K == 0) {
      combine_token<T>(a.dest_row, a.gate, n0, a.k, a.R_cap, stg, o, a.d, threadIdx.x, kThreads);
    } else {
      // the same sums as combine_token, with the K slot loads issued first
      for (int u = threadIdx.x; u < units; u += kThreads) {
        float acc[U];
#pragma unroll
        for (int i = 0; i < U; ++i) acc[i] = 0.0f;
        uint4 v[K];
#pragma unroll
        for (int j = 0; j < K; ++j) v[j] = ld16(stg + (size_t)j * a.d + u * U);
#pragma unroll
        for (int j = 0; j < K; ++j) {
          if (a.dest_row[n0 + j] >= a.R_cap) continue;
          const float gj = a.gate[n0 + j];
          const T* e = reinterpret_cast<const T*>(&v[j]);
#pragma unroll
          for (int i = 0; i < U; ++i) acc[i] = __builtin_fmaf(gj, to_f32<T>(e[i]), acc[i]);
        }
        uint4 outv;
        T* ov = reinterpret_cast<T*>(&outv);
#pragma unroll
        for (int i = 0; i < U; ++i) ov[i] = from_f32<T>(acc[i]);
        st16(o + u * U, outv);
      }
    }
  }
}

// ---------------------------------------------------------------- MX rows
struct MxArgs {
  const void* src;  // bf16 or fp32 values
  uint8_t* codes;
  uint8_t* scales;
  int64_t rows, K;
};

// The 8 values of 16-byte unit u of the source as floats.
template <typename T>
__device__ __forceinline__ void mx_unit(const void* src, int64_t u, float* v) {
  if constexpr (sizeof(T) == 2) {
    const uint4 q = ld16(reinterpret_cast<const bf16_t*>(src) + u * 8);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float* p = reinterpret_cast<const float*>(src) + u * 8;
    const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void mx_quantize_kernel(MxArgs a) {
  // one 16-byte unit (8 values) per thread; 4 threads per 32-value block
  const int64_t units = a.rows * (a.K / 8);
  for (int64_t u0 = (int64_t)blockIdx.x * kThreads; u0 < units; u0 += (int64_t)gridDim.x * kThreads) {
    const int64_t u = u0 + threadIdx.x;
    const bool have = u < units;  // units % 4 == 0 and u0 % 4 == 0
    float v[8];
    float amax = 0.0f;
    if (have) {
      mx_unit<T>(a.src, u, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    if (have) {
      const int sh = mx_shared_exp(amax);
      const uint32_t lo = e4m3_pack4(v[0], v[1], v[2], v[3], sh);
      const uint32_t hi = e4m3_pack4(v[4], v[5], v[6], v[7], sh);
      *reinterpret_cast<uint2*>(a.codes + u * 8) = make_uint2(lo, hi);
      if ((u & 3) == 0) a.scales[u >> 2] = (uint8_t)(sh + 127);
    }
  }
}

}  // namespace

// ---------------------------------------------------------------- launchers
mok_status launch_gather(int prec, const SrcTable& src, int T_src, int d, int k, int E_local,
                         int R_cap, const int32_t* row_src, const int32_t* offsets, void* dst,
                         uint8_t* dst_scale, hipStream_t stream, mok_trace* tr) {
  if (R_cap == 0) return MOK_OK;
  GatherArgs a;
  a.src = src;
  a.row_src = row_src;
  a.offsets = offsets;
  a.dst = dst;
  a.dst_scale = dst_scale;
  a.T_src = T_src;
  a.d = d;
  a.k = k;
  a.E_local = E_local;
  a.R_cap = R_cap;
  a.rows_per_block = prec == MOK_MXFP8 ? kGatherRows : 4;
  // (one workgroup per row group: measured faster for the MX gather than a
  // persistent grid of 4, 8 or 16 workgroups per CU)
  dim3 grid((R_cap + a.rows_per_block - 1) / a.rows_per_block);
  if (prec == MOK_F32)
    hipLaunchKernelGGL(gather_kernel<float>, grid, dim3(kThreads), 0, stream, a);
  else if (prec == MOK_BF16)
    hipLaunchKernelGGL(gather_kernel<bf16_t>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(gather_mx_kernel, grid, dim3(kThreads), 0, stream, a);
  trace_mark(tr, "gather", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

mok_status launch_push(int prec, const void* y, const int32_t* dest_row, int64_t N,
                       const DstTable& staging, int T_src, int d, int k, int R_cap,
                       hipStream_t stream, mok_trace* tr) {
  if (N == 0) return MOK_OK;
  PushArgs a;
  a.y = y;
  a.dest_row = dest_row;
  a.staging = staging;
  a.N = N;
  a.T_src = T_src;
  a.d = d;
  a.k = k;
  a.R_cap = R_cap;
  a.items_per_block = 4;
  dim3 grid((unsigned)((N + a.items_per_block - 1) / a.items_per_block));
  if (prec == MOK_F32)
    hipLaunchKernelGGL(push_kernel<float>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(push_kernel<bf16_t>, grid, dim3(kThreads), 0, stream, a);
  trace_mark(tr, "push", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

mok_status launch_combine(int prec, const int32_t* dest_row, const float* gate,
                          const DstTable& staging, const DstTable& out, int T_src, int d, int k,
                          int own_lo, int own_n, int R_cap, hipStream_t stream,
                          mok_trace* tr) {
  CombineArgs a;
  a.dest_row = dest_row;
  a.gate = gate;
  a.staging = staging;
  a.out = out;
  a.T_src = T_src;
  a.d = d;
  a.k = k;
  a.own_lo = own_lo;
  a.R_cap = R_cap;
  a.n_tok = (int64_t)own_n * T_src;
  if (a.n_tok == 0) return MOK_OK;
  const int cus = device_cus();
  if (cus <= 0) return MOK_EDEVICE;
  const int64_t wgs = (int64_t)cus * kCombineWgsPerCu;
  dim3 grid((unsigned)(a.n_tok < wgs ? a.n_tok : wgs));
  if (prec == MOK_F32) {
    hipLaunchKernelGGL((combine_kernel<float, 0>), grid, dim3(kThreads), 0, stream, a);
  } else {
    switch (k) {
      case 2: hipLaunchKernelGGL((combine_kernel<bf16_t, 2>), grid, dim3(kThreads), 0, stream, a); break;
      case 4: hipLaunchKernelGGL((combine_kernel<bf16_t, 4>), grid, dim3(kThreads), 0, stream, a); break;
      case 6: hipLaunchKernelGGL((combine_kernel<bf16_t, 6>), grid, dim3(kThreads), 0, stream, a); break;
      case 8: hipLaunchKernelGGL((combine_kernel<bf16_t, 8>), grid, dim3(kThreads), 0, stream, a); break;
      default: hipLaunchKernelGGL((combine_kernel<bf16_t, 0>), grid, dim3(kThreads), 0, stream, a);
    }
  }
  trace_mark(tr, "combine", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

mok_status launch_mx_quantize(int64_t rows, int64_t K, const void* src, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream, bool f32) {
  MxArgs a;
  a.src = src;
  a.codes = codes;
  a.scales = scales;
  a.rows = rows;
  a.K = K;
  int64_t units = rows * (K / 8);
  if (units == 0) return MOK_OK;
  int64_t blocks = (units + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  if (f32)
    hipLaunchKernelGGL(mx_quantize_kernel<float>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(mx_quantize_kernel<bf16_t>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

}  // namespace mok
