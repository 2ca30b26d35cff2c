// Expert-contiguous layout: per-expert histogram, exclusive scan, stable rank.
//
// kucoin article, section 01: before a grouped GEMM can run, the system counts
// the tokens of every expert, decides where they go and groups each expert's
// tokens together.  Section 02: with pull dispatch the receiver only needs the
// (source, position) of every token and picks its own placement, ordered by
// local expert.  Here every routed item n = (s*T_src + t)*k + j whose expert
// is local gets a row; rows of one expert keep ascending n (a stable counting
// sort), so the layout is a pure function of the routing.
//
// Three launches, all integer work:
//   1. count : one wave per chunk of kChunk items -> per-chunk expert histogram
//   2. scan  : one block; per expert an exclusive scan over chunks, then over
//              experts -> counts, offsets, per-(chunk, expert) base rows
//   3. place : one wave per chunk; 64 items at a time, a wave-ballot multisplit
//              on the 8 bits of the local expert id gives each lane its peers
//              with the same key, rank = popcount(peers below me), then the
//              per-expert cursor advances by the group size.
#include "mok_internal.h"

namespace mok {

namespace {

// items per chunk: one wave counts and places a chunk.  Measured: 2048 /
// 1024 / 512 gave 72 / 60 / 61 us for the three launches on the mid-size
// layer (98304 items) and 66 / 55 / 58 us on the 256-expert share (smaller
// chunks mean more waves but a longer scan over them).
constexpr int kChunk = 1024;

struct LayoutArgs {
  const int32_t* topk;     // [N]
  const int32_t* e2l;      // [E]
  int32_t* counts;         // [E_local]
  int32_t* offsets;        // [E_local+1]
  int32_t* row_src;        // [R_cap]
  int32_t* dest_row;       // [N]
  int32_t* chunk_base;     // [nchunk][E_local] workspace
  int32_t* status;
  int64_t N;
  int E, E_local, R_cap, nchunk;
};

__device__ __forceinline__ int local_expert(const LayoutArgs& a, int64_t n, bool report) {
  int e = a.topk[n];
  if (e < 0 || e >= a.E) {
    if (report) latch(a.status, MOK_EROUTE);
    return -1;
  }
  int le = a.e2l[e];
  if (le >= a.E_local) {  // a malformed expert_to_local entry: treated as remote
    if (report) latch(a.status, MOK_EROUTE);
    return -1;
  }
  return le < 0 ? -1 : le;
}

__global__ __launch_bounds__(64) void layout_count(LayoutArgs a) {
  __shared__ int hist[256];
  const int lane = threadIdx.x;
  for (int e = lane; e < a.E_local; e += 64) hist[e] = 0;
  __syncthreads();
  const int64_t n0 = (int64_t)blockIdx.x * kChunk;
  const int64_t n1 = n0 + kChunk < a.N ? n0 + kChunk : a.N;
  for (int64_t n = n0 + lane; n < n1; n += 64) {
    int le = local_expert(a, n, true);
    if (le >= 0) atomicAdd(&hist[le], 1);
  }
  __syncthreads();
  for (int e = lane; e < a.E_local; e += 64)
    a.chunk_base[(int64_t)blockIdx.x * a.E_local + e] = hist[e];
}

// Exclusive scan of the per-chunk counts of every local expert (over chunks,
// then over experts).  The 256 threads split each expert's column of chunk
// counts into segments: tpe = 256 / E_local threads per expert, each summing
// a contiguous run of chunks; the segment sums are scanned in LDS, and every
// thread then writes the global starting rows of its chunks.
__global__ __launch_bounds__(256) void layout_scan(LayoutArgs a) {
  __shared__ int part[256];
  __shared__ int off[257];
  const int tid = threadIdx.x;
  const int tpe = 256 / a.E_local;  // E_local <= 256
  const int e = tid / tpe, sub = tid % tpe;
  const bool act = e < a.E_local;
  const int L = (a.nchunk + tpe - 1) / tpe;
  const int c0 = sub * L, c1 = min(a.nchunk, c0 + L);
  int sum = 0;
  if (act)
    for (int c = c0; c < c1; ++c) sum += a.chunk_base[(int64_t)c * a.E_local + e];
  part[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int x = 0; x < a.E_local; ++x) {
      off[x] = run;
      for (int q = 0; q < tpe; ++q) run += part[x * tpe + q];
    }
    off[a.E_local] = run;
    if (run > a.R_cap) latch(a.status, MOK_ECAPACITY);
  }
  __syncthreads();
  if (act) {
    int run = off[e];
    for (int q = 0; q < sub; ++q) run += part[e * tpe + q];
    for (int c = c0; c < c1; ++c) {
      const int64_t i = (int64_t)c * a.E_local + e;
      const int v = a.chunk_base[i];
      a.chunk_base[i] = run;
      run += v;
    }
    if (sub == 0) {
      a.counts[e] = off[e + 1] - off[e];
      a.offsets[e] = off[e];
    }
  }
  if (tid == 0) a.offsets[a.E_local] = off[a.E_local];
}

__global__ __launch_bounds__(64) void layout_place(LayoutArgs a) {
  __shared__ int cursor[256];
  const int lane = threadIdx.x;
  for (int e = lane; e < a.E_local; e += 64)
    cursor[e] = a.chunk_base[(int64_t)blockIdx.x * a.E_local + e];
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t n0 = (int64_t)blockIdx.x * kChunk;
  const int64_t n1 = n0 + kChunk < a.N ? n0 + kChunk : a.N;
  for (int64_t base = n0; base < n1; base += 64) {
    const int64_t n = base + lane;
    const bool in = n < n1;
    const int le = in ? local_expert(a, n, false) : -1;
    const bool valid = le >= 0;
    // peers: lanes with the same (valid) key
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      uint64_t m = __ballot(valid && ((le >> b) & 1));
      peers &= ((le >> b) & 1) ? m : ~m;
    }
    int row = -1;
    if (valid) {
      const int rank = __popcll(peers & below);
      row = cursor[le] + rank;
    }
    __syncthreads();  // every lane has read its cursor before the leaders advance it
    if (valid) {
      const int cnt = __popcll(peers);
      const int leader = 63 - __clzll(peers);  // highest lane of the group
      if (leader == lane) cursor[le] += cnt;
    }
    __syncthreads();
    if (in) {
      // a local item past the capacity keeps its row number (>= R_cap): the
      // consumers skip it, where -1 would read it as a remote slot
      if (valid && row < a.R_cap) a.row_src[row] = (int32_t)n;
      a.dest_row[n] = valid ? row : -1;
    }
  }
}

}  // namespace

size_t layout_ws_bytes(int64_t N, int E_local) {
  int64_t nchunk = (N + kChunk - 1) / kChunk;
  if (nchunk < 1) nchunk = 1;
  return (size_t)nchunk * (size_t)E_local * sizeof(int32_t);
}

mok_status launch_layout(int64_t N, int E, int E_local, int R_cap, const int32_t* topk,
                         const int32_t* e2l, int32_t* counts, int32_t* offsets, int32_t* row_src,
                         int32_t* dest_row, void* ws, int32_t* status, hipStream_t stream,
                         mok_trace* tr) {
  LayoutArgs a;
  a.topk = topk;
  a.e2l = e2l;
  a.counts = counts;
  a.offsets = offsets;
  a.row_src = row_src;
  a.dest_row = dest_row;
  a.chunk_base = reinterpret_cast<int32_t*>(ws);
  a.status = status;
  a.N = N;
  a.E = E;
  a.E_local = E_local;
  a.R_cap = R_cap;
  a.nchunk = (int)((N + kChunk - 1) / kChunk);
  if (a.nchunk > 0) hipLaunchKernelGGL(layout_count, dim3(a.nchunk), dim3(64), 0, stream, a);
  trace_mark(tr, "layout_count", stream);
  hipLaunchKernelGGL(layout_scan, dim3(1), dim3(256), 0, stream, a);
  trace_mark(tr, "layout_scan", stream);
  if (a.nchunk > 0) hipLaunchKernelGGL(layout_place, dim3(a.nchunk), dim3(64), 0, stream, a);
  trace_mark(tr, "layout_place", stream);
  return hipGetLastError() == hipSuccess ? MOK_OK : MOK_EDEVICE;
}

}  // namespace mok
