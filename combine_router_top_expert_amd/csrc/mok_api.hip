// C ABI of the library (declared in include/mok.h): argument validation,
// workspace carving and launch sequencing.  No allocation, no host sync.
#include <string.h>

#include <mutex>

#include "mok_internal.h"

using namespace mok;

namespace {

constexpr int kTuneMax = 64;  // candidates per tuned parameter

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t act_bytes(int prec) { return prec == MOK_F32 ? 4 : 2; }

bool valid_cfg(const mok_config* c) {
  if (!c) return false;
  if (c->S < 1 || c->S > MOK_MAX_SOURCES || c->T_src < 0) return false;
  if (c->d <= 0 || c->d % 64 != 0) return false;
  if (c->I <= 0 || c->I % 64 != 0) return false;
  if (c->E < 1 || c->E > 512) return false;
  if (c->k < 1 || c->k > 16 || c->k > c->E) return false;
  if (c->E_local < 1 || c->E_local > 256 || c->E_local > c->E) return false;
  if (c->prec != MOK_F32 && c->prec != MOK_BF16 && c->prec != MOK_MXFP8) return false;
  if (c->R_cap < 0) return false;
  int64_t N = (int64_t)c->S * c->T_src * c->k;
  if (N > 0x7FFFFFFF) return false;  // items are indexed by int32
  if (c->ring_bytes < 0) return false;
  if (c->ring_bytes > 0 && c->minibatch_rows < 1) return false;
  if (c->comm_wgs < 0 || c->gemm_wgs < 0 || c->wait_limit_us < 0) return false;
  if (c->bwd_ring_bytes < 0) return false;
  if (c->bwd_ring_bytes > 0 && c->minibatch_rows < 1) return false;
  return true;
}

struct Ws {
  size_t layout, xperm, xscale, hscale, ring, ring_ctr, dy, dab, dz, dwr, r_ident, r_counts, r_offsets,
      r_row_src, r_dest_row, r_scratch, bx, bh, wpart, wpart_down, worder, bwin, bring, mx_dyq,
      mx_dys, mx_dabq, mx_dabs, mx_dabT, mx_dabTs, mx_xT, mx_xTs, mx_dyT, mx_dyTs, mx_hT,
      mx_hTs, total;
};

// The bf16 backward runs through the ring (window by window) when cfg has one.
bool bwd_through_ring(const mok_config* c) {
  return c->bwd_ring_bytes > 0 && c->prec == MOK_BF16 && c->R_cap > 0;
}

Ws ws_layout(const mok_config* c) {
  Ws w;
  const int64_t N = (int64_t)c->S * c->T_src * c->k;
  const size_t R = (size_t)c->R_cap;
  size_t off = 0;
  w.layout = off;
  off += align256(layout_ws_bytes(N, c->E_local));
  const size_t base = off;
  // forward pieces
  size_t f = base;
  w.xperm = f;
  f += align256(c->prec == MOK_MXFP8 ? R * c->d : R * c->d * act_bytes(c->prec));
  w.xscale = f;
  f += align256(c->prec == MOK_MXFP8 ? R * (c->d / 32) : 0);
  w.hscale = f;  // MXFP8: scales of h, one region per call of the ring path
  f += align256(c->prec == MOK_MXFP8 ? R * (c->I / 32) * (c->ring_bytes > 0 ? kRingMaxCalls : 1)
                                     : 0);
  w.ring = f;
  w.ring_ctr = f;
  if (c->ring_bytes > 0) {
    f += align256((size_t)c->ring_bytes);
    w.ring_ctr = f;
    f += align256(ring_meta_bytes(c->R_cap, c->E_local, c->minibatch_rows));
  }
  // backward pieces (same region); through the ring, dy, dab and the
  // transposed token rows are a window's, in the ring region at the end
  const bool bring = bwd_through_ring(c);
  size_t b = base;
  w.dy = b;
  if (!bring) b += align256(R * c->d * act_bytes(c->prec));
  w.dab = b;
  if (!bring) b += align256(R * 2 * c->I * act_bytes(c->prec));
  w.dz = b;
  b += align256((size_t)N * sizeof(float));
  w.dwr = b;
  b += align256(((size_t)N / 64 + c->E) * c->d * sizeof(float));
  w.r_ident = b;
  b += align256((size_t)c->E * sizeof(int32_t));
  w.r_counts = b;
  b += align256((size_t)c->E * sizeof(int32_t));
  w.r_offsets = b;
  b += align256((size_t)(c->E + 1) * sizeof(int32_t));
  w.r_row_src = b;
  b += align256((size_t)N * sizeof(int32_t));
  w.r_dest_row = b;
  b += align256((size_t)N * sizeof(int32_t));
  w.r_scratch = b;
  b += align256(c->E <= 256 ? layout_ws_bytes(N, c->E) : 0);
  w.bx = b;
  if (!bring && c->prec != MOK_MXFP8)
    b += align256(c->prec == MOK_BF16 ? (size_t)c->d * xt_ld(c->R_cap, c->E_local) * 2
                                      : R * c->d * act_bytes(c->prec));
  // h transposed like the token rows, for the down projection's weight
  // gradient (one-launch bf16 backward)
  w.bh = b;
  if (!bring && c->prec == MOK_BF16) b += align256((size_t)c->I * xt_ld(c->R_cap, c->E_local) * 2);
  w.wpart = b;
  b += align256(c->prec == MOK_BF16 ? wgrad_partial_bytes(c->R_cap, c->d, c->I) : 0);
  // through the ring both weight gradients keep their partials until the
  // last window: the down projection's get a region of their own (half size)
  w.wpart_down = b;
  if (bring) b += align256(wgrad_partial_bytes(c->R_cap, c->d, c->I) / 2);
  w.worder = b;
  b += align256((size_t)c->E_local * sizeof(int32_t));
  w.bwin = b;
  b += align256((size_t)(4 + c->E_local) * sizeof(int32_t));
  w.bring = b;
  if (bring) b += align256((size_t)c->bwd_ring_bytes);
  // MXFP8 backward: the quantised rows of dy and da | db and the weight
  // gradients' operands transposed (every expert's rows padded to 128
  // columns), each E4M3 codes + E8M0 scales per 32
  const bool mx = c->prec == MOK_MXFP8;
  const size_t cols = mx ? (size_t)bwd_mx_cols(c->R_cap, c->E_local) : 0;
  const size_t d = (size_t)c->d, I2 = 2 * (size_t)c->I;
  size_t* const regions[12] = {&w.mx_dyq, &w.mx_dys, &w.mx_dabq, &w.mx_dabs,
                               &w.mx_dabT, &w.mx_dabTs, &w.mx_xT, &w.mx_xTs, &w.mx_dyT,
                               &w.mx_dyTs, &w.mx_hT, &w.mx_hTs};
  const size_t bytes[12] = {R * d, R * d / 32, R * I2, R * I2 / 32,
                            I2 * cols, I2 * cols / 32, d * cols, d * cols / 32, d * cols,
                            d * cols / 32, I2 / 2 * cols, I2 / 2 * cols / 32};
  for (int i = 0; i < 12; ++i) {
    *regions[i] = b;
    if (mx) b += align256(bytes[i]);
  }
  w.total = f > b ? f : b;
  return w;
}

template <class Tab>
bool fill_table(Tab* tab, const void* const* ptrs, int S) {
  if (!ptrs) return false;
  memset(tab, 0, sizeof(*tab));
  for (int s = 0; s < S; ++s) tab->p[s] = (decltype(tab->p[0]))ptrs[s];
  return true;
}

bool own_range_ok(const mok_config* c, int own_lo, int own_n) {
  return own_lo >= 0 && own_n >= 0 && own_lo + own_n <= c->S;
}

// Per-source pointer arrays.  Which sources have items routed to a local
// expert is known on the device only, so a call that pulls from or pushes
// to the sources needs all S entries (when there are tokens at all); the
// final combine and the per-token sums touch the own sources only.
bool all_sources_set(const void* const* p, int S, int T_src) {
  if (!p) return false;
  if (T_src == 0) return true;
  for (int s = 0; s < S; ++s)
    if (!p[s]) return false;
  return true;
}

bool own_sources_set(const void* const* p, int own_lo, int own_n, int T_src) {
  if (own_n == 0 || T_src == 0) return true;
  if (!p) return false;
  for (int s = own_lo; s < own_lo + own_n; ++s)
    if (!p[s]) return false;
  return true;
}

}  // namespace

extern "C" {

const char* mok_version(void) { return "mok 0.1 gfx950"; }

size_t mok_workspace_bytes(const mok_config* cfg) {
  if (!valid_cfg(cfg)) return 0;
  return ws_layout(cfg).total;
}

mok_status mok_route(const mok_config* cfg, int32_t T, const void* x, const void* w_router,
                     const float* bias, int32_t* topk_idx, float* topk_gate, void* stream) {
  if (!valid_cfg(cfg) || T < 0) return MOK_EINVAL;
  if (T > 0 && (!x || !w_router || !topk_idx || !topk_gate)) return MOK_EINVAL;
  trace_mark(cfg->trace, "start", (hipStream_t)stream);
  SrcTable src;
  memset(&src, 0, sizeof(src));
  src.p[0] = x;
  const int rprec = cfg->prec == MOK_F32 ? MOK_F32 : MOK_BF16;
  return launch_route(rprec, src, 0, T > 0 ? T : 1, T, cfg->d, cfg->E, cfg->k, w_router, bias,
                      topk_idx, topk_gate, (hipStream_t)stream, cfg->trace);
}

mok_status mok_layout(const mok_config* cfg, const int32_t* topk_idx_all,
                      const int32_t* expert_to_local, int32_t* counts, int32_t* offsets,
                      int32_t* row_src, int32_t* dest_row, void* ws, int32_t* dev_status,
                      void* stream) {
  if (!valid_cfg(cfg)) return MOK_EINVAL;
  const int64_t N = (int64_t)cfg->S * cfg->T_src * cfg->k;
  if (!expert_to_local || !counts || !offsets || !ws) return MOK_EINVAL;
  if (N > 0 && (!topk_idx_all || !dest_row)) return MOK_EINVAL;
  if (cfg->R_cap > 0 && !row_src) return MOK_EINVAL;
  return launch_layout(N, cfg->E, cfg->E_local, cfg->R_cap, topk_idx_all, expert_to_local, counts,
                       offsets, row_src, dest_row, (char*)ws + ws_layout(cfg).layout, dev_status,
                       (hipStream_t)stream, cfg->trace);
}

mok_status mok_dispatch(const mok_config* cfg, const void* const* src_x, const int32_t* row_src,
                        const int32_t* offsets, void* x_perm, uint8_t* x_scale,
                        int32_t* dev_status, void* stream) {
  (void)dev_status;
  if (!valid_cfg(cfg)) return MOK_EINVAL;
  if (cfg->R_cap == 0) return MOK_OK;
  SrcTable src;
  if (!all_sources_set(src_x, cfg->S, cfg->T_src)) return MOK_EINVAL;
  if (!fill_table(&src, src_x, cfg->S) || !row_src || !offsets || !x_perm) return MOK_EINVAL;
  if (cfg->prec == MOK_MXFP8 && !x_scale) return MOK_EINVAL;
  trace_mark(cfg->trace, "start", (hipStream_t)stream);
  return launch_gather(cfg->prec, src, cfg->T_src, cfg->d, cfg->k, cfg->E_local, cfg->R_cap,
                       row_src, offsets, x_perm, x_scale, (hipStream_t)stream, cfg->trace);
}

mok_status mok_expert_ffn(const mok_config* cfg, const void* x_perm, const uint8_t* x_scale,
                          const int32_t* offsets, const mok_expert_weights* w, void* h,
                          uint8_t* h_scale, void* ab, void* y, int32_t* dev_status,
                          void* stream) {
  (void)dev_status;
  if (!valid_cfg(cfg) || !w || !offsets) return MOK_EINVAL;
  if (cfg->R_cap == 0) return MOK_OK;
  if (!x_perm || !w->w_gate || !w->w_up || !w->w_down || !h || !y) return MOK_EINVAL;
  if (cfg->prec == MOK_MXFP8) {
    if (!x_scale || !h_scale || !w->s_gate || !w->s_up || !w->s_down) return MOK_EINVAL;
    trace_mark(cfg->trace, "start", (hipStream_t)stream);
    return launch_ffn_mx(cfg->d, cfg->I, cfg->E_local, cfg->R_cap, (const uint8_t*)x_perm,
                         x_scale, offsets, nullptr, w, (uint8_t*)h, h_scale, ab, y, nullptr,
                         cfg->T_src, cfg->k, (hipStream_t)stream, cfg->trace);
  }
  trace_mark(cfg->trace, "start", (hipStream_t)stream);
  return launch_ffn(cfg->prec, cfg->d, cfg->I, cfg->E_local, cfg->R_cap, x_perm, offsets, nullptr,
                    w->w_gate, w->w_up, w->w_down, h, ab, y, nullptr, cfg->T_src, cfg->k,
                    (hipStream_t)stream, cfg->trace);
}

mok_status mok_combine(const mok_config* cfg, const void* y, const int32_t* dest_row,
                       const float* topk_gate, void* const* staging, int32_t own_lo,
                       int32_t own_n, void* const* out, int32_t* dev_status, void* stream) {
  (void)dev_status;
  if (!valid_cfg(cfg) || !own_range_ok(cfg, own_lo, own_n)) return MOK_EINVAL;
  const int64_t N = (int64_t)cfg->S * cfg->T_src * cfg->k;
  if (N == 0) return MOK_OK;
  DstTable stg, o;
  if (!fill_table(&stg, (const void* const*)staging, cfg->S) || !dest_row) return MOK_EINVAL;
  // the push reaches every source with a local row; the combine the own ones
  if (y && !all_sources_set((const void* const*)staging, cfg->S, cfg->T_src)) return MOK_EINVAL;
  if (own_n > 0) {
    if (!topk_gate || !own_sources_set((const void* const*)staging, own_lo, own_n, cfg->T_src) ||
        !own_sources_set((const void* const*)out, own_lo, own_n, cfg->T_src))
      return MOK_EINVAL;
  }
  const int prec = cfg->prec == MOK_F32 ? MOK_F32 : MOK_BF16;
  hipStream_t st = (hipStream_t)stream;
  if (y) {
    mok_status rc = launch_push(prec, y, dest_row, N, stg, cfg->T_src, cfg->d, cfg->k, cfg->R_cap,
                                st, cfg->trace);
    if (rc != MOK_OK) return rc;
  }
  if (own_n == 0) return MOK_OK;
  fill_table(&o, (const void* const*)out, cfg->S);
  return launch_combine(prec, dest_row, topk_gate, stg, o, cfg->T_src, cfg->d, cfg->k, own_lo,
                        own_n, cfg->R_cap, st, cfg->trace);
}

}  // extern "C"

namespace {

// Arguments of one forward call (the state, per-source tables and outputs).
mok_status check_call(const mok_config* cfg, int32_t own_lo, int32_t own_n,
                      const void* const* src_x, const mok_fwd_state* st, void* const* staging,
                      void* const* out) {
  if (!own_range_ok(cfg, own_lo, own_n)) return MOK_EINVAL;
  if (!src_x || !st || !staging) return MOK_EINVAL;
  if (!st->topk_idx || !st->topk_gate || !st->counts || !st->offsets || !st->dest_row)
    return MOK_EINVAL;
  if (cfg->R_cap > 0 && (!st->row_src || !st->h)) return MOK_EINVAL;
  // the pull reads and the push writes any source with a local row; the
  // router and the final combine touch the own sources
  if (cfg->R_cap > 0 && (!all_sources_set(src_x, cfg->S, cfg->T_src) ||
                         !all_sources_set((const void* const*)staging, cfg->S, cfg->T_src)))
    return MOK_EINVAL;
  if (!own_sources_set(src_x, own_lo, own_n, cfg->T_src) ||
      !own_sources_set((const void* const*)staging, own_lo, own_n, cfg->T_src) ||
      !own_sources_set((const void* const*)out, own_lo, own_n, cfg->T_src))
    return MOK_EINVAL;
  return MOK_OK;
}

// Router of the own sources, then the layout of all sources' items.
mok_status route_and_layout(const mok_config* cfg, int32_t own_lo, int32_t own_n,
                            const void* const* src_x, const void* w_router, const float* bias,
                            const int32_t* expert_to_local, const mok_fwd_state* st,
                            void* layout_ws, int32_t* dev_status, hipStream_t sm, mok_trace* tr) {
  const int64_t per_src = (int64_t)cfg->T_src * cfg->k;
  const int rprec = cfg->prec == MOK_F32 ? MOK_F32 : MOK_BF16;
  SrcTable src;
  fill_table(&src, src_x, cfg->S);
  mok_status rc = launch_route(rprec, src, own_lo, cfg->T_src, own_n * cfg->T_src, cfg->d, cfg->E,
                               cfg->k, w_router, bias, st->topk_idx + own_lo * per_src,
                               st->topk_gate + own_lo * per_src, sm, tr);
  if (rc != MOK_OK) return rc;
  return launch_layout((int64_t)cfg->S * cfg->T_src * cfg->k, cfg->E, cfg->E_local, cfg->R_cap,
                       st->topk_idx, expert_to_local, st->counts, st->offsets, st->row_src,
                       st->dest_row, layout_ws, dev_status, sm, tr);
}

// One call's descriptor for the ring kernel.
// Where the forward writes h's MX scales: the caller's buffer when the state
// has one (kept for the backward), else call c's region of the workspace.
uint8_t* h_scale_of(const mok_config* cfg, const mok_fwd_state* st, char* wsb, int c) {
  if (st->h_scale) return st->h_scale;
  return (uint8_t*)(wsb + ws_layout(cfg).hscale) + (size_t)c * cfg->R_cap * (cfg->I / 32);
}

RingCall ring_call(const mok_config* cfg, int32_t own_lo, int32_t own_n, const void* const* src_x,
                   const mok_fwd_state* st, void* const* staging, void* const* out,
                   uint8_t* h_scale) {
  RingCall c;
  memset(&c, 0, sizeof(c));
  fill_table(&c.src, src_x, cfg->S);
  fill_table(&c.staging, (const void* const*)staging, cfg->S);
  if (out) fill_table(&c.out, (const void* const*)out, cfg->S);
  c.row_src = st->row_src;
  c.offsets = st->offsets;
  c.dest_row = st->dest_row;
  c.gate = st->topk_gate;
  c.h = st->h;
  c.h_scale = h_scale;
  c.ab = st->ab;  // a | b for the backward pass (bf16 and MXFP8), or null
  c.own_lo = own_lo;
  c.own_n = own_n;
  return c;
}

// The ring launch of n_calls calls (descriptors on the host).
mok_status run_ring(const mok_config* cfg, int n_calls, const RingCall* calls,
                    const mok_expert_weights* w, char* wsb, int32_t* dev_status, hipStream_t sm,
                    mok_trace* tr) {
  const Ws wl = ws_layout(cfg);
  RingPlan p;
  memset(&p, 0, sizeof(p));
  p.prec = cfg->prec;
  p.n_calls = n_calls;
  p.calls = calls;
  p.d = cfg->d;
  p.I = cfg->I;
  p.E_local = cfg->E_local;
  p.R_cap = cfg->R_cap;
  p.T_src = cfg->T_src;
  p.k = cfg->k;
  p.mb = cfg->minibatch_rows;
  p.ring_bytes = cfg->ring_bytes;
  p.comm_wgs = cfg->comm_wgs;
  p.gemm_wgs = cfg->gemm_wgs;
  p.wait_limit_us = cfg->wait_limit_us;
  p.ring = wsb + wl.ring;
  p.meta = wsb + wl.ring_ctr;
  p.status = dev_status;
  p.w = w;
  return launch_ring_fwd(p, sm, tr);
}

// The final weighted combine of a ring launch's last call (the earlier
// calls' combines run inside the ring kernel).
mok_status last_combine(const mok_config* cfg, const RingCall& c, hipStream_t sm, mok_trace* tr) {
  if (c.own_n == 0) return MOK_OK;
  return launch_combine(cfg->prec == MOK_F32 ? MOK_F32 : MOK_BF16, c.dest_row, c.gate, c.staging,
                        c.out, cfg->T_src, cfg->d, cfg->k, c.own_lo, c.own_n, cfg->R_cap, sm, tr);
}

// The forward pass.  layout_ws: the layout kernels' scratch (the start of ws,
// or the no-allocation entry point's static array); ws may then be null on
// the paths that use no other workspace (bf16, no ring).
mok_status layer_fwd(const mok_config* cfg, int32_t own_lo, int32_t own_n,
                     const void* const* src_x, const void* w_router, const float* bias,
                     const int32_t* expert_to_local, const mok_expert_weights* w,
                     const mok_fwd_state* st, void* const* staging, void* const* out, void* ws,
                     void* layout_ws, int32_t* dev_status, void* stream) {
  if (!valid_cfg(cfg)) return MOK_EINVAL;
  if (!w_router || !expert_to_local || !w || !layout_ws) return MOK_EINVAL;
  if (!ws && (cfg->prec != MOK_BF16 || cfg->ring_bytes > 0)) return MOK_EINVAL;
  mok_status rc = check_call(cfg, own_lo, own_n, src_x, st, staging, out);
  if (rc != MOK_OK) return rc;
  const bool ring = cfg->ring_bytes > 0 && cfg->R_cap > 0;
  if (ring) {  // ring path: bf16 / MXFP8
    if (!dev_status) return MOK_EINVAL;
    rc = ring_check(cfg->prec, cfg->d, cfg->I, cfg->minibatch_rows, cfg->ring_bytes, cfg->comm_wgs,
                    cfg->gemm_wgs, nullptr, nullptr);
    if (rc != MOK_OK) return rc;
  }
  hipStream_t sm = (hipStream_t)stream;
  mok_trace* tr = cfg->trace;
  trace_mark(tr, "start", sm);
  const int rprec = cfg->prec == MOK_F32 ? MOK_F32 : MOK_BF16;
  rc = route_and_layout(cfg, own_lo, own_n, src_x, w_router, bias, expert_to_local, st, layout_ws,
                        dev_status, sm, tr);
  if (rc != MOK_OK) return rc;
  const Ws wl = ws_layout(cfg);
  char* wsb = (char*)ws;
  if (ring) {
    // one persistent launch: dispatch workgroups fill ring slots, GEMM
    // workgroups run GEMM1 + SwiGLU and GEMM2 and push to staging, and the
    // dispatch side runs the final weighted combine once the pushes are in
    const RingCall c = ring_call(cfg, own_lo, own_n, src_x, st, staging, out,
                                 h_scale_of(cfg, st, wsb, 0));
    rc = run_ring(cfg, 1, &c, w, wsb, dev_status, sm, tr);
    if (rc != MOK_OK) return rc;
    return last_combine(cfg, c, sm, tr);
  }
  DstTable stg;
  fill_table(&stg, (const void* const*)staging, cfg->S);
  if (cfg->R_cap > 0) {
    SrcTable src;
    fill_table(&src, src_x, cfg->S);
    if (cfg->prec == MOK_MXFP8) {
      rc = launch_gather(cfg->prec, src, cfg->T_src, cfg->d, cfg->k, cfg->E_local, cfg->R_cap,
                         st->row_src, st->offsets, wsb + wl.xperm, (uint8_t*)(wsb + wl.xscale), sm,
                         tr);
      if (rc != MOK_OK) return rc;
      rc = launch_ffn_mx(cfg->d, cfg->I, cfg->E_local, cfg->R_cap, (const uint8_t*)(wsb + wl.xperm),
                         (const uint8_t*)(wsb + wl.xscale), st->offsets, st->row_src, w,
                         (uint8_t*)st->h, h_scale_of(cfg, st, wsb, 0), st->ab, nullptr, &stg,
                         cfg->T_src, cfg->k, sm, tr);
    } else if (cfg->prec == MOK_BF16) {
      // the pull dispatch runs inside GEMM1: its A rows are read from the sources
      rc = launch_ffn_bf16(cfg->d, cfg->I, cfg->E_local, cfg->R_cap, nullptr, &src, cfg->T_src,
                           cfg->k, st->offsets, st->row_src, w->w_gate, w->w_up, w->w_down, st->h,
                           st->ab, nullptr, &stg, sm, tr);
    } else {
      rc = launch_gather(cfg->prec, src, cfg->T_src, cfg->d, cfg->k, cfg->E_local, cfg->R_cap,
                         st->row_src, st->offsets, wsb + wl.xperm, nullptr, sm, tr);
      if (rc != MOK_OK) return rc;
      rc = launch_ffn(cfg->prec, cfg->d, cfg->I, cfg->E_local, cfg->R_cap, wsb + wl.xperm,
                      st->offsets, st->row_src, w->w_gate, w->w_up, w->w_down, st->h, st->ab,
                      nullptr, &stg, cfg->T_src, cfg->k, sm, tr);
    }
    if (rc != MOK_OK) return rc;
  }
  if (own_n == 0) return MOK_OK;
  DstTable o;
  fill_table(&o, (const void* const*)out, cfg->S);
  return launch_combine(rprec, st->dest_row, st->topk_gate, stg, o, cfg->T_src, cfg->d, cfg->k,
                        own_lo, own_n, cfg->R_cap, sm, tr);
}

// Scratch of the no-allocation forward entry point: the layout kernels'
// per-chunk expert counts.  One copy per GPU, held until the process ends;
// host code uses only the per-device address from hipGetSymbolAddress.
constexpr size_t kStaticScratchBytes = MOK_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, null until looked up

// The current device's address of `scratch`, looked up once per device with
// that device current.  Null if the runtime cannot give it.
void* static_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

mok_status mok_layer_fwd(const mok_config* cfg, int32_t own_lo, int32_t own_n,
                         const void* const* src_x, const void* w_router, const float* bias,
                         const int32_t* expert_to_local, const mok_expert_weights* w,
                         const mok_fwd_state* st, void* const* staging, void* const* out,
                         void* ws, int32_t* dev_status, void* stream) {
  if (!valid_cfg(cfg) || !ws) return MOK_EINVAL;
  return layer_fwd(cfg, own_lo, own_n, src_x, w_router, bias, expert_to_local, w, st, staging,
                   out, ws, (char*)ws + ws_layout(cfg).layout, dev_status, stream);
}

mok_status mok_layer_fwd_macro(const mok_config* cfg, int32_t n_calls,
                               const mok_layer_call* calls, const void* w_router,
                               const float* bias, const int32_t* expert_to_local,
                               const mok_expert_weights* w, void* ws, int32_t* dev_status,
                               void* stream) {
  if (!valid_cfg(cfg) || !calls || n_calls < 1 || n_calls > MOK_MAX_CALLS) return MOK_EINVAL;
  if (cfg->ring_bytes <= 0 || (cfg->prec != MOK_BF16 && cfg->prec != MOK_MXFP8)) return MOK_EINVAL;
  if (!w_router || !expert_to_local || !w || !ws || !dev_status) return MOK_EINVAL;
  for (int c = 0; c < n_calls; ++c) {
    const mok_status rc = check_call(cfg, calls[c].own_lo, calls[c].own_n, calls[c].src_x,
                                     calls[c].st, calls[c].staging, calls[c].out);
    if (rc != MOK_OK) return rc;
  }
  if (cfg->R_cap > 0) {
    const mok_status rc = ring_check(cfg->prec, cfg->d, cfg->I, cfg->minibatch_rows,
                                     cfg->ring_bytes, cfg->comm_wgs, cfg->gemm_wgs, nullptr,
                                     nullptr);
    if (rc != MOK_OK) return rc;
  }
  hipStream_t sm = (hipStream_t)stream;
  mok_trace* tr = cfg->trace;
  trace_mark(tr, "start", sm);
  const Ws wl = ws_layout(cfg);
  char* wsb = (char*)ws;
  // every call's routing and layout first (the layout scratch is reused in
  // stream order), then one ring launch for all of them
  for (int c = 0; c < n_calls; ++c) {
    const mok_status rc = route_and_layout(cfg, calls[c].own_lo, calls[c].own_n, calls[c].src_x,
                                           w_router, bias, expert_to_local, calls[c].st,
                                           wsb + wl.layout, dev_status, sm, tr);
    if (rc != MOK_OK) return rc;
  }
  if (cfg->R_cap == 0) {  // no rows: only the combines of remote slots
    for (int c = 0; c < n_calls; ++c) {
      if (calls[c].own_n == 0) continue;
      DstTable stg, o;
      fill_table(&stg, (const void* const*)calls[c].staging, cfg->S);
      fill_table(&o, (const void* const*)calls[c].out, cfg->S);
      const mok_status rc =
          launch_combine(MOK_BF16, calls[c].st->dest_row, calls[c].st->topk_gate, stg, o,
                         cfg->T_src, cfg->d, cfg->k, calls[c].own_lo, calls[c].own_n, cfg->R_cap,
                         sm, tr);
      if (rc != MOK_OK) return rc;
    }
    return MOK_OK;
  }
  RingCall rc_calls[MOK_MAX_CALLS];
  for (int c = 0; c < n_calls; ++c)
    rc_calls[c] = ring_call(cfg, calls[c].own_lo, calls[c].own_n, calls[c].src_x, calls[c].st,
                            calls[c].staging, calls[c].out,
                            h_scale_of(cfg, calls[c].st, wsb, c));
  const mok_status rc = run_ring(cfg, n_calls, rc_calls, w, wsb, dev_status, sm, tr);
  if (rc != MOK_OK) return rc;
  return last_combine(cfg, rc_calls[n_calls - 1], sm, tr);
}

mok_status mok_layer_fwd_noalloc(const mok_config* cfg, int32_t own_lo, int32_t own_n,
                                 const void* const* src_x, const void* w_router,
                                 const float* bias, const int32_t* expert_to_local,
                                 const mok_expert_weights* w, const mok_fwd_state* st,
                                 void* const* staging, void* const* out, int32_t* dev_status,
                                 void* stream) {
  if (!valid_cfg(cfg)) return MOK_EINVAL;
  // the bf16 layer without the ring: the layout's counts are its only scratch
  if (cfg->prec != MOK_BF16 || cfg->ring_bytes != 0) return MOK_EINVAL;
  const int64_t N = (int64_t)cfg->S * cfg->T_src * cfg->k;
  if (layout_ws_bytes(N, cfg->E_local) > kStaticScratchBytes) return MOK_ESCRATCH;
  void* scr = static_scratch();
  if (!scr) return MOK_EDEVICE;
  return layer_fwd(cfg, own_lo, own_n, src_x, w_router, bias, expert_to_local, w, st, staging,
                   out, nullptr, scr, dev_status, stream);
}

mok_status mok_layer_bwd(const mok_config* cfg, int32_t own_lo, int32_t own_n,
                         const void* const* d_out, const void* const* src_x,
                         const void* w_router, const int32_t* expert_to_local,
                         const mok_expert_weights* w, const mok_fwd_state* st,
                         void* const* staging, float* d_gate, void* const* dx_stage,
                         void* const* d_x, float* dw_gate, float* dw_up, float* dw_down,
                         float* dw_router, void* ws, int32_t* dev_status, void* stream) {
  (void)expert_to_local;
  if (!valid_cfg(cfg) || !own_range_ok(cfg, own_lo, own_n)) return MOK_EINVAL;
  if (!d_out || !src_x || !w_router || !w || !st || !staging || !d_gate || !dx_stage || !ws)
    return MOK_EINVAL;
  const bool mx = cfg->prec == MOK_MXFP8;
  if (mx) {
    if (!w->wt_down || !w->st_down || !w->wt_gu || !w->st_gu || !st->h_scale) return MOK_EINVAL;
    if (cfg->d % 128 != 0) return MOK_ESHAPE;  // dh contracts over d in 128-wide stages
  }
  if (!dw_gate || !dw_up || !dw_down || !st->ab || !st->h) return MOK_EINVAL;
  if (!st->topk_idx || !st->topk_gate || !st->offsets || !st->dest_row) return MOK_EINVAL;
  if (cfg->R_cap > 0 && !st->row_src) return MOK_EINVAL;
  // the pulls and pushes reach every source with a local row; the per-token
  // sums and the router gradient the own ones
  if (cfg->R_cap > 0 &&
      (!all_sources_set(d_out, cfg->S, cfg->T_src) || !all_sources_set(src_x, cfg->S, cfg->T_src) ||
       !all_sources_set((const void* const*)staging, cfg->S, cfg->T_src) ||
       !all_sources_set((const void* const*)dx_stage, cfg->S, cfg->T_src)))
    return MOK_EINVAL;
  if (!own_sources_set(src_x, own_lo, own_n, cfg->T_src) ||
      !own_sources_set((const void* const*)dx_stage, own_lo, own_n, cfg->T_src) ||
      !own_sources_set((const void* const*)d_x, own_lo, own_n, cfg->T_src))
    return MOK_EINVAL;
  if (dw_router && cfg->E > 256) return MOK_EINVAL;  // router layout holds at most 256 experts
  BwdPlan p;
  memset(&p, 0, sizeof(p));
  p.prec = cfg->prec;
  p.S = cfg->S;
  p.T_src = cfg->T_src;
  p.d = cfg->d;
  p.E = cfg->E;
  p.k = cfg->k;
  p.I = cfg->I;
  p.E_local = cfg->E_local;
  p.R_cap = cfg->R_cap;
  p.own_lo = own_lo;
  p.own_n = own_n;
  fill_table(&p.d_out, d_out, cfg->S);
  fill_table(&p.src_x, src_x, cfg->S);
  fill_table(&p.staging, (const void* const*)staging, cfg->S);
  fill_table(&p.dx_stage, (const void* const*)dx_stage, cfg->S);
  if (own_n > 0) fill_table(&p.d_x, (const void* const*)d_x, cfg->S);
  p.w_router = w_router;
  p.wg = w->w_gate;
  p.wu = w->w_up;
  p.wd = w->w_down;
  // transposed weights: required by MXFP8, optional for bf16 (both or none)
  if (cfg->prec == MOK_BF16 && (!w->wt_down) != (!w->wt_gu)) return MOK_EINVAL;
  if (cfg->prec != MOK_F32) {
    p.wt_down = w->wt_down;
    p.wt_gu = w->wt_gu;
  }
  p.topk_idx = st->topk_idx;
  p.topk_gate = st->topk_gate;
  p.offsets = st->offsets;
  p.row_src = st->row_src;
  p.dest_row = st->dest_row;
  p.h = st->h;
  p.ab = st->ab;
  p.d_gate = d_gate;
  p.dw_gate = dw_gate;
  p.dw_up = dw_up;
  p.dw_down = dw_down;
  p.dw_router = dw_router;
  const Ws wl = ws_layout(cfg);
  char* wsb = (char*)ws;
  p.dy = wsb + wl.dy;
  p.dab = wsb + wl.dab;
  p.dz = (float*)(wsb + wl.dz);
  p.dwr_part = (float*)(wsb + wl.dwr);
  p.r_ident = (int32_t*)(wsb + wl.r_ident);
  p.r_counts = (int32_t*)(wsb + wl.r_counts);
  p.r_offsets = (int32_t*)(wsb + wl.r_offsets);
  p.r_row_src = (int32_t*)(wsb + wl.r_row_src);
  p.r_dest_row = (int32_t*)(wsb + wl.r_dest_row);
  p.r_scratch = wsb + wl.r_scratch;
  p.x_perm = wsb + wl.bx;
  p.hT = cfg->prec == MOK_BF16 && !bwd_through_ring(cfg) ? wsb + wl.bh : nullptr;
  p.wg_part = (float*)(wsb + wl.wpart);
  p.wg_order = (int32_t*)(wsb + wl.worder);
  p.status = dev_status;
  if (bwd_through_ring(cfg)) {
    // windows of whole minibatches through the ring: dy, dab and the
    // transposed token rows of a window in its slots (rows r - lo)
    int slots = 0, rows = 0, nwin = 0;
    int64_t cols = 0;
    if (!bwd_ring_geometry(cfg->bwd_ring_bytes, cfg->d, cfg->I, cfg->E_local, cfg->minibatch_rows,
                           cfg->R_cap, &slots, &rows, &cols, &nwin))
      return MOK_EINVAL;
    char* ring = wsb + wl.bring;
    p.dy = ring;
    p.dab = ring + align256((size_t)rows * cfg->d * 2);
    p.x_perm = (char*)p.dab + align256((size_t)rows * 2 * cfg->I * 2);
    p.win = (int32_t*)(wsb + wl.bwin);
    p.wd_part = (float*)(wsb + wl.wpart_down);
    p.win_rows = rows;
    p.win_cols = cols;
    p.win_mb = cfg->minibatch_rows;
    p.win_slots = slots;
    p.n_win = nwin;
  }
  if (mx) {
    p.mx_hs = st->h_scale;
    p.mx_st_down = w->st_down;
    p.mx_st_gu = w->st_gu;
    p.mx_dyq = (uint8_t*)(wsb + wl.mx_dyq);
    p.mx_dys = (uint8_t*)(wsb + wl.mx_dys);
    p.mx_dabq = (uint8_t*)(wsb + wl.mx_dabq);
    p.mx_dabs = (uint8_t*)(wsb + wl.mx_dabs);
    p.mx_cols = bwd_mx_cols(cfg->R_cap, cfg->E_local);
    p.mx_dabT = (uint8_t*)(wsb + wl.mx_dabT);
    p.mx_dabTs = (uint8_t*)(wsb + wl.mx_dabTs);
    p.mx_xT = (uint8_t*)(wsb + wl.mx_xT);
    p.mx_xTs = (uint8_t*)(wsb + wl.mx_xTs);
    p.mx_dyT = (uint8_t*)(wsb + wl.mx_dyT);
    p.mx_dyTs = (uint8_t*)(wsb + wl.mx_dyTs);
    p.mx_hT = (uint8_t*)(wsb + wl.mx_hT);
    p.mx_hTs = (uint8_t*)(wsb + wl.mx_hTs);
  }
  p.tr = cfg->trace;
  if (cfg->aux && !mx) {
    const mok_aux* a = cfg->aux;
    if (!a->stream || a->stream == stream || !a->events[0] || !a->events[1] || !a->events[2])
      return MOK_EINVAL;
    p.aux = (hipStream_t)a->stream;
    for (int i = 0; i < 3; ++i) p.aux_ev[i] = (hipEvent_t)a->events[i];
  }
  trace_mark(p.tr, "start", (hipStream_t)stream);
  return launch_bwd(p, (hipStream_t)stream);
}

mok_status mok_prepare_bwd(const mok_config* cfg, const void* w_gate, const void* w_up,
                           const void* w_down, void* wt_down, uint8_t* st_down, void* wt_gu,
                           uint8_t* st_gu, void* stream) {
  if (!valid_cfg(cfg)) return MOK_EINVAL;
  if (!w_gate || !w_up || !w_down || !wt_down || !wt_gu) return MOK_EINVAL;
  if (cfg->prec == MOK_MXFP8) {
    if (!st_down || !st_gu) return MOK_EINVAL;
    if (cfg->d % 128 != 0) return MOK_ESHAPE;
    return launch_mx_prepare_bwd(cfg->E_local, cfg->d, cfg->I, w_gate, w_up, w_down,
                                 (uint8_t*)wt_down, st_down, (uint8_t*)wt_gu, st_gu,
                                 (hipStream_t)stream);
  }
  if (cfg->prec != MOK_BF16) return MOK_EINVAL;
  return launch_prepare_bwd_bf16(cfg->E_local, cfg->d, cfg->I, w_gate, w_up, w_down, wt_down,
                                 wt_gu, (hipStream_t)stream);
}

mok_status mok_tune_fwd(const mok_config* cfg, const int32_t* mbs, int32_t n_mb,
                        const int32_t* comms, int32_t n_comm, int32_t reps, size_t ws_bytes,
                        int32_t own_lo, int32_t own_n, const void* const* src_x,
                        const void* w_router, const float* bias, const int32_t* expert_to_local,
                        const mok_expert_weights* w, const mok_fwd_state* st,
                        void* const* staging, void* const* out, void* ws, int32_t* dev_status,
                        void* stream, mok_config* best, float* times_ms) {
  if (!valid_cfg(cfg) || !best || !dev_status || cfg->ring_bytes <= 0 || cfg->R_cap <= 0)
    return MOK_EINVAL;
  if (reps < 1 || reps > 1000) return MOK_EINVAL;
  if ((mbs && (n_mb < 1 || n_mb > kTuneMax)) || (comms && (n_comm < 1 || n_comm > kTuneMax)))
    return MOK_EINVAL;
  const int cus = device_cus();
  if (cus <= 0) return MOK_EDEVICE;
  // default grid: the minibatch sizes of the 256-expert share's sweep, up to
  // the sizes where two full waves of GEMM1 tiles fit in one minibatch on 256
  // CUs (2 x 240 tiles of 256 rows x 256 columns over 2I = 4096 columns: about
  // 7.7k rows), and dispatch sides of 1/16 .. 1/4 of the CUs; sizes the ring
  // cannot hold are skipped
  const int32_t mb_def[7] = {64, 128, 256, 512, 1024, 2048, 4096};
  const int32_t comm_def[4] = {cus / 16 > 0 ? cus / 16 : 1, cus / 8 > 0 ? cus / 8 : 1,
                               3 * cus / 16 > 0 ? 3 * cus / 16 : 1, cus / 4 > 0 ? cus / 4 : 1};
  if (!mbs) {
    mbs = mb_def;
    n_mb = 7;
  }
  if (!comms) {
    comms = comm_def;
    n_comm = 4;
  }
  hipStream_t sm = (hipStream_t)stream;
  hipEvent_t ev[2] = {nullptr, nullptr};
  if (hipEventCreate(&ev[0]) != hipSuccess || hipEventCreate(&ev[1]) != hipSuccess) {
    if (ev[0]) (void)hipEventDestroy(ev[0]);
    return MOK_EDEVICE;
  }
  mok_status result = MOK_EINVAL;  // until one candidate ran
  float best_ms = 0.0f;
  for (int i = 0; i < n_mb; ++i)
    for (int j = 0; j < n_comm; ++j) {
      const int idx = i * n_comm + j;
      if (times_ms) times_ms[idx] = -1.0f;
      mok_config c = *cfg;
      c.minibatch_rows = mbs[i];
      c.comm_wgs = comms[j];
      c.gemm_wgs = 0;
      c.trace = nullptr;
      // a candidate the ring cannot take (no slot of that minibatch, a
      // split beyond the CUs) or whose counters outgrow ws is skipped
      if (c.minibatch_rows < 1 || c.comm_wgs < 1 || mok_workspace_bytes(&c) > ws_bytes ||
          ring_check(c.prec, c.d, c.I, c.minibatch_rows, c.ring_bytes, c.comm_wgs, c.gemm_wgs,
                     nullptr, nullptr) != MOK_OK)
        continue;
      mok_status rc = MOK_OK;
      for (int r = 0; r <= reps && rc == MOK_OK; ++r) {  // call 0 warms up
        if (r == 1 && hipEventRecord(ev[0], sm) != hipSuccess) rc = MOK_EDEVICE;
        if (rc == MOK_OK)
          rc = mok_layer_fwd(&c, own_lo, own_n, src_x, w_router, bias, expert_to_local, w, st,
                             staging, out, ws, dev_status, stream);
      }
      int32_t h_status = 0;
      if (rc == MOK_OK && (hipEventRecord(ev[1], sm) != hipSuccess ||
                           hipMemcpyAsync(&h_status, dev_status, sizeof(int32_t),
                                          hipMemcpyDeviceToHost, sm) != hipSuccess ||
                           hipStreamSynchronize(sm) != hipSuccess))
        rc = MOK_EDEVICE;
      if (rc == MOK_OK && h_status != 0) rc = (mok_status)h_status;
      float ms = 0.0f;
      if (rc == MOK_OK && hipEventElapsedTime(&ms, ev[0], ev[1]) != hipSuccess) rc = MOK_EDEVICE;
      if (rc != MOK_OK) {
        result = rc;
        goto done;
      }
      ms /= (float)reps;
      if (times_ms) times_ms[idx] = ms;
      if (result != MOK_OK || ms < best_ms) {
        best_ms = ms;
        *best = c;
        best->trace = cfg->trace;
        result = MOK_OK;
      }
    }
done:
  // (a failed destroy leaves nothing the caller could act on; the result stands)
  (void)hipEventDestroy(ev[0]);
  (void)hipEventDestroy(ev[1]);
  return result;
}

mok_status mok_ring_layout(const mok_config* cfg, size_t* offset, size_t* slot_bytes,
                           int32_t* nslot) {
  if (!valid_cfg(cfg) || cfg->ring_bytes <= 0 || !offset || !slot_bytes || !nslot)
    return MOK_EINVAL;
  if (cfg->prec != MOK_BF16 && cfg->prec != MOK_MXFP8) return MOK_EINVAL;
  const int64_t sb = ring_slot_bytes(cfg->prec, cfg->d, cfg->minibatch_rows);
  const int64_t n = cfg->ring_bytes / sb;
  if (n < 1) return MOK_EINVAL;
  *offset = ws_layout(cfg).ring;
  *slot_bytes = (size_t)sb;
  *nslot = n > (1 << 30) ? (1 << 30) : (int32_t)n;
  return MOK_OK;
}

mok_status mok_hbm_stream(int32_t mode, void* dst, const void* src, int64_t bytes,
                          void* stream) {
  if (mode < 0 || mode > 2 || bytes < 0 || bytes % 16 != 0) return MOK_EINVAL;
  if (bytes == 0) return MOK_OK;
  if (!dst || (mode != 1 && !src)) return MOK_EINVAL;
  if (((uintptr_t)dst | (uintptr_t)src) % 16 != 0) return MOK_EINVAL;
  return launch_stream(mode, dst, src, bytes, (hipStream_t)stream);
}

mok_status mok_mfma_probe(int32_t kind, int32_t constant, int64_t iters, int32_t workgroups,
                          float* out, void* stream) {
  if ((kind != 0 && kind != 1) || (constant != 0 && constant != 1) || iters <= 0 ||
      workgroups <= 0 || !out)
    return MOK_EINVAL;
  return launch_mfma_probe(kind, constant, iters, workgroups, out, (hipStream_t)stream);
}

mok_status mok_mx_quantize(int64_t rows, int64_t K, const void* src, uint8_t* codes,
                           uint8_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 32 != 0) return MOK_EINVAL;
  if (rows == 0) return MOK_OK;
  if (!src || !codes || !scales) return MOK_EINVAL;
  // 16-byte loads of the values, 8-byte stores of the codes
  if ((uintptr_t)src % 16 != 0 || (uintptr_t)codes % 8 != 0) return MOK_EINVAL;
  return launch_mx_quantize(rows, K, src, codes, scales, (hipStream_t)stream);
}

mok_status mok_mx_quantize_f32(int64_t rows, int64_t K, const float* src, uint8_t* codes,
                               uint8_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 32 != 0) return MOK_EINVAL;
  if (rows == 0) return MOK_OK;
  if (!src || !codes || !scales) return MOK_EINVAL;
  if ((uintptr_t)src % 16 != 0 || (uintptr_t)codes % 8 != 0) return MOK_EINVAL;
  return launch_mx_quantize(rows, K, src, codes, scales, (hipStream_t)stream, true);
}

}  // extern "C"
