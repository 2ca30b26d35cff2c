// Internal launchers (one per kernel family); the C ABI in mok_api.hip
// validates arguments and sequences these.
#pragma once

#include "mok_common.h"

namespace mok {

int route_geometry(int E, int T, int* EL, int* ESETS, int* TB, int* dc);
size_t route_smem_bytes(int E, int T);
// Routes T consecutive tokens starting at token 0 of source src_lo (sources
// of T_src tokens each, contiguous in the table).
mok_status launch_route(int prec, const SrcTable& src, int src_lo, int T_src, int T, int d,
                        int E, int k, const void* w, const float* bias, int32_t* topk_idx,
                        float* topk_gate, hipStream_t stream, mok_trace* tr = nullptr);

size_t layout_ws_bytes(int64_t N, int E_local);
mok_status launch_layout(int64_t N, int E, int E_local, int R_cap, const int32_t* topk,
                         const int32_t* e2l, int32_t* counts, int32_t* offsets, int32_t* row_src,
                         int32_t* dest_row, void* ws, int32_t* status, hipStream_t stream,
                         mok_trace* tr = nullptr);

mok_status launch_gather(int prec, const SrcTable& src, int T_src, int d, int k, int E_local,
                         int R_cap, const int32_t* row_src, const int32_t* offsets, void* dst,
                         uint8_t* dst_scale, hipStream_t stream, mok_trace* tr = nullptr);
mok_status launch_push(int prec, const void* y, const int32_t* dest_row, int64_t N,
                       const DstTable& staging, int T_src, int d, int k, int R_cap,
                       hipStream_t stream, mok_trace* tr = nullptr);
mok_status launch_combine(int prec, const int32_t* dest_row, const float* gate,
                          const DstTable& staging, const DstTable& out, int T_src, int d, int k,
                          int own_lo, int own_n, int R_cap, hipStream_t stream,
                          mok_trace* tr = nullptr);
mok_status launch_mx_quantize(int64_t rows, int64_t K, const void* src, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream, bool f32 = false);

int grouped_mtiles_bound(int R_cap, int E_local);
mok_status launch_ffn(int prec, int d, int I, int E_local, int R_cap, const void* x,
                      const int32_t* offsets, const int32_t* row_src, const void* wg,
                      const void* wu, const void* wd, void* h, void* ab, void* y,
                      const DstTable* staging, int T_src, int k, hipStream_t stream,
                      mok_trace* tr = nullptr);
mok_status launch_ffn_mx(int d, int I, int E_local, int R_cap, const uint8_t* xq,
                         const uint8_t* xs, const int32_t* offsets, const int32_t* row_src,
                         const mok_expert_weights* w, uint8_t* hq, uint8_t* hs, void* ab, void* y,
                         const DstTable* staging, int T_src, int k, hipStream_t stream,
                         mok_trace* tr = nullptr);

// MX GEMM over grouped rows on the scaled matrix cores: out[r][n] = sum over
// k < K of A[r][k] B_e[n][k] for the rows r of each local expert e, A and B
// E4M3 codes (K-major, B [E_local, N, K]) with E8M0 scales per 32 along k;
// bf16 out stored at y + r ldy, or pushed to the staging rows of the items.
mok_status launch_mx_rows_gemm(const uint8_t* aq, const uint8_t* as, const uint8_t* bq,
                               const uint8_t* bs, int K, int N, int E_local, int R_cap,
                               const int32_t* offsets, const int32_t* row_src, void* y, int ldy,
                               const DstTable* push, int T_src, int k, hipStream_t stream,
                               mok_trace* tr, const char* name);

// bf16 forward GEMMs on the pipelined engine; x == null gathers the A rows
// from the source table through row_src.
mok_status launch_ffn_bf16(int d, int I, int E_local, int R_cap, const void* x,
                           const SrcTable* src, int T_src, int k, const int32_t* offsets,
                           const int32_t* row_src, const void* wg, const void* wu, const void* wd,
                           void* h, void* ab, void* y, const DstTable* staging,
                           hipStream_t stream, mok_trace* tr = nullptr);

// Persistent ring kernel of the forward pass (gather + GEMM1 + SwiGLU +
// GEMM2 + push + final weighted combine in one launch, for one or several
// layer calls in a row; see mok_ring.hip).
constexpr int kRingMaxCalls = MOK_MAX_CALLS;
struct RingCall {       // one layer call (macrobatch) through the ring
  SrcTable src;         // S source buffers [T_src, d]
  DstTable staging;     // S staging buffers [T_src*k, d]
  DstTable out;         // S outputs [T_src, d] (own entries)
  const int32_t* row_src;
  const int32_t* offsets;
  const int32_t* dest_row;
  const float* gate;
  void* h;              // [R_cap, I] (MX: codes)
  uint8_t* h_scale;     // MX: [R_cap, I/32]
  void* ab;             // [R_cap, 2I] bf16 a | b (bf16 and MXFP8 layers), or null
  int own_lo, own_n;
};
struct RingPlan {
  int prec;
  int n_calls;
  const RingCall* calls;  // host array [n_calls]
  int d, I, E_local, R_cap, T_src, k;
  int mb;                 // minibatch rows
  int64_t ring_bytes;
  int comm_wgs, gemm_wgs, wait_limit_us;
  void* ring;             // ring_bytes of workspace
  void* meta;             // ring_meta_bytes() of workspace: counters and call descriptors
  int32_t* status;
  const mok_expert_weights* w;
};
int64_t ring_slot_bytes(int prec, int d, int mb);
// Compute units of the current device (0 if the runtime cannot tell).
int device_cus();
int ring_max_minibatches(int R_cap, int E_local, int mb);
// Counters and call descriptors of the ring kernel, for up to kRingMaxCalls calls.
size_t ring_meta_bytes(int R_cap, int E_local, int mb);
// Argument check of the ring path (also run by launch_ring_fwd); the auto
// split of workgroups is returned through comm_out / gemm_out.
mok_status ring_check(int prec, int d, int I, int mb, int64_t ring_bytes, int comm_wgs,
                      int gemm_wgs, int* comm_out, int* gemm_out);
mok_status launch_ring_fwd(const RingPlan& p, hipStream_t stream, mok_trace* tr = nullptr);

// HBM streaming probe (mok_stream.hip): mode 0 read, 1 write, 2 copy.
mok_status launch_stream(int mode, void* dst, const void* src, int64_t bytes, hipStream_t stream);
mok_status launch_mfma_probe(int kind, int constant, int64_t iters, int workgroups, float* out,
                             hipStream_t stream);

struct BwdPlan {
  int prec;
  int S, T_src, d, E, k, I, E_local, R_cap;
  int own_lo, own_n;
  SrcTable d_out, src_x;
  DstTable staging, dx_stage, d_x;
  const void* w_router;
  const void *wg, *wu, *wd;
  const int32_t* topk_idx;
  const float* topk_gate;
  const int32_t* offsets;
  const int32_t* row_src;
  const int32_t* dest_row;
  const void* h;
  const void* ab;
  float* d_gate;
  float *dw_gate, *dw_up, *dw_down, *dw_router;
  // workspace pieces
  void* dy;      // [R_cap, d]
  void* dab;     // [R_cap, 2I]
  float* dz;     // [own tokens, k]
  float* dwr_part;  // [N_own/64 + E, d] per-chunk partial router gradients
  // router layout of the own items over all E experts (workspace)
  int32_t *r_ident, *r_counts, *r_offsets, *r_row_src, *r_dest_row;
  void* r_scratch;
  void* x_perm;     // bf16: [d, xt_ld] token rows gathered again, transposed, for the wgrad GEMM
  void* hT;         // bf16: [I, xt_ld] h transposed the same way (one-launch backward), or null
  float* wg_part;   // [R_cap / 4096, 2I, d] split-K partials of the weight gradients
  float* wd_part;   // the down projection's partials ([R_cap / 4096, d, I]): wg_part in one
                    // launch (reduced before it is reused); a region of its own through the
                    // ring, where both sets are reduced after the last window
  int32_t* wg_order;  // [E_local] local experts by routed rows, descending
  int32_t* status;  // device status word (may be null)
  // ring windows (win != null): the backward runs window by window, dy, dab
  // and the transposed token rows of a window in the ring (rows r - lo)
  int32_t* win;       // [3 + E_local + 1]: lo, hi, window index, clipped offsets
  int win_rows;       // rows of a window, at most (slots x minibatch rows)
  int64_t win_cols;   // leading dimension of the window's transposed token rows
  int win_mb, win_slots, n_win;
  // MXFP8 backward (prec == MOK_MXFP8): E4M3 codes + E8M0 scales per 32
  const uint8_t* mx_hs;                     // [R_cap, I/32] the forward's h scales
  // the weights transposed (mok_prepare_bwd): W_down^T [E_local, I, d] and
  // [W_gate; W_up]^T [E_local, d, 2I]; bf16 (optional, null = read W
  // n-contiguous) or MXFP8 codes with the scales below
  const void *wt_down, *wt_gu;
  const uint8_t *mx_st_down, *mx_st_gu;     // MXFP8: [.., d/32], [.., 2I/32]
  uint8_t *mx_dyq, *mx_dys;                 // dy rows along d
  uint8_t *mx_dabq, *mx_dabs;               // [da|db] rows along 2I
  int64_t mx_cols;                          // columns of the transposed operands
  uint8_t *mx_dabT, *mx_dabTs, *mx_xT, *mx_xTs, *mx_dyT, *mx_dyTs, *mx_hT, *mx_hTs;
  mok_trace* tr;    // host-side trace, may be null
  hipStream_t aux;      // second stream for the work beside the GEMMs, or null
  hipEvent_t aux_ev[3]; // fork/join events of the second stream
};
mok_status launch_bwd(const BwdPlan& p, hipStream_t stream);
// Leading dimension of the transposed token rows of the gate/up weight
// gradients ([d, xt_ld] bf16): every expert's rows padded to 64 columns.
inline int64_t xt_ld(int R_cap, int E_local) {
  return ((int64_t)R_cap + 63) / 64 * 64 + 64 * (int64_t)E_local;
}
// The token rows (rows == null) or a row-major [R_cap, width] matrix (h),
// transposed per expert into [width, xt_ld] with every expert's rows padded
// to 64 columns.
mok_status launch_gather_t(const BwdPlan& p, void* xT, hipStream_t stream, int max_blocks = 0,
                           const void* rows = nullptr, int width = 0);
mok_status launch_bwd_gemms_bf16(const BwdPlan& p, const void* x_perm, hipStream_t stream,
                                 hipEvent_t before_wgrad = nullptr, hipEvent_t after_dx = nullptr);
// Pieces of the bf16 backward GEMMs (one launch, or one ring window each).
mok_status launch_bwd_dgrad(const BwdPlan& p, hipStream_t stream);
mok_status launch_bwd_wgrad(const BwdPlan& p, const void* x_perm, hipStream_t stream, bool order,
                            bool reduce);
mok_status launch_bwd_reduce(const BwdPlan& p, hipStream_t stream);
mok_status launch_bwd_window(const BwdPlan& p, int w, hipStream_t stream);
mok_status launch_swiglu_bwd(const BwdPlan& p, hipStream_t stream);
// MXFP8 backward GEMMs (dh, SwiGLU backward, dx push, weight gradients) and
// their transposed operands; columns of those operands: every local expert's
// rows padded to 128.
mok_status launch_bwd_mx_gemms(const BwdPlan& p, hipStream_t stream);
int64_t bwd_mx_cols(int R_cap, int E_local);
mok_status launch_mx_prepare_bwd(int E_local, int d, int I, const void* w_gate, const void* w_up,
                                 const void* w_down, uint8_t* wt_down, uint8_t* st_down,
                                 uint8_t* wt_gu, uint8_t* st_gu, hipStream_t stream);
mok_status launch_prepare_bwd_bf16(int E_local, int d, int I, const void* w_gate, const void* w_up,
                                   const void* w_down, void* wt_down, void* wt_gu,
                                   hipStream_t stream);
// Geometry of the backward's ring windows for cfg (bf16, ring_bytes > 0):
// slots of minibatch_rows rows, each holding dy and da | db rows and the
// transposed token rows; false if the ring holds no slot.
bool bwd_ring_geometry(int64_t ring_bytes, int d, int I, int E_local, int mb, int R_cap,
                       int* slots, int* rows, int64_t* cols, int* n_win);
size_t wgrad_partial_bytes(int R_cap, int d, int I);

}  // namespace mok
