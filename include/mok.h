/*
 * mok.h -- C ABI of the MI355X (gfx950) fused MoE layer: route -> expert-
 * contiguous layout -> gather (pull dispatch) -> SwiGLU expert grouped GEMM ->
 * gate-weighted combine, forward and backward, deterministic.
 *
 * The operations follow the Mixture-of-Kittens write-ups:
 *   [K01] LeFeng.com article on kucoin.com, section 01 ("the communication tax
 *         of MoE"): the router picks a few experts per token; the system counts
 *         the tokens of each expert, decides where they go and groups each
 *         expert's tokens together so that a grouped GEMM gets ordered input;
 *         dispatch and combine in the forward pass, two more rounds in reverse
 *         in the backward pass.
 *   [K02] same article, section 02: pull dispatch (the receiver only needs to
 *         know which source holds a token and where, and chooses its own
 *         placement, ordered by local expert), push combine, pull
 *         reverse-combine and push reverse-dispatch; a fixed-size ring token
 *         buffer whose slots are reused as soon as compute and combine are
 *         done; a minibatch size; SMs split between communication and compute
 *         sides that hand off through on-GPU counters; MXFP8 quantisation fused
 *         into the dispatch, grouped-GEMM and SwiGLU data paths.
 *   [K03] same article, section 03: the measured layer consists of scheduling,
 *         routing, the expert FFN, the combine and the final weighted combine.
 *   [M-P] miku-ai.ru article, section "Производительность и масштабируемость":
 *         identical inputs give bit-identical results.
 *
 * Conventions for every entry point
 *   - Memory: the caller owns every buffer (device memory unless stated).
 *     The library allocates and frees nothing, keeps no global mutable state
 *     and never synchronises the host with the device (except the tuner,
 *     mok_tune_fwd, which runs off the timed path).
 *   - Execution: work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and runs asynchronously.
 *   - Errors: invalid arguments are rejected before anything is enqueued with
 *     a negative mok_status.  Conditions that only the device can see (more
 *     routed rows than R_cap, an expert id out of range, a bounded wait that
 *     timed out) are latched into `*dev_status` (a device int32 the caller
 *     zeroes; the first error code written wins) and the affected kernels skip
 *     the offending work instead of writing out of bounds.
 *   - Sizes that depend on routing (rows per expert, R) stay on the device;
 *     the host passes capacities only.
 *   - Layout: all matrices are row-major.  Expert weights are stored with the
 *     contraction dimension innermost for the forward pass: W_gate, W_up are
 *     [E_local, I, d], W_down is [E_local, d, I].
 *   - Determinism: every reduction runs in a fixed order; no floating-point
 *     atomics.  Two runs give bit-identical outputs.
 *   - Source buffers: S simulated source ranks, each a separate device buffer
 *     of T_src tokens, passed as a host array of S device pointers (up to
 *     MOK_MAX_SOURCES).  Item n = (s * T_src + t) * k + j names slot j of
 *     token t of source s.  Which sources have items routed to a local
 *     expert is known on the device only, so a call that pulls rows from the
 *     sources or pushes rows to them (mok_dispatch, the push of mok_combine,
 *     mok_layer_fwd, mok_layer_bwd) needs all S entries of those arrays
 *     non-NULL whenever T_src > 0 and R_cap > 0; arrays read or written for
 *     the own sources only (out, d_x) need their own entries only.  Any NULL
 *     entry a call needs is MOK_EINVAL before anything is enqueued.  With
 *     T_src = 0 (an empty batch) the per-source device pointers may be NULL;
 *     the state arrays must still be non-NULL.
 */
#ifndef MOK_H
#define MOK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOK_MAX_SOURCES 64
#define MOK_MX_BLOCK 32
#define MOK_MAX_CALLS 8     /* layer calls (macrobatches) of one mok_layer_fwd_macro */

typedef enum {
  MOK_OK = 0,
  MOK_EINVAL = -1,     /* null pointer, bad size, unsupported combination */
  MOK_ESHAPE = -2,     /* shape constraint violated (e.g. d % 32 for MXFP8) */
  MOK_EDEVICE = -3,    /* HIP runtime error at launch */
  MOK_ECAPACITY = -4,  /* device-latched: routed rows exceed R_cap */
  MOK_ETIMEOUT = -5,   /* device-latched: a bounded wait in the fused kernel ran out */
  MOK_EROUTE = -6,     /* device-latched: an expert id outside [0, E) in routing input */
  MOK_ESCRATCH = -7    /* mok_layer_fwd_noalloc: cfg needs more than its static scratch */
} mok_status;

typedef enum {
  MOK_F32 = 0,   /* fp32 tokens, weights, outputs; fp32 GEMMs */
  MOK_BF16 = 1,  /* bf16 tokens, weights, outputs; bf16 MFMA with fp32 accumulation */
  MOK_MXFP8 = 2  /* bf16 tokens/outputs in HBM; E4M3 elements + one E8M0 scale per 32
                    along the contraction dim inside the expert GEMMs */
} mok_prec;

/* Optional per-kernel timing [tracing]: when mok_config.trace is non-NULL,
 * every entry point records events[count] on its stream at its start and
 * after each kernel it launches, stores the name of the kernel that ended at
 * that event in names[count] (static strings) and increments count, while
 * count < capacity.  events are caller-created hipEvent_t handles. */
typedef struct mok_trace {
  void** events;
  const char** names;
  int32_t capacity;
  int32_t count;
  int32_t* from;          /* optional [capacity]: from[i] = the index of the previous event
                             recorded on the same stream (the start of kernel i), -1 for the
                             first event of a stream; NULL = not kept.  With a second stream
                             (mok_aux) durations are elapsed(events[from[i]], events[i]). */
  void* last_stream[2];   /* bookkeeping of the library (zero-initialise): the last two */
  int32_t last_idx[2];    /* streams seen and their latest event index */
} mok_trace;

/* Optional second stream of the backward pass (caller-owned).  With
 * mok_config.aux non-NULL, the bf16 mok_layer_bwd runs the steps that do not
 * feed the next GEMM -- the transposed re-gather of the token rows, the
 * router-gradient layout, the per-token dx sum and the router weight
 * gradient -- on `stream`, beside the dgrad/wgrad GEMMs on the call's
 * stream, ordered by the three events; the call's stream then waits for the
 * second one, so work enqueued after the call sees every output.  `stream`
 * must differ from the call's stream and have the default priority;
 * `events` are hipEvent_t handles (timing may be disabled), re-recorded by
 * every call.  Results are bit-identical with and without it. */
typedef struct mok_aux {
  void* stream;
  void* events[3];
} mok_aux;

typedef struct mok_config {
  int32_t S;              /* source token buffers (simulated source ranks), 1..MOK_MAX_SOURCES */
  int32_t T_src;          /* tokens per source buffer */
  int32_t d;              /* hidden size: multiple of 64 (MOK_EINVAL otherwise); the MXFP8
                             expert FFN and the MXFP8 ring need a multiple of 128 (MOK_ESHAPE) */
  int32_t E;              /* experts in the layer, 1..512 */
  int32_t k;              /* experts chosen per token, 1..min(E, 16) */
  int32_t I;              /* SwiGLU intermediate size per expert: multiple of 64; of 128 for
                             the MXFP8 expert FFN (MOK_ESHAPE) */
  int32_t E_local;        /* experts whose FFN runs on this GPU, 1..256 */
  int32_t prec;           /* mok_prec */
  int32_t R_cap;          /* row capacity of every routed-row buffer */
  int32_t minibatch_rows; /* fused path: at most this many rows of one expert per minibatch */
  int64_t ring_bytes;     /* fused path (persistent ring kernel, bf16 and MXFP8): bytes of the
                             ring of token slots, at least one slot of minibatch_rows rows;
                             0 = staged path (one launch per step) */
  int32_t comm_wgs;       /* fused path: dispatch/combine workgroups (0 = CUs / 8 for bf16,
                             CUs / 4 for MXFP8, whose dispatch also quantises) */
  int32_t gemm_wgs;       /* fused path: grouped-GEMM workgroups (0 = the remaining CUs);
                             comm_wgs + gemm_wgs must not exceed the CU count */
  int32_t wait_limit_us;  /* fused path: bound of every device-side wait in microseconds;
                             on expiry MOK_ETIMEOUT is latched and the kernel returns
                             (0 = 2 s) */
  mok_trace* trace;       /* optional kernel timing, NULL = off (host memory) */
  mok_aux* aux;           /* optional second stream of the backward pass, NULL = one stream */
  int64_t bwd_ring_bytes; /* bf16 backward through a ring of this many bytes: the routed rows
                             run in windows of whole minibatches (minibatch_rows, a multiple
                             of 64) whose dy, da | db and transposed token rows occupy the
                             ring's slots, reused window after window, instead of buffers of
                             R_cap rows; 0 = one launch per step over all rows.  The results
                             are bit-identical either way.  The ring must hold one slot
                             (MOK_EINVAL otherwise); aux is not used on this path */
} mok_config;

/* Expert weights of the E_local local experts (see Layout above).  For
 * MOK_MXFP8 the three matrices hold E4M3 codes (uint8, same shapes) and
 * s_gate, s_up, s_down their E8M0 scales ([E_local, I, d/32] and
 * [E_local, d, I/32]); otherwise the s_* pointers are NULL.
 * The backward (mok_layer_bwd) contracts W_down over d and W_gate, W_up over
 * I, and can read them transposed, from mok_prepare_bwd: wt_down
 * [E_local, I, d] = W_down^T and wt_gu [E_local, d, 2I] = [W_gate; W_up]^T.
 * MOK_MXFP8: E4M3 codes, blocks of 32 along the last axis, with st_down
 * [E_local, I, d/32] and st_gu [E_local, d, 2I/32]; required by the MXFP8
 * backward.  MOK_BF16: bf16 values (st_* unused), optional (both or
 * neither): with them the dh and dx GEMMs read their weights k-contiguous,
 * with bit-identical results.  NULL otherwise. */
typedef struct mok_expert_weights {
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const uint8_t* s_gate;
  const uint8_t* s_up;
  const uint8_t* s_down;
  const void* wt_down;
  const uint8_t* st_down;
  const void* wt_gu;
  const uint8_t* st_gu;
} mok_expert_weights;

/* State the forward pass leaves for the backward pass (all caller-owned). */
typedef struct mok_fwd_state {
  int32_t* topk_idx;   /* [S*T_src*k]: in for non-own sources, out for own sources */
  float* topk_gate;    /* [S*T_src*k] fp32, same split */
  int32_t* counts;     /* [E_local] routed rows per local expert */
  int32_t* offsets;    /* [E_local+1] exclusive scan of counts; offsets[E_local] = R */
  int32_t* row_src;    /* [R_cap] row -> item n */
  int32_t* dest_row;   /* [S*T_src*k] item n -> row, -1 for remote experts (>= R_cap: dropped) */
  void* h;             /* [R_cap, I] SwiGLU output in the activation dtype (bf16 / f32) */
  void* ab;            /* [R_cap, 2I] pre-activation a | b in the activation dtype (bf16 for
                          MOK_MXFP8), or NULL */
  uint8_t* h_scale;    /* MOK_MXFP8: [R_cap, I/32] E8M0 scales of h (h holds its E4M3
                          codes), kept for the backward; NULL = the forward keeps them in
                          its workspace only.  Unused otherwise. */
} mok_fwd_state;

/* Bytes of device workspace the calls below need for `cfg` (256-byte aligned
 * pointer expected).  Covers layout scratch, gathered rows, intermediates of
 * the backward pass and, when cfg->ring_bytes > 0, the ring and its counters. */
size_t mok_workspace_bytes(const mok_config* cfg);

/* Router [K01 router; K03 routing].  For T tokens x [T, d] (fp32 for MOK_F32,
 * else bf16) and router weights w_router [E, d] (same dtype), bias [E] fp32 or
 * NULL:  z[t][e] = fp32 chain (z = 0; for i ascending z = fma(x_i, w_i, z))
 * then z += bias[e];  topk_idx[t][0..k) = the k largest z, ties to the lower
 * expert id, slot 0 largest;  topk_gate[t][j] = softmax over all E experts
 * renormalised over the chosen k (= softmax of the chosen logits), fp32. */
mok_status mok_route(const mok_config* cfg, int32_t T, const void* x, const void* w_router,
                     const float* bias, int32_t* topk_idx, float* topk_gate, void* stream);

/* Expert-contiguous layout [K01 count / place / group; K02 receiver-chosen
 * placement ordered by local expert].  Input: routing of all S sources
 * topk_idx_all [S*T_src*k] and expert_to_local [E] (local index, -1 remote).
 * Output: counts [E_local], offsets [E_local+1], row_src [R_cap] (row -> n),
 * dest_row [S*T_src*k] (n -> row, or -1 if the expert is remote).  Rows of an
 * expert are in ascending n (a stable counting sort).  R > R_cap latches
 * MOK_ECAPACITY: rows past R_cap are not written to row_src, their items keep
 * their row number (>= R_cap) in dest_row, and every later step skips them
 * (a dropped slot adds nothing to the output and has a zero gate gradient);
 * a bad expert id latches MOK_EROUTE.  ws: workspace. */
mok_status mok_layout(const mok_config* cfg, const int32_t* topk_idx_all,
                      const int32_t* expert_to_local, int32_t* counts, int32_t* offsets,
                      int32_t* row_src, int32_t* dest_row, void* ws, int32_t* dev_status,
                      void* stream);

/* Pull dispatch [K02 pull dispatch]: x_perm[r] = src_x[s][t] for every routed
 * row r < R (n = row_src[r]).  src_x: host array of S device pointers, each
 * [T_src, d] in the activation dtype.  x_perm: [R_cap, d] activation dtype, or
 * for MOK_MXFP8 [R_cap, d] E4M3 codes with x_scale [R_cap, d/32] E8M0 (the
 * quantisation is fused into the gather [K02 MXFP8]); x_scale NULL otherwise. */
mok_status mok_dispatch(const mok_config* cfg, const void* const* src_x, const int32_t* row_src,
                        const int32_t* offsets, void* x_perm, uint8_t* x_scale,
                        int32_t* dev_status, void* stream);

/* Expert FFN as grouped GEMMs [K01 grouped GEMM; K02 SwiGLU]: for each local
 * expert e and its rows [offsets[e], offsets[e+1]):
 *   a = x W_gate[e]^T, b = x W_up[e]^T (fp32 accumulation); h = silu(a) * b;
 *   y = h W_down[e]^T.
 * h [R_cap, I] (activation dtype; for MOK_MXFP8 h_scale [R_cap, I/32] holds
 * its scales and h its E4M3 codes, quantised from fp32 in the GEMM epilogue),
 * ab [R_cap, 2I] a | b (activation dtype) or NULL, y [R_cap, d] (activation
 * dtype; bf16 for MOK_MXFP8). */
mok_status mok_expert_ffn(const mok_config* cfg, const void* x_perm, const uint8_t* x_scale,
                          const int32_t* offsets, const mok_expert_weights* w, void* h,
                          uint8_t* h_scale, void* ab, void* y, int32_t* dev_status, void* stream);

/* Push combine + final weighted combine [K02 push combine; K03 final weighted
 * combine].  Push: staging[s][t*k+j] = y[dest_row[n]] for every routed item
 * (staging: host array of S device pointers, each [T_src*k, d] activation
 * dtype; rows of remote items are not written: the GPU holding that expert
 * pushes them).  Final combine for the own sources s in [own_lo,
 * own_lo+own_n):  out[s][t] = sum over j ascending of topk_gate[n] *
 * staging[s][t*k+j], fp32, rounded once, over every slot except local rows
 * dropped beyond R_cap (dest_row[n] >= R_cap); a remote slot (dest_row[n] ==
 * -1) is read as its pusher left it, so the caller fills or zeroes it.
 * out: host array of S device pointers ([T_src, d]); only own entries used.
 * y may be NULL to skip the push (staging already filled). */
mok_status mok_combine(const mok_config* cfg, const void* y, const int32_t* dest_row,
                       const float* topk_gate, void* const* staging, int32_t own_lo,
                       int32_t own_n, void* const* out, int32_t* dev_status, void* stream);

/* Whole forward pass of the layer on this GPU's share.  Routes the own
 * sources [own_lo, own_lo+own_n) (their topk written into st->topk_idx /
 * st->topk_gate; the other sources' routing is read from there), builds the
 * layout, gathers, runs the expert FFN, pushes every local row to `staging`
 * and final-combines the own sources into `out`.  With cfg->ring_bytes == 0
 * the steps run as separate kernels; with ring_bytes > 0 the gather, the FFN
 * and the push run in one persistent kernel whose workgroups are split into
 * dispatch/combine and grouped-GEMM roles handing minibatches over through a
 * fixed ring of expert-contiguous slots and device-scope counters [K02]; the
 * final weighted combine follows as its own launch.
 * Results are bit-identical between the two paths, across ring sizes and
 * minibatch sizes. */
mok_status mok_layer_fwd(const mok_config* cfg, int32_t own_lo, int32_t own_n,
                         const void* const* src_x, const void* w_router, const float* bias,
                         const int32_t* expert_to_local, const mok_expert_weights* w,
                         const mok_fwd_state* st, void* const* staging, void* const* out,
                         void* ws, int32_t* dev_status, void* stream);

/* One layer call of mok_layer_fwd_macro: the arguments of mok_layer_fwd that
 * differ between calls (all host memory; the tables are host arrays of S
 * device pointers as for mok_layer_fwd). */
typedef struct mok_layer_call {
  int32_t own_lo, own_n;         /* own sources of the call */
  const void* const* src_x;      /* S source buffers [T_src, d] */
  const mok_fwd_state* st;       /* the call's forward state */
  void* const* staging;          /* S staging buffers [T_src*k, d] */
  void* const* out;              /* S outputs [T_src, d] (own entries) */
} mok_layer_call;

/* Macrobatch pipelining [K02: the combine of the previous macrobatch runs
 * concurrently with the dispatch of the next]: the forward pass of n_calls
 * layer calls (1..MOK_MAX_CALLS; consecutive layer calls or microbatches
 * with the same configuration and weights, each with its own sources,
 * state, staging rows and outputs) through one ring.  The routing and
 * layout of every call run first; then one persistent launch pulls,
 * computes and pushes the minibatches of call 0, 1, ... in order, and its
 * dispatch/combine workgroups run the final weighted combine of call i
 * while they pull the rows of call i + 1 (the last call's combine, with
 * nothing left to overlap, is a launch of its own after that kernel).  Needs cfg->ring_bytes > 0 and
 * prec MOK_BF16 or MOK_MXFP8 (MOK_EINVAL otherwise); the ring's counters
 * and per-call descriptors are part of mok_workspace_bytes(cfg).  Results
 * (state, staging rows, outputs) are bit-identical to n_calls separate
 * mok_layer_fwd calls.  Calls must not share outputs or state. */
mok_status mok_layer_fwd_macro(const mok_config* cfg, int32_t n_calls,
                               const mok_layer_call* calls, const void* w_router,
                               const float* bias, const int32_t* expert_to_local,
                               const mok_expert_weights* w, void* ws, int32_t* dev_status,
                               void* stream);

/* mok_layer_fwd without a workspace argument, for callers that cannot
 * allocate device memory at all: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, kernels and
 * results as mok_layer_fwd with ring_bytes == 0 and prec == MOK_BF16 (the
 * path whose only scratch is the layout's per-chunk expert counts); any other
 * precision or a ring is MOK_EINVAL.  The scratch is a static device array
 * of MOK_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends; it fits ceil(S*T_src*k / 1024) * E_local * 4 bytes, so a
 * cfg needing more returns MOK_ESCRATCH before anything is enqueued.  The
 * call itself allocates nothing (its first call on a device looks up that
 * device's copy of the array once).  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (two streams, or two threads)
 * race and give undefined results; calls in stream order do not.  The array
 * keeps the last call's contents; every value a call reads from it is
 * written by the same call first. */
#define MOK_NOALLOC_SCRATCH_BYTES (4u << 20)
mok_status mok_layer_fwd_noalloc(const mok_config* cfg, int32_t own_lo, int32_t own_n,
                                 const void* const* src_x, const void* w_router,
                                 const float* bias, const int32_t* expert_to_local,
                                 const mok_expert_weights* w, const mok_fwd_state* st,
                                 void* const* staging, void* const* out, int32_t* dev_status,
                                 void* stream);

/* Backward pass [K01 two more rounds in reverse; K02 pull reverse-combine and
 * push reverse-dispatch].  Inputs: d_out (host array of S device pointers
 * [T_src, d], the upstream gradient; sources whose rows are routed here are
 * read), src_x, w_router, expert_to_local, the weights, the forward state and
 * `staging` as the forward pass left them; for own items whose expert is
 * remote, their d_gate entry and dx_stage row as the GPU holding that expert
 * wrote them (read, never written here).  Outputs:
 *   d_gate [S*T_src*k] fp32: dL/dg for every local item (others untouched);
 *   dx_stage (host array of S device pointers [T_src*k, d], activation
 *     dtype): the pushed input gradient of every local row;
 *   d_x (host array of S pointers [T_src, d]): for own sources, the sum over
 *     the slots of dx_stage plus the router path sum_j dz_j w_router[e_j],
 *     dz_j = g_j (dg_j - sum_i g_i dg_i), over every slot except local rows
 *     dropped beyond R_cap;
 *   dw_gate, dw_up [E_local, I, d], dw_down [E_local, d, I] fp32 (overwritten);
 *   dw_router [E, d] fp32 over the own tokens (overwritten), or NULL.
 * MOK_MXFP8 [K02 MXFP8 in the GEMM data paths; K03 the backward in MXFP8]:
 * the four expert GEMMs run on the scaled matrix cores, each operand E4M3
 * with one E8M0 scale per 32 along its contraction axis, quantised from the
 * stored bf16 values: dy and [da|db] along the row, the weight gradients'
 * operands along the expert's rows (blocks of 32 from the expert's first
 * row, zero padded), h as the forward's GEMM2 read it.  It needs st->ab,
 * st->h_scale and the prepared wt_* / st_* weights (MOK_EINVAL otherwise),
 * and d % 128 == 0, I % 64 == 0 (MOK_ESHAPE); bwd_ring_bytes and aux are not
 * used.  The rows, the router path and the outputs are bf16 as for MOK_BF16.
 * MOK_F32, MOK_BF16 and MOK_MXFP8 are supported. */
mok_status mok_layer_bwd(const mok_config* cfg, int32_t own_lo, int32_t own_n,
                         const void* const* d_out, const void* const* src_x,
                         const void* w_router, const int32_t* expert_to_local,
                         const mok_expert_weights* w, const mok_fwd_state* st,
                         void* const* staging, float* d_gate, void* const* dx_stage,
                         void* const* d_x, float* dw_gate, float* dw_up, float* dw_down,
                         float* dw_router, void* ws, int32_t* dev_status, void* stream);

/* Transposed weights of the backward [K01 the backward of the expert FFN;
 * K02 MXFP8 in the GEMM data paths]: from the bf16 weights w_gate, w_up
 * [E_local, I, d] and w_down [E_local, d, I] (cfg->E_local, d, I), writes
 * wt_down [E_local, I, d] = W_down^T and wt_gu [E_local, d, 2I] =
 * [W_gate; W_up]^T.  cfg->prec MOK_BF16: bf16 copies (st_down, st_gu
 * unused).  MOK_MXFP8 (d % 128 == 0, else MOK_ESHAPE): their E4M3 codes with
 * st_down [E_local, I, d/32] and st_gu [E_local, d, 2I/32] (OCP MX v1.0
 * blocks of 32 along the last axis; shared exponent floor(log2 amax) - 8,
 * nearest E4M3 with ties to even, saturating).  MOK_F32: MOK_EINVAL.
 * Caller-owned outputs; run once per weight update, off the step. */
mok_status mok_prepare_bwd(const mok_config* cfg, const void* w_gate, const void* w_up,
                           const void* w_down, void* wt_down, uint8_t* st_down, void* wt_gu,
                           uint8_t* st_gu, void* stream);

/* Tuner of the fused path's minibatch size and workgroup split [K02: the
 * split of SMs between the communication and compute sides is set directly,
 * and the minibatch size trades a long wait for the first computation
 * (too large) against too few GEMM tasks to keep the SMs busy (too small);
 * K03: the right minibatch size and number of communication SMs change with
 * the hidden size, top-k and expert size].  Off the
 * timed path, and unlike every other entry point it synchronises the host
 * with `stream`.  For each candidate (mbs[i], comms[j]) -- cfg with
 * minibatch_rows = mbs[i], comm_wgs = comms[j], gemm_wgs = 0 (the remaining
 * CUs) -- it runs mok_layer_fwd once to warm up and then `reps` times
 * (1..1000) between two HIP events, with the arguments of mok_layer_fwd.
 * mbs / comms: host arrays of 1..64 entries, or NULL for {64, 128, 256, 512,
 * 1024, 2048, 4096} rows and {1/16, 1/8, 3/16, 1/4} of the CUs.  cfg->ring_bytes and
 * cfg->R_cap must be > 0.  ws_bytes: size of ws; a candidate whose
 * mok_workspace_bytes exceeds it, or that the ring cannot take (no slot of
 * that many rows, a split beyond the CUs), is skipped.  Outputs:
 * *best = cfg with the fastest candidate's two fields (host), times_ms
 * [n_mb*n_comm] (host, row i*n_comm + j; NULL allowed) the mean milliseconds
 * per call or -1 for a skipped candidate.  The forward outputs and state
 * are those of one mok_layer_fwd call: they do not depend on the tunables.
 * Returns MOK_EINVAL if no candidate could run; a status the device latched
 * during a candidate (read back after it) is returned and tuning stops. */
mok_status mok_tune_fwd(const mok_config* cfg, const int32_t* mbs, int32_t n_mb,
                        const int32_t* comms, int32_t n_comm, int32_t reps, size_t ws_bytes,
                        int32_t own_lo, int32_t own_n, const void* const* src_x,
                        const void* w_router, const float* bias, const int32_t* expert_to_local,
                        const mok_expert_weights* w, const mok_fwd_state* st,
                        void* const* staging, void* const* out, void* ws, int32_t* dev_status,
                        void* stream, mok_config* best, float* times_ms);

/* Where the fused path keeps its ring inside the workspace, for inspection
 * [K02 ring token buffer]: the ring of cfg (ring_bytes > 0, bf16 or MXFP8)
 * starts *offset bytes into ws and holds *nslot slots of *slot_bytes bytes.
 * After mok_layer_fwd, minibatch m (the m-th run of at most minibatch_rows
 * consecutive rows of one local expert, experts in order) is in slot
 * m % nslot unless a later minibatch reused the slot.  A slot holds its
 * rows in order: bf16 rows of d values, or for MOK_MXFP8 minibatch_rows * d
 * E4M3 codes followed by minibatch_rows * d/32 E8M0 scales.  Host only;
 * MOK_EINVAL if cfg has no ring or the ring holds no slot. */
mok_status mok_ring_layout(const mok_config* cfg, size_t* offset, size_t* slot_bytes,
                           int32_t* nslot);

/* HBM streaming probe: a reference rate for the layer's data-movement
 * kernels.  Moves `bytes` (a multiple of 16) with 16-byte vector loads and
 * stores, the access of those kernels, from a persistent grid of a few
 * workgroups per CU that walks 32 KiB chunks with a grid stride.  mode 0:
 * read src (dst must hold `bytes` too; a word is written there only in the
 * unlikely case that a lane's folded words equal a fixed pattern); 1: write
 * dst; 2: copy src to dst.  Pointers 16-byte aligned, device memory.
 * MOK_EINVAL on a bad mode, size or pointer. */
mok_status mok_hbm_stream(int32_t mode, void* dst, const void* src, int64_t bytes, void* stream);

/* Matrix-core rate probe: a reference rate for the expert GEMMs.  Launches
 * `workgroups` workgroups of 256 threads (one per CU gives one wave per
 * SIMD); every wave runs `iters` rounds of 16 MFMAs on operands held in
 * registers, with no memory traffic, so the rate reflects what the matrix
 * cores sustain under the chip's power limit.  kind 0: bf16
 * (32x32x16, 32768 flops each); kind 1: E4M3 with unit E8M0 scales
 * (32x32x64, 131072 flops each).  constant 0: hashed operand values
 * (random-looking data, the layer's case); 1: every operand 1.0, which makes
 * out exact.  out: device memory, workgroups * 256 floats, one sum of its
 * accumulators per thread.  MOK_EINVAL on a bad kind, flag, count or null
 * out. */
mok_status mok_mfma_probe(int32_t kind, int32_t constant, int64_t iters, int32_t workgroups,
                          float* out, void* stream);

/* MX quantisation of rows of bf16 values (weight preparation off the timed
 * path, and the same codec as the fused activation paths):  src [rows, K]
 * bf16 (K % 32 == 0), 16-byte aligned -> codes [rows, K] E4M3 (8-byte
 * aligned), scales [rows, K/32] E8M0; MOK_EINVAL otherwise.
 * Per block of 32: shared = clamp(floor(log2 max|v|) - 8, -127, 127) (-127 for
 * an all-zero block), scale byte = shared + 127, code = E4M3 of v / 2^shared,
 * nearest, ties to even, saturating at +-448 (OCP Microscaling v1.0). */
mok_status mok_mx_quantize(int64_t rows, int64_t K, const void* src, uint8_t* codes,
                           uint8_t* scales, void* stream);

/* The same MX quantisation of rows of fp32 values (the codec the GEMM1
 * epilogue applies to h, which it forms in fp32): src [rows, K] fp32, 16-byte
 * aligned (K % 32 == 0); outputs, alignment and errors as mok_mx_quantize.
 * Inputs are finite (a NaN gets an unspecified code). */
mok_status mok_mx_quantize_f32(int64_t rows, int64_t K, const float* src, uint8_t* codes,
                               uint8_t* scales, void* stream);

/* Library version string (static storage). */
const char* mok_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOK_H */
