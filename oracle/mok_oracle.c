/*
 * CPU oracle of the fused MoE layer: route -> expert-contiguous layout ->
 * gather -> SwiGLU expert FFN -> gate-weighted combine, and its backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library; the HIP library never does,
 * and the two share no code.  Plain, single-threaded, unblocked loops in
 * float64, except where a step is defined in a narrower precision:
 *   - router logits are an fp32 chain (the precision the GPU kernel decides
 *     top-k in), so that expert selection can be compared bit for bit;
 *   - stored intermediates (h, y, out) are rounded to the storage dtype the
 *     layer keeps them in (fp32, bf16 or MXFP8), once, round-to-nearest-even.
 * Precision code MOKREF_EXACT turns every rounding off (float64 throughout,
 * logits included); it exists for the finite-difference and closed-form pins.
 *
 * Sources (pages on the Mixture-of-Kittens MoE kernel):
 *   - LeFeng.com article on kucoin.com, section 01 ("the communication tax of
 *     MoE"): a router picks a few experts per token; the system counts tokens
 *     per expert, decides their placement, groups each expert's tokens
 *     together so a grouped GEMM can run; dispatch and combine in the forward
 *     pass, two more rounds in reverse in the backward pass.
 *   - same article, section 02: pull dispatch / push combine, pull
 *     reverse-combine / push reverse-dispatch; SwiGLU and MXFP8 activation
 *     quantisation in the dispatch, grouped-GEMM and SwiGLU data paths.
 *   - same article, section 03: the measured layer is scheduling, routing,
 *     expert FFN, combine and the final weighted combine.
 *   - miku-ai.ru article, section "Производительность и масштабируемость":
 *     results are bit-for-bit reproducible.
 * Readings where the pages are silent (score function, tie rule, row order,
 * MX scale rule, ...) are listed at the top of each function.
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MOKREF_F32 0
#define MOKREF_BF16 1
#define MOKREF_MXFP8 2
#define MOKREF_EXACT 3

#define MX_BLOCK 32

/* ------------------------------------------------------------------ rounding */

/* Round a float64 to the nearest bf16 value (8 significant bits), ties to
 * even, returned as a double.  bf16 has fp32's exponent range. */
double mokref_round_bf16(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  double a = fabs(v);
  if (a < ldexp(1.0, -126)) {
    /* subnormal range: fixed quantum 2^-133 */
    double r = nearbyint(ldexp(v, 133));
    return ldexp(r, -133);
  }
  int e;
  double m = frexp(v, &e); /* v = m * 2^e, 0.5 <= |m| < 1 */
  double r = nearbyint(ldexp(m, 8));
  return ldexp(r, e - 8);
}

/* ------------------------------------------------------------------ e4m3 / e8m0 */

/* OCP 8-bit float E4M3 ("fn" variant): 1 sign, 4 exponent bits (bias 7), 3
 * mantissa bits, no infinities, S.1111.111 is NaN; largest finite 448. */
double mokref_e4m3_decode(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(8.0 + m, e - 10);
  return s ? -v : v;
}

/* Nearest E4M3 code to v, ties to the even code, magnitudes above 448
 * saturate to +-448 (the MX conversion rule for E4M3 elements). */
int mokref_e4m3_encode(double v) {
  int sign = signbit(v) ? 0x80 : 0;
  double a = fabs(v);
  if (isnan(v)) return 0x7F;
  if (a >= 448.0) return sign | 0x7E;
  /* quantum of the binade holding a (binades below 2^-6 share quantum 2^-9) */
  int e;
  frexp(a, &e); /* a = m 2^e, m in [0.5,1) -> floor(log2 a) = e-1 */
  int fl = (a == 0.0) ? -6 : e - 1;
  if (fl < -6) fl = -6;
  double q = ldexp(1.0, fl - 3);
  double r = nearbyint(a / q) * q; /* exact: a/q is a scaling by 2^k */
  if (r > 448.0) r = 448.0;
  /* r is an E4M3 value: find its code */
  int code;
  if (r < ldexp(1.0, -6)) {
    code = (int)nearbyint(ldexp(r, 9));
  } else {
    int e2;
    double m2 = frexp(r, &e2); /* r = m2 2^e2 */
    int ex = e2 - 1 + 7;
    int mant = (int)nearbyint(ldexp(m2, 4)) - 8;
    code = (ex << 3) | mant;
  }
  return sign | code;
}

/* MX block quantisation (OCP Microscaling v1.0 rule): per block of 32
 * contiguous values, shared exponent = floor(log2(max|v|)) - 8 (8 = largest
 * E4M3 exponent), clamped to [-127, 127]; all-zero blocks get -127.  The scale
 * byte (E8M0) is shared + 127; each element is E4M3(v / 2^shared).
 * v: [rows, K] (K a multiple of 32), codes: [rows, K], scales: [rows, K/32]. */
void mokref_mx_quantize(int64_t rows, int64_t K, const double* v, uint8_t* codes,
                        uint8_t* scales) {
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < K / MX_BLOCK; ++b) {
      const double* blk = v + r * K + b * MX_BLOCK;
      double amax = 0.0;
      for (int i = 0; i < MX_BLOCK; ++i)
        if (fabs(blk[i]) > amax) amax = fabs(blk[i]);
      int shared;
      if (amax == 0.0) {
        shared = -127;
      } else {
        int e;
        frexp(amax, &e);
        shared = (e - 1) - 8;
        if (shared < -127) shared = -127;
        if (shared > 127) shared = 127;
      }
      scales[r * (K / MX_BLOCK) + b] = (uint8_t)(shared + 127);
      for (int i = 0; i < MX_BLOCK; ++i)
        codes[r * K + b * MX_BLOCK + i] = (uint8_t)mokref_e4m3_encode(ldexp(blk[i], -shared));
    }
  }
}

void mokref_mx_dequantize(int64_t rows, int64_t K, const uint8_t* codes, const uint8_t* scales,
                          double* v) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < K; ++i) {
      int shared = (int)scales[r * (K / MX_BLOCK) + i / MX_BLOCK] - 127;
      v[r * K + i] = ldexp(mokref_e4m3_decode(codes[r * K + i]), shared);
    }
}

/* Round one vector the way the layer stores it in precision `prec`. */
static void store_round(int prec, int64_t n, double* v) {
  if (prec == MOKREF_EXACT) return;
  for (int64_t i = 0; i < n; ++i)
    v[i] = (prec == MOKREF_F32) ? (double)(float)v[i] : mokref_round_bf16(v[i]);
}

/* MXFP8 round trip of one row of length K (quantise then dequantise). */
static void mx_roundtrip(int64_t K, double* v) {
  uint8_t* c = (uint8_t*)malloc((size_t)K);
  uint8_t* s = (uint8_t*)malloc((size_t)(K / MX_BLOCK));
  mokref_mx_quantize(1, K, v, c, s);
  mokref_mx_dequantize(1, K, c, s, v);
  free(c);
  free(s);
}

/* ------------------------------------------------------------------ routing */

/* Router logits z[t][e] = x_t . Wr_e + bias_e.
 * Reading (the pages only say a router picks a few experts per token): the
 * logits are an fp32 chain, z = 0; for i ascending z = fma(x_i, w_i, z); then
 * one fp32 add of the bias.  For bf16 inputs every product is exact in fp32.
 * MOKREF_EXACT: the same sum in float64.  Output stored as double. */
void mokref_logits(int64_t T, int64_t d, int64_t E, const float* x, const float* wr,
                   const float* bias, int prec, double* z) {
  for (int64_t t = 0; t < T; ++t)
    for (int64_t e = 0; e < E; ++e) {
      if (prec == MOKREF_EXACT) {
        double acc = 0.0;
        for (int64_t i = 0; i < d; ++i) acc += (double)x[t * d + i] * (double)wr[e * d + i];
        z[t * E + e] = acc + (bias ? (double)bias[e] : 0.0);
      } else {
        float acc = 0.0f;
        for (int64_t i = 0; i < d; ++i) acc = fmaf(x[t * d + i], wr[e * d + i], acc);
        if (bias) acc = acc + bias[e];
        z[t * E + e] = (double)acc;
      }
    }
}

/* Does logit a (expert ea) rank before logit b (expert eb)?  Reading: larger
 * logit first, lower expert id first on equal logits.  The pages say nothing
 * of non-numbers; here a NaN logit ranks after every number (-inf included)
 * and NaNs rank among themselves by expert id, so that every token still gets
 * k distinct valid experts. */
static int ranks_before(double a, int64_t ea, double b, int64_t eb) {
  if (isnan(a) || isnan(b)) return isnan(b) && (!isnan(a) || ea < eb);
  return a > b || (a == b && ea < eb);
}

/* Top-k selection: slot j = 0 holds the first expert in the order above.
 * Picks the first unselected expert k times. */
void mokref_topk(int64_t T, int64_t E, int64_t k, const double* z, int32_t* idx) {
  char* used = (char*)malloc((size_t)E);
  for (int64_t t = 0; t < T; ++t) {
    memset(used, 0, (size_t)E);
    for (int64_t j = 0; j < k; ++j) {
      int64_t best = -1;
      for (int64_t e = 0; e < E; ++e) {
        if (used[e]) continue;
        if (best < 0 || ranks_before(z[t * E + e], e, z[t * E + best], best)) best = e;
      }
      used[best] = 1;
      idx[t * k + j] = (int32_t)best;
    }
  }
  free(used);
}

/* Gates: softmax over all E experts renormalised over the k chosen ones.  The
 * renormalisation cancels the unchosen experts' terms, so this is the softmax
 * of the chosen logits, computed as such in float64:
 * g_j = exp(z_j - z_0) / sum_i exp(z_i - z_0), with z_0 the slot-0 logit.  A
 * NaN among the unchosen logits then leaves the gates alone. */
void mokref_gates(int64_t T, int64_t E, int64_t k, const double* z, const int32_t* idx,
                  double* g) {
  for (int64_t t = 0; t < T; ++t) {
    const double z0 = z[t * E + idx[t * k]];
    double tot = 0.0;
    for (int64_t j = 0; j < k; ++j) tot += exp(z[t * E + idx[t * k + j]] - z0);
    for (int64_t j = 0; j < k; ++j) g[t * k + j] = exp(z[t * E + idx[t * k + j]] - z0) / tot;
  }
}

/* Route T tokens: logits, top-k, gates.  z may be NULL (scratch allocated). */
void mokref_route(int64_t T, int64_t d, int64_t E, int64_t k, const float* x, const float* wr,
                  const float* bias, int prec, int32_t* idx, double* gate) {
  double* z = (double*)malloc(sizeof(double) * (size_t)(T * E));
  mokref_logits(T, d, E, x, wr, bias, prec, z);
  mokref_topk(T, E, k, z, idx);
  mokref_gates(T, E, k, z, idx, gate);
  free(z);
}

/* ------------------------------------------------------------------ layout */

/* Expert-contiguous layout (kucoin article, section 01: count tokens per
 * expert, decide placement, group each expert's tokens; section 02: the
 * receiver chooses the placement and orders rows per local expert).
 * Items n = (s*T_src + t)*k + j in ascending n; an item is a routed row here
 * when expert_to_local[topk[n]] >= 0.  Reading: rows of one expert keep
 * ascending n (ascending source, token, slot) -- a stable counting sort.
 * Outputs: counts[E_local], offsets[E_local+1] (exclusive scan), row_src[R]
 * (row -> n), dest_row[S*T_src*k] (n -> row, -1 when the expert is remote).
 * Returns R, or -1 when an expert id is out of range, or -2 when R > R_cap. */
int64_t mokref_layout(int64_t S, int64_t T_src, int64_t k, int64_t E, const int32_t* topk,
                      const int32_t* e2l, int64_t E_local, int64_t R_cap, int32_t* counts,
                      int32_t* offsets, int32_t* row_src, int32_t* dest_row) {
  int64_t N = S * T_src * k;
  for (int64_t e = 0; e < E_local; ++e) counts[e] = 0;
  for (int64_t n = 0; n < N; ++n) {
    if (topk[n] < 0 || topk[n] >= E) return -1;
    int32_t le = e2l[topk[n]];
    if (le >= 0) counts[le] += 1;
  }
  offsets[0] = 0;
  for (int64_t e = 0; e < E_local; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int64_t R = offsets[E_local];
  if (R > R_cap) return -2;
  int32_t* cursor = (int32_t*)calloc((size_t)(E_local > 0 ? E_local : 1), sizeof(int32_t));
  for (int64_t n = 0; n < N; ++n) {
    int32_t le = e2l[topk[n]];
    if (le < 0) {
      dest_row[n] = -1;
      continue;
    }
    int32_t row = offsets[le] + cursor[le]++;
    row_src[row] = (int32_t)n;
    dest_row[n] = row;
  }
  free(cursor);
  return R;
}

/* ------------------------------------------------------------------ expert FFN */

static double silu(double a) { return a / (1.0 + exp(-a)); }
static double sigmoid(double a) { return 1.0 / (1.0 + exp(-a)); }

/* One routed row through one expert's SwiGLU FFN (kucoin article, section 02
 * names SwiGLU in the expert path; the formula is the usual gated one):
 *   a = W_gate x, b = W_up x          (W_gate, W_up: [I, d])
 *   h = silu(a) * b                   -> stored in the layer's dtype
 *   y = W_down h                      (W_down: [d, I]) -> stored dtype
 * prec MXFP8: x is MX-quantised along d, h along I (from its fp32 value);
 * the weights passed in are already the dequantised MX values.
 * a, b, h may be NULL. */
void mokref_ffn_row(int64_t d, int64_t I, int prec, const float* x, const float* wg,
                    const float* wu, const float* wd, double* a_out, double* b_out,
                    double* h_out, double* y) {
  double* xv = (double*)malloc(sizeof(double) * (size_t)d);
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  for (int64_t i = 0; i < d; ++i) xv[i] = (double)x[i];
  if (prec == MOKREF_MXFP8) mx_roundtrip(d, xv);
  for (int64_t i = 0; i < I; ++i) {
    double a = 0.0, b = 0.0;
    for (int64_t c = 0; c < d; ++c) {
      a += xv[c] * (double)wg[i * d + c];
      b += xv[c] * (double)wu[i * d + c];
    }
    if (a_out) a_out[i] = a;
    if (b_out) b_out[i] = b;
    h[i] = silu(a) * b;
  }
  if (prec == MOKREF_MXFP8) {
    for (int64_t i = 0; i < I; ++i) h[i] = (double)(float)h[i];
    mx_roundtrip(I, h);
  } else {
    store_round(prec, I, h);
  }
  if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)I);
  for (int64_t c = 0; c < d; ++c) {
    double acc = 0.0;
    for (int64_t i = 0; i < I; ++i) acc += h[i] * (double)wd[c * I + i];
    y[c] = acc;
  }
  store_round(prec == MOKREF_MXFP8 ? MOKREF_BF16 : prec, d, y);
  free(xv);
  free(h);
}

/* ------------------------------------------------------------------ layer forward */

/* Forward outputs of a list of tokens.
 * tok_x: [n_tok, d] the tokens' rows; topk/gate: [n_tok, k] their routing;
 * e2l: [E] expert -> local index (-1 remote); weights of the local experts
 * (wg, wu: [E_local, I, d], wd: [E_local, d, I]).
 * peer_y: [n_tok, k, d] or NULL (= zeros): for a slot whose expert is remote,
 *    the row that the GPU holding that expert pushed into the token's source
 *    (kucoin article, section 02, push combine: every expert's output lands in
 *    the source's buffer, so the source's combine reads all k slots).
 * y: [n_tok, k, d] the expert output of each (token, slot) -- what the push
 *    combine delivers to the token's source, in the stored dtype; the peer's
 *    row when the slot's expert is remote;
 * out: [n_tok, d] the final weighted combine out = sum_j g_j y_j over all k
 *    slots (kucoin article, section 03 lists it as its own step), float64 sum
 *    rounded once to the output dtype. */
void mokref_fwd_tokens(int64_t n_tok, int64_t d, int64_t E, int64_t k, int64_t I, int prec,
                       const float* tok_x, const int32_t* topk, const double* gate,
                       const int32_t* e2l, const float* wg, const float* wu, const float* wd,
                       const double* peer_y, double* y, double* out) {
  for (int64_t t = 0; t < n_tok; ++t) {
    double* o = out + t * d;
    for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      double* yj = y + (t * k + j) * d;
      int32_t e = topk[t * k + j];
      int32_t le = (e >= 0 && e < E) ? e2l[e] : -1;
      if (le < 0) {
        for (int64_t c = 0; c < d; ++c) yj[c] = peer_y ? peer_y[(t * k + j) * d + c] : 0.0;
      } else {
        mokref_ffn_row(d, I, prec, tok_x + t * d, wg + le * I * d, wu + le * I * d,
                       wd + le * d * I, NULL, NULL, NULL, yj);
      }
      for (int64_t c = 0; c < d; ++c) o[c] += gate[t * k + j] * yj[c];
    }
    store_round(prec == MOKREF_MXFP8 ? MOKREF_BF16 : prec, d, o);
  }
}

/* ------------------------------------------------------------------ backward */

/* Backward of one routed row (chain rule of mokref_ffn_row without its
 * roundings, float64).  Inputs: the row's token x [d], its gate g, the
 * upstream gradient of the token's output dout [d].  The reverse-combine
 * brings dy = g * dout to the expert (kucoin article, section 02: pull
 * reverse-combine).  Outputs (any may be NULL):
 *   dx [d]   = W_gate^T da + W_up^T db  (pushed back by the reverse dispatch)
 *   dg       = dout . y                 (gradient of the token's gate)
 *   dy [d], h [I], da [I], db [I]       (the wgrad operands)
 * with dh = W_down^T dy, s = sigmoid(a), da = dh * b * s * (1 + a (1 - s)),
 * db = dh * silu(a). */
void mokref_bwd_row(int64_t d, int64_t I, const float* x, double g, const float* dout,
                    const float* wg, const float* wu, const float* wd, double* dx, double* dg,
                    double* dy_out, double* h_out, double* da_out, double* db_out) {
  double* a = (double*)malloc(sizeof(double) * (size_t)I);
  double* b = (double*)malloc(sizeof(double) * (size_t)I);
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  double* y = (double*)malloc(sizeof(double) * (size_t)d);
  double* dy = (double*)malloc(sizeof(double) * (size_t)d);
  double* da = (double*)malloc(sizeof(double) * (size_t)I);
  double* db = (double*)malloc(sizeof(double) * (size_t)I);
  mokref_ffn_row(d, I, MOKREF_EXACT, x, wg, wu, wd, a, b, h, y);
  double s = 0.0;
  for (int64_t c = 0; c < d; ++c) s += (double)dout[c] * y[c];
  if (dg) *dg = s;
  for (int64_t c = 0; c < d; ++c) dy[c] = g * (double)dout[c];
  for (int64_t i = 0; i < I; ++i) {
    double dh = 0.0;
    for (int64_t c = 0; c < d; ++c) dh += dy[c] * (double)wd[c * I + i];
    double sg = sigmoid(a[i]);
    da[i] = dh * b[i] * sg * (1.0 + a[i] * (1.0 - sg));
    db[i] = dh * silu(a[i]);
  }
  if (dx) {
    for (int64_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t i = 0; i < I; ++i)
        acc += da[i] * (double)wg[i * d + c] + db[i] * (double)wu[i * d + c];
      dx[c] = acc;
    }
  }
  if (dy_out) memcpy(dy_out, dy, sizeof(double) * (size_t)d);
  if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)I);
  if (da_out) memcpy(da_out, da, sizeof(double) * (size_t)I);
  if (db_out) memcpy(db_out, db, sizeof(double) * (size_t)I);
  free(a); free(b); free(h); free(y); free(dy); free(da); free(db);
}

/* Router backward of one token: gates g_j = softmax over the chosen logits, so
 * dz_j = g_j (dg_j - sum_i g_i dg_i) on the chosen experts and 0 elsewhere
 * (the selection itself is piecewise constant).  dx_router = sum_j dz_j Wr_e_j.
 * dz: [k] out; dxr: [d] out (may be NULL). */
void mokref_router_bwd_token(int64_t d, int64_t k, const int32_t* idx, const double* g,
                             const double* dg, const float* wr, double* dz, double* dxr) {
  double m = 0.0;
  for (int64_t j = 0; j < k; ++j) m += g[j] * dg[j];
  for (int64_t j = 0; j < k; ++j) dz[j] = g[j] * (dg[j] - m);
  if (dxr) {
    for (int64_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t j = 0; j < k; ++j) acc += dz[j] * (double)wr[(int64_t)idx[j] * d + c];
      dxr[c] = acc;
    }
  }
}

/* Backward of a list of tokens (float64, no roundings).
 * Per token: for each slot whose expert is local, the row backward above;
 * for a slot whose expert is remote, the GPU holding that expert computes
 * the same row backward and writes its gate gradient and pushes its input
 * gradient back to the token's source (kucoin article, section 02: pull
 * reverse-combine, push reverse-dispatch): those arrive as peer_dg [n_tok, k]
 * and peer_dx [n_tok, k, d] (either may be NULL = zeros).
 * d_gate[t][j] = the slot's gate gradient; dx[t] = sum_j dx_row_j + the
 * router path through dz = g (dg - sum g dg).  dz: [n_tok, k] out. */
void mokref_bwd_tokens(int64_t n_tok, int64_t d, int64_t E, int64_t k, int64_t I,
                       const float* tok_x, const float* tok_dout, const int32_t* topk,
                       const double* gate, const int32_t* e2l, const float* wr, const float* wg,
                       const float* wu, const float* wd, const double* peer_dg,
                       const double* peer_dx, double* d_gate, double* dz, double* dx) {
  double* dxr = (double*)malloc(sizeof(double) * (size_t)d);
  double* dxj = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t t = 0; t < n_tok; ++t) {
    double* o = dx + t * d;
    for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      int32_t le = e2l[topk[t * k + j]];
      if (le < 0) {
        d_gate[t * k + j] = peer_dg ? peer_dg[t * k + j] : 0.0;
        if (peer_dx)
          for (int64_t c = 0; c < d; ++c) o[c] += peer_dx[(t * k + j) * d + c];
        continue;
      }
      mokref_bwd_row(d, I, tok_x + t * d, gate[t * k + j], tok_dout + t * d, wg + le * I * d,
                     wu + le * I * d, wd + le * d * I, dxj, &d_gate[t * k + j], NULL, NULL,
                     NULL, NULL);
      for (int64_t c = 0; c < d; ++c) o[c] += dxj[c];
    }
    mokref_router_bwd_token(d, k, topk + t * k, gate + t * k, d_gate + t * k, wr, dz + t * k, dxr);
    for (int64_t c = 0; c < d; ++c) o[c] += dxr[c];
  }
  free(dxr);
  free(dxj);
}

/* Weight gradients of one local expert from its routed rows (float64):
 *   dW_down += dy h^T, dW_gate += da x^T, dW_up += db x^T, rows in the order
 * given.  rows_x: [n, d] the rows' tokens; rows_g: [n]; rows_dout: [n, d].
 * Outputs (zeroed here): dwg, dwu [I, d], dwd [d, I]. */
void mokref_expert_wgrad(int64_t n, int64_t d, int64_t I, const float* rows_x,
                         const double* rows_g, const float* rows_dout, const float* wg,
                         const float* wu, const float* wd, double* dwg, double* dwu,
                         double* dwd) {
  double* dy = (double*)malloc(sizeof(double) * (size_t)d);
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  double* da = (double*)malloc(sizeof(double) * (size_t)I);
  double* db = (double*)malloc(sizeof(double) * (size_t)I);
  memset(dwg, 0, sizeof(double) * (size_t)(I * d));
  memset(dwu, 0, sizeof(double) * (size_t)(I * d));
  memset(dwd, 0, sizeof(double) * (size_t)(I * d));
  for (int64_t r = 0; r < n; ++r) {
    const float* x = rows_x + r * d;
    mokref_bwd_row(d, I, x, rows_g[r], rows_dout + r * d, wg, wu, wd, NULL, NULL, dy, h, da, db);
    for (int64_t c = 0; c < d; ++c)
      for (int64_t i = 0; i < I; ++i) dwd[c * I + i] += dy[c] * h[i];
    for (int64_t i = 0; i < I; ++i)
      for (int64_t c = 0; c < d; ++c) {
        dwg[i * d + c] += da[i] * (double)x[c];
        dwu[i * d + c] += db[i] * (double)x[c];
      }
  }
  free(dy); free(h); free(da); free(db);
}

/* Selected columns of one expert's weight gradients (float64), for checks at
 * sizes where the whole gradient is too slow: the same sums as
 * mokref_expert_wgrad, restricted to the intermediate indices sel[0..n_sel):
 *   dwg_sel[q][c] = dW_gate[sel[q]][c], dwu_sel[q][c] = dW_up[sel[q]][c],
 *   dwd_sel[c][q] = dW_down[c][sel[q]],
 * rows in the order given.  Per row only a, b, h, dh, da, db at the selected
 * indices are formed (dy = g dout as in the row backward). */
void mokref_expert_wgrad_cols(int64_t n, int64_t d, int64_t I, const float* rows_x,
                              const double* rows_g, const float* rows_dout, const float* wg,
                              const float* wu, const float* wd, int64_t n_sel,
                              const int32_t* sel, double* dwg_sel, double* dwu_sel,
                              double* dwd_sel) {
  double* dy = (double*)malloc(sizeof(double) * (size_t)d);
  memset(dwg_sel, 0, sizeof(double) * (size_t)(n_sel * d));
  memset(dwu_sel, 0, sizeof(double) * (size_t)(n_sel * d));
  memset(dwd_sel, 0, sizeof(double) * (size_t)(n_sel * d));
  for (int64_t r = 0; r < n; ++r) {
    const float* x = rows_x + r * d;
    for (int64_t c = 0; c < d; ++c) dy[c] = rows_g[r] * (double)rows_dout[r * d + c];
    for (int64_t q = 0; q < n_sel; ++q) {
      const int64_t i = sel[q];
      double a = 0.0, b = 0.0, dh = 0.0;
      for (int64_t c = 0; c < d; ++c) {
        a += (double)x[c] * (double)wg[i * d + c];
        b += (double)x[c] * (double)wu[i * d + c];
      }
      for (int64_t c = 0; c < d; ++c) dh += dy[c] * (double)wd[c * I + i];
      const double h = silu(a) * b;
      const double sg = sigmoid(a);
      const double da = dh * b * sg * (1.0 + a * (1.0 - sg));
      const double db = dh * silu(a);
      for (int64_t c = 0; c < d; ++c) {
        dwg_sel[q * d + c] += da * (double)x[c];
        dwu_sel[q * d + c] += db * (double)x[c];
        dwd_sel[c * n_sel + q] += dy[c] * h;
      }
    }
  }
  free(dy);
}

/* MX round trip of a vector of n values quantised in blocks of 32 along it,
 * the last block padded with zeros (the layout pads every expert's rows to
 * whole blocks). */
static void mx_roundtrip_padded(int64_t n, double* v) {
  const int64_t np = (n + MX_BLOCK - 1) / MX_BLOCK * MX_BLOCK;
  double* t = (double*)calloc((size_t)(np > 0 ? np : 1), sizeof(double));
  memcpy(t, v, sizeof(double) * (size_t)n);
  if (np > 0) mx_roundtrip(np, t);
  memcpy(v, t, sizeof(double) * (size_t)n);
  free(t);
}

/* Columns of a row-major [n, cols] matrix as [cols][n] copies, each
 * MX-quantised along the rows (zero padded to whole blocks) when quant. */
static double* column_copies(int64_t n, int64_t cols, const double* m, int quant) {
  double* o = (double*)malloc(sizeof(double) * (size_t)(n * cols > 0 ? n * cols : 1));
  for (int64_t c = 0; c < cols; ++c) {
    for (int64_t r = 0; r < n; ++r) o[c * n + r] = m[r * cols + c];
    if (quant) mx_roundtrip_padded(n, o + c * n);
  }
  return o;
}

/* MXFP8 backward of one local expert's routed rows (kucoin article, section
 * 03: the layer's backward in MXFP8).  The pages fix only that the backward
 * runs in MXFP8; the reading taken: every GEMM quantises both operands to
 * E4M3 with one E8M0 scale per 32 elements along its contraction axis, from
 * the values the layer stores (bf16), and accumulates exactly; results are
 * stored in bf16 (rows) or kept exact (weight gradients):
 *   dy   = bf16(g dout)
 *   dh   = bf16(MX_d(dy) . MX_d(W_down^T))          contraction over d
 *   da, db from dh and the saved a, b (bf16) -> bf16
 *   dx   = bf16(MX_2I([da|db]) . MX_2I([W_gate; W_up]^T))   over 2I
 *   dW_gate|up = MX_rows([da|db]^T) . MX_rows(X^T)  over the expert's rows
 *   dW_down    = MX_rows(dy^T) . MX_rows(h^T)       over the expert's rows
 * where MX_rows quantises each column in blocks of 32 consecutive rows of
 * the expert, zero padded, and h is the forward's h as its GEMM2 used it.
 * quant = 0 turns every MX quantisation and bf16 rounding off: the exact
 * backward of mokref_bwd_row / mokref_expert_wgrad.
 * rows_a, rows_b, rows_h [n, I]; wg, wu [I, d], wd [d, I] (the bf16 weights,
 * not their forward MX values).  Outputs: dx [n, d] (the rows' input
 * gradients), dwg, dwu [I, d], dwd [d, I]. */
void mokref_expert_bwd_mx(int64_t n, int64_t d, int64_t I, int quant, const float* rows_x,
                          const double* rows_g, const float* rows_dout, const double* rows_a,
                          const double* rows_b, const double* rows_h, const float* wg,
                          const float* wu, const float* wd, double* dx, double* dwg,
                          double* dwu, double* dwd) {
  const int64_t I2 = 2 * I;
  double* wdt = (double*)malloc(sizeof(double) * (size_t)(I * d));   /* [I][d] */
  double* wgut = (double*)malloc(sizeof(double) * (size_t)(d * I2)); /* [d][2I] */
  for (int64_t i = 0; i < I; ++i)
    for (int64_t c = 0; c < d; ++c) wdt[i * d + c] = (double)wd[c * I + i];
  for (int64_t c = 0; c < d; ++c)
    for (int64_t i = 0; i < I2; ++i)
      wgut[c * I2 + i] = i < I ? (double)wg[i * d + c] : (double)wu[(i - I) * d + c];
  if (quant) {
    for (int64_t i = 0; i < I; ++i) mx_roundtrip(d, wdt + i * d);
    for (int64_t c = 0; c < d; ++c) mx_roundtrip(I2, wgut + c * I2);
  }
  double* dy = (double*)malloc(sizeof(double) * (size_t)(n * d > 0 ? n * d : 1));
  double* dab = (double*)malloc(sizeof(double) * (size_t)(n * I2 > 0 ? n * I2 : 1));
  double* q = (double*)malloc(sizeof(double) * (size_t)(d > I2 ? d : I2));
  for (int64_t r = 0; r < n; ++r) {
    double* dyr = dy + r * d;
    for (int64_t c = 0; c < d; ++c) dyr[c] = rows_g[r] * (double)rows_dout[r * d + c];
    if (quant) store_round(MOKREF_BF16, d, dyr);
    memcpy(q, dyr, sizeof(double) * (size_t)d);
    if (quant) mx_roundtrip(d, q);
    double* dabr = dab + r * I2;
    for (int64_t i = 0; i < I; ++i) {
      double dh = 0.0;
      for (int64_t c = 0; c < d; ++c) dh += q[c] * wdt[i * d + c];
      double a = rows_a[r * I + i], b = rows_b[r * I + i];
      if (quant) {
        dh = mokref_round_bf16(dh);
        a = mokref_round_bf16(a);
        b = mokref_round_bf16(b);
      }
      const double sg = sigmoid(a);
      dabr[i] = dh * b * sg * (1.0 + a * (1.0 - sg));
      dabr[I + i] = dh * silu(a);
    }
    if (quant) store_round(MOKREF_BF16, I2, dabr);
    memcpy(q, dabr, sizeof(double) * (size_t)I2);
    if (quant) mx_roundtrip(I2, q);
    for (int64_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t i = 0; i < I2; ++i) acc += q[i] * wgut[c * I2 + i];
      dx[r * d + c] = quant ? mokref_round_bf16(acc) : acc;
    }
  }
  /* weight gradients: every column of [da|db], X, dy and h quantised along
   * the rows once ([column][row] copies), then one dot product per element */
  double* cab = column_copies(n, I2, dab, quant);
  double* cx = (double*)malloc(sizeof(double) * (size_t)(n * d > 0 ? n * d : 1));
  for (int64_t c = 0; c < d; ++c) {
    for (int64_t r = 0; r < n; ++r) cx[c * n + r] = (double)rows_x[r * d + c];
    if (quant) mx_roundtrip_padded(n, cx + c * n);
  }
  double* cdy = column_copies(n, d, dy, quant);
  double* ch = column_copies(n, I, rows_h, quant);
  for (int64_t i = 0; i < I2; ++i)
    for (int64_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t r = 0; r < n; ++r) acc += cab[i * n + r] * cx[c * n + r];
      if (i < I) dwg[i * d + c] = acc; else dwu[(i - I) * d + c] = acc;
    }
  for (int64_t c = 0; c < d; ++c)
    for (int64_t i = 0; i < I; ++i) {
      double acc = 0.0;
      for (int64_t r = 0; r < n; ++r) acc += cdy[c * n + r] * ch[i * n + r];
      dwd[c * I + i] = acc;
    }
  free(cab); free(cx); free(cdy); free(ch);
  free(wdt); free(wgut); free(dy); free(dab); free(q);
}

/* Router weight gradient over the tokens routed here: dWr[e] = sum_t dz_t,e x_t
 * with dz from mokref_router_bwd_token (tokens in the order given).
 * dwr: [E, d] out (zeroed here). */
void mokref_router_wgrad(int64_t n_tok, int64_t d, int64_t E, int64_t k, const float* tok_x,
                         const int32_t* topk, const double* dz, double* dwr) {
  memset(dwr, 0, sizeof(double) * (size_t)(E * d));
  for (int64_t t = 0; t < n_tok; ++t)
    for (int64_t j = 0; j < k; ++j) {
      int64_t e = topk[t * k + j];
      for (int64_t c = 0; c < d; ++c) dwr[e * d + c] += dz[t * k + j] * (double)tok_x[t * d + c];
    }
}
