/*
 * moe_oracle.c -- a plain, slow, fp64 CPU oracle for the forward and backward
 * passes of one Mixture-of-Experts block on one GPU's share of tokens.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and
 * the CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or helper with the HIP library, and neither includes or
 * links the other.
 *
 * What it follows (page title, then section):
 *   [P1] "How MegaDLMs Implements Mixture of Experts (MoE) Architectures"
 *        - "Routing Mechanisms: Top-K vs Expert Choice": the TopKRouter scores
 *          every expert for every token with one trained linear map, applies a
 *          softmax and keeps the k best experts per token, handing the
 *          dispatcher probability weights plus a routing map; the
 *          ExpertChoiceRouter lets every expert pick its tokens by score.
 *        - "Core MoE Layer Architecture" (MoELayer): permute tokens to their
 *          experts, run the local experts, unpermute back to sequence order.
 *        - "Activation Checkpointing and Constraints": the dropless mode, in
 *          which every token reaches every expert it selected; the layer is
 *          trained, and moe_layer_recompute re-runs its forward inside the
 *          backward pass (the backward below differentiates that forward).
 *   [P3] "Expert Parallelism > Key Parameters"
 *        - capacity_factor paragraph: each expert holds capacity_factor times
 *          the expected average load; tokens above it are dropped and their
 *          contribution is zeroed.
 *        - top_k paragraph: an always-used shared expert next to the routed
 *          top-k experts.
 *
 * Readings taken where the pages are silent:
 *   - selection key is the logit value; ties go to the lower expert index;
 *     comparisons are IEEE (so -0 == +0);
 *   - SOFTMAX_ALL: weight = softmax over all E experts at the chosen index,
 *     not renormalised; SOFTMAX_TOPK: softmax over the k chosen logits only;
 *   - capacity C = ceil(cf * T * k / E), cf == 0 means dropless;
 *   - drop priority follows token order, then slot order within a token;
 *   - permuted rows are expert-major, ascending token inside an expert;
 *   - expert FFN: GELU (exact erf form) or SwiGLU (gate rows first, then up
 *     rows), no biases; the shared expert is added with weight 1;
 *   - ExpertChoice scores are the per-token softmax over E; expert e keeps the
 *     C best tokens by (score desc, token asc), stored in ascending token order.
 *
 * Everything floating point is fp64.  fp32 and bf16 inputs are read from their
 * bit patterns and widened exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

#define ORC_GELU 0
#define ORC_SWIGLU 1

#define ORC_SOFTMAX_ALL 0
#define ORC_SOFTMAX_TOPK 1

int orc_version(void) { return 1; }

/* Exact widening of element i of a fp32 or bf16 buffer. */
static double ld(const void *p, int64_t i, int dt) {
  if (dt == ORC_F32) return (double)((const float *)p)[i];
  uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* [P1] Routing Mechanisms: the router scores every expert for every token with
 * one trained linear map (no bias of its own; the optional bias is an input).
 * logits[t,e] = sum_i x[t,i] * W_r[e,i]  (+ bias).  bias_stride 0: bias[e];
 * bias_stride E: bias[t*E+e]; bias NULL: no bias. */
void orc_logits(int T, int d, int E, int dt, const void *x, const void *wr,
                const float *bias, int64_t bias_stride, double *logits) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      double s = 0.0;
      for (int i = 0; i < d; ++i)
        s += ld(x, (int64_t)t * d + i, dt) * ld(wr, (int64_t)e * d + i, dt);
      if (bias) s += (double)bias[(int64_t)t * bias_stride + e];
      logits[(int64_t)t * E + e] = s;
    }
  }
}

/* Softmax over one row of n values, fp64. */
static void softmax_row(int n, const double *l, double *p) {
  double m = l[0];
  for (int i = 1; i < n; ++i)
    if (l[i] > m) m = l[i];
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += exp(l[i] - m);
  for (int i = 0; i < n; ++i) p[i] = exp(l[i] - m) / s;
}

void orc_softmax(int T, int E, const double *logits, double *p) {
  for (int t = 0; t < T; ++t) softmax_row(E, logits + (int64_t)t * E, p + (int64_t)t * E);
}

/* "a beats b": larger value, or equal value (IEEE ==, so -0 == +0) and the
 * lower index. */
static int beats(double va, int ia, double vb, int ib) {
  if (va > vb) return 1;
  if (va == vb && ia < ib) return 1;
  return 0;
}

/* [P1] Routing Mechanisms: top-k experts per token.  Slot j holds the j-th
 * best expert: repeated selection of the best not-yet-chosen expert. */
void orc_topk(int T, int E, int k, const double *logits, int32_t *idx) {
  char *taken = (char *)malloc((size_t)E);
  for (int t = 0; t < T; ++t) {
    const double *l = logits + (int64_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || beats(l[e], e, l[best], best)) best = e;
      }
      taken[best] = 1;
      idx[(int64_t)t * k + j] = best;
    }
  }
  free(taken);
}

/* Gate weights for the chosen experts.
 * SOFTMAX_ALL: w_j = softmax(l)[idx_j] over all E, not renormalised.
 * SOFTMAX_TOPK: w = softmax(l[idx_0..idx_{k-1}]). */
void orc_gate_weights(int T, int E, int k, int mode, const double *logits,
                      const int32_t *idx, double *w) {
  double *p = (double *)malloc(sizeof(double) * (size_t)(E > k ? E : k));
  double *sel = (double *)malloc(sizeof(double) * (size_t)k);
  for (int t = 0; t < T; ++t) {
    const double *l = logits + (int64_t)t * E;
    const int32_t *ix = idx + (int64_t)t * k;
    if (mode == ORC_SOFTMAX_ALL) {
      softmax_row(E, l, p);
      for (int j = 0; j < k; ++j) w[(int64_t)t * k + j] = p[ix[j]];
    } else {
      for (int j = 0; j < k; ++j) sel[j] = l[ix[j]];
      softmax_row(k, sel, p);
      for (int j = 0; j < k; ++j) w[(int64_t)t * k + j] = p[j];
    }
  }
  free(p);
  free(sel);
}

/* [P3] capacity_factor: capacity = cf times the expected average load T*k/E,
 * rounded up.  cf == 0 selects the dropless mode ([P1] Constraints); -1 is
 * returned for "no limit". */
int64_t orc_capacity(double cf, int T, int k, int E) {
  if (cf == 0.0) return -1;
  return (int64_t)ceil(cf * (double)T * (double)k / (double)E);
}

/* [P1] Token Dispatching (token_permutation) with the [P3] drop rule.
 * Assignments are visited in token order, then slot order.  A running count
 * per expert gives each assignment its rank; it is kept iff rank < cap (cap
 * < 0: always).  Kept assignments are laid out expert-major, ascending token
 * inside an expert.
 * Outputs: slot_row[T*k] (row, or -1 if dropped), row_token[N], and per expert
 * the kept count, the full load, and the exclusive offsets [E+1].
 * Returns N, the number of kept assignments. */
int64_t orc_dispatch_topk(int T, int E, int k, int64_t cap, const int32_t *idx,
                          int32_t *slot_row, int32_t *row_token,
                          int32_t *expert_count, int32_t *expert_load,
                          int32_t *expert_offset) {
  int64_t A = (int64_t)T * k;
  int32_t *rank = (int32_t *)malloc(sizeof(int32_t) * (size_t)(A > 0 ? A : 1));
  for (int e = 0; e < E; ++e) expert_load[e] = 0;
  for (int64_t a = 0; a < A; ++a) {
    int e = idx[a];
    rank[a] = expert_load[e];
    expert_load[e] += 1;
  }
  for (int e = 0; e < E; ++e) {
    int64_t c = expert_load[e];
    if (cap >= 0 && c > cap) c = cap;
    expert_count[e] = (int32_t)c;
  }
  expert_offset[0] = 0;
  for (int e = 0; e < E; ++e) expert_offset[e + 1] = expert_offset[e] + expert_count[e];
  for (int64_t a = 0; a < A; ++a) {
    int e = idx[a];
    if (cap >= 0 && rank[a] >= cap) {
      slot_row[a] = -1;
    } else {
      int32_t row = expert_offset[e] + rank[a];
      slot_row[a] = row;
      row_token[row] = (int32_t)(a / k);
    }
  }
  free(rank);
  return expert_offset[E];
}

/* [P1] Routing Mechanisms (ExpertChoiceRouter): expert e keeps the C tokens
 * with the best score in column e, by (score desc, token asc), by repeated
 * selection; the kept tokens are stored in ascending token order. */
void orc_ec_select(int T, int E, int C, const double *scores, int32_t *ec_token) {
  char *taken = (char *)malloc((size_t)(T > 0 ? T : 1));
  for (int e = 0; e < E; ++e) {
    memset(taken, 0, (size_t)T);
    for (int c = 0; c < C; ++c) {
      int best = -1;
      for (int t = 0; t < T; ++t) {
        if (taken[t]) continue;
        if (best < 0 || beats(scores[(int64_t)t * E + e], t, scores[(int64_t)best * E + e], best))
          best = t;
      }
      taken[best] = 1;
    }
    int c = 0;
    for (int t = 0; t < T; ++t)
      if (taken[t]) ec_token[(int64_t)e * C + c++] = t;
  }
  free(taken);
}

static double gelu(double z) { return 0.5 * z * (1.0 + erf(z / sqrt(2.0))); }
static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One expert FFN on one token row, fp64, no biases.
 * GELU:   h = gelu(W1 x),              W1 [dff, d]
 * SwiGLU: h = silu(Wg x) * (Wu x),     W1 [2*dff, d], gate rows first
 * y = W2 h,                            W2 [d, dff] */
void orc_ffn_row(int d, int dff, int act, int dt, const void *x, int64_t x_off,
                 const void *w1, int64_t w1_off, const void *w2, int64_t w2_off,
                 double *y) {
  double *h = (double *)malloc(sizeof(double) * (size_t)dff);
  for (int n = 0; n < dff; ++n) {
    double g = 0.0;
    for (int i = 0; i < d; ++i) g += ld(w1, w1_off + (int64_t)n * d + i, dt) * ld(x, x_off + i, dt);
    if (act == ORC_GELU) {
      h[n] = gelu(g);
    } else {
      double u = 0.0;
      for (int i = 0; i < d; ++i)
        u += ld(w1, w1_off + (int64_t)(dff + n) * d + i, dt) * ld(x, x_off + i, dt);
      h[n] = silu(g) * u;
    }
  }
  for (int o = 0; o < d; ++o) {
    double s = 0.0;
    for (int n = 0; n < dff; ++n) s += ld(w2, w2_off + (int64_t)o * dff + n, dt) * h[n];
    y[o] = s;
  }
  free(h);
}

/* [P1] MoELayer forward + token_unpermutation, for the listed tokens only:
 *   y[t] = sum over kept slots j of w[t,j] * FFN_{idx[t,j]}(x_t)
 *          + FFN_shared(x_t)            ([P3] top_k paragraph, weight 1)
 * Dropped slots (slot_row == -1) contribute nothing ([P3] capacity_factor).
 * w1 is [E, n_up*dff, d], w2 is [E, d, dff]; ws1/ws2 (shared expert, SwiGLU
 * or GELU per `act`) are used when dffs > 0. */
void orc_moe_rows_topk(int d, int E, int k, int dff, int dffs, int act, int dt,
                       const void *x, const int32_t *idx, const double *w,
                       const int32_t *slot_row, const void *w1, const void *w2,
                       const void *ws1, const void *ws2, int ntok,
                       const int32_t *toks, double *y) {
  int64_t w1_sz = (int64_t)(act == ORC_SWIGLU ? 2 : 1) * dff * d;
  int64_t w2_sz = (int64_t)d * dff;
  (void)E;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < ntok; ++i) {
    int t = toks[i];
    double *yt = y + (int64_t)i * d;
    double *tmp = (double *)malloc(sizeof(double) * (size_t)d);
    for (int o = 0; o < d; ++o) yt[o] = 0.0;
    for (int j = 0; j < k; ++j) {
      int64_t a = (int64_t)t * k + j;
      if (slot_row[a] < 0) continue;
      int e = idx[a];
      orc_ffn_row(d, dff, act, dt, x, (int64_t)t * d, w1, e * w1_sz, w2, e * w2_sz, tmp);
      for (int o = 0; o < d; ++o) yt[o] += w[a] * tmp[o];
    }
    if (dffs > 0) {
      orc_ffn_row(d, dffs, act, dt, x, (int64_t)t * d, ws1, 0, ws2, 0, tmp);
      for (int o = 0; o < d; ++o) yt[o] += tmp[o];
    }
    free(tmp);
  }
}

/* ExpertChoice form of the same: token t receives S[t,e] * FFN_e(x_t) from
 * every expert e whose kept list holds t, in ascending e; a token no expert
 * picked receives only the shared expert (or 0).  scores is [T,E]. */
void orc_moe_rows_ec(int T, int d, int E, int C, int dff, int dffs, int act, int dt,
                     const void *x, const int32_t *ec_token, const double *scores,
                     const void *w1, const void *w2, const void *ws1, const void *ws2,
                     int ntok, const int32_t *toks, double *y) {
  int64_t w1_sz = (int64_t)(act == ORC_SWIGLU ? 2 : 1) * dff * d;
  int64_t w2_sz = (int64_t)d * dff;
  (void)T;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < ntok; ++i) {
    int t = toks[i];
    double *yt = y + (int64_t)i * d;
    double *tmp = (double *)malloc(sizeof(double) * (size_t)d);
    for (int o = 0; o < d; ++o) yt[o] = 0.0;
    for (int e = 0; e < E; ++e) {
      int hit = 0;
      for (int c = 0; c < C; ++c)
        if (ec_token[(int64_t)e * C + c] == t) hit = 1;
      if (!hit) continue;
      orc_ffn_row(d, dff, act, dt, x, (int64_t)t * d, w1, e * w1_sz, w2, e * w2_sz, tmp);
      for (int o = 0; o < d; ++o) yt[o] += scores[(int64_t)t * E + e] * tmp[o];
    }
    if (dffs > 0) {
      orc_ffn_row(d, dffs, act, dt, x, (int64_t)t * d, ws1, 0, ws2, 0, tmp);
      for (int o = 0; o < d; ++o) yt[o] += tmp[o];
    }
    free(tmp);
  }
}

/* ==========================================================================
 * Backward pass (gradients of a scalar loss L given dL/dy).
 *
 * The pages train these layers ([P1] "Activation Checkpointing and
 * Constraints": moe_layer_recompute re-runs the layer's forward inside the
 * backward pass).  What is differentiated is the forward above:
 *   y[t] = sum over kept slots j of w[t,j] * FFN_{e(t,j)}(x_t) + FFN_s(x_t)
 *   w    = gate weights from logits = x W_r^T (+ bias)
 * The choice of experts (top-k, ExpertChoice selection, capacity drops) is a
 * piecewise-constant function of the logits and is held fixed; only the
 * weights, the expert FFNs and the router's linear layer carry gradient.
 * Everything is fp64; dy is read from its fp32 / bf16 bits exactly.
 * ========================================================================== */

static double phi_cdf(double z) { return 0.5 * (1.0 + erf(z / sqrt(2.0))); }
static double phi_pdf(double z) { return exp(-0.5 * z * z) / sqrt(2.0 * acos(-1.0)); }
/* d/dz of z * Phi(z) */
static double gelu_grad(double z) { return phi_cdf(z) + z * phi_pdf(z); }
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }
/* d/dz of z * sigmoid(z) */
static double silu_grad(double z) {
  double s = sigmoid(z);
  return s + z * s * (1.0 - s);
}

/* Backward of one expert FFN on one row (forward: orc_ffn_row).
 *   z = W1 x  (SwiGLU: a = Wg x, b = Wu x),  h = act(z),  out = W2 h
 * Given g = dL/d(out) [d]:
 *   dh = W2^T g;  GELU: dz = dh * gelu'(z);
 *   SwiGLU: da = dh * b * silu'(a), db = dh * silu(a)
 *   dW2 += g h^T,  dW1 += dz x^T,  dx += W1^T dz
 * Accumulators may be NULL.  `out` (NULL to skip) receives the forward
 * output, which the gate gradient needs. */
void orc_ffn_row_bwd(int d, int dff, int act, int dt, const void *x, int64_t x_off,
                     const void *w1, int64_t w1_off, const void *w2, int64_t w2_off,
                     const double *g, double *dw1, double *dw2, double *dx, double *out) {
  const int n_up = act == ORC_SWIGLU ? 2 : 1;
  double *z = (double *)malloc(sizeof(double) * (size_t)n_up * dff);
  double *h = (double *)malloc(sizeof(double) * (size_t)dff);
  double *dz = (double *)malloc(sizeof(double) * (size_t)n_up * dff);
  for (int n = 0; n < n_up * dff; ++n) {
    double s = 0.0;
    for (int i = 0; i < d; ++i) s += ld(w1, w1_off + (int64_t)n * d + i, dt) * ld(x, x_off + i, dt);
    z[n] = s;
  }
  for (int n = 0; n < dff; ++n) h[n] = act == ORC_GELU ? gelu(z[n]) : silu(z[n]) * z[dff + n];
  if (out) {
    for (int o = 0; o < d; ++o) {
      double s = 0.0;
      for (int n = 0; n < dff; ++n) s += ld(w2, w2_off + (int64_t)o * dff + n, dt) * h[n];
      out[o] = s;
    }
  }
  for (int n = 0; n < dff; ++n) {
    double dh = 0.0;
    for (int o = 0; o < d; ++o) dh += ld(w2, w2_off + (int64_t)o * dff + n, dt) * g[o];
    if (act == ORC_GELU) {
      dz[n] = dh * gelu_grad(z[n]);
    } else {
      dz[n] = dh * z[dff + n] * silu_grad(z[n]);
      dz[dff + n] = dh * silu(z[n]);
    }
  }
  if (dw2)
    for (int o = 0; o < d; ++o)
      for (int n = 0; n < dff; ++n) dw2[(int64_t)o * dff + n] += g[o] * h[n];
  if (dw1)
    for (int n = 0; n < n_up * dff; ++n)
      for (int i = 0; i < d; ++i) dw1[(int64_t)n * d + i] += dz[n] * ld(x, x_off + i, dt);
  if (dx)
    for (int n = 0; n < n_up * dff; ++n)
      for (int i = 0; i < d; ++i) dx[i] += ld(w1, w1_off + (int64_t)n * d + i, dt) * dz[n];
  free(z);
  free(h);
  free(dz);
}

/* Gradient of the top-k gate weights with respect to the logits, one token
 * at a time, the expert choice held fixed ([P1] Routing Mechanisms).
 * SOFTMAX_ALL:  w_j = p[idx_j], p = softmax(l): with g_e = sum of dw_j over
 *               the slots choosing e, dl_e = p_e * (g_e - sum_i p_i g_i).
 * SOFTMAX_TOPK: w = softmax(l[idx]): dl[idx_j] = w_j * (dw_j - sum_i w_i dw_i),
 *               every other logit gets 0. */
void orc_gate_bwd_topk(int T, int E, int k, int mode, const double *logits, const int32_t *idx,
                       const double *dw, double *dlogits) {
  double *p = (double *)malloc(sizeof(double) * (size_t)(E > k ? E : k));
  double *sel = (double *)malloc(sizeof(double) * (size_t)k);
  double *g = (double *)malloc(sizeof(double) * (size_t)E);
  for (int t = 0; t < T; ++t) {
    const double *l = logits + (int64_t)t * E;
    const int32_t *ix = idx + (int64_t)t * k;
    const double *dwt = dw + (int64_t)t * k;
    double *dl = dlogits + (int64_t)t * E;
    for (int e = 0; e < E; ++e) dl[e] = 0.0;
    if (mode == ORC_SOFTMAX_ALL) {
      softmax_row(E, l, p);
      for (int e = 0; e < E; ++e) g[e] = 0.0;
      for (int j = 0; j < k; ++j) g[ix[j]] += dwt[j];
      double s = 0.0;
      for (int e = 0; e < E; ++e) s += p[e] * g[e];
      for (int e = 0; e < E; ++e) dl[e] = p[e] * (g[e] - s);
    } else {
      for (int j = 0; j < k; ++j) sel[j] = l[ix[j]];
      softmax_row(k, sel, p);
      double s = 0.0;
      for (int j = 0; j < k; ++j) s += p[j] * dwt[j];
      for (int j = 0; j < k; ++j) dl[ix[j]] += p[j] * (dwt[j] - s);
    }
  }
  free(p);
  free(sel);
  free(g);
}

/* ExpertChoice: the weight of (t, e) is S[t,e] = softmax(l[t,:])_e for the
 * pairs the experts chose.  g[t,e] = dL/dw(t,e) for chosen pairs, else 0;
 * dl_e = S_e * (g_e - sum_i S_i g_i).  dw_ec [E,C] follows ec_token [E,C]. */
void orc_gate_bwd_ec(int T, int E, int C, const double *logits, const int32_t *ec_token,
                     const double *dw_ec, double *dlogits) {
  double *g = (double *)calloc((size_t)T * E + 1, sizeof(double));
  double *p = (double *)malloc(sizeof(double) * (size_t)E);
  for (int e = 0; e < E; ++e)
    for (int c = 0; c < C; ++c) g[(int64_t)ec_token[(int64_t)e * C + c] * E + e] += dw_ec[(int64_t)e * C + c];
  for (int t = 0; t < T; ++t) {
    softmax_row(E, logits + (int64_t)t * E, p);
    double s = 0.0;
    for (int e = 0; e < E; ++e) s += p[e] * g[(int64_t)t * E + e];
    for (int e = 0; e < E; ++e) dlogits[(int64_t)t * E + e] = p[e] * (g[(int64_t)t * E + e] - s);
  }
  free(g);
  free(p);
}

/* The whole backward pass for top-k routing, serial (small problems).
 * Inputs as in the forward (logits fp64 [T,E], idx and slot_row [T,k] from
 * the dispatch, slot_row -1 = dropped), dy [T,d] in dtype.
 * Outputs (fp64, overwritten): dx [T,d], dwr [E,d], dlogits [T,E],
 * dw1 [E,n_up*dff,d], dw2 [E,d,dff], dws1 / dws2 (shared expert, when
 * dffs > 0), d_slot_w [T,k] = dL/dw per slot (0 for dropped slots). */
void orc_moe_bwd_topk(int T, int d, int E, int k, int dff, int dffs, int act, int dt, int mode,
                      const void *x, const void *wr, const double *logits, const int32_t *idx,
                      const int32_t *slot_row, const void *w1, const void *w2, const void *ws1,
                      const void *ws2, const void *dy, double *dx, double *dwr, double *dlogits,
                      double *dw1, double *dw2, double *dws1, double *dws2, double *d_slot_w) {
  const int n_up = act == ORC_SWIGLU ? 2 : 1;
  const int64_t w1_sz = (int64_t)n_up * dff * d, w2_sz = (int64_t)d * dff;
  double *w = (double *)malloc(sizeof(double) * ((size_t)T * k + 1));
  double *g = (double *)malloc(sizeof(double) * (size_t)d);
  double *out = (double *)malloc(sizeof(double) * (size_t)d);
  memset(dx, 0, sizeof(double) * (size_t)T * d);
  memset(dwr, 0, sizeof(double) * (size_t)E * d);
  memset(dw1, 0, sizeof(double) * (size_t)E * w1_sz);
  memset(dw2, 0, sizeof(double) * (size_t)E * w2_sz);
  if (dffs > 0) {
    memset(dws1, 0, sizeof(double) * (size_t)n_up * dffs * d);
    memset(dws2, 0, sizeof(double) * (size_t)d * dffs);
  }
  orc_gate_weights(T, E, k, mode, logits, idx, w);
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < k; ++j) {
      const int64_t a = (int64_t)t * k + j;
      d_slot_w[a] = 0.0;
      if (slot_row[a] < 0) continue; /* dropped: no term, no gradient */
      const int e = idx[a];
      for (int o = 0; o < d; ++o) g[o] = w[a] * ld(dy, (int64_t)t * d + o, dt);
      orc_ffn_row_bwd(d, dff, act, dt, x, (int64_t)t * d, w1, e * w1_sz, w2, e * w2_sz, g,
                      dw1 + e * w1_sz, dw2 + e * w2_sz, dx + (int64_t)t * d, out);
      double s = 0.0;
      for (int o = 0; o < d; ++o) s += ld(dy, (int64_t)t * d + o, dt) * out[o];
      d_slot_w[a] = s;
    }
    if (dffs > 0) {
      for (int o = 0; o < d; ++o) g[o] = ld(dy, (int64_t)t * d + o, dt);
      orc_ffn_row_bwd(d, dffs, act, dt, x, (int64_t)t * d, ws1, 0, ws2, 0, g, dws1, dws2,
                      dx + (int64_t)t * d, NULL);
    }
  }
  orc_gate_bwd_topk(T, E, k, mode, logits, idx, d_slot_w, dlogits);
  /* router: logits = x W_r^T, so dx += dlogits W_r and dW_r = dlogits^T x */
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      const double gl = dlogits[(int64_t)t * E + e];
      for (int i = 0; i < d; ++i) {
        dx[(int64_t)t * d + i] += gl * ld(wr, (int64_t)e * d + i, dt);
        dwr[(int64_t)e * d + i] += gl * ld(x, (int64_t)t * d + i, dt);
      }
    }
  free(w);
  free(g);
  free(out);
}

/* The same for ExpertChoice: expert e's rows are the tokens ec_token[e,:],
 * weighted by S[t,e] = softmax(logits[t,:])_e; d_slot_w [E,C] follows
 * ec_token. */
void orc_moe_bwd_ec(int T, int d, int E, int C, int dff, int dffs, int act, int dt,
                    const void *x, const void *wr, const double *logits, const int32_t *ec_token,
                    const void *w1, const void *w2, const void *ws1, const void *ws2, const void *dy,
                    double *dx, double *dwr, double *dlogits, double *dw1, double *dw2, double *dws1,
                    double *dws2, double *d_slot_w) {
  const int n_up = act == ORC_SWIGLU ? 2 : 1;
  const int64_t w1_sz = (int64_t)n_up * dff * d, w2_sz = (int64_t)d * dff;
  double *S = (double *)malloc(sizeof(double) * ((size_t)T * E + 1));
  double *g = (double *)malloc(sizeof(double) * (size_t)d);
  double *out = (double *)malloc(sizeof(double) * (size_t)d);
  memset(dx, 0, sizeof(double) * (size_t)T * d);
  memset(dwr, 0, sizeof(double) * (size_t)E * d);
  memset(dw1, 0, sizeof(double) * (size_t)E * w1_sz);
  memset(dw2, 0, sizeof(double) * (size_t)E * w2_sz);
  if (dffs > 0) {
    memset(dws1, 0, sizeof(double) * (size_t)n_up * dffs * d);
    memset(dws2, 0, sizeof(double) * (size_t)d * dffs);
  }
  orc_softmax(T, E, logits, S);
  for (int e = 0; e < E; ++e)
    for (int c = 0; c < C; ++c) {
      const int64_t a = (int64_t)e * C + c;
      const int t = ec_token[a];
      const double we = S[(int64_t)t * E + e];
      for (int o = 0; o < d; ++o) g[o] = we * ld(dy, (int64_t)t * d + o, dt);
      orc_ffn_row_bwd(d, dff, act, dt, x, (int64_t)t * d, w1, e * w1_sz, w2, e * w2_sz, g,
                      dw1 + e * w1_sz, dw2 + e * w2_sz, dx + (int64_t)t * d, out);
      double s = 0.0;
      for (int o = 0; o < d; ++o) s += ld(dy, (int64_t)t * d + o, dt) * out[o];
      d_slot_w[a] = s;
    }
  if (dffs > 0)
    for (int t = 0; t < T; ++t) {
      for (int o = 0; o < d; ++o) g[o] = ld(dy, (int64_t)t * d + o, dt);
      orc_ffn_row_bwd(d, dffs, act, dt, x, (int64_t)t * d, ws1, 0, ws2, 0, g, dws1, dws2,
                      dx + (int64_t)t * d, NULL);
    }
  orc_gate_bwd_ec(T, E, C, logits, ec_token, d_slot_w, dlogits);
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      const double gl = dlogits[(int64_t)t * E + e];
      for (int i = 0; i < d; ++i) {
        dx[(int64_t)t * d + i] += gl * ld(wr, (int64_t)e * d + i, dt);
        dwr[(int64_t)e * d + i] += gl * ld(x, (int64_t)t * d + i, dt);
      }
    }
  free(S);
  free(g);
  free(out);
}

/* Sampled checks of large problems, token by token: dx[t] (experts, shared
 * expert and router), dlogits[t] and dL/dw of each of t's slots, for the
 * listed tokens only (top-k).  Outputs are [ntok, d], [ntok, E], [ntok, k]. */
void orc_moe_bwd_tokens_topk(int d, int E, int k, int dff, int dffs, int act, int dt, int mode,
                             const void *x, const void *wr, const double *logits, const int32_t *idx,
                             const int32_t *slot_row, const void *w1, const void *w2, const void *ws1,
                             const void *ws2, const void *dy, int ntok, const int32_t *toks,
                             double *dx, double *dlogits, double *d_slot_w) {
  const int n_up = act == ORC_SWIGLU ? 2 : 1;
  const int64_t w1_sz = (int64_t)n_up * dff * d, w2_sz = (int64_t)d * dff;
#pragma omp parallel for schedule(dynamic, 1)
  for (int q = 0; q < ntok; ++q) {
    const int t = toks[q];
    double *g = (double *)malloc(sizeof(double) * (size_t)d);
    double *out = (double *)malloc(sizeof(double) * (size_t)d);
    double *w = (double *)malloc(sizeof(double) * (size_t)k);
    double *dxt = dx + (int64_t)q * d;
    double *dwt = d_slot_w + (int64_t)q * k;
    double *dl = dlogits + (int64_t)q * E;
    for (int i = 0; i < d; ++i) dxt[i] = 0.0;
    orc_gate_weights(1, E, k, mode, logits + (int64_t)t * E, idx + (int64_t)t * k, w);
    for (int j = 0; j < k; ++j) {
      const int64_t a = (int64_t)t * k + j;
      dwt[j] = 0.0;
      if (slot_row[a] < 0) continue;
      const int e = idx[a];
      for (int o = 0; o < d; ++o) g[o] = w[j] * ld(dy, (int64_t)t * d + o, dt);
      orc_ffn_row_bwd(d, dff, act, dt, x, (int64_t)t * d, w1, e * w1_sz, w2, e * w2_sz, g, NULL, NULL,
                      dxt, out);
      double s = 0.0;
      for (int o = 0; o < d; ++o) s += ld(dy, (int64_t)t * d + o, dt) * out[o];
      dwt[j] = s;
    }
    if (dffs > 0) {
      for (int o = 0; o < d; ++o) g[o] = ld(dy, (int64_t)t * d + o, dt);
      orc_ffn_row_bwd(d, dffs, act, dt, x, (int64_t)t * d, ws1, 0, ws2, 0, g, NULL, NULL, dxt, NULL);
    }
    orc_gate_bwd_topk(1, E, k, mode, logits + (int64_t)t * E, idx + (int64_t)t * k, dwt, dl);
    for (int e = 0; e < E; ++e)
      for (int i = 0; i < d; ++i) dxt[i] += dl[e] * ld(wr, (int64_t)e * d + i, dt);
    free(g);
    free(out);
    free(w);
  }
}

/* Sampled elements of one expert's weight gradients.  The expert's rows are
 * the tokens row_tok[0..nrows) with gate weights row_w (1 for the shared
 * expert); g_row = row_w * dy[t].
 *   which 1: dW1[r][c] = sum over rows of dz_row[r] * x_row[c]
 *   which 2: dW2[r][c] = sum over rows of g_row[r] * h_row[c]
 * w1e / w2e point at the expert's own matrices. */
void orc_ffn_dw_elems(int d, int dff, int act, int dt, const void *x, const void *dy, const void *w1e,
                      const void *w2e, int nrows, const int32_t *row_tok, const double *row_w, int which,
                      int nelem, const int32_t *rr, const int32_t *cc, double *out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int q = 0; q < nelem; ++q) {
    const int r = rr[q], c = cc[q];
    /* the hidden unit whose pre-activations this element needs */
    const int n = which == 1 ? (r % dff) : c;
    double acc = 0.0;
    for (int m = 0; m < nrows; ++m) {
      const int t = row_tok[m];
      const int64_t xo = (int64_t)t * d;
      double a = 0.0, b = 0.0;
      for (int i = 0; i < d; ++i) a += ld(w1e, (int64_t)n * d + i, dt) * ld(x, xo + i, dt);
      if (act == ORC_SWIGLU)
        for (int i = 0; i < d; ++i) b += ld(w1e, (int64_t)(dff + n) * d + i, dt) * ld(x, xo + i, dt);
      if (which == 2) {
        const double h = act == ORC_GELU ? gelu(a) : silu(a) * b;
        acc += row_w[m] * ld(dy, xo + r, dt) * h;
      } else {
        double dh = 0.0;
        for (int o = 0; o < d; ++o) dh += ld(w2e, (int64_t)o * dff + n, dt) * row_w[m] * ld(dy, xo + o, dt);
        double dz;
        if (act == ORC_GELU) dz = dh * gelu_grad(a);
        else if (r < dff) dz = dh * b * silu_grad(a);
        else dz = dh * silu(a);
        acc += dz * ld(x, xo + c, dt);
      }
    }
    out[q] = acc;
  }
}

/* ExpertChoice form of orc_moe_bwd_tokens_topk: token t's experts are those
 * whose kept list holds t (weight S[t,e]); d_slot_w is [ntok, E] (0 where
 * expert e did not choose t). */
void orc_moe_bwd_tokens_ec(int d, int E, int C, int dff, int dffs, int act, int dt, const void *x,
                           const void *wr, const double *logits, const int32_t *ec_token, const void *w1,
                           const void *w2, const void *ws1, const void *ws2, const void *dy, int ntok,
                           const int32_t *toks, double *dx, double *dlogits, double *d_slot_w) {
  const int n_up = act == ORC_SWIGLU ? 2 : 1;
  const int64_t w1_sz = (int64_t)n_up * dff * d, w2_sz = (int64_t)d * dff;
#pragma omp parallel for schedule(dynamic, 1)
  for (int q = 0; q < ntok; ++q) {
    const int t = toks[q];
    double *g = (double *)malloc(sizeof(double) * (size_t)d);
    double *out = (double *)malloc(sizeof(double) * (size_t)d);
    double *S = (double *)malloc(sizeof(double) * (size_t)E);
    double *dxt = dx + (int64_t)q * d;
    double *gw = d_slot_w + (int64_t)q * E;
    double *dl = dlogits + (int64_t)q * E;
    for (int i = 0; i < d; ++i) dxt[i] = 0.0;
    softmax_row(E, logits + (int64_t)t * E, S);
    for (int e = 0; e < E; ++e) {
      gw[e] = 0.0;
      int hit = 0;
      for (int c = 0; c < C; ++c)
        if (ec_token[(int64_t)e * C + c] == t) hit = 1;
      if (!hit) continue;
      for (int o = 0; o < d; ++o) g[o] = S[e] * ld(dy, (int64_t)t * d + o, dt);
      orc_ffn_row_bwd(d, dff, act, dt, x, (int64_t)t * d, w1, e * w1_sz, w2, e * w2_sz, g, NULL, NULL,
                      dxt, out);
      double s = 0.0;
      for (int o = 0; o < d; ++o) s += ld(dy, (int64_t)t * d + o, dt) * out[o];
      gw[e] = s;
    }
    if (dffs > 0) {
      for (int o = 0; o < d; ++o) g[o] = ld(dy, (int64_t)t * d + o, dt);
      orc_ffn_row_bwd(d, dffs, act, dt, x, (int64_t)t * d, ws1, 0, ws2, 0, g, NULL, NULL, dxt, NULL);
    }
    double s = 0.0;
    for (int e = 0; e < E; ++e) s += S[e] * gw[e];
    for (int e = 0; e < E; ++e) dl[e] = S[e] * (gw[e] - s);
    for (int e = 0; e < E; ++e)
      for (int i = 0; i < d; ++i) dxt[i] += dl[e] * ld(wr, (int64_t)e * d + i, dt);
    free(g);
    free(out);
    free(S);
  }
}
