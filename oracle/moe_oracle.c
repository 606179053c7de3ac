/*
 * moe_oracle.c -- a plain, slow, fp64 CPU oracle for the forward pass of one
 * Mixture-of-Experts block on one GPU's share of tokens.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and
 * the CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or helper with the HIP library, and neither includes or
 * links the other.
 *
 * What it follows (page title, then section):
 *   [P1] "How MegaDLMs Implements Mixture of Experts (MoE) Architectures"
 *        - "Routing Mechanisms: Top-K vs Expert Choice": the TopKRouter turns
 *          tokens into dense gate logits with a learned linear layer, applies a
 *          softmax and keeps the k best experts per token, handing the
 *          dispatcher probability weights plus a routing map; the
 *          ExpertChoiceRouter lets every expert pick its tokens by score.
 *        - "Core MoE Layer Architecture" (MoELayer): permute tokens to their
 *          experts, run the local experts, unpermute back to sequence order.
 *        - "Activation Checkpointing and Constraints": the dropless mode, in
 *          which every token reaches every expert it selected.
 *   [P3] "Expert Parallelism > Key Parameters"
 *        - capacity_factor paragraph: each expert holds capacity_factor times
 *          the expected average load; tokens above it are dropped and their
 *          contribution is zeroed.
 *        - top_k paragraph: an always-used shared expert next to the routed
 *          top-k experts.
 *
 * Readings taken where the pages are silent (each is listed in the design doc):
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

/* [P1] Routing Mechanisms: dense gate logits through a learned linear layer.
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
