/*
 * moe.h -- C ABI of the MI355X (gfx950) forward and backward passes of one
 * Mixture-of-Experts block on one GPU's share of tokens and its local experts.
 *
 * The operations follow two pages:
 *   [P1] "How MegaDLMs Implements Mixture of Experts (MoE) Architectures"
 *   [P3] "Expert Parallelism > Key Parameters"
 * and are cited by page and section at each entry point.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensors are dense row-major device buffers.  Weights use the
 *   [out_features, in_features] layout, so every contraction reads both
 *   operands along their contiguous inner dimension.
 * - Floating-point tensors hold `cfg->dtype` elements (fp32 or bf16) unless
 *   the argument says fp32.  Indices are int32.
 * - The caller owns every buffer.  The library never allocates, frees or
 *   synchronises; every call only enqueues work on `stream` (a hipStream_t
 *   passed as void*, NULL = the null stream) and returns.
 * - Arguments are checked on the host before anything is enqueued.  A failed
 *   check returns MOE_ERR_INVALID_ARG (or MOE_ERR_UNSUPPORTED for a valid but
 *   unimplemented combination) and enqueues nothing.  A failed launch returns
 *   MOE_ERR_HIP.  No exception crosses the ABI.
 * - The host never learns how many assignments survive the capacity limit:
 *   buffers indexed by permuted row are sized for moe_max_rows() rows, and
 *   expert_offset[E] (device) holds the number actually used.
 * - Same inputs give bitwise-identical outputs (no floating-point atomics).
 * - Pointers to floating-point tensors must be 16-byte aligned; d_model and
 *   d_ff (and d_ff_shared) must be multiples of 8.  Widths of 2^22 or more,
 *   moe_max_rows() of 2^25 - 256 or more, or any GEMM operand past 2^31
 *   elements return MOE_ERR_UNSUPPORTED (32-bit offsets).
 * - T = 0 is valid: every call returns MOE_OK and buffers whose size is zero
 *   may be NULL; moe_permute still writes the (zero) counts and offsets.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* a host-side check failed; nothing was enqueued */
  MOE_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. E > 256)        */
  MOE_ERR_WORKSPACE = 3,   /* workspace/scratch smaller than required          */
  MOE_ERR_HIP = 4,         /* a HIP launch failed                              */
  MOE_ERR_NOALLOC_LIMIT = 5 /* the allocation-free entry point's static scratch
                               is smaller than this configuration needs       */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
typedef enum { MOE_ACT_GELU = 0, MOE_ACT_SWIGLU = 1 } moe_act;

/* [P1] "Routing Mechanisms: Top-K vs Expert Choice": the TopKRouter (softmax
 * and top-k per token) and the ExpertChoiceRouter (each expert picks tokens).
 * SOFTMAX_ALL: gate weight = softmax over all E logits at the chosen expert
 *              (not renormalised over the k chosen).
 * SOFTMAX_TOPK: gate weights = softmax over the k chosen logits.            */
typedef enum {
  MOE_TOPK_SOFTMAX_ALL = 0,
  MOE_TOPK_SOFTMAX_TOPK = 1,
  MOE_EXPERT_CHOICE = 2
} moe_routing;

/* The problem statement: [P1] "Configuration-Driven MoE Activation"
 * (num_moe_experts, moe_shared_expert_intermediate_size) and [P3] (num_experts,
 * top_k, capacity_factor). */
typedef struct {
  int32_t num_tokens;      /* T >= 0: tokens on this GPU                         */
  int32_t d_model;         /* d: token width, multiple of 8                      */
  int32_t num_experts;     /* E: local experts, 1..256                           */
  int32_t top_k;           /* k: experts per token, 1..min(E,16) (top-k modes)   */
  int32_t d_ff;            /* expert hidden width, multiple of 8                 */
  int32_t d_ff_shared;     /* shared expert hidden width, 0 = no shared expert   */
  double capacity_factor;  /* [P3] capacity_factor; 0 = dropless ([P1]
                              "Activation Checkpointing and Constraints").
                              A double, so that the capacity below is the
                              same ceil(cf*T*k/E) a caller computes from
                              the factor it wrote (a float32 factor such as
                              1.2 is stored slightly high and can round the
                              capacity up by one)                             */
  int32_t ec_capacity;     /* ExpertChoice: tokens per expert, 1..T             */
  int32_t dtype;           /* moe_dtype of x, weights and activations            */
  int32_t act;             /* moe_act of the routed and the shared experts       */
  int32_t routing;         /* moe_routing                                        */
} moe_config;

/* Number of permuted rows buffers must hold: T*k dropless, min(T*k, E*C) with
 * capacity C = ceil(capacity_factor*T*k/E), E*ec_capacity for ExpertChoice. */
int64_t moe_max_rows(const moe_config *cfg);

/* Capacity C = ceil(cf*T*k/E) of [P3] "Key Parameters" (capacity_factor: cf
 * times the expected average load), or -1 when dropless or ExpertChoice.
 * Evaluated in IEEE double as ((cf*T)*k)/E. */
int64_t moe_capacity(const moe_config *cfg);

/* --------------------------------------------------------------------------
 * moe_route -- [P1] "Routing Mechanisms: Top-K vs Expert Choice".
 *
 * logits[t,e] = sum_i x[t,i] * w_router[e,i] (+ bias), fp32 accumulation.
 *   x         [T,d] dtype, or NULL: then `logits` is an INPUT and only the gate
 *             below runs on it (bias is then ignored).
 *   w_router  [E,d] dtype (ignored when x is NULL).
 *   logit_bias fp32, NULL = none; bias_row_stride 0: bias[e] for every token,
 *             E: bias[t*E+e].
 *   logits    [T,E] fp32 output (or input, see x).
 * Top-k modes: topk_idx [T,k] int32 gets the k best experts by logit, slot j
 *   the j-th best, equal logits going to the lower expert index (IEEE
 *   equality, -0 == +0); topk_w [T,k] fp32 gets the gate weights (see
 *   moe_routing).  scores/ec_token/ec_w are ignored and may be NULL.
 * ExpertChoice: scores [E,T] fp32, expert-major (row e holds expert e's
 *   score of every token) = softmax over E per token; expert e keeps the
 *   ec_capacity tokens with the largest score in its row (equal scores to
 *   the lower token), stored in ascending token order in ec_token [E,C];
 *   ec_w [E,C] fp32 = their scores.  Requires T <= 16384.  topk_* ignored.
 * ------------------------------------------------------------------------ */
moe_status moe_route(const moe_config *cfg, const void *x, const void *w_router,
                     const float *logit_bias, int64_t bias_row_stride, float *logits,
                     int32_t *topk_idx, float *topk_w, float *scores, int32_t *ec_token,
                     float *ec_w, void *stream);

/* Bytes of device scratch moe_permute needs (per-block counts and ranks). */
moe_status moe_permute_scratch_bytes(const moe_config *cfg, size_t *bytes);

/* --------------------------------------------------------------------------
 * moe_permute -- [P1] "Token Dispatching and Communication"
 * (token_permutation, the single-GPU part) with the [P3] capacity_factor drop
 * rule (overflow assignments are dropped and contribute zero).
 *
 * Top-k modes (reads topk_idx [T,k]):
 *   Assignments (t,j) compete for capacity in token order, then slot order.
 *   rank(t,j) = number of earlier assignments to the same expert; kept iff
 *   rank < C (always when dropless).  Kept rows are expert-major, ascending
 *   token inside an expert:
 *     expert_load[E]    assignments per expert before dropping
 *     expert_count[E]   kept rows per expert = min(load, C)
 *     expert_offset[E+1] exclusive scan of expert_count; [E] = rows used
 *     slot_row [T,k]    row of (t,j), or -1 when dropped (the drop mask)
 *     row_token[rows]   token of each row
 *     x_perm [rows,d]   x[row_token[r]] for r < expert_offset[E]
 *   ec_token, ec_w, slot_w, tok_ptr are ignored (may be NULL).
 * ExpertChoice (reads ec_token [E,C], ec_w [E,C]):
 *   row e*C+i holds token ec_token[e,i]; expert_count = expert_load = C;
 *   tok_ptr [T+1] and slot_row/slot_w [E*C] form a per-token list (CSR) of the
 *   rows holding that token and their weights, in ascending expert order.
 * scratch: moe_permute_scratch_bytes() bytes of device memory, 16-B aligned.
 * ------------------------------------------------------------------------ */
moe_status moe_permute(const moe_config *cfg, const void *x, const int32_t *topk_idx,
                       const int32_t *ec_token, const float *ec_w, void *x_perm,
                       int32_t *row_token, int32_t *slot_row, float *slot_w, int32_t *tok_ptr,
                       int32_t *expert_count, int32_t *expert_load, int32_t *expert_offset,
                       void *scratch, size_t scratch_bytes, void *stream);

/* --------------------------------------------------------------------------
 * moe_permute_noalloc -- moe_permute for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments and results without the scratch
 * pair.  Its per-block counts and ranks live in a static device array of
 * MOE_PERMUTE_NOALLOC_MAX_BYTES that each GPU the library runs on holds until
 * the process ends; the call itself allocates nothing.  A configuration whose
 * moe_permute_scratch_bytes() exceeds that maximum returns
 * MOE_ERR_NOALLOC_LIMIT and enqueues nothing (about 1.7 M assignments T*k
 * with 256 experts; ExpertChoice and T*k <= 8192 use no scratch at all).
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind: calls enqueued on one stream are ordered, but two calls that
 * overlap on one GPU (different streams or host threads without ordering)
 * race and give undefined results.
 * ------------------------------------------------------------------------ */
#define MOE_PERMUTE_NOALLOC_MAX_BYTES (8u << 20)
moe_status moe_permute_noalloc(const moe_config *cfg, const void *x, const int32_t *topk_idx,
                               const int32_t *ec_token, const float *ec_w, void *x_perm,
                               int32_t *row_token, int32_t *slot_row, float *slot_w, int32_t *tok_ptr,
                               int32_t *expert_count, int32_t *expert_load, int32_t *expert_offset,
                               void *stream);

/* Bytes of device workspace moe_expert_ffn needs for this configuration:
 * room for the fp32 partial tiles of GEMM tiles cut along K.
 *   bf16, >= 192 rows per expert on average, and a reduction length (d_model
 *   for the up projection, d_ff for the down projection) >= 8192: the tiles
 *   of the last, partial round of workgroups are cut; 256 tiles of 256 KiB.
 *   bf16, <= 128 rows per expert on average, K a multiple of 64: the
 *   weight-streaming kernel cuts its tiles when there are too few to fill
 *   the GPU; 512 tiles of 64 x 256 fp32: 32 MiB.
 * The larger of the two applies; 0 for every other configuration.  When the
 * configuration also admits packed weights (moe_pack_weights), the figure
 * covers moe_expert_ffn_packed as well, whose kernel choice can differ. */
moe_status moe_expert_ffn_workspace_bytes(const moe_config *cfg, size_t *bytes);

/* --------------------------------------------------------------------------
 * moe_expert_ffn -- [P1] "Core MoE Layer Architecture" (MoELayer step 2: the
 * local experts process their dispatched tokens).  For every expert e, rows
 * [expert_offset[e], expert_offset[e+1]) of x_perm go through
 *   GELU:   h = gelu(x W1_e^T)                   (exact erf form)
 *   SwiGLU: h = silu(x Wg_e^T) * (x Wu_e^T)      (W1_e rows: gate, then up)
 *   y = h W2_e^T
 * with fp32 accumulation; h and y are rounded to dtype once.
 *   x_perm [rows,d], w1 [E, n_up*d_ff, d] (n_up = 2 for SwiGLU), w2 [E, d, d_ff],
 *   expert_offset [E+1] int32 (device), h [rows,d_ff] (workspace the caller
 *   owns), y_perm [rows,d].  rows = moe_max_rows(cfg).
 *   workspace: moe_expert_ffn_workspace_bytes() bytes of device memory,
 *   256-B aligned (NULL when that is 0); MOE_ERR_WORKSPACE when too small.
 *   Its contents need no initialisation and are scratch afterwards; two
 *   calls in flight at once need two workspaces.
 * Results are deterministic: a K-split tile adds its pieces in K order.
 * The shared expert ([P3] "Key Parameters", top_k paragraph: a shared expert
 * every token uses) is this call with num_experts = 1, top_k = 1, dropless,
 * d_ff = d_ff_shared, expert_offset = {0, T} and x_perm = x.
 * ------------------------------------------------------------------------ */
moe_status moe_expert_ffn(const moe_config *cfg, const void *x_perm, const int32_t *expert_offset,
                          const void *w1, const void *w2, void *h, void *y_perm, void *workspace,
                          size_t workspace_bytes, void *stream);

/* --------------------------------------------------------------------------
 * Packed expert weights for inference: the same computation as
 * moe_expert_ffn / moe_layer_fwd ([P1] "Core MoE Layer Architecture",
 * MoELayer step 2), with each weight matrix rearranged once, when it is
 * loaded, into the order in which the expert GEMMs stream it, so that every
 * K stage of a weight tile is one contiguous block of memory.
 *
 * Packed order of one weight (per expert e, column tile j, K slice s):
 *   column tiles of 256 weight rows; SwiGLU's W1 tile j holds gate rows
 *   [128 j, 128 j + 128) then the matching up rows; K slices of 32; each
 *   (e, j, s) is a block of 256 x 32 bf16 (16 KB) at byte
 *   ((e * tiles + j) * (K / 32) + s) * 16384, whose 16-B chunk q holds row
 *   q / 4 of the tile at K elements 32 s + 8 ((q % 4) ^ ((q / 16) % 4)) .. +8.
 *   Tile rows past the weight's output width are zero.
 * The packed path also keeps the expert activations K-blocked: a [rows, K]
 * bf16 matrix is stored as [K/32][rows][32] (row r, column k at element
 * ((k / 32) * rows + r) * 32 + k % 32), so a K stage of any run of
 * consecutive rows is one contiguous block too.  moe_permute_packed writes
 * x_perm in that order (rows = moe_max_rows()), and the packed FFN keeps h in
 * it ([d_ff/32][rows][32]); y_perm stays row-major for moe_unpermute.
 * Requirements: dtype bf16, d_model and the FFN width (d_ff, or d_ff_shared
 * for the shared expert's weights) multiples of 64; otherwise
 * MOE_ERR_UNSUPPORTED.  Results are bitwise identical to the unpacked entry
 * points on the same weights (h and x_perm up to their order).  Training
 * (moe_layer_fwd_train, moe_layer_bwd) takes the unpacked weights.
 * ------------------------------------------------------------------------ */
typedef enum {
  MOE_PACK_W1 = 0,        /* w1 [E, n_up*d_ff, d]             */
  MOE_PACK_W2 = 1,        /* w2 [E, d, d_ff]                  */
  MOE_PACK_SHARED_W1 = 2, /* ws1 [n_up*d_ff_shared, d]        */
  MOE_PACK_SHARED_W2 = 3  /* ws2 [d, d_ff_shared]             */
} moe_pack_which;
/* Bytes of the packed form of weight `which` (a moe_pack_which):
 * E * tiles * (K / 32) * 16384 with K its input width and tiles =
 * ceil(d_ff / 128) for SwiGLU's W1, ceil(output width / 256) otherwise.
 * MOE_ERR_INVALID_ARG for an unknown `which` or a shared weight when
 * d_ff_shared == 0. */
moe_status moe_packed_weight_bytes(const moe_config *cfg, int32_t which, size_t *bytes);
/* Enqueues the rearrangement of weight `which` from `w` (unpacked layout, as
 * moe_expert_ffn / moe_layer_fwd take it) into `packed`
 * (moe_packed_weight_bytes() bytes, caller-owned, 16-byte aligned, not
 * overlapping w; every byte is written).  w is only read. */
moe_status moe_pack_weights(const moe_config *cfg, int32_t which, const void *w, void *packed, void *stream);
/* moe_permute with x_perm written K-blocked ([d/32][moe_max_rows()][32]);
 * every other output, the arguments and the scratch as moe_permute. */
moe_status moe_permute_packed(const moe_config *cfg, const void *x, const int32_t *topk_idx,
                              const int32_t *ec_token, const float *ec_w, void *x_perm, int32_t *row_token,
                              int32_t *slot_row, float *slot_w, int32_t *tok_ptr, int32_t *expert_count,
                              int32_t *expert_load, int32_t *expert_offset, void *scratch, size_t scratch_bytes,
                              void *stream);
/* moe_expert_ffn on packed weights: w1_packed / w2_packed from
 * moe_pack_weights(MOE_PACK_W1 / MOE_PACK_W2); x_perm_kblocked = 1 when
 * x_perm is K-blocked (moe_permute_packed), 0 when it is row-major
 * [rows, d] (moe_permute, or x itself for the shared expert; other values:
 * MOE_ERR_INVALID_ARG).  h (same size as for moe_expert_ffn) is written
 * K-blocked.  y_perm, the workspace size and the results as moe_expert_ffn. */
moe_status moe_expert_ffn_packed(const moe_config *cfg, const void *x_perm, int32_t x_perm_kblocked,
                                 const int32_t *expert_offset, const void *w1_packed, const void *w2_packed,
                                 void *h, void *y_perm, void *workspace, size_t workspace_bytes, void *stream);

/* --------------------------------------------------------------------------
 * moe_unpermute -- [P1] "Token Dispatching and Communication"
 * (token_unpermutation) and "Core MoE Layer Architecture" step 3.
 *   y[t] = sum over t's slots s with slot_row[s] >= 0, in slot order, of
 *          slot_w[s] * y_perm[slot_row[s]]   (+ y_shared[t] if given)
 * fp32 accumulation, one rounding to dtype.  Dropped slots contribute zero
 * ([P3] capacity_factor paragraph); a token with no kept slot gets 0.
 *   tok_ptr NULL: token t's slots are [t*k, t*k+k) (top-k: slot_row [T,k],
 *                 slot_w = topk_w [T,k]);
 *   tok_ptr [T+1]: slots [tok_ptr[t], tok_ptr[t+1]) (ExpertChoice CSR).
 *   y_shared [T,d] or NULL; y [T,d].
 * ------------------------------------------------------------------------ */
moe_status moe_unpermute(const moe_config *cfg, const void *y_perm, const int32_t *tok_ptr,
                         const int32_t *slot_row, const float *slot_w, const void *y_shared,
                         void *y, void *stream);

/* Byte offsets of every intermediate inside moe_layer_fwd's workspace, so a
 * caller can inspect routing, permutation and expert outputs afterwards.
 * Unused entries (e.g. scores under top-k) have size 0 and repeat an offset. */
typedef struct {
  size_t logits, topk_idx, topk_w, scores, ec_token, ec_w;
  size_t x_perm, row_token, slot_row, slot_w, tok_ptr;
  size_t expert_count, expert_load, expert_offset, shared_offset;
  size_t h, y_perm, shared_h, shared_y, scratch, scratch_bytes;
  size_t ffn_scratch, ffn_scratch_bytes;               /* moe_expert_ffn workspace */
  size_t shared_ffn_scratch, shared_ffn_scratch_bytes; /* ... of the shared expert */
  size_t z, shared_z; /* pre-activations [rows, n_up*d_ff], [T, n_up*d_ff_shared]
                         kept by moe_layer_fwd_train */
  size_t stamp;       /* int32 written by the forward's last step: which of
                         moe_layer_fwd / moe_layer_fwd_train filled z */
  size_t total; /* bytes the workspace must hold */
} moe_workspace_layout;

moe_status moe_layer_workspace(const moe_config *cfg, moe_workspace_layout *layout);

/* --------------------------------------------------------------------------
 * moe_layer_fwd -- the whole MoE block forward ([P1] "Core MoE Layer
 * Architecture": MoELayer / MoELayerExpertChoice): route, permute, routed
 * experts, shared expert (when d_ff_shared > 0, weight 1), unpermute; no
 * host synchronisation.  The shared expert reads only x, so it runs on a
 * side stream beside the rest (forked from `stream` at the start, joined
 * back before the combine; P1's shared-expert overlap): the call is
 * asynchronous on `stream` as a whole.  The side stream and its two events
 * are created once per device and host thread and kept.
 *   x [T,d], w_router [E,d], logit_bias as in moe_route, w1/w2 as in
 *   moe_expert_ffn, ws1 [n_up*d_ff_shared, d] / ws2 [d, d_ff_shared] (NULL
 *   when d_ff_shared == 0), y [T,d] output.
 *   workspace: moe_layer_workspace().total bytes, 256-B aligned.
 * ------------------------------------------------------------------------ */
moe_status moe_layer_fwd(const moe_config *cfg, const void *x, const void *w_router,
                         const float *logit_bias, int64_t bias_row_stride, const void *w1,
                         const void *w2, const void *ws1, const void *ws2, void *y,
                         void *workspace, size_t workspace_bytes, void *stream);
/* moe_layer_fwd on packed expert weights (moe_pack_weights: MOE_PACK_W1,
 * MOE_PACK_W2, and for a shared expert MOE_PACK_SHARED_W1 / _W2); the router
 * weights stay unpacked.  Its steps are moe_route, moe_permute_packed and
 * moe_expert_ffn_packed (the workspace's x_perm and h regions then hold
 * K-blocked matrices), the shared expert's moe_expert_ffn_packed on x and
 * moe_unpermute.  Workspace (moe_layer_workspace) and y as moe_layer_fwd. */
moe_status moe_layer_fwd_packed(const moe_config *cfg, const void *x, const void *w_router,
                                const float *logit_bias, int64_t bias_row_stride, const void *w1_packed,
                                const void *w2_packed, const void *ws1_packed, const void *ws2_packed, void *y,
                                void *workspace, size_t workspace_bytes, void *stream);

/* --------------------------------------------------------------------------
 * Backward pass ([P1] "Activation Checkpointing and Constraints": the layer
 * is trained, and its recompute mode re-runs the forward inside the backward
 * pass).  moe_layer_bwd differentiates moe_layer_fwd for an upstream
 * gradient dy = dL/dy, re-running the expert GEMM1 (the pre-activations are
 * recomputed, not kept).  The choice of experts (top-k, ExpertChoice
 * selection, capacity drops) is held fixed: it is piecewise constant in the
 * logits.  Gradients flow through
 *   - the gate weights ([P1] "Routing Mechanisms": softmax over the logits):
 *     SOFTMAX_ALL  dl_e = p_e (g_e - sum_i p_i g_i), g_e = dL/dw of the slot
 *                  that chose e (p = softmax of the logits);
 *     SOFTMAX_TOPK dl[idx_j] = w_j (dL/dw_j - sum_i w_i dL/dw_i), others 0;
 *     ExpertChoice dl_e = S_e (g_e - sum_i S_i g_i), S = the scores;
 *     with dL/dw of a kept slot = <dy[t], y_perm[row]> and 0 when dropped;
 *   - the expert FFNs (GELU / SwiGLU as in moe_expert_ffn), the shared
 *     expert (weight 1) and the router's linear layer logits = x W_r^T.
 *
 * Layout of the backward workspace.  Routed rows keep the forward's
 * expert-major order, but expert e's block starts at poff[e], a multiple of
 * 32 (pad rows are zero), so every weight-gradient contraction covers whole
 * 32-row stages.  Offsets are bytes from the workspace start; rows of the
 * row buffers = padded_rows (moe_max_rows() + 31 * E); shared-expert buffers
 * have shared_rows = T rounded up to 32 rows.
 *   poff [E+1] int32        slot_prow [slots] int32 (padded row or -1)
 *   roff [E+1] int32        offsets the recomputed GEMM1 runs over: poff, or
 *                           all zero when the forward kept its
 *                           pre-activations (shared_roff: the same for the
 *                           shared expert's {0, rows})
 *   prow_src [padded_rows] int32  forward row of each padded row (-1: pad;
 *                           written when recompute = 0)
 *   d_slot_w [slots] fp32   dL/dw per slot (top-k [T,k]; ExpertChoice the
 *                           CSR order of moe_permute)
 *   dlogits [T,E] fp32      dL/dlogits; the gradient of a logit bias is its
 *                           sum over tokens ([E] bias) or dlogits itself
 *   dx_router [T,d] fp32    dlogits W_r
 *   router_part             fp32 partials of dW_r over chunks of 512 tokens
 *   xp, dyp, dxp [padded_rows, d]   expert inputs, output gradients (w dy),
 *                           input gradients
 *   z [padded_rows, n_up*d_ff]      pre-activations, then dL/dz
 *   dh [padded_rows, d_ff]          dL/dh, then the recomputed h
 *   xs, dys, dxs, zs, dhs   the same for the shared expert
 * ------------------------------------------------------------------------ */
typedef struct {
  size_t poff, roff, slot_prow, prow_src, d_slot_w, dlogits, dx_router, router_offset, router_part;
  size_t xp, dyp, z, dh, dxp;
  size_t shared_offset, shared_roff, xs, dys, zs, dhs, dxs;
  size_t scratch, scratch_bytes, shared_scratch, shared_scratch_bytes;
  size_t padded_rows, shared_rows; /* row counts, not bytes */
  size_t total;                    /* bytes the workspace must hold */
} moe_bwd_layout;
moe_status moe_layer_bwd_workspace(const moe_config *cfg, moe_bwd_layout *layout);
/* moe_layer_fwd_train -- moe_layer_fwd for training: the same outputs
 * (within bf16 rounding: the activation is applied to the pre-activations
 * after their rounding to dtype), and the expert pre-activations z are kept
 * in the workspace (layout.z, layout.shared_z) so that moe_layer_bwd can skip
 * recomputing them (recompute = 0).  Arguments as moe_layer_fwd. */
moe_status moe_layer_fwd_train(const moe_config *cfg, const void *x, const void *w_router,
                               const float *logit_bias, int64_t bias_row_stride, const void *w1,
                               const void *w2, const void *ws1, const void *ws2, void *y, void *workspace,
                               size_t workspace_bytes, void *stream);
/* moe_layer_bwd -- gradients of the whole block.
 *   x, w_router, w1, w2, ws1, ws2: as given to moe_layer_fwd.
 *   fwd_workspace: the workspace of a moe_layer_fwd or moe_layer_fwd_train
 *     call on the same inputs (its routing, permutation and y_perm are read;
 *     nothing is written).
 *   recompute: 1 re-runs the expert GEMM1; 0 reads the pre-activations a
 *     training forward kept.  The forward's last step stamps the workspace
 *     with which forward ran, and the device checks that stamp: after a
 *     plain moe_layer_fwd, recompute = 0 re-runs GEMM1 as well, so the
 *     gradients never come from stale pre-activations.
 *   dy [T,d] dtype: dL/dy.
 *   Outputs (dtype, overwritten): dx [T,d], dw_router [E,d],
 *     dw1 [E, n_up*d_ff, d], dw2 [E, d, d_ff], dws1 / dws2 (shared expert,
 *     NULL when d_ff_shared == 0).  T = 0 writes zero weight gradients.
 *   workspace: moe_layer_bwd_workspace().total bytes, 256-B aligned.
 * The shared expert's backward runs on the side stream of moe_layer_fwd
 * beside the routed part and is joined before dx is assembled.  Results are
 * deterministic. */
moe_status moe_layer_bwd(const moe_config *cfg, const void *x, const void *w_router, const void *w1,
                         const void *w2, const void *ws1, const void *ws2, const void *fwd_workspace,
                         size_t fwd_workspace_bytes, const void *dy, void *dx, void *dw_router, void *dw1,
                         void *dw2, void *dws1, void *dws2, int32_t recompute, void *workspace,
                         size_t workspace_bytes, void *stream);
const char *moe_status_string(moe_status s);
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
