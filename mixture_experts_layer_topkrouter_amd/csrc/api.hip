// C ABI entry points (include/moe.h): host-side validation, workspace
// layout and the enqueue sequence of the forward pass.  Every check runs
// before anything is enqueued; nothing here allocates device memory, frees
// or waits on the host (moe_layer_fwd with a shared expert creates one side
// stream and two events per device and host thread, once).
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"

// Scratch of moe_permute_noalloc: one copy per GPU, resident for the life of
// the process.  Host code never uses this name as an address (on the host
// it is only a stand-in); noalloc_scratch() looks up the device address.
static __device__ __align__(256) unsigned char scratch[MOE_PERMUTE_NOALLOC_MAX_BYTES];

namespace {

using moe::kEcMaxTokens;
using moe::kMaxExperts;
using moe::kMaxTopK;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(const moe_config *c) { return c->dtype == MOE_F32 ? 4 : 2; }

// Shape checks shared by every entry point.
moe_status check_config(const moe_config *c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->num_tokens < 0 || c->d_model <= 0 || c->num_experts <= 0 || c->d_ff <= 0 || c->d_ff_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (c->d_model % 8 || c->d_ff % 8 || c->d_ff_shared % 8) return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->act != MOE_ACT_GELU && c->act != MOE_ACT_SWIGLU) return MOE_ERR_INVALID_ARG;
  if (!(c->capacity_factor >= 0.0) || !isfinite(c->capacity_factor)) return MOE_ERR_INVALID_ARG;
  if (c->routing == MOE_EXPERT_CHOICE) {
    if (c->num_tokens < 1 || c->ec_capacity < 1 || c->ec_capacity > c->num_tokens) return MOE_ERR_INVALID_ARG;
    if (c->num_tokens > kEcMaxTokens) return MOE_ERR_UNSUPPORTED;
  } else if (c->routing == MOE_TOPK_SOFTMAX_ALL || c->routing == MOE_TOPK_SOFTMAX_TOPK) {
    if (c->top_k < 1 || c->top_k > c->num_experts) return MOE_ERR_INVALID_ARG;
    if (c->top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  } else {
    return MOE_ERR_INVALID_ARG;
  }
  if (c->num_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int64_t capacity_of(const moe_config *c) {
  if (c->routing == MOE_EXPERT_CHOICE || c->capacity_factor == 0.0) return -1;
  const double v = ceil(c->capacity_factor * static_cast<double>(c->num_tokens) * static_cast<double>(c->top_k) /
                        static_cast<double>(c->num_experts));
  return static_cast<int64_t>(v);
}

int64_t max_rows_of(const moe_config *c) {
  if (c->routing == MOE_EXPERT_CHOICE) return static_cast<int64_t>(c->num_experts) * c->ec_capacity;
  const int64_t a = static_cast<int64_t>(c->num_tokens) * c->top_k;
  const int64_t cap = capacity_of(c);
  if (cap < 0) return a;
  const int64_t lim = cap * c->num_experts;
  return a < lim ? a : lim;
}

// 32-bit element offsets inside the GEMM kernels must not overflow, and the
// byte offsets of a tile's A rows must stay below the 2^31-byte range of the
// range-checked loads that turn pad rows into zeros: 256 row-major rows of
// width below 2^22, or K-blocked slices of fewer than 2^25 - 256 rows.
bool gemm_fits(const moe_config *c, int64_t rows, int dff) {
  const int64_t lim = INT32_MAX;
  const int64_t n_up = c->act == MOE_ACT_SWIGLU ? 2 : 1;
  const int64_t wlim = int64_t{1} << 22, rlim = (int64_t{1} << 25) - 256;
  return rows * c->d_model < lim && rows * dff < lim && n_up * dff * c->d_model < lim && c->d_model < wlim &&
         dff < wlim && rows < rlim;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

moe_status route_impl(const moe_config *cfg, const void *x, const void *w_router, const float *bias,
                      int64_t bias_stride, float *logits, int32_t *topk_idx, float *topk_w, float *scores,
                      int32_t *ec_token, float *ec_w, void *stream) {
  const int T = cfg->num_tokens, E = cfg->num_experts;
  if (T == 0) return MOE_OK;  // nothing to route; empty buffers may be NULL
  if (!logits) return MOE_ERR_INVALID_ARG;
  if (x) {
    if (!w_router || !aligned16(x) || !aligned16(w_router)) return MOE_ERR_INVALID_ARG;
    if (bias && bias_stride != 0 && bias_stride != E) return MOE_ERR_INVALID_ARG;
  }
  if (cfg->routing == MOE_EXPERT_CHOICE) {
    if (!scores || !ec_token || !ec_w) return MOE_ERR_INVALID_ARG;
  } else if (!topk_idx || !topk_w) {
    return MOE_ERR_INVALID_ARG;
  }
  moe::RouteArgs a{};
  a.dtype = cfg->dtype;
  a.x = x;
  a.wr = w_router;
  a.bias = x ? bias : nullptr;
  a.bias_stride = bias_stride;
  a.T = T;
  a.d = cfg->d_model;
  a.E = E;
  a.k = cfg->routing == MOE_EXPERT_CHOICE ? 0 : cfg->top_k;
  a.routing = cfg->routing;
  a.C = cfg->ec_capacity;
  a.logits = logits;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.scores = scores;
  a.ec_token = ec_token;
  a.ec_w = ec_w;
  return hip_status(moe::launch_route(a, static_cast<hipStream_t>(stream)));
}

moe_status permute_impl(const moe_config *cfg, const void *x, const int32_t *topk_idx, const int32_t *ec_token,
                        const float *ec_w, void *x_perm, int32_t *row_token, int32_t *slot_row, float *slot_w,
                        int32_t *tok_ptr, int32_t *expert_count, int32_t *expert_load, int32_t *expert_offset,
                        void *scratch, size_t scratch_bytes, void *stream, bool kblocked = false) {
  if (!expert_count || !expert_load || !expert_offset) return MOE_ERR_INVALID_ARG;
  const int64_t kb_rows = kblocked ? max_rows_of(cfg) : 0;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const bool empty = cfg->num_tokens == 0;  // only the (zero) counts and offsets are written
  if (!empty && (!x || !x_perm || !row_token || !slot_row)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_INVALID_ARG;
  if (cfg->routing == MOE_EXPERT_CHOICE) {
    if (!ec_token || !ec_w || !slot_w || !tok_ptr) return MOE_ERR_INVALID_ARG;
    moe::PermuteEcArgs a{};
    a.T = cfg->num_tokens;
    a.E = cfg->num_experts;
    a.C = cfg->ec_capacity;
    a.row_bytes = static_cast<size_t>(cfg->d_model) * elem_bytes(cfg);
    a.x = x;
    a.ec_token = ec_token;
    a.ec_w = ec_w;
    a.x_perm = x_perm;
    a.row_token = row_token;
    a.slot_row = slot_row;
    a.tok_ptr = tok_ptr;
    a.expert_count = expert_count;
    a.expert_load = expert_load;
    a.expert_offset = expert_offset;
    a.slot_w = slot_w;
    a.kb_rows = kb_rows;
    return hip_status(moe::launch_permute_ec(a, st));
  }
  if (!empty && !topk_idx) return MOE_ERR_INVALID_ARG;
  const size_t need = moe::permute_scratch_bytes(cfg->num_tokens, cfg->top_k, cfg->num_experts);
  if (need > 0 && (!scratch || scratch_bytes < need)) return MOE_ERR_WORKSPACE;
  if (scratch && !aligned16(scratch)) return MOE_ERR_INVALID_ARG;
  const int64_t A = static_cast<int64_t>(cfg->num_tokens) * cfg->top_k;
  const int64_t nblk = (A + moe::kPermuteBlock - 1) / moe::kPermuteBlock;
  moe::PermuteArgs a{};
  a.T = cfg->num_tokens;
  a.k = cfg->top_k;
  a.E = cfg->num_experts;
  a.cap = capacity_of(cfg);
  a.row_bytes = static_cast<size_t>(cfg->d_model) * elem_bytes(cfg);
  a.x = x;
  a.topk_idx = topk_idx;
  a.x_perm = x_perm;
  a.row_token = row_token;
  a.slot_row = slot_row;
  a.expert_count = expert_count;
  a.expert_load = expert_load;
  a.expert_offset = expert_offset;
  a.kb_rows = kb_rows;
  a.blk = static_cast<int32_t *>(scratch);
  a.rank = reinterpret_cast<int32_t *>(static_cast<char *>(scratch) +
                                       align256(static_cast<size_t>(nblk * cfg->num_experts) * 4));
  return hip_status(moe::launch_permute_topk(a, st));
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
void *noalloc_scratch() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

// Packed expert weights: bf16, and every dimension a packed GEMM contracts
// over or tiles a multiple of 64.
bool packable(const moe_config *c, int dff) { return c->dtype == MOE_BF16 && c->d_model % 64 == 0 && dff % 64 == 0; }

// The FFN scratch of a configuration covers both weight orders: the packed
// one may run another kernel (and so need another scratch) than the plain.
size_t ffn_scratch_of(const moe_config *c) {
  const int64_t rows = max_rows_of(c);
  size_t need = moe::ffn_scratch_bytes(c->dtype, c->num_experts, c->d_model, c->d_ff, rows);
  if (packable(c, c->d_ff))
    need = std::max(need, moe::ffn_scratch_bytes(c->dtype, c->num_experts, c->d_model, c->d_ff, rows, true));
  return need;
}

moe_status ffn_impl(const moe_config *cfg, const void *x_perm, const int32_t *expert_offset, const void *w1,
                    const void *w2, void *h, void *y_perm, void *workspace, size_t workspace_bytes,
                    void *stream, void *z = nullptr, bool packed = false, bool x_kblocked = false) {
  if (packed && (!packable(cfg, cfg->d_ff) || z)) return MOE_ERR_UNSUPPORTED;
  if (max_rows_of(cfg) == 0) return MOE_OK;  // no rows: nothing to compute, empty buffers may be NULL
  if (!x_perm || !expert_offset || !w1 || !w2 || !h || !y_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(w1) || !aligned16(w2) || !aligned16(h) || !aligned16(y_perm))
    return MOE_ERR_INVALID_ARG;
  const int64_t rows = max_rows_of(cfg);
  if (!gemm_fits(cfg, rows, cfg->d_ff)) return MOE_ERR_UNSUPPORTED;
  const size_t need = ffn_scratch_of(cfg);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MOE_ERR_INVALID_ARG;
  moe::FfnArgs a{};
  a.dtype = cfg->dtype;
  a.act = cfg->act;
  a.E = cfg->num_experts;
  a.d = cfg->d_model;
  a.d_ff = cfg->d_ff;
  a.max_rows = rows;
  a.x_perm = x_perm;
  a.expert_offset = expert_offset;
  a.w1 = w1;
  a.w2 = w2;
  a.h = h;
  a.y_perm = y_perm;
  a.scratch = workspace;
  a.scratch_bytes = workspace_bytes;
  a.z = z;
  a.packed = packed;
  a.x_kb = packed && x_kblocked;
  return hip_status(moe::launch_expert_ffn(a, static_cast<hipStream_t>(stream)));
}

// Shapes of the weight that `which` names (moe_pack_which).
moe_status pack_args(const moe_config *cfg, int32_t which, moe::PackArgs *a) {
  const bool swiglu = cfg->act == MOE_ACT_SWIGLU;
  const int d = cfg->d_model;
  switch (which) {
    case MOE_PACK_W1: *a = {cfg->num_experts, (swiglu ? 2 : 1) * cfg->d_ff, cfg->d_ff, d, swiglu, nullptr, nullptr}; break;
    case MOE_PACK_W2: *a = {cfg->num_experts, d, d, cfg->d_ff, false, nullptr, nullptr}; break;
    case MOE_PACK_SHARED_W1:
      *a = {1, (swiglu ? 2 : 1) * cfg->d_ff_shared, cfg->d_ff_shared, d, swiglu, nullptr, nullptr};
      break;
    case MOE_PACK_SHARED_W2: *a = {1, d, d, cfg->d_ff_shared, false, nullptr, nullptr}; break;
    default: return MOE_ERR_INVALID_ARG;
  }
  const bool shared = which == MOE_PACK_SHARED_W1 || which == MOE_PACK_SHARED_W2;
  if (shared && cfg->d_ff_shared == 0) return MOE_ERR_INVALID_ARG;
  if (!packable(cfg, shared ? cfg->d_ff_shared : cfg->d_ff)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status unpermute_impl(const moe_config *cfg, const void *y_perm, const int32_t *tok_ptr,
                          const int32_t *slot_row, const float *slot_w, const void *y_shared, void *y,
                          void *stream, int32_t *stamp = nullptr, int32_t stamp_val = 0) {
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!y_perm || !slot_row || !slot_w || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_perm) || !aligned16(y) || (y_shared && !aligned16(y_shared))) return MOE_ERR_INVALID_ARG;
  if (cfg->routing == MOE_EXPERT_CHOICE && !tok_ptr) return MOE_ERR_INVALID_ARG;
  moe::CombineArgs a{};
  a.dtype = cfg->dtype;
  a.T = cfg->num_tokens;
  a.d = cfg->d_model;
  a.k = cfg->routing == MOE_EXPERT_CHOICE ? 0 : cfg->top_k;
  a.y_perm = y_perm;
  a.tok_ptr = cfg->routing == MOE_EXPERT_CHOICE ? tok_ptr : nullptr;
  a.slot_row = slot_row;
  a.slot_w = slot_w;
  a.y_shared = y_shared;
  a.y = y;
  a.rows = max_rows_of(cfg);
  a.nslots = cfg->routing == MOE_EXPERT_CHOICE ? static_cast<int64_t>(cfg->num_experts) * cfg->ec_capacity
                                                : static_cast<int64_t>(cfg->num_tokens) * cfg->top_k;
  a.stamp = stamp;
  a.stamp_val = stamp_val;
  return hip_status(moe::launch_combine(a, static_cast<hipStream_t>(stream)));
}

// One side stream (default priority) and its fork / join events per device
// and host thread, created on first use and kept for the life of the
// process.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

SideStream *side_stream() {
  constexpr int kMaxDevices = 64;
  thread_local SideStream per_device[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  SideStream &s = per_device[dev];
  if (!s.stream) {
    if (hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&s.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&s.join, hipEventDisableTiming) != hipSuccess)
      return nullptr;
  }
  return &s;
}

moe_config shared_config(const moe_config *cfg) {
  moe_config s = *cfg;
  s.num_experts = 1;
  s.top_k = 1;
  s.capacity_factor = 0.0;
  s.routing = MOE_TOPK_SOFTMAX_ALL;
  s.d_ff = cfg->d_ff_shared;
  s.d_ff_shared = 0;
  s.ec_capacity = 0;
  return s;
}

void make_layout(const moe_config *c, moe_workspace_layout *L) {
  const size_t T = static_cast<size_t>(c->num_tokens), E = static_cast<size_t>(c->num_experts);
  const size_t d = static_cast<size_t>(c->d_model), s = elem_bytes(c);
  const bool ec = c->routing == MOE_EXPERT_CHOICE;
  const size_t k = ec ? 0 : static_cast<size_t>(c->top_k);
  const size_t C = ec ? static_cast<size_t>(c->ec_capacity) : 0;
  const size_t rows = static_cast<size_t>(max_rows_of(c));
  const size_t nslots = ec ? E * C : T * k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  memset(L, 0, sizeof(*L));
  L->logits = take(T * E * 4);
  L->topk_idx = take(T * k * 4);
  L->topk_w = take(T * k * 4);
  L->scores = take(ec ? T * E * 4 : 0);
  L->ec_token = take(E * C * 4);
  L->ec_w = take(E * C * 4);
  L->x_perm = take(rows * d * s);
  L->row_token = take(rows * 4);
  L->slot_row = take(nslots * 4);
  L->slot_w = take(ec ? nslots * 4 : 0);
  L->tok_ptr = take(ec ? (T + 1) * 4 : 0);
  L->expert_count = take(E * 4);
  L->expert_load = take(E * 4);
  L->expert_offset = take((E + 1) * 4);
  L->shared_offset = take(c->d_ff_shared ? 2 * 4 : 0);
  L->h = take(rows * static_cast<size_t>(c->d_ff) * s);
  L->y_perm = take(rows * d * s);
  L->shared_h = take(c->d_ff_shared ? T * static_cast<size_t>(c->d_ff_shared) * s : 0);
  L->shared_y = take(c->d_ff_shared ? T * d * s : 0);
  // pre-activations kept by a training forward (moe_layer_fwd_train)
  const size_t n_up = c->act == MOE_ACT_SWIGLU ? 2 : 1;
  L->z = take(rows * n_up * static_cast<size_t>(c->d_ff) * s);
  L->shared_z = take(c->d_ff_shared ? T * n_up * static_cast<size_t>(c->d_ff_shared) * s : 0);
  L->stamp = take(4);
  L->scratch_bytes = ec ? 0 : moe::permute_scratch_bytes(c->num_tokens, c->top_k, c->num_experts);
  L->scratch = take(L->scratch_bytes);
  // the shared expert FFN runs beside the routed one (side stream), so each
  // has its own scratch region
  L->ffn_scratch_bytes = ffn_scratch_of(c);
  L->ffn_scratch = take(L->ffn_scratch_bytes);
  if (c->d_ff_shared) {
    const moe_config sc = shared_config(c);
    L->shared_ffn_scratch_bytes = ffn_scratch_of(&sc);
  }
  L->shared_ffn_scratch = take(L->shared_ffn_scratch_bytes);
  L->total = off;
}

// ---------------------------------------------------------------------------
// Backward pass: layout of its workspace.
int64_t padded_rows_of(const moe_config *c) {
  return max_rows_of(c) + static_cast<int64_t>(moe::kPadRows - 1) * c->num_experts;
}

int64_t round_rows(int64_t v) { return (v + moe::kPadRows - 1) / moe::kPadRows * moe::kPadRows; }

moe::BwdGemm bwd_gemm(const moe_config *c, int kind) {
  moe::BwdGemm g{};
  g.kind = kind;
  g.dtype = c->dtype;
  return g;
}

// The grouped GEMMs of one expert set's backward (routed: E experts over
// padded rows; shared: one expert over T rounded up): their split scratch.
size_t ffn_bwd_scratch(const moe_config *c, int E, int64_t rows, int dff) {
  const int n_up = c->act == MOE_ACT_SWIGLU ? 2 : 1, d = c->d_model;
  size_t need = 0;
  moe::BwdGemm g = bwd_gemm(c, moe::BWD_NT);
  g.E = E;
  g.max_rows = rows;
  g.N = n_up * dff;
  g.K = d;
  need = std::max(need, moe::bwd_gemm_scratch_bytes(g));
  g.kind = moe::BWD_NN;
  g.N = dff;
  need = std::max(need, moe::bwd_gemm_scratch_bytes(g));
  g.N = d;
  g.K = n_up * dff;
  need = std::max(need, moe::bwd_gemm_scratch_bytes(g));
  g.kind = moe::BWD_TN;
  g.M = d;
  g.N = dff;
  need = std::max(need, moe::bwd_gemm_scratch_bytes(g));
  g.M = n_up * dff;
  g.N = d;
  need = std::max(need, moe::bwd_gemm_scratch_bytes(g));
  return need;
}

void make_bwd_layout(const moe_config *c, moe_bwd_layout *L) {
  const size_t T = static_cast<size_t>(c->num_tokens), E = static_cast<size_t>(c->num_experts);
  const size_t d = static_cast<size_t>(c->d_model), s = elem_bytes(c);
  const size_t n_up = c->act == MOE_ACT_SWIGLU ? 2 : 1;
  const bool ec = c->routing == MOE_EXPERT_CHOICE;
  const size_t nslots = ec ? E * static_cast<size_t>(c->ec_capacity) : T * static_cast<size_t>(c->top_k);
  const size_t P = static_cast<size_t>(padded_rows_of(c));
  const size_t dff = static_cast<size_t>(c->d_ff), dffs = static_cast<size_t>(c->d_ff_shared);
  const size_t Ts = dffs ? static_cast<size_t>(round_rows(c->num_tokens)) : 0;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  memset(L, 0, sizeof(*L));
  L->padded_rows = P;
  L->shared_rows = Ts;
  L->poff = take((E + 1) * 4);
  L->roff = take((E + 1) * 4);
  L->slot_prow = take(nslots * 4);
  L->prow_src = take(P * 4);
  L->d_slot_w = take(nslots * 4);
  L->dlogits = take(T * E * 4);
  L->dx_router = take(T * d * 4);
  L->router_offset = take(2 * 4);
  L->router_part = take(static_cast<size_t>((c->num_tokens + moe::kRouterChunk - 1) / moe::kRouterChunk) * E * d * 4);
  L->xp = take(P * d * s);
  L->dyp = take(P * d * s);
  L->z = take(P * n_up * dff * s);
  L->dh = take(P * dff * s);
  L->dxp = take(P * d * s);
  L->shared_offset = take(dffs ? 2 * 4 : 0);
  L->shared_roff = take(dffs ? 2 * 4 : 0);
  L->xs = take(Ts * d * s);
  L->dys = take(Ts * d * s);
  L->zs = take(Ts * n_up * dffs * s);
  L->dhs = take(Ts * dffs * s);
  L->dxs = take(Ts * d * s);
  L->scratch_bytes = ffn_bwd_scratch(c, c->num_experts, static_cast<int64_t>(P), c->d_ff);
  L->scratch = take(L->scratch_bytes);
  L->shared_scratch_bytes = dffs ? ffn_bwd_scratch(c, 1, static_cast<int64_t>(Ts), c->d_ff_shared) : 0;
  L->shared_scratch = take(L->shared_scratch_bytes);
  L->total = off;
}

// Backward of one expert set (the routed experts, or the shared expert as one
// expert): recompute z = x W1^T, dh = dy W2, the activation backward
// (z -> dz, dh -> h), dx = dz W1, dW2 = dy^T h, dW1 = dz^T x.  Rows of expert
// e are [offs[e], offs[e+1]), multiples of 32, pad rows zero.
moe_status ffn_bwd_impl(const moe_config *c, int E, int dff, int64_t rows, const int32_t *offs, const void *w1,
                        const void *w2, void *xp, void *dyp, void *z, void *dh, void *dxp, void *dw1, void *dw2,
                        void *scratch, size_t scratch_bytes, hipStream_t st, const void *z_saved,
                        const int32_t *z_src, int64_t z_rows, const int32_t *roff, const int32_t *stamp) {
  const int n_up = c->act == MOE_ACT_SWIGLU ? 2 : 1, d = c->d_model;
  moe::BwdGemm g = bwd_gemm(c, moe::BWD_NT);
  g.offs = offs;
  g.E = E;
  g.max_rows = rows;
  g.scratch = scratch;
  g.scratch_bytes = scratch_bytes;
  // z = xp W1^T (the recomputed forward).  When the caller asks for the
  // kept pre-activations this GEMM runs over roff, which the device set to
  // all zeros after reading the forward's stamp if a training forward kept
  // z (its workgroups then exit at once), and to offs otherwise.
  {
    g.offs = z_saved ? roff : offs;
    g.A = xp;
    g.lda = d;
    g.B = w1;
    g.ldb = d;
    g.b_stride = static_cast<int64_t>(n_up) * dff * d;
    g.C = z;
    g.ldc = static_cast<int64_t>(n_up) * dff;
    g.N = n_up * dff;
    g.K = d;
    if (moe::launch_bwd_gemm(g, st) != hipSuccess) return MOE_ERR_HIP;
    g.offs = offs;
  }
  // dh = dyp W2   (W2_e [d, dff]: K = d rows, N = dff columns)
  g.kind = moe::BWD_NN;
  g.A = dyp;
  g.lda = d;
  g.B = w2;
  g.ldb = dff;
  g.b_stride = static_cast<int64_t>(d) * dff;
  g.C = dh;
  g.ldc = dff;
  g.N = dff;
  g.K = d;
  if (moe::launch_bwd_gemm(g, st) != hipSuccess) return MOE_ERR_HIP;
  const int act = c->act == MOE_ACT_SWIGLU ? 2 : 1;  // ACT_SWIGLU / ACT_GELU of the kernels
  if (moe::launch_act_bwd(c->dtype, act, z, dh, offs + E, rows, dff, z_saved, z_src, z_rows, st,
                          z_saved ? stamp : nullptr) != hipSuccess)
    return MOE_ERR_HIP;
  // dxp = dz W1   (W1_e [n_up*dff, d]: K = n_up*dff rows, N = d columns)
  g.A = z;
  g.lda = static_cast<int64_t>(n_up) * dff;
  g.B = w1;
  g.ldb = d;
  g.b_stride = static_cast<int64_t>(n_up) * dff * d;
  g.C = dxp;
  g.ldc = d;
  g.N = d;
  g.K = n_up * dff;
  if (moe::launch_bwd_gemm(g, st) != hipSuccess) return MOE_ERR_HIP;
  // dW2_e = dyp_e^T h_e   [d, dff]
  g.kind = moe::BWD_TN;
  g.A = dyp;
  g.lda = d;
  g.B = dh;
  g.ldb = dff;
  g.C = dw2;
  g.ldc = dff;
  g.c_stride = static_cast<int64_t>(d) * dff;
  g.M = d;
  g.N = dff;
  g.K = 0;
  if (moe::launch_bwd_gemm(g, st) != hipSuccess) return MOE_ERR_HIP;
  // dW1_e = dz_e^T xp_e   [n_up*dff, d]
  g.A = z;
  g.lda = static_cast<int64_t>(n_up) * dff;
  g.B = xp;
  g.ldb = d;
  g.C = dw1;
  g.ldc = d;
  g.c_stride = static_cast<int64_t>(n_up) * dff * d;
  g.M = n_up * dff;
  g.N = d;
  if (moe::launch_bwd_gemm(g, st) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status layer_fwd_impl(const moe_config *cfg, const void *x, const void *w_router, const float *logit_bias,
                          int64_t bias_row_stride, const void *w1, const void *w2, const void *ws1,
                          const void *ws2, void *y, void *workspace, size_t workspace_bytes, void *stream,
                          bool train, bool packed = false) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (packed && (!packable(cfg, cfg->d_ff) || (cfg->d_ff_shared > 0 && !packable(cfg, cfg->d_ff_shared))))
    return MOE_ERR_UNSUPPORTED;
  if (cfg->num_tokens == 0) return MOE_OK;  // empty batch: nothing to do, empty buffers may be NULL
  if (!x || !w_router || !w1 || !w2 || !y || !workspace) return MOE_ERR_INVALID_ARG;
  if (cfg->d_ff_shared > 0 && (!ws1 || !ws2)) return MOE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MOE_ERR_INVALID_ARG;
  if (bias_row_stride != 0 && bias_row_stride != cfg->num_experts) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w1) || !aligned16(w2) || !aligned16(y))
    return MOE_ERR_INVALID_ARG;
  if (cfg->d_ff_shared > 0 && (!aligned16(ws1) || !aligned16(ws2))) return MOE_ERR_INVALID_ARG;
  moe_workspace_layout L;
  make_layout(cfg, &L);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  const int64_t rows = max_rows_of(cfg);
  if (!gemm_fits(cfg, rows, cfg->d_ff)) return MOE_ERR_UNSUPPORTED;
  moe_config sc = shared_config(cfg);
  if (cfg->d_ff_shared > 0 && !gemm_fits(&sc, cfg->num_tokens, cfg->d_ff_shared)) return MOE_ERR_UNSUPPORTED;

  char *ws = static_cast<char *>(workspace);
  auto P = [&](size_t off) { return static_cast<void *>(ws + off); };
  const bool ec = cfg->routing == MOE_EXPERT_CHOICE;
  float *logits = static_cast<float *>(P(L.logits));
  int32_t *topk_idx = static_cast<int32_t *>(P(L.topk_idx));
  float *topk_w = static_cast<float *>(P(L.topk_w));
  float *scores = static_cast<float *>(P(L.scores));
  int32_t *ec_token = static_cast<int32_t *>(P(L.ec_token));
  float *ec_w = static_cast<float *>(P(L.ec_w));
  int32_t *slot_row = static_cast<int32_t *>(P(L.slot_row));
  float *slot_w = ec ? static_cast<float *>(P(L.slot_w)) : topk_w;
  int32_t *tok_ptr = static_cast<int32_t *>(P(L.tok_ptr));
  int32_t *expert_offset = static_cast<int32_t *>(P(L.expert_offset));

  // Shared expert ([P3] top_k paragraph; overlapped as P1's shared-expert
  // overlap): it reads only x, so it is forked onto a side stream right away
  // and runs beside routing, permutation and the routed experts; the main
  // stream waits for it just before the combine.
  hipStream_t main_st = static_cast<hipStream_t>(stream);
  const void *y_shared = nullptr;
  hipEvent_t join = nullptr;
  if (cfg->d_ff_shared > 0) {
    SideStream *side = side_stream();
    if (!side) return MOE_ERR_HIP;
    if (hipEventRecord(side->fork, main_st) != hipSuccess ||
        hipStreamWaitEvent(side->stream, side->fork, 0) != hipSuccess)
      return MOE_ERR_HIP;
    int32_t *so = static_cast<int32_t *>(P(L.shared_offset));
    if (moe::launch_fill_offsets(so, cfg->num_tokens, side->stream) != hipSuccess) return MOE_ERR_HIP;
    s = ffn_impl(&sc, x, so, ws1, ws2, P(L.shared_h), P(L.shared_y), P(L.shared_ffn_scratch),
                 L.shared_ffn_scratch_bytes, side->stream, train ? P(L.shared_z) : nullptr, packed);
    if (s != MOE_OK) return s;
    if (hipEventRecord(side->join, side->stream) != hipSuccess) return MOE_ERR_HIP;
    join = side->join;
    y_shared = P(L.shared_y);
  }
  s = route_impl(cfg, x, w_router, logit_bias, bias_row_stride, logits, topk_idx, topk_w, scores, ec_token, ec_w,
                 stream);
  if (s != MOE_OK) return s;
  s = permute_impl(cfg, x, topk_idx, ec_token, ec_w, P(L.x_perm), static_cast<int32_t *>(P(L.row_token)), slot_row,
                   static_cast<float *>(P(L.slot_w)), tok_ptr, static_cast<int32_t *>(P(L.expert_count)),
                   static_cast<int32_t *>(P(L.expert_load)), expert_offset, P(L.scratch), L.scratch_bytes, stream,
                   packed);
  if (s != MOE_OK) return s;
  s = ffn_impl(cfg, P(L.x_perm), expert_offset, w1, w2, P(L.h), P(L.y_perm), P(L.ffn_scratch),
               L.ffn_scratch_bytes, stream, train ? P(L.z) : nullptr, packed, packed);
  if (s != MOE_OK) return s;
  if (join && hipStreamWaitEvent(main_st, join, 0) != hipSuccess) return MOE_ERR_HIP;
  return unpermute_impl(cfg, P(L.y_perm), tok_ptr, slot_row, slot_w, y_shared, y, stream,
                        static_cast<int32_t *>(P(L.stamp)), train ? moe::kStampTrain : moe::kStampPlain);
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return 7; }

const char *moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_NOALLOC_LIMIT: return "larger than the allocation-free entry point's static scratch";
  }
  return "unknown status";
}

int64_t moe_max_rows(const moe_config *cfg) {
  if (check_config(cfg) != MOE_OK) return -1;
  return max_rows_of(cfg);
}

int64_t moe_capacity(const moe_config *cfg) {
  if (check_config(cfg) != MOE_OK) return -1;
  return capacity_of(cfg);
}

moe_status moe_route(const moe_config *cfg, const void *x, const void *w_router, const float *logit_bias,
                     int64_t bias_row_stride, float *logits, int32_t *topk_idx, float *topk_w, float *scores,
                     int32_t *ec_token, float *ec_w, void *stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  return route_impl(cfg, x, w_router, logit_bias, bias_row_stride, logits, topk_idx, topk_w, scores, ec_token,
                    ec_w, stream);
}

moe_status moe_permute_scratch_bytes(const moe_config *cfg, size_t *bytes) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = cfg->routing == MOE_EXPERT_CHOICE
               ? 0
               : moe::permute_scratch_bytes(cfg->num_tokens, cfg->top_k, cfg->num_experts);
  return MOE_OK;
}

moe_status moe_permute(const moe_config *cfg, const void *x, const int32_t *topk_idx, const int32_t *ec_token,
                       const float *ec_w, void *x_perm, int32_t *row_token, int32_t *slot_row, float *slot_w,
                       int32_t *tok_ptr, int32_t *expert_count, int32_t *expert_load, int32_t *expert_offset,
                       void *scratch, size_t scratch_bytes, void *stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  return permute_impl(cfg, x, topk_idx, ec_token, ec_w, x_perm, row_token, slot_row, slot_w, tok_ptr,
                      expert_count, expert_load, expert_offset, scratch, scratch_bytes, stream);
}

moe_status moe_permute_packed(const moe_config *cfg, const void *x, const int32_t *topk_idx, const int32_t *ec_token,
                              const float *ec_w, void *x_perm, int32_t *row_token, int32_t *slot_row, float *slot_w,
                              int32_t *tok_ptr, int32_t *expert_count, int32_t *expert_load, int32_t *expert_offset,
                              void *scratch, size_t scratch_bytes, void *stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!packable(cfg, cfg->d_ff)) return MOE_ERR_UNSUPPORTED;
  return permute_impl(cfg, x, topk_idx, ec_token, ec_w, x_perm, row_token, slot_row, slot_w, tok_ptr,
                      expert_count, expert_load, expert_offset, scratch, scratch_bytes, stream, true);
}

moe_status moe_permute_noalloc(const moe_config *cfg, const void *x, const int32_t *topk_idx,
                               const int32_t *ec_token, const float *ec_w, void *x_perm, int32_t *row_token,
                               int32_t *slot_row, float *slot_w, int32_t *tok_ptr, int32_t *expert_count,
                               int32_t *expert_load, int32_t *expert_offset, void *stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  const size_t need = cfg->routing == MOE_EXPERT_CHOICE
                          ? 0
                          : moe::permute_scratch_bytes(cfg->num_tokens, cfg->top_k, cfg->num_experts);
  if (need > MOE_PERMUTE_NOALLOC_MAX_BYTES) return MOE_ERR_NOALLOC_LIMIT;
  void *ws = nullptr;
  if (need > 0 && !(ws = noalloc_scratch())) return MOE_ERR_HIP;
  return permute_impl(cfg, x, topk_idx, ec_token, ec_w, x_perm, row_token, slot_row, slot_w, tok_ptr, expert_count,
                      expert_load, expert_offset, ws, need, stream);
}

moe_status moe_expert_ffn_workspace_bytes(const moe_config *cfg, size_t *bytes) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = ffn_scratch_of(cfg);
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_config *cfg, const void *x_perm, const int32_t *expert_offset,
                          const void *w1, const void *w2, void *h, void *y_perm, void *workspace,
                          size_t workspace_bytes, void *stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  return ffn_impl(cfg, x_perm, expert_offset, w1, w2, h, y_perm, workspace, workspace_bytes, stream);
}

moe_status moe_packed_weight_bytes(const moe_config *cfg, int32_t which, size_t *bytes) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  moe::PackArgs a{};
  if ((s = pack_args(cfg, which, &a)) != MOE_OK) return s;
  *bytes = moe::packed_weight_bytes(a.E, a.n_out, a.K, a.swiglu);
  return MOE_OK;
}

moe_status moe_pack_weights(const moe_config *cfg, int32_t which, const void *w, void *packed, void *stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  moe::PackArgs a{};
  if ((s = pack_args(cfg, which, &a)) != MOE_OK) return s;
  if (!w || !packed || w == packed || !aligned16(w) || !aligned16(packed)) return MOE_ERR_INVALID_ARG;
  a.src = w;
  a.dst = packed;
  return hip_status(moe::launch_pack_weights(a, static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_ffn_packed(const moe_config *cfg, const void *x_perm, int32_t x_perm_kblocked,
                                 const int32_t *expert_offset, const void *w1_packed, const void *w2_packed, void *h,
                                 void *y_perm, void *workspace, size_t workspace_bytes, void *stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (x_perm_kblocked != 0 && x_perm_kblocked != 1) return MOE_ERR_INVALID_ARG;
  return ffn_impl(cfg, x_perm, expert_offset, w1_packed, w2_packed, h, y_perm, workspace, workspace_bytes, stream,
                  nullptr, true, x_perm_kblocked == 1);
}

moe_status moe_unpermute(const moe_config *cfg, const void *y_perm, const int32_t *tok_ptr,
                         const int32_t *slot_row, const float *slot_w, const void *y_shared, void *y,
                         void *stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  return unpermute_impl(cfg, y_perm, tok_ptr, slot_row, slot_w, y_shared, y, stream);
}

moe_status moe_layer_workspace(const moe_config *cfg, moe_workspace_layout *layout) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!layout) return MOE_ERR_INVALID_ARG;
  make_layout(cfg, layout);
  return MOE_OK;
}

moe_status moe_layer_fwd(const moe_config *cfg, const void *x, const void *w_router, const float *logit_bias,
                         int64_t bias_row_stride, const void *w1, const void *w2, const void *ws1,
                         const void *ws2, void *y, void *workspace, size_t workspace_bytes, void *stream) {
  return layer_fwd_impl(cfg, x, w_router, logit_bias, bias_row_stride, w1, w2, ws1, ws2, y, workspace,
                        workspace_bytes, stream, false);
}

moe_status moe_layer_fwd_packed(const moe_config *cfg, const void *x, const void *w_router,
                                const float *logit_bias, int64_t bias_row_stride, const void *w1_packed,
                                const void *w2_packed, const void *ws1_packed, const void *ws2_packed, void *y,
                                void *workspace, size_t workspace_bytes, void *stream) {
  return layer_fwd_impl(cfg, x, w_router, logit_bias, bias_row_stride, w1_packed, w2_packed, ws1_packed, ws2_packed,
                        y, workspace, workspace_bytes, stream, false, true);
}

moe_status moe_layer_fwd_train(const moe_config *cfg, const void *x, const void *w_router, const float *logit_bias,
                               int64_t bias_row_stride, const void *w1, const void *w2, const void *ws1,
                               const void *ws2, void *y, void *workspace, size_t workspace_bytes, void *stream) {
  return layer_fwd_impl(cfg, x, w_router, logit_bias, bias_row_stride, w1, w2, ws1, ws2, y, workspace,
                        workspace_bytes, stream, true);
}

moe_status moe_layer_bwd_workspace(const moe_config *cfg, moe_bwd_layout *layout) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!layout) return MOE_ERR_INVALID_ARG;
  make_bwd_layout(cfg, layout);
  return MOE_OK;
}

moe_status moe_layer_bwd(const moe_config *cfg, const void *x, const void *w_router, const void *w1,
                         const void *w2, const void *ws1, const void *ws2, const void *fwd_workspace,
                         size_t fwd_workspace_bytes, const void *dy, void *dx, void *dw_router, void *dw1,
                         void *dw2, void *dws1, void *dws2, int32_t recompute, void *workspace,
                         size_t workspace_bytes, void *stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  const bool shared = cfg->d_ff_shared > 0;
  if (!w_router || !w1 || !w2 || !dw_router || !dw1 || !dw2) return MOE_ERR_INVALID_ARG;
  if (shared && (!ws1 || !ws2 || !dws1 || !dws2)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(w_router) || !aligned16(w1) || !aligned16(w2) || !aligned16(dw_router) || !aligned16(dw1) ||
      !aligned16(dw2))
    return MOE_ERR_INVALID_ARG;
  if (shared && (!aligned16(ws1) || !aligned16(ws2) || !aligned16(dws1) || !aligned16(dws2)))
    return MOE_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int T = cfg->num_tokens, E = cfg->num_experts, d = cfg->d_model;
  const int n_up = cfg->act == MOE_ACT_SWIGLU ? 2 : 1;
  const size_t es = elem_bytes(cfg);
  if (T == 0) {  // no tokens: every weight gradient is zero
    if (moe::launch_zero(dw_router, static_cast<size_t>(E) * d * es, st) != hipSuccess ||
        moe::launch_zero(dw1, static_cast<size_t>(E) * n_up * cfg->d_ff * d * es, st) != hipSuccess ||
        moe::launch_zero(dw2, static_cast<size_t>(E) * d * cfg->d_ff * es, st) != hipSuccess)
      return MOE_ERR_HIP;
    if (shared && (moe::launch_zero(dws1, static_cast<size_t>(n_up) * cfg->d_ff_shared * d * es, st) != hipSuccess ||
                   moe::launch_zero(dws2, static_cast<size_t>(d) * cfg->d_ff_shared * es, st) != hipSuccess))
      return MOE_ERR_HIP;
    return MOE_OK;
  }
  if (!x || !dy || !dx || !fwd_workspace || !workspace) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dx)) return MOE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || (reinterpret_cast<uintptr_t>(fwd_workspace) & 255u) != 0)
    return MOE_ERR_INVALID_ARG;
  moe_workspace_layout F;
  make_layout(cfg, &F);
  if (fwd_workspace_bytes < F.total) return MOE_ERR_WORKSPACE;
  moe_bwd_layout L;
  make_bwd_layout(cfg, &L);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  const int64_t prows = static_cast<int64_t>(L.padded_rows);
  if (!gemm_fits(cfg, prows, cfg->d_ff)) return MOE_ERR_UNSUPPORTED;
  moe_config sc = shared_config(cfg);
  if (shared && !gemm_fits(&sc, static_cast<int64_t>(L.shared_rows), cfg->d_ff_shared)) return MOE_ERR_UNSUPPORTED;

  const char *fw = static_cast<const char *>(fwd_workspace);
  char *ws = static_cast<char *>(workspace);
  auto F_ = [&](size_t off) { return static_cast<const void *>(fw + off); };
  auto P = [&](size_t off) { return static_cast<void *>(ws + off); };
  const bool ec = cfg->routing == MOE_EXPERT_CHOICE;
  const int32_t *tok_ptr = ec ? static_cast<const int32_t *>(F_(F.tok_ptr)) : nullptr;
  const int32_t *slot_row = static_cast<const int32_t *>(F_(F.slot_row));
  const float *slot_w = static_cast<const float *>(ec ? F_(F.slot_w) : F_(F.topk_w));
  const int32_t *count = static_cast<const int32_t *>(F_(F.expert_count));
  const int64_t nslots = ec ? static_cast<int64_t>(E) * cfg->ec_capacity : static_cast<int64_t>(T) * cfg->top_k;
  int32_t *poff = static_cast<int32_t *>(P(L.poff));
  int32_t *slot_prow = static_cast<int32_t *>(P(L.slot_prow));
  float *d_slot_w = static_cast<float *>(P(L.d_slot_w));
  float *dlogits = static_cast<float *>(P(L.dlogits));
  float *dx_router = static_cast<float *>(P(L.dx_router));
  const int32_t *stamp = static_cast<const int32_t *>(F_(F.stamp));

  // Shared expert: depends only on x and dy, so it runs on the side stream
  // beside the routed part and is joined before dx is assembled.
  hipEvent_t join = nullptr;
  if (shared) {
    SideStream *side = side_stream();
    if (!side) return MOE_ERR_HIP;
    if (hipEventRecord(side->fork, st) != hipSuccess || hipStreamWaitEvent(side->stream, side->fork, 0) != hipSuccess)
      return MOE_ERR_HIP;
    const int64_t Ts = static_cast<int64_t>(L.shared_rows);
    int32_t *so = static_cast<int32_t *>(P(L.shared_offset));
    int32_t *sro = static_cast<int32_t *>(P(L.shared_roff));
    if (moe::launch_fill_offsets(so, static_cast<int32_t>(Ts), side->stream) != hipSuccess ||
        (!recompute && moe::launch_fill_offsets(sro, static_cast<int32_t>(Ts), side->stream, stamp) != hipSuccess) ||
        moe::launch_pad_copy(x, P(L.xs), T, Ts, static_cast<size_t>(d) * es, side->stream) != hipSuccess ||
        moe::launch_pad_copy(dy, P(L.dys), T, Ts, static_cast<size_t>(d) * es, side->stream) != hipSuccess)
      return MOE_ERR_HIP;
    s = ffn_bwd_impl(&sc, 1, cfg->d_ff_shared, Ts, so, ws1, ws2, P(L.xs), P(L.dys), P(L.zs), P(L.dhs), P(L.dxs),
                     dws1, dws2, P(L.shared_scratch), L.shared_scratch_bytes, side->stream,
                     recompute ? nullptr : F_(F.shared_z), nullptr, T, sro, stamp);
    if (s != MOE_OK) return s;
    if (hipEventRecord(side->join, side->stream) != hipSuccess) return MOE_ERR_HIP;
    join = side->join;
  }

  // padded offsets, then the combine's backward (dL/dw per slot, w*dy and x
  // into the padded rows), then zero pad rows
  int32_t *roff = static_cast<int32_t *>(P(L.roff));
  if (moe::launch_bwd_offsets(count, E, max_rows_of(cfg), poff, st, recompute ? nullptr : stamp, roff) != hipSuccess)
    return MOE_ERR_HIP;
  moe::BwdUnpermuteArgs u{};
  u.dtype = cfg->dtype;
  u.T = T;
  u.d = d;
  u.k = ec ? 0 : cfg->top_k;
  u.E = E;
  u.ec_capacity = ec ? cfg->ec_capacity : 0;
  u.rows = max_rows_of(cfg);
  u.prows = prows;
  u.nslots = nslots;
  u.dy = dy;
  u.x = x;
  u.y_perm = F_(F.y_perm);
  u.tok_ptr = tok_ptr;
  u.slot_row = slot_row;
  u.topk_idx = static_cast<const int32_t *>(F_(F.topk_idx));
  u.offs = static_cast<const int32_t *>(F_(F.expert_offset));
  u.poff = poff;
  u.slot_w = slot_w;
  u.dyp = P(L.dyp);
  u.xp = P(L.xp);
  u.d_slot_w = d_slot_w;
  u.slot_prow = slot_prow;
  int32_t *prow_src = recompute ? nullptr : static_cast<int32_t *>(P(L.prow_src));
  u.prow_src = prow_src;
  if (moe::launch_unpermute_bwd(u, st) != hipSuccess) return MOE_ERR_HIP;
  if (moe::launch_pad_zero(poff, count, E, prows, static_cast<size_t>(d) * es, P(L.xp), P(L.dyp), prow_src, st) !=
      hipSuccess)
    return MOE_ERR_HIP;

  // gate gradient, then the router's linear layer
  moe::RouterBwdArgs r{};
  r.T = T;
  r.E = E;
  r.k = ec ? 0 : cfg->top_k;
  r.routing = cfg->routing;
  r.ec_capacity = ec ? cfg->ec_capacity : 0;
  r.nslots = nslots;
  r.logits = static_cast<const float *>(F_(F.logits));
  r.scores = ec ? static_cast<const float *>(F_(F.scores)) : nullptr;
  r.topk_w = ec ? nullptr : static_cast<const float *>(F_(F.topk_w));
  r.d_slot_w = d_slot_w;
  r.topk_idx = ec ? nullptr : static_cast<const int32_t *>(F_(F.topk_idx));
  r.tok_ptr = tok_ptr;
  r.slot_row = slot_row;
  r.dlogits = dlogits;
  if (moe::launch_router_bwd(r, st) != hipSuccess) return MOE_ERR_HIP;
  int32_t *ro = static_cast<int32_t *>(P(L.router_offset));
  if (moe::launch_fill_offsets(ro, T, st) != hipSuccess) return MOE_ERR_HIP;
  {
    // dx_router = dlogits W_r  (fp32 [T,E] x [E,d])
    moe::GenGemmArgs g{};
    g.A = dlogits;
    g.a_rs = E;
    g.a_ks = 1;
    g.B = w_router;
    g.b_ks = d;
    g.b_cs = 1;
    g.C = dx_router;
    g.c_rs = d;
    g.offs = ro;
    g.E = 1;
    g.mode = 0;
    g.max_rows = T;
    g.N = d;
    g.K = E;
    if (moe::launch_gemm_generic(g, 0, cfg->dtype, 0, st) != hipSuccess) return MOE_ERR_HIP;
    // dW_r = dlogits^T x  ([E,T] x [T,d]): fp32 partials over chunks of
    // kRouterChunk tokens, computed side by side, then added in chunk order
    const int chunks = (T + moe::kRouterChunk - 1) / moe::kRouterChunk;
    moe::GenGemmArgs h{};
    h.A = dlogits;
    h.a_rs = 1;
    h.a_ks = E;
    h.B = x;
    h.b_ks = d;
    h.b_cs = 1;
    h.C = P(L.router_part);
    h.c_rs = d;
    h.c_es = static_cast<int64_t>(E) * d;
    h.offs = nullptr;
    h.kchunk = moe::kRouterChunk;
    h.E = chunks;
    h.mode = 1;
    h.max_rows = T;
    h.M = E;
    h.N = d;
    if (moe::launch_gemm_generic(h, 0, cfg->dtype, 0, st) != hipSuccess) return MOE_ERR_HIP;
    if (moe::launch_sum_partials(static_cast<const float *>(P(L.router_part)), chunks, static_cast<int64_t>(E) * d,
                                 cfg->dtype, dw_router, st) != hipSuccess)
      return MOE_ERR_HIP;
  }

  // routed experts
  s = ffn_bwd_impl(cfg, E, cfg->d_ff, prows, poff, w1, w2, P(L.xp), P(L.dyp), P(L.z), P(L.dh), P(L.dxp), dw1, dw2,
                   P(L.scratch), L.scratch_bytes, st, recompute ? nullptr : F_(F.z), prow_src, max_rows_of(cfg), roff,
                   stamp);
  if (s != MOE_OK) return s;

  // dx: the permutation's backward (each token gathers its copies'
  // gradients) + the router term + the shared expert's
  if (join && hipStreamWaitEvent(st, join, 0) != hipSuccess) return MOE_ERR_HIP;
  moe::GatherDxArgs gx{};
  gx.dtype = cfg->dtype;
  gx.T = T;
  gx.d = d;
  gx.k = ec ? 0 : cfg->top_k;
  gx.prows = prows;
  gx.nslots = nslots;
  gx.tok_ptr = tok_ptr;
  gx.slot_prow = slot_prow;
  gx.dxp = P(L.dxp);
  gx.dx_shared = shared ? P(L.dxs) : nullptr;
  gx.dx_router = dx_router;
  gx.dx = dx;
  return hip_status(moe::launch_gather_dx(gx, st));
}

}  // extern "C"
