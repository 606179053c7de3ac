// Internal launchers of the gfx950 kernels (host side).  The C ABI in
// include/moe.h validates arguments and then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kEcMaxTokens = 16384;      // ExpertChoice: score column held in LDS
constexpr int kSplitUnits = 256;        // grouped GEMM: most workgroups in one round (one per CU)
constexpr int kPermuteBlock = 1024;      // assignments per counting block
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 16;

struct RouteArgs {
  int dtype;  // 0 fp32, 1 bf16
  const void *x, *wr;
  const float *bias;
  int64_t bias_stride;
  int T, d, E, k, routing, C;
  float *logits;
  int32_t *topk_idx;
  float *topk_w;
  float *scores;
  int32_t *ec_token;
  float *ec_w;
};
hipError_t launch_route(const RouteArgs &a, hipStream_t st);

struct PermuteArgs {
  int T, k, E;
  int64_t cap;              // -1: dropless
  size_t row_bytes;         // d * element size
  const void *x;
  const int32_t *topk_idx;
  void *x_perm;
  int32_t *row_token, *slot_row, *expert_count, *expert_load, *expert_offset;
  int32_t *blk;             // scratch [nblk][E]
  int32_t *rank;            // scratch [T*k]
  int64_t kb_rows;          // > 0: x_perm K-blocked over this many rows ([d/32][kb_rows][32])
};
size_t permute_scratch_bytes(int T, int k, int E);
hipError_t launch_permute_topk(const PermuteArgs &a, hipStream_t st);

struct PermuteEcArgs {
  int T, E, C;
  size_t row_bytes;
  const void *x;
  const int32_t *ec_token;
  const float *ec_w;
  void *x_perm;
  int32_t *row_token, *slot_row, *tok_ptr, *expert_count, *expert_load, *expert_offset;
  float *slot_w;
  int64_t kb_rows;  // > 0: x_perm K-blocked, as in PermuteArgs
};
hipError_t launch_permute_ec(const PermuteEcArgs &a, hipStream_t st);

struct FfnArgs {
  int dtype, act;
  int E, d, d_ff;
  int64_t max_rows;
  const void *x_perm;
  const int32_t *expert_offset;
  const void *w1, *w2;
  void *h, *y_perm;
  void *scratch;  // ffn_scratch_bytes() bytes, 256-B aligned
  size_t scratch_bytes;
  void *z;        // optional [max_rows, n_up*d_ff]: keep the pre-activations
  bool packed;    // w1 / w2 in the packed order of launch_pack_weights (bf16,
                  // d and d_ff multiples of 64, no z); h is then K-blocked
                  // ([d_ff/32][max_rows][32])
  bool x_kb;      // packed only: x_perm K-blocked ([d/32][max_rows][32])
};
size_t ffn_scratch_bytes(int dtype, int E, int d, int d_ff, int64_t max_rows, bool packed = false);
hipError_t launch_expert_ffn(const FfnArgs &a, hipStream_t st);

// Expert weights [E][n_rows][K] (bf16) -> the packed tile-major order the
// forward GEMMs read as whole contiguous stages (gemm_common.h describes it).
// SwiGLU: n_rows = 2 n_out, gate rows first; otherwise n_rows = n_out.
struct PackArgs {
  int E, n_rows, n_out, K;
  bool swiglu;
  const void *src;
  void *dst;
};
size_t packed_weight_bytes(int E, int n_out, int K, bool swiglu);
hipError_t launch_pack_weights(const PackArgs &a, hipStream_t st);

struct CombineArgs {
  int dtype;
  int T, d, k;
  const void *y_perm;
  const int32_t *tok_ptr, *slot_row;
  const float *slot_w;
  const void *y_shared;
  void *y;
  int64_t rows;    // rows of y_perm
  int64_t nslots;  // entries of slot_row / slot_w
  int32_t *stamp;  // optional: workgroup 0 writes stamp_val here once the
  int32_t stamp_val;  // combine has been enqueued (the forward's last step)
};
hipError_t launch_combine(const CombineArgs &a, hipStream_t st);

// Stamps moe_layer_fwd / moe_layer_fwd_train leave in their workspace: the
// backward reads the saved pre-activations only after a training forward
// (kStampTrain) and recomputes them otherwise.
constexpr int32_t kStampPlain = 0x3e5f0000, kStampTrain = 0x3e5f0001;

// Fills a small int32 device array (used for the shared expert's {0, T}).
// With `stamp` given, dst = {0, 0} when *stamp == kStampTrain (device-side).
hipError_t launch_fill_offsets(int32_t *dst, int32_t t, hipStream_t st, const int32_t *stamp = nullptr);

// ---- backward pass (backward.hip) ----------------------------------------
// Expert blocks of the backward's row layout start on multiples of this many
// rows (zero pad rows), so the weight-gradient GEMMs contract over whole
// 32-row K stages.
constexpr int kPadRows = 32;

struct BwdUnpermuteArgs {
  int dtype, T, d, k, E;
  int ec_capacity;  // > 0: ExpertChoice (row r belongs to expert r / C)
  int64_t rows, prows, nslots;
  const void *dy, *x, *y_perm;
  const int32_t *tok_ptr, *slot_row, *topk_idx, *offs, *poff;
  const float *slot_w;
  void *dyp, *xp;
  float *d_slot_w;
  int32_t *slot_prow;
  int32_t *prow_src;  // optional [prows]: compact row of each padded row
};
hipError_t launch_unpermute_bwd(const BwdUnpermuteArgs &a, hipStream_t st);

struct RouterBwdArgs {
  int T, E, k, routing, ec_capacity;
  int64_t nslots;
  const float *logits, *scores, *topk_w, *d_slot_w;
  const int32_t *topk_idx, *tok_ptr, *slot_row;
  float *dlogits;
};
hipError_t launch_router_bwd(const RouterBwdArgs &a, hipStream_t st);

struct GatherDxArgs {
  int dtype, T, d, k;
  int64_t prows, nslots;
  const int32_t *tok_ptr, *slot_prow;
  const void *dxp, *dx_shared;
  const float *dx_router;
  void *dx;
};
hipError_t launch_gather_dx(const GatherDxArgs &a, hipStream_t st);

// poff = padded exclusive offsets; with roff given, also roff = poff, or all
// zeros when *stamp == kStampTrain (the recompute GEMM then has no rows).
hipError_t launch_bwd_offsets(const int32_t *count, int E, int64_t max_rows, int32_t *poff, hipStream_t st,
                              const int32_t *stamp = nullptr, int32_t *roff = nullptr);
hipError_t launch_pad_zero(const int32_t *poff, const int32_t *count, int E, int64_t prows, size_t row_bytes,
                           void *b0, void *b1, int32_t *prow_src, hipStream_t st);
hipError_t launch_pad_copy(const void *src, void *dst, int64_t rows, int64_t prows, size_t row_bytes,
                           hipStream_t st);
// z_src (the saved pre-activations) is read when given and, if `stamp` is
// given too, only when *stamp == kStampTrain; otherwise z is read in place.
hipError_t launch_act_bwd(int dtype, int act, void *z, void *dh, const int32_t *rows_of, int64_t prows, int dff,
                          const void *z_src, const int32_t *src, int64_t src_rows, hipStream_t st,
                          const int32_t *stamp = nullptr);
hipError_t launch_act_fwd(int dtype, int act, const void *z, void *h, const int32_t *rows_of, int64_t max_rows,
                          int dff, hipStream_t st);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t st);

// Generic grouped GEMM C(r, c) = sum_k A(r, k) B(k, c), element strides:
//   A(r, k) = A[r*a_rs + k*a_ks],  B(k, c) = B[e*b_es + k*b_ks + c*b_cs],
//   C(r, c) = C[e*c_es + r*c_rs + c]  (e = the group; c_es used in mode 1).
// mode 0: group e owns rows [offs[e], offs[e+1]) (< max_rows), K fixed.
// mode 1: group e contracts over [offs[e], offs[e+1]) (< max_rows) and owns
//         a dense M x N block of C; offs NULL: over [e*kchunk, (e+1)*kchunk).
struct GenGemmArgs {
  const void *A;
  int64_t a_rs, a_ks;
  const void *B;
  int64_t b_ks, b_cs, b_es;
  void *C;
  int64_t c_rs, c_es;
  const int32_t *offs;
  int E, mode;
  int64_t max_rows;
  int M, N, K;
  int64_t kchunk;
  int m_tiles, n_tiles;  // set by the launcher
};
// dtypes: 0 fp32, 1 bf16 (A, B, C).
hipError_t launch_gemm_generic(GenGemmArgs g, int a_dt, int b_dt, int c_dt, hipStream_t st);
// out[j] = sum over g < groups of part[g*n + j], in a fixed order (c_dt 0 fp32, 1 bf16).
hipError_t launch_sum_partials(const float *part, int groups, int64_t n, int c_dt, void *out, hipStream_t st);
// Token chunk of the router weight gradient dW_r = dlogits^T x: each chunk's
// fp32 partial is computed on its own, then the chunks are added in order.
constexpr int kRouterChunk = 512;

// The grouped GEMMs of the backward pass: bf16 shapes the direct-to-LDS
// MFMA kernels take run there (gemm.hip), the rest on the generic kernel.
//   kind NT: C[r,:] = A[r,:] B_e^T   (B_e [N, K], the forward's layout)
//   kind NN: C[r,:] = A[r,:] B_e     (B_e [K, N])
//   kind TN: C_e = A[rows_e,:]^T B[rows_e,:]  (C_e [M, N], contraction over
//            the group's rows, which start on multiples of kPadRows)
enum { BWD_NT = 0, BWD_NN = 1, BWD_TN = 2 };
struct BwdGemm {
  int kind, dtype;
  const void *A, *B;
  void *C;
  int64_t lda, ldb, ldc;   // row strides (elements)
  int64_t b_stride;        // per-group B elements (NT, NN)
  int64_t c_stride;        // per-group C elements (TN)
  const int32_t *offs;
  int E;
  int64_t max_rows;        // rows (NT, NN) or contraction rows (TN) bound
  int M, N, K;             // TN: C_e is M x N; NT / NN: N outputs, K contraction
  void *scratch;
  size_t scratch_bytes;
};
size_t bwd_gemm_scratch_bytes(const BwdGemm &g);
hipError_t launch_bwd_gemm(const BwdGemm &g, hipStream_t st);

}  // namespace moe
