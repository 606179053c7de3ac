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
};
size_t ffn_scratch_bytes(int dtype, int E, int d, int d_ff, int64_t max_rows);
hipError_t launch_expert_ffn(const FfnArgs &a, hipStream_t st);

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
};
hipError_t launch_combine(const CombineArgs &a, hipStream_t st);

// Fills a small int32 device array (used for the shared expert's {0, T}).
hipError_t launch_fill_offsets(int32_t *dst, int32_t t, hipStream_t st);

}  // namespace moe
