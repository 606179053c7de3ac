// Router: gate logits, softmax and top-k per token (TopKRouter), or softmax
// scores plus a per-expert top-C selection (ExpertChoiceRouter).
//
// "How MegaDLMs Implements Mixture of Experts (MoE) Architectures", section
// "Routing Mechanisms: Top-K vs Expert Choice": the TopKRouter computes dense
// gate logits with a learned linear layer, applies a softmax and keeps the k
// best experts per token (probability weights + routing map); the
// ExpertChoiceRouter lets each expert choose its tokens by routing score.
//
// gfx950 design:
// * logits: bf16 MFMA 16x16x32 with fp32 accumulation.  A block owns 16*MT
//   tokens and all E (padded to 16*NT) experts; its four waves split the
//   contraction over d by interleaved 32-wide steps and their partial tiles
//   are summed in LDS in a fixed wave order, so results are deterministic.
//   The router weight is tiny and stays in L2; x is streamed once from HBM.
// * the gate runs on the logits tile while it is still in LDS: one wave per
//   token, lane l holds experts l, l+64, l+128, l+192; each of the k picks is a
//   64-lane butterfly arg-max under the order (value desc, index asc) with IEEE
//   comparisons (so -0 == +0), which is a strict total order, so every lane
//   agrees on the winner.
// * ExpertChoice: one workgroup per expert keeps its score column in LDS,
//   finds the C-th largest score by an 8-bit radix select (scores are >= 0,
//   so their bit patterns order like the values), then compacts the chosen
//   tokens in ascending order with block prefix sums.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;

// Gate for `rows` tokens whose logits sit in LDS (row stride ld).
__device__ void gate_rows(const float *tile, int ld, int rows, int t0, int T, int E, int k,
                          int routing, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
                          float *__restrict__ scores) {
  const int l = lane_id();
  const int nw = blockDim.x / kWave;
  for (int r = wave_id(); r < rows; r += nw) {
    const int t = t0 + r;
    if (t >= T) break;
    const float *row = tile + r * ld;
    float v[4];
    bool valid[4], taken[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = l + kWave * q;
      valid[q] = e < E;
      v[q] = valid[q] ? row[e] : 0.f;
      taken[q] = !valid[q];
    }
    if (routing == 2) {  // ExpertChoice scores: softmax over E
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (valid[q]) m = fmaxf(m, v[q]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (valid[q]) s += expf(v[q] - m);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
      s = __shfl(s, 0, kWave);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (valid[q]) scores[(int64_t)t * E + l + kWave * q] = expf(v[q] - m) / s;
      continue;
    }
    int my_idx = -1;
    float my_val = 0.f;
    for (int j = 0; j < k; ++j) {
      bool have = false;
      float bv = 0.f;
      int bi = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // q ascending is index ascending: a strict '>' keeps the lower index on ties
        if (!taken[q] && (!have || v[q] > bv)) {
          have = true;
          bv = v[q];
          bi = l + kWave * q;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        const int oh = __shfl_xor(have ? 1 : 0, o, kWave);
        if (oh && (!have || ov > bv || (ov == bv && oi < bi))) {
          have = true;
          bv = ov;
          bi = oi;
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (bi == l + kWave * q) taken[q] = true;
      if (l == j) {
        my_idx = bi;
        my_val = bv;
      }
    }
    const float top = __shfl(my_val, 0, kWave);
    float w;
    if (routing == 0) {  // softmax over all E, read at the chosen experts
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (valid[q]) s += expf(v[q] - top);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
      s = __shfl(s, 0, kWave);
      w = expf(my_val - top) / s;
    } else {  // softmax over the k chosen logits
      const float ex = (l < k) ? expf(my_val - top) : 0.f;
      float s = 0.f;
      for (int jj = 0; jj < k; ++jj) s += __shfl(ex, jj, kWave);
      w = ex / s;
    }
    if (l < k) {
      topk_idx[(int64_t)t * k + l] = my_idx;
      topk_w[(int64_t)t * k + l] = w;
    }
  }
}

// Adds the bias, writes the logits and leaves them in LDS for the gate.
__device__ void finish_logits(float *tile, int ld, int rows, int t0, int T, int E, const float *bias,
                              int64_t bias_stride, float *logits) {
  for (int i = threadIdx.x; i < rows * E; i += blockDim.x) {
    const int r = i / E, e = i - (i / E) * E;
    const int t = t0 + r;
    if (t >= T) continue;
    float v = tile[r * ld + e];
    if (bias) v += bias[(int64_t)t * bias_stride + e];
    tile[r * ld + e] = v;
    logits[(int64_t)t * E + e] = v;
  }
  __syncthreads();
}

template <int MT, int NT>
__global__ __launch_bounds__(kRouteThreads) void route_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, const float *__restrict__ bias,
    int64_t bias_stride, int T, int d, int E, int k, int routing, float *__restrict__ logits,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, float *__restrict__ scores) {
  constexpr int BT = 16 * MT, EP = 16 * NT;
  __shared__ float tile[BT * EP];
  const int l = lane_id(), w = wave_id();
  const int t0 = blockIdx.x * BT;
  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ksteps = (d + 31) / 32;
  const bf16x8 zero = {};
#pragma unroll 2
  for (int s = w; s < ksteps; s += 4) {
    const int kk = s * 32 + (l >> 4) * 8;
    const bool kin = kk < d;
    bf16x8 a[MT], b[NT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int row = t0 + m * 16 + (l & 15);
      a[m] = (kin && row < T) ? *reinterpret_cast<const bf16x8 *>(x + (int64_t)row * d + kk) : zero;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int e = n * 16 + (l & 15);
      b[n] = (kin && e < E) ? *reinterpret_cast<const bf16x8 *>(wr + (int64_t)e * d + kk) : zero;
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], b[n], acc[m][n], 0, 0, 0);
  }
  // fixed-order sum of the four waves' partial tiles
  for (int ww = 0; ww < kRouteThreads / kWave; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int id = (m * 16 + (l >> 4) * 4 + r) * EP + n * 16 + (l & 15);
            tile[id] = (ww == 0 ? 0.f : tile[id]) + acc[m][n][r];
          }
    }
    __syncthreads();
  }
  finish_logits(tile, EP, BT, t0, T, E, bias, bias_stride, logits);
  gate_rows(tile, EP, BT, t0, T, E, k, routing, topk_idx, topk_w, scores);
}

constexpr int kF32Rows = 16;

__global__ __launch_bounds__(kRouteThreads) void route_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    int64_t bias_stride, int T, int d, int E, int k, int routing, float *__restrict__ logits,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, float *__restrict__ scores) {
  __shared__ float tile[kF32Rows * 256];
  const int t0 = blockIdx.x * kF32Rows;
  for (int i = threadIdx.x; i < kF32Rows * E; i += blockDim.x) {
    const int r = i / E, e = i - (i / E) * E;
    const int t = t0 + r;
    float s = 0.f;
    if (t < T)
      for (int kk = 0; kk < d; ++kk) s = fmaf(x[(int64_t)t * d + kk], wr[(int64_t)e * d + kk], s);
    tile[r * E + e] = s;
  }
  __syncthreads();
  finish_logits(tile, E, kF32Rows, t0, T, E, bias, bias_stride, logits);
  gate_rows(tile, E, kF32Rows, t0, T, E, k, routing, topk_idx, topk_w, scores);
}

// Gate only: the logits are an input.
__global__ __launch_bounds__(kRouteThreads) void gate_only_kernel(
    const float *__restrict__ logits, int T, int E, int k, int routing, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, float *__restrict__ scores) {
  __shared__ float tile[kF32Rows * 256];
  const int t0 = blockIdx.x * kF32Rows;
  for (int i = threadIdx.x; i < kF32Rows * E; i += blockDim.x) {
    const int r = i / E, e = i - (i / E) * E;
    const int t = t0 + r;
    tile[r * E + e] = (t < T) ? logits[(int64_t)t * E + e] : 0.f;
  }
  __syncthreads();
  gate_rows(tile, E, kF32Rows, t0, T, E, k, routing, topk_idx, topk_w, scores);
}

constexpr int kEcThreads = 1024;

// ExpertChoice selection: expert e (one workgroup) keeps the C tokens with the
// largest scores[t,e] (equal scores: lower token), in ascending token order.
__global__ __launch_bounds__(kEcThreads) void ec_select_kernel(const float *__restrict__ scores, int T,
                                                               int E, int C, int32_t *__restrict__ ec_token,
                                                               float *__restrict__ ec_w) {
  __shared__ uint32_t key[kEcMaxTokens];
  __shared__ int hist[256];
  __shared__ int scan_tmp[kEcThreads / kWave + 1];
  __shared__ uint32_t sel_state[2];
  const int e = blockIdx.x;
  for (int t = threadIdx.x; t < T; t += blockDim.x) key[t] = __float_as_uint(scores[(int64_t)t * E + e]);
  uint32_t prefix = 0, pmask = 0;
  int need = C;  // rank (1-based, from the top) of the wanted key among those matching the prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int t = threadIdx.x; t < T; t += blockDim.x) {
      const uint32_t kv = key[t];
      if ((kv & pmask) == prefix) atomicAdd(&hist[(kv >> shift) & 255u], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int cum = 0, b = 255;
      for (; b > 0; --b) {
        if (cum + hist[b] >= need) break;
        cum += hist[b];
      }
      sel_state[0] = static_cast<uint32_t>(b);
      sel_state[1] = static_cast<uint32_t>(need - cum);
    }
    __syncthreads();
    prefix |= sel_state[0] << shift;
    pmask |= 255u << shift;
    need = static_cast<int>(sel_state[1]);
    __syncthreads();
  }
  // prefix is the C-th largest key; `need` of the keys equal to it are taken
  // (the lowest tokens), every key above it is taken.
  const int per = (T + kEcThreads - 1) / kEcThreads;
  const int b0 = min(T, static_cast<int>(threadIdx.x) * per), b1 = min(T, b0 + per);
  int n_eq = 0;
  for (int t = b0; t < b1; ++t) n_eq += (key[t] == prefix);
  int tot;
  int eq_rank = block_excl_scan(n_eq, scan_tmp, &tot);
  int n_sel = 0;
  {
    int er = eq_rank;
    for (int t = b0; t < b1; ++t) {
      const uint32_t kv = key[t];
      if (kv > prefix) ++n_sel;
      else if (kv == prefix) { if (er < need) ++n_sel; ++er; }
    }
  }
  int pos = block_excl_scan(n_sel, scan_tmp, &tot);
  {
    int er = eq_rank;
    for (int t = b0; t < b1; ++t) {
      const uint32_t kv = key[t];
      bool take = false;
      if (kv > prefix) take = true;
      else if (kv == prefix) { take = er < need; ++er; }
      if (take) {
        ec_token[(int64_t)e * C + pos] = t;
        ec_w[(int64_t)e * C + pos] = __uint_as_float(kv);
        ++pos;
      }
    }
  }
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  if (a.x == nullptr) {
    const int blocks = (a.T + kF32Rows - 1) / kF32Rows;
    gate_only_kernel<<<blocks, kRouteThreads, 0, st>>>(a.logits, a.T, a.E, a.k, a.routing, a.topk_idx,
                                                       a.topk_w, a.scores);
  } else if (a.dtype == 0) {
    const int blocks = (a.T + kF32Rows - 1) / kF32Rows;
    route_f32_kernel<<<blocks, kRouteThreads, 0, st>>>(
        static_cast<const float *>(a.x), static_cast<const float *>(a.wr), a.bias, a.bias_stride, a.T,
        a.d, a.E, a.k, a.routing, a.logits, a.topk_idx, a.topk_w, a.scores);
  } else {
    int nt = 1;
    while (nt * 16 < a.E) nt <<= 1;
    int mt = 1;
    if ((a.T + 63) / 64 >= 256 && nt <= 8) mt = 4;
    else if ((a.T + 31) / 32 >= 256 && nt <= 16) mt = 2;
    const int blocks = (a.T + 16 * mt - 1) / (16 * mt);
    const uint16_t *x = static_cast<const uint16_t *>(a.x);
    const uint16_t *wr = static_cast<const uint16_t *>(a.wr);
#define MOE_ROUTE_CASE(MT_, NT_)                                                                     \
  if (mt == MT_ && nt == NT_) {                                                                      \
    route_bf16_kernel<MT_, NT_><<<blocks, kRouteThreads, 0, st>>>(x, wr, a.bias, a.bias_stride, a.T, \
                                                                  a.d, a.E, a.k, a.routing,          \
                                                                  a.logits, a.topk_idx, a.topk_w,    \
                                                                  a.scores);                         \
  }
    MOE_ROUTE_CASE(1, 1) MOE_ROUTE_CASE(1, 2) MOE_ROUTE_CASE(1, 4) MOE_ROUTE_CASE(1, 8) MOE_ROUTE_CASE(1, 16)
    MOE_ROUTE_CASE(2, 1) MOE_ROUTE_CASE(2, 2) MOE_ROUTE_CASE(2, 4) MOE_ROUTE_CASE(2, 8) MOE_ROUTE_CASE(2, 16)
    MOE_ROUTE_CASE(4, 1) MOE_ROUTE_CASE(4, 2) MOE_ROUTE_CASE(4, 4) MOE_ROUTE_CASE(4, 8)
#undef MOE_ROUTE_CASE
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.routing != 2) return err;
  ec_select_kernel<<<a.E, kEcThreads, 0, st>>>(a.scores, a.T, a.E, a.C, a.ec_token, a.ec_w);
  return hipGetLastError();
}

}  // namespace moe
