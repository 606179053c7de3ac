// Router: gate logits, softmax and top-k per token (TopKRouter), or softmax
// scores plus a per-expert top-C selection (ExpertChoiceRouter).
//
// "How MegaDLMs Implements Mixture of Experts (MoE) Architectures", section
// "Routing Mechanisms: Top-K vs Expert Choice": the TopKRouter scores every
// expert for every token with one trained linear map, applies a softmax and keeps the k
// best experts per token (probability weights + routing map); the
// ExpertChoiceRouter lets each expert choose its tokens by routing score.
//
// gfx950 design:
// * logits: bf16 MFMA 16x16x32 with fp32 accumulation.  A block owns 16*MT
//   tokens and all E (padded to 16*NT) experts; its eight waves split the
//   contraction over d by interleaved 32-wide steps, each with several steps
//   of loads in flight, and their partial tiles are summed in LDS in a fixed
//   wave order, so results are deterministic.
//   The router weight is tiny and stays in L2; x is streamed once from HBM.
// * the gate runs on the logits tile while it is still in LDS: one wave per
//   token, lane l holds experts l, l+64, l+128, l+192; each of the k picks is a
//   wave arg-max under the order (value desc, index asc) with IEEE comparisons
//   (so -0 == +0), a strict total order.  The wave reductions (arg-max, max,
//   sum) run on DPP lane shifts inside rows of 16 lanes plus two row
//   broadcasts, a few cycles per step instead of an LDS-crossbar round trip
//   per butterfly level; lane 63 ends with the result, which readlane makes
//   wave-uniform.  The order of the steps is fixed, so sums are
//   deterministic.
// * ExpertChoice: one workgroup per expert keeps its score column in LDS,
//   finds the C-th largest score by an 8-bit radix select (scores are >= 0,
//   so their bit patterns order like the values), then compacts the chosen
//   tokens in ascending order with block prefix sums.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;

// The DPP moves of common.h on floats and ints (a lane whose source lane is
// out of range, or outside the row mask, keeps its own value).
constexpr int kRowShr1 = kDppRowShr1, kRowShr2 = kDppRowShr2, kRowShr4 = kDppRowShr4, kRowShr8 = kDppRowShr8;
constexpr int kRowBcast15 = kDppRowBcast15, kRowBcast31 = kDppRowBcast31;

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_move<CTRL, ROWS>(__float_as_int(v)));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_i(int v) {
  return dpp_move<CTRL, ROWS>(v);
}

// (vb, ib) ranks before (va, ia): larger value, equal values by lower index.
__device__ __forceinline__ bool ranks_before(float vb, int ib, float va, int ia) {
  return vb > va || (vb == va && ib < ia);
}

// Wave arg-max of (v, i) under ranks_before; returns it wave-uniform.  Row
// shifts 1, 2, 4, 8 leave each row's best in its lane 15, the two row
// broadcasts carry rows 0 and 2 into rows 1 and 3, then row 1 into 2 and 3.
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
#define MOE_ARGMAX_STEP(C, R)                   \
  {                                             \
    const float ov = dpp_f<C, R>(v);            \
    const int oi = dpp_i<C, R>(i);              \
    if (ranks_before(ov, oi, v, i)) {           \
      v = ov;                                   \
      i = oi;                                   \
    }                                           \
  }
  MOE_ARGMAX_STEP(kRowShr1, 0xf)
  MOE_ARGMAX_STEP(kRowShr2, 0xf)
  MOE_ARGMAX_STEP(kRowShr4, 0xf)
  MOE_ARGMAX_STEP(kRowShr8, 0xf)
  MOE_ARGMAX_STEP(kRowBcast15, 0xa)
  MOE_ARGMAX_STEP(kRowBcast31, 0xc)
#undef MOE_ARGMAX_STEP
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}

__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f<kRowShr1, 0xf>(v));
  v = fmaxf(v, dpp_f<kRowShr2, 0xf>(v));
  v = fmaxf(v, dpp_f<kRowShr4, 0xf>(v));
  v = fmaxf(v, dpp_f<kRowShr8, 0xf>(v));
  v = fmaxf(v, dpp_f<kRowBcast15, 0xa>(v));
  v = fmaxf(v, dpp_f<kRowBcast31, 0xc>(v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Wave sum in a fixed order.  A shifted-in value is added only where the
// source lane exists (the DPP keeps the lane's own value elsewhere, which
// must not be added twice).
__device__ __forceinline__ float wave_sum_dpp(float v) {
  const int l = lane_id() & 15, row = lane_id() >> 4;
  float o;
  o = dpp_f<kRowShr1, 0xf>(v);
  if (l >= 1) v += o;
  o = dpp_f<kRowShr2, 0xf>(v);
  if (l >= 2) v += o;
  o = dpp_f<kRowShr4, 0xf>(v);
  if (l >= 4) v += o;
  o = dpp_f<kRowShr8, 0xf>(v);
  if (l >= 8) v += o;
  o = dpp_f<kRowBcast15, 0xa>(v);
  if (row & 1) v += o;
  o = dpp_f<kRowBcast31, 0xc>(v);
  if (row >= 2) v += o;
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

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
      m = wave_max_dpp(m);
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (valid[q]) s += expf(v[q] - m);
      s = wave_sum_dpp(s);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (valid[q]) scores[(int64_t)t * E + l + kWave * q] = expf(v[q] - m) / s;
      continue;
    }
    int my_idx = -1;
    float my_val = 0.f, top = 0.f;
    for (int j = 0; j < k; ++j) {
      // this lane's best untaken candidate; lanes without one offer
      // (-inf, INT_MAX), which every real candidate ranks before
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // q ascending is index ascending: a strict '>' keeps the lower index on ties
        if (!taken[q] && (bi == 0x7fffffff || v[q] > bv)) {
          bv = v[q];
          bi = l + kWave * q;
        }
      }
      wave_argmax(bv, bi);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (bi == l + kWave * q) taken[q] = true;
      if (j == 0) top = bv;
      if (l == j) {
        my_idx = bi;
        my_val = bv;
      }
    }
    float w;
    if (routing == 0) {  // softmax over all E, read at the chosen experts
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (valid[q]) s += expf(v[q] - top);
      s = wave_sum_dpp(s);
      w = expf(my_val - top) / s;
    } else {  // softmax over the k chosen logits, added in slot order
      const float ex = (l < k) ? expf(my_val - top) : 0.f;
      float s = 0.f;
      for (int jj = 0; jj < k; ++jj) s += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), jj));
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

// Logits: 8 waves per block split the contraction over d by interleaved
// 32-wide steps (wave w takes steps w, w+8, ...).  Each wave keeps D steps of
// operand fragments in flight in a register ring (load step j+D, then
// multiply step j), so a CU holds tens of KB of x loads in flight: enough to
// stream x at HBM speed instead of waiting on one step at a time.
constexpr int kRouteBf16Threads = 512;

template <int MT, int NT>
__global__ __launch_bounds__(kRouteBf16Threads) void route_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, const float *__restrict__ bias,
    int64_t bias_stride, int T, int d, int E, int k, int routing, float *__restrict__ logits,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, float *__restrict__ scores) {
  constexpr int BT = 16 * MT, EP = 16 * NT;
  constexpr int NW = kRouteBf16Threads / kWave;
  // logits tile row pitch: 4 rows apart (the row groups of a 16x16 MFMA
  // result) land 16 banks apart, so the tile write is conflict-free
  constexpr int LD = EP + 4;
  constexpr int RED = (NW / 2) * MT * NT * kWave;  // float4s of the reduction buffer
  static_assert(BT * LD <= RED * 4 || RED == 0, "logits tile fits in the reduction buffer");
  // steps in flight per wave: as many as fit next to the accumulators in
  // about 192 registers (4 per fragment), at most 16 (with 16 tokens, 16
  // experts and d = 4096, every load of a wave is in flight at once)
  constexpr int D_FIT = (192 - 4 * MT * NT) / (4 * (MT + NT));
  constexpr int D = D_FIT < 1 ? 1 : (D_FIT > 16 ? 16 : D_FIT);
  __shared__ f32x4 red[RED];  // partial tiles, then the logits tile
  float *tile = reinterpret_cast<float *>(red);
  const int l = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
  const int t0 = blockIdx.x * BT;
  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ksteps = (d + 31) / 32;
  const int nsteps = ksteps > w ? (ksteps - w + NW - 1) / NW : 0;  // this wave's steps
  const bf16x8 zero = {};
  bf16x8 a[D][MT], b[D][NT];
  // fragments of this wave's step j (zero past the end of d or of the rows)
  auto load = [&](bf16x8 (&fa)[MT], bf16x8 (&fb)[NT], int j) {
    const int kk = (w + j * NW) * 32 + (l >> 4) * 8;
    const bool kin = j < nsteps && kk < d;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int row = t0 + m * 16 + (l & 15);
      fa[m] = (kin && row < T) ? *reinterpret_cast<const bf16x8 *>(x + (int64_t)row * d + kk) : zero;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int e = n * 16 + (l & 15);
      fb[n] = (kin && e < E) ? *reinterpret_cast<const bf16x8 *>(wr + (int64_t)e * d + kk) : zero;
    }
  };
#pragma unroll
  for (int i = 0; i < D; ++i) load(a[i], b[i], i);
  for (int j0 = 0; j0 < nsteps; j0 += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if (j0 + i < nsteps) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int n = 0; n < NT; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][m], b[i][n], acc[m][n], 0, 0, 0);
        load(a[i], b[i], j0 + i + D);
      }
    }
  }
  // Sum of the waves' partial tiles by a fixed tree (waves h..2h-1 hand
  // theirs to waves 0..h-1, h = 4, 2, 1), so the result is deterministic.
  // Partials travel in accumulator order: each lane moves whole float4s to
  // consecutive addresses.
#pragma unroll
  for (int h = NW / 2; h >= 1; h >>= 1) {
    if (w >= h && w < 2 * h) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) red[((w - h) * MT * NT + m * NT + n) * kWave + l] = acc[m][n];
    }
    __syncthreads();
    if (w < h) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[m][n] += red[(w * MT * NT + m * NT + n) * kWave + l];
    }
    __syncthreads();
  }
  if (w == 0) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) tile[(m * 16 + (l >> 4) * 4 + r) * LD + n * 16 + (l & 15)] = acc[m][n][r];
  }
  __syncthreads();
  finish_logits(tile, LD, BT, t0, T, E, bias, bias_stride, logits);
  gate_rows(tile, LD, BT, t0, T, E, k, routing, topk_idx, topk_w, scores);
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
    // Softmax scores of one expert share their top bits, so most lanes hit
    // the same bin: the lanes of a wave with equal bins are found with one
    // ballot per bin bit and only the lowest of them adds the group's count.
    for (int t0 = 0; t0 < T; t0 += blockDim.x) {
      const int t = t0 + threadIdx.x;
      const uint32_t kv = t < T ? key[t] : 0u;
      const bool match = t < T && (kv & pmask) == prefix;
      const uint32_t bin = (kv >> shift) & 255u;
      uint64_t peers = __ballot(match);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const bool bit = (bin >> b) & 1u;
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
      }
      if (match && (peers & lanemask_lt()) == 0) atomicAdd(&hist[bin], __popcll(peers));
    }
    __syncthreads();
    if (wave_id() == 0) {
      // bins from the top: lane l holds bins 255-4l .. 252-4l; a suffix
      // count over them finds the bin that holds the need-th largest key
      const int l = lane_id();
      int h[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        h[q] = hist[255 - (4 * l + q)];
        sum += h[q];
      }
      const int incl = wave_incl_scan(sum);
      const int excl = incl - sum;
      const uint64_t hit = __ballot(excl < need && need <= incl);
      // every key matching the prefix is in some bin and at least `need` of
      // them do, so one lane is hit; without a hit bin 0 is taken, as the
      // sequential search did
      const int src = hit ? __ffsll(static_cast<unsigned long long>(hit)) - 1 : kWave - 1;
      if (l == src) {
        int cum = excl, q = 0;
        for (; q < 3; ++q) {
          if (cum + h[q] >= need) break;
          cum += h[q];
        }
        sel_state[0] = static_cast<uint32_t>(255 - (4 * l + q));
        sel_state[1] = static_cast<uint32_t>(need - cum);
      }
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
    // 16*mt tokens per block: larger token tiles re-read the router weight
    // (all E rows, from L2) fewer times, as long as 256 blocks remain
    int mt = 1;
    if ((a.T + 63) / 64 >= 256 && nt <= 8) mt = 4;
    else if ((a.T + 31) / 32 >= 256 && nt <= 16) mt = 2;
    const int blocks = (a.T + 16 * mt - 1) / (16 * mt);
    const uint16_t *x = static_cast<const uint16_t *>(a.x);
    const uint16_t *wr = static_cast<const uint16_t *>(a.wr);
#define MOE_ROUTE_CASE(MT_, NT_)                                                                     \
  if (mt == MT_ && nt == NT_) {                                                                      \
    route_bf16_kernel<MT_, NT_><<<blocks, kRouteBf16Threads, 0, st>>>(x, wr, a.bias, a.bias_stride, a.T, \
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
