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
// * logits: bf16 MFMA 16x16x32 with fp32 accumulation.  A workgroup of four
//   waves owns 16*MT tokens and all E experts (padded to 16*NT); K advances in
//   64-wide stages that direct-to-LDS loads copy into a deep LDS ring as whole
//   128-B lines, so x streams from HBM once in full lines with tens of KB in
//   flight per CU, and the small router weight comes from L2 the same way.
//   The output tiles are dealt to the waves (when there are fewer than four,
//   the waves split the stages as well and add their partials in a fixed
//   order), so results are deterministic.
// * the gate runs on the logits tile while it is still in LDS, 16 lanes per
//   token (a DPP row), so a wave gates four tokens at once: each of the k
//   picks is a row arg-max under the order (value desc, index asc) with IEEE
//   comparisons (so -0 == +0), a strict total order, taken by four row
//   rotations; softmax sums are added in a fixed order and broadcast.
// * ExpertChoice: the scores are stored expert-major, so one workgroup per
//   expert reads its contiguous score row into LDS and finds the C-th largest
//   score by a radix select (scores are >= 0, so their bit patterns order
//   like the values) that skips the bits all keys share, then compacts the
//   chosen tokens in ascending order with block prefix sums.
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

// Gate over a tile of logits in LDS (row r = token t0 + r, row stride ld
// floats), 16 lanes per token: lane j of a DPP row (16 lanes) holds experts
// j, j+16, ..., so a wave gates four tokens at once.  Each of the k picks is
// an arg-max under (value desc, index asc) with IEEE comparisons (so
// -0 == +0), a strict total order: every lane offers its best untaken
// candidate and four row rotations (8, 4, 2, 1) leave the row's best in every
// lane of the row.  Lane j of the row keeps pick j.  Sums (softmax
// denominators) are taken in a fixed order (row shifts into lane 15) and
// broadcast from lane 15, so every slot of a token divides by the same sum.
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

__device__ __forceinline__ void row_argmax(float &v, int &i) {
#define MOE_ROW_ARGMAX_STEP(C)            \
  {                                       \
    const float ov = dpp_f<C, 0xf>(v);    \
    const int oi = dpp_i<C, 0xf>(i);      \
    if (ranks_before(ov, oi, v, i)) {     \
      v = ov;                             \
      i = oi;                             \
    }                                     \
  }
  MOE_ROW_ARGMAX_STEP(kRowRor8)
  MOE_ROW_ARGMAX_STEP(kRowRor4)
  MOE_ROW_ARGMAX_STEP(kRowRor2)
  MOE_ROW_ARGMAX_STEP(kRowRor1)
#undef MOE_ROW_ARGMAX_STEP
}

__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp_f<kRowRor8, 0xf>(v));
  v = fmaxf(v, dpp_f<kRowRor4, 0xf>(v));
  v = fmaxf(v, dpp_f<kRowRor2, 0xf>(v));
  v = fmaxf(v, dpp_f<kRowRor1, 0xf>(v));
  return v;
}

// Sum over the 16 lanes of each row in a fixed order (row shifts 1, 2, 4, 8
// into lane 15), then lane 15's value to every lane of its row (ds_swizzle,
// bit mode: lane = (lane & 0x10) | 0xf inside each half-wave).
__device__ __forceinline__ float row_sum(float v) {
  const int l = lane_id() & 15;
  float o;
  o = dpp_f<kRowShr1, 0xf>(v);
  if (l >= 1) v += o;
  o = dpp_f<kRowShr2, 0xf>(v);
  if (l >= 2) v += o;
  o = dpp_f<kRowShr4, 0xf>(v);
  if (l >= 4) v += o;
  o = dpp_f<kRowShr8, 0xf>(v);
  if (l >= 8) v += o;
  constexpr int kBcast15 = (0x10 << 0) | (0x0f << 5);  // and_mask 0x10, or_mask 0x0f, xor_mask 0
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), kBcast15));
}

// NT: values per lane (experts padded to 16 * NT).  rows tokens of the tile.
template <int NT>
__device__ __forceinline__ void gate_tile(float *tile, int ld, int rows, int t0, int T, int E, int k, int routing,
                          int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, float *__restrict__ scores) {
  const int j = lane_id() & 15;
  const int rw = wave_id() * 4 + (lane_id() >> 4);  // row of this lane group
  const int groups = (blockDim.x / kWave) * 4;
  for (int r = rw; r < rows; r += groups) {
    const int t = t0 + r;
    if (t >= T) break;  // rows ascend with r: the rest of this lane group's rows are past T too
    float *row = tile + r * ld;
    float v[NT];
    uint32_t taken = 0;  // bit q: expert j + 16q is taken (or past E)
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int e = j + 16 * q;
      v[q] = e < E ? row[e] : 0.f;
      if (e >= E) taken |= 1u << q;
    }
    if (routing == 2) {  // ExpertChoice scores: softmax over E
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < NT; ++q)
        if (!(taken >> q & 1u)) m = fmaxf(m, v[q]);
      m = row_max(m);
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < NT; ++q) {
        v[q] = (taken >> q & 1u) ? 0.f : expf(v[q] - m);
        s += v[q];
      }
      s = row_sum(s);
      // into the tile in place of the logits; store_scores_t writes them out
      // expert-major
#pragma unroll
      for (int q = 0; q < NT; ++q)
        if (!(taken >> q & 1u)) row[j + 16 * q] = v[q] / s;
      continue;
    }
    int my_idx = -1;
    float my_val = 0.f, top = 0.f;
    for (int p = 0; p < k; ++p) {
      // this lane's best untaken candidate; a lane without one offers
      // (-inf, INT_MAX), which every real candidate ranks before
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < NT; ++q) {
        // q ascending is index ascending: a strict '>' keeps the lower index on ties
        if (!(taken >> q & 1u) && (bi == 0x7fffffff || v[q] > bv)) {
          bv = v[q];
          bi = j + 16 * q;
        }
      }
      row_argmax(bv, bi);
      if ((bi & 15) == j && bi < 16 * NT) taken |= 1u << (bi >> 4);
      if (p == 0) top = bv;
      if (j == p) {
        my_idx = bi;
        my_val = bv;
      }
    }
    float w;
    if (routing == 0) {  // softmax over all E, read at the chosen experts
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < NT; ++q)
        if (j + 16 * q < E) s += expf(v[q] - top);
      s = row_sum(s);
      w = expf(my_val - top) / s;
    } else {  // softmax over the k chosen logits
      const float ex = (j < k) ? expf(my_val - top) : 0.f;
      w = ex / row_sum(ex);
    }
    if (j < k) {
      topk_idx[(int64_t)t * k + j] = my_idx;
      topk_w[(int64_t)t * k + j] = w;
    }
  }
}

// ExpertChoice scores of a tile (rows tokens, in LDS after gate_tile) to
// scores[e, t] (expert-major): consecutive threads take consecutive tokens of
// one expert, so each expert's run of the tile is one contiguous store.
template <int ROWS>
__device__ __forceinline__ void store_scores_t(const float *tile, int ld, int t0, int T, int E,
                                               float *__restrict__ scores) {
  __syncthreads();
  for (int i = threadIdx.x; i < ROWS * E; i += blockDim.x) {
    const int e = i / ROWS, r = i - (i / ROWS) * ROWS;
    if (t0 + r < T) scores[(int64_t)e * T + t0 + r] = tile[r * ld + e];
  }
}

// Adds the bias, writes the logits and leaves them in LDS for the gate.
// Thread i takes expert e = i % E of rows i / E, i / E + blockDim / E, ...
// when E divides the block (one bias load per row step, no division in the
// loop); otherwise a plain flat loop.
__device__ __forceinline__ void finish_logits(float *tile, int ld, int rows, int t0, int T, int E, const float *bias,
                                              int64_t bias_stride, float *logits) {
  const int nthr = blockDim.x;
  if (nthr % E == 0) {
    const int e = threadIdx.x % E, rstep = nthr / E;
    const float b0 = (bias && bias_stride == 0) ? bias[e] : 0.f;
    for (int r = threadIdx.x / E; r < rows; r += rstep) {
      const int t = t0 + r;
      if (t >= T) break;
      float v = tile[r * ld + e];
      if (bias) v += bias_stride == 0 ? b0 : bias[(int64_t)t * bias_stride + e];
      tile[r * ld + e] = v;
      logits[(int64_t)t * E + e] = v;
    }
  } else {
    for (int i = threadIdx.x; i < rows * E; i += nthr) {
      const int r = i / E, e = i - (i / E) * E;
      const int t = t0 + r;
      if (t >= T) continue;
      float v = tile[r * ld + e];
      if (bias) v += bias[(int64_t)t * bias_stride + e];
      tile[r * ld + e] = v;
      logits[(int64_t)t * E + e] = v;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// bf16 logits.  A workgroup of NW waves owns BT = 16*MT tokens and all E
// experts, padded to EP = 16*NT rows of W_r (padding rows repeat row E-1;
// their logits are never read).  K advances in stages of KB bytes per row
// (64 or 128 elements): a stage holds the BT x rows and the EP W_r rows,
// copied into an LDS ring of NS stages by direct-to-LDS loads
// (global_load_lds_dwordx4).  One load instruction fills 64/(KB/16) rows
// with whole 128-B lines, so the token rows stream from HBM in full lines;
// the stage for step s + NS - 1 is requested as step s starts, which keeps
// NS - 1 stages in flight per CU.  The 16-B chunk c of row r is stored at
// c ^ ((r >> 1) & 7) (128-B rows) or c ^ (r & 15) (256-B rows), so the 16
// rows a ds_read_b128 serves together fall on 16 distinct 16-B bank slots.
// MFMA 16x16x32 (bf16, fp32 accumulation): the MT x NT output tiles are
// dealt to the waves; when there are fewer tiles than waves, the waves also
// split the K stages (stage s to wave group s % KS) and their partial tiles
// are added in a fixed order.  The logits tile then goes through the bias,
// the global store and the gate while it sits in LDS.
template <int MT, int NT, int NS, int NW, int KB>
__global__ __launch_bounds__(NW * kWave) void route_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, const float *__restrict__ bias,
    int64_t bias_stride, int T, int d, int E, int k, int routing, float *__restrict__ logits,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, float *__restrict__ scores) {
  static_assert(KB == 128 || KB == 256, "128- or 256-byte rows");
  constexpr int KC = KB / 2;                        // K elements per stage
  constexpr int CPR = KB / 16;                      // 16-B chunks per row
  constexpr int RPI = kWave / CPR;                  // rows per load instruction
  constexpr int BT = 16 * MT, EP = 16 * NT;
  constexpr int ROWS = BT + EP;                     // staged rows per stage
  static_assert(BT % RPI == 0 && EP % RPI == 0, "an instruction stays inside x or W_r");
  constexpr int NI = ROWS / RPI;                    // load instructions per stage
  constexpr int LPW_LO = NI / NW, NHI = NI % NW;    // waves w < NHI issue LPW_LO + 1
  constexpr int LPW = LPW_LO + (NHI ? 1 : 0);
  static_assert((NS - 2) * LPW <= 63, "vmcnt range");
  constexpr int SB = ROWS * KB;                     // stage bytes
  constexpr int TILES = MT * NT;
  constexpr int KS = TILES >= NW ? 1 : NW / TILES;  // waves sharing a tile (K split)
  constexpr int TPW = TILES * KS / NW;              // tiles per wave
  constexpr int WG = NW / KS;                       // waves per K slice
  constexpr int LD = EP + 4;                        // logits tile row pitch (floats)
  static_assert(BT * LD * 4 <= NS * SB, "logits tile fits in the ring");
  static_assert(KS == 1 || (KS - 1) * WG * TPW * kWave * 16 <= NS * SB, "partials fit in the ring");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * SB];

  const int l = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
  const int t0 = blockIdx.x * BT;
  const int S = (d + KC - 1) / KC;                   // stages
  const int nchunk = d / 8;                          // 16-B chunks per row (d is a multiple of 8)
  const int nld = LPW_LO + (w < NHI ? 1 : 0);        // this wave's loads per stage (wave-uniform)
  auto swz = [](int r) { return KB == 128 ? (r >> 1) & 7 : r & 15; };

  // instruction i = w + NW*j covers staged rows RPI*i .. +RPI-1; lane l ->
  // row RPI*i + l/CPR, stored chunk l%CPR, which holds logical chunk
  // (l%CPR) ^ swz(row)
  const uint32_t ring_lds = lds_addr_of(ring);
  uint32_t voff[LPW];
  bool is_x[LPW];
  int lchunk[LPW];
#pragma unroll
  for (int jj = 0; jj < LPW; ++jj) {
    const int i = min(w + NW * jj, NI - 1);
    const int r = RPI * i + l / CPR;
    const int c = (l % CPR) ^ swz(r);
    lchunk[jj] = c;
    is_x[jj] = i < BT / RPI;  // wave-uniform: x rows come first
    if (r < BT) voff[jj] = static_cast<uint32_t>((min(t0 + r, T - 1) - t0) * static_cast<int64_t>(d) * 2 + c * 16);
    else voff[jj] = static_cast<uint32_t>(min(r - BT, E - 1) * static_cast<int64_t>(d) * 2 + c * 16);
  }
  const char *xb = reinterpret_cast<const char *>(x) + static_cast<int64_t>(t0) * d * 2;
  const char *wb = reinterpret_cast<const char *>(wr);
  // stage s -> ring slot s % NS; a stage whose chunks run past d (the last one
  // when d % KC != 0) reads a clamped chunk there, whose products are zeroed
  // below
  auto issue = [&](int s) {
    const uint32_t slot = ring_lds + static_cast<uint32_t>((s % NS) * SB);
    const bool tail = (s + 1) * KC > d;
#pragma unroll
    for (int jj = 0; jj < LPW; ++jj) {
      if (jj == LPW - 1 && NHI && w >= NHI) break;  // wave-uniform
      const int i = w + NW * jj;
      // with one load per wave per stage, a wave whose rows are all padding
      // rows of W_r (experts E..EP-1, whose logits are never read) skips it:
      // it then has no loads in flight, and the waits of the other waves
      // still cover every row that is read
      if constexpr (LPW == 1 && NHI == 0)
        if (!is_x[jj] && RPI * i - BT >= E) break;
      uint32_t off = voff[jj];
      if (tail) {
        const int over = s * CPR + lchunk[jj] - (nchunk - 1);  // chunks past the last real one
        if (over > 0) off -= static_cast<uint32_t>(over * 16);
      }
      dma16(off, (is_x[jj] ? xb : wb) + static_cast<int64_t>(s) * KB, slot + i * 1024);
    }
  };

  const int kslice = w / WG;
  f32x4 acc[TPW];
#pragma unroll
  for (int jj = 0; jj < TPW; ++jj) acc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int frow = l & 15;
  auto frag = [&](const uint8_t *slot, int row, int ks) -> bf16x8 {
    const int c = ks * 4 + (l >> 4);
    return *reinterpret_cast<const bf16x8 *>(slot + row * KB + ((c ^ swz(row)) << 4));
  };

  for (int s = 0; s < NS - 1 && s < S; ++s) issue(s);
  for (int s = 0; s < S; ++s) {
    if (s + NS - 2 < S) {
      if (NHI == 0 || nld == LPW) wait_vm<(NS - 2) * LPW>();
      else wait_vm<(NS - 2) * LPW_LO>();
    } else {
      wait_vm<0>();
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (s + NS - 1 < S) issue(s + NS - 1);  // refills slot (s-1) % NS: every wave is past reading it
    if (KS > 1 && s % KS != kslice) continue;
    const uint8_t *slot = ring + (s % NS) * SB;
    const bool tail = (s + 1) * KC > d;
#pragma unroll
    for (int ks = 0; ks < KC / 32; ++ks) {
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj) {
        const int q = (w % WG) + WG * jj;
        const int m = q / NT, n = q - (q / NT) * NT;
        bf16x8 a = frag(slot, m * 16 + frow, ks);
        const bf16x8 b = frag(slot, BT + n * 16 + frow, ks);
        if (tail && s * KC + (ks * 4 + (l >> 4)) * 8 >= d) a = bf16x8{};
        acc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[jj], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // the ring is free: partial tiles, then the logits tile
  float *red = reinterpret_cast<float *>(ring);
  if constexpr (KS > 1) {
    // K slices 1..KS-1 hand their partial tiles over; slice 0 adds them in
    // slice order (accumulator layout, one float4 per lane)
    if (kslice > 0) {
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj)
        reinterpret_cast<f32x4 *>(red)[(((kslice - 1) * WG + (w % WG)) * TPW + jj) * kWave + l] = acc[jj];
    }
    __syncthreads();
    if (kslice == 0) {
      for (int ksl = 1; ksl < KS; ++ksl)
#pragma unroll
        for (int jj = 0; jj < TPW; ++jj)
          acc[jj] += reinterpret_cast<const f32x4 *>(red)[(((ksl - 1) * WG + w) * TPW + jj) * kWave + l];
    }
    __syncthreads();
  }
  float *tile = red;
  if (kslice == 0) {
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) {
      const int q = (w % WG) + WG * jj;
      const int m = q / NT, n = q - (q / NT) * NT;
#pragma unroll
      for (int r = 0; r < 4; ++r) tile[(m * 16 + (l >> 4) * 4 + r) * LD + n * 16 + (l & 15)] = acc[jj][r];
    }
  }
  __syncthreads();
  finish_logits(tile, LD, BT, t0, T, E, bias, bias_stride, logits);
  gate_tile<NT>(tile, LD, BT, t0, T, E, k, routing, topk_idx, topk_w, scores);
  if (routing == 2) store_scores_t<BT>(tile, LD, t0, T, E, scores);
}

constexpr int kF32Rows = 16;

// fp32 logits: the workgroup's 16 token rows and the router's rows are
// staged through LDS in 64-wide chunks of d (coalesced loads, one memory
// round trip per chunk); thread i owns logits i, i + 256, ... of the tile
// (row i / E, expert i % E) and adds its products in d order.
constexpr int kF32Chunk = 64;

template <int NT>
__global__ __launch_bounds__(kRouteThreads) void route_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    int64_t bias_stride, int T, int d, int E, int k, int routing, float *__restrict__ logits,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, float *__restrict__ scores) {
  constexpr int DC = kF32Chunk;
  __shared__ float tile[kF32Rows * 256];
  __shared__ float sx[kF32Rows][DC + 1];
  __shared__ float sw[16 * NT][DC + 1];
  const int t0 = blockIdx.x * kF32Rows;
  float acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = 0.f;
  for (int c0 = 0; c0 < d; c0 += DC) {
    const int n = min(DC, d - c0);
    __syncthreads();  // every thread is done with the previous chunk
    for (int q = threadIdx.x; q < kF32Rows * DC; q += kRouteThreads) {
      const int r = q / DC, kk = q - (q / DC) * DC;
      sx[r][kk] = (t0 + r < T && kk < n) ? x[static_cast<int64_t>(t0 + r) * d + c0 + kk] : 0.f;
    }
    for (int q = threadIdx.x; q < E * DC; q += kRouteThreads) {
      const int e = q / DC, kk = q - (q / DC) * DC;
      sw[e][kk] = kk < n ? wr[static_cast<int64_t>(e) * d + c0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int i = threadIdx.x + j * kRouteThreads;
      if (i >= kF32Rows * E) continue;
      const int r = i / E, e = i - (i / E) * E;
      if (t0 + r >= T) continue;
      for (int kk = 0; kk < n; ++kk) acc[j] = fmaf(sx[r][kk], sw[e][kk], acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int i = threadIdx.x + j * kRouteThreads;
    if (i < kF32Rows * E) tile[(i / E) * E + i % E] = t0 + i / E < T ? acc[j] : 0.f;
  }
  __syncthreads();
  finish_logits(tile, E, kF32Rows, t0, T, E, bias, bias_stride, logits);
  gate_tile<NT>(tile, E, kF32Rows, t0, T, E, k, routing, topk_idx, topk_w, scores);
  if (routing == 2) store_scores_t<kF32Rows>(tile, E, t0, T, E, scores);
}

// Gate only: the logits are an input.
template <int NT>
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
  gate_tile<NT>(tile, E, kF32Rows, t0, T, E, k, routing, topk_idx, topk_w, scores);
  if (routing == 2) store_scores_t<kF32Rows>(tile, E, t0, T, E, scores);
}

constexpr int kEcThreads = 1024;

// ExpertChoice selection, one workgroup per expert e: the C tokens with the
// largest scores[e, t] (equal scores: lower token), in ascending token order.
// The expert's score row is contiguous (expert-major scores) and is read
// once into LDS as 32-bit keys; scores are >= 0, so their bit patterns order
// like the values.  The C-th largest key is found by a radix select from the
// top, up to 11 bits per pass.  While the row is read, every key already
// goes into the histogram of bits [19, 30) (the first digit when every key
// is below 2.0, i.e. bit 30 and up are clear, as for softmax scores, and
// the keys differ in a bit at or above 22); otherwise the bits every key
// shares (block-wide AND and OR) are skipped and the first digit is
// histogrammed again below them.  The keys of the first pass's threshold
// digit are copied to a candidate list (keys above it are selected
// outright), in any order, since the later passes only count them; those
// passes, over the candidates only, run in wave 0 alone (no workgroup
// barriers) while the list fits kEcWaveCand entries.
// Finally the tokens whose key is above the threshold, and the lowest tokens
// whose key equals it, are compacted in ascending token order.
constexpr int kEcDigitBits = 11;
constexpr int kEcBins = 1 << kEcDigitBits;
constexpr int kEcFusedShift = 19;      // the histogram taken while reading: bits [19, 30)
constexpr int kEcWaveCand = 4096;      // later passes in one wave up to this many candidates

// The digit (histogram of kEcBins bins in LDS) that holds the need-th
// largest key, found by one wave from the top: lane l first sums the 32 bins
// bins-1-32l .. bins-32-32l (eight 16-B reads), a wave scan of the sums
// picks the lane whose group holds it, then lane q (< 32) takes bin
// bins-1-32src-q of that group and a second scan picks the bin.  Returns the
// digit and the rank of the wanted key inside it (every lane).
__device__ __forceinline__ void ec_find_digit(const int *hist, int need, int *digit, int *rank) {
  const int l = lane_id();
  const int lo = kEcBins - 32 * (l + 1);  // this lane's group: bins lo .. lo+31
  int sum = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int4 v = *reinterpret_cast<const int4 *>(hist + lo + 4 * q);
    sum += v.x + v.y + v.z + v.w;
  }
  const int incl = wave_incl_scan(sum);
  const int excl = incl - sum;
  const uint64_t hit = __ballot(excl < need && need <= incl);
  const int src = hit ? __ffsll(static_cast<unsigned long long>(hit)) - 1 : kWave - 1;
  const int base = __builtin_amdgcn_readlane(excl, src);
  const int bin = kEcBins - 1 - 32 * src - l;  // lanes 0..31: the group's bins from the top
  const int h = l < 32 ? hist[bin] : 0;
  const int c = wave_incl_scan(h) + base;
  const uint64_t hit2 = __ballot(l < 32 && c - h < need && need <= c);
  const int q = hit2 ? __ffsll(static_cast<unsigned long long>(hit2)) - 1 : 31;
  *digit = __builtin_amdgcn_readlane(bin, q);
  *rank = need - __builtin_amdgcn_readlane(c - h, q);
}

// Thread i's run of entries [b0, b1) of src[0, n), runs of a multiple of 4
// entries (at most kEcPer), read with 16-B LDS loads into v (entries past
// the run hold whatever follows in the array, which the kEcMaxTokens bound
// keeps inside it).
constexpr int kEcPer = kEcMaxTokens / kEcThreads;
static_assert(kEcPer % 4 == 0, "runs of whole 16-B loads");
__device__ __forceinline__ void load_run(const uint32_t *src, int n, uint32_t (&v)[kEcPer], int *b0, int *b1) {
  const int per = ((n + kEcThreads - 1) / kEcThreads + 3) & ~3;
  *b0 = min(n, static_cast<int>(threadIdx.x) * per);
  *b1 = min(n, *b0 + per);
  const int at = static_cast<int>(threadIdx.x) * per;  // at + per <= kEcMaxTokens
#pragma unroll
  for (int q = 0; q < kEcPer; q += 4) {
    if (q < per) {
      const u32x4 w = *reinterpret_cast<const u32x4 *>(src + at + q);
      v[q] = w[0];
      v[q + 1] = w[1];
      v[q + 2] = w[2];
      v[q + 3] = w[3];
    } else {
      v[q] = v[q + 1] = v[q + 2] = v[q + 3] = 0u;
    }
  }
}

// LDS operations of one wave complete in order; this makes the compiler keep
// them in order too and waits for them (a wave-only "barrier").
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__global__ __launch_bounds__(kEcThreads) void ec_select_kernel(const float *__restrict__ scores, int T,
                                                               int E, int C, int32_t *__restrict__ ec_token,
                                                               float *__restrict__ ec_w) {
  __shared__ __attribute__((aligned(16))) uint32_t key[kEcMaxTokens];
  __shared__ __attribute__((aligned(16))) uint32_t cand[kEcMaxTokens];
  __shared__ __attribute__((aligned(16))) int hist[kEcBins];
  __shared__ int scan_tmp[kEcThreads / kWave + 1];
  __shared__ uint32_t red[2][kEcThreads / kWave];
  __shared__ uint32_t sel_state[3];
  __shared__ int ncand;
  const int e = blockIdx.x;
  const int nw = kEcThreads / kWave;
  const float *row = scores + (int64_t)e * T;
  for (int i = threadIdx.x; i < kEcBins; i += kEcThreads) hist[i] = 0;
  if (threadIdx.x == 0) ncand = 0;
  __syncthreads();  // the histogram is clear before the first key goes in
  uint32_t kand = ~0u, kor = 0u;
  constexpr uint32_t kFusedMask = kEcBins - 1;
  if ((T & 3) == 0 && (reinterpret_cast<uintptr_t>(row) & 15) == 0) {
    for (int i = threadIdx.x; i < T / 4; i += kEcThreads) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(row + 4 * i);
      *reinterpret_cast<u32x4 *>(key + 4 * i) = v;
      kand &= v[0] & v[1] & v[2] & v[3];
      kor |= v[0] | v[1] | v[2] | v[3];
#pragma unroll
      for (int q = 0; q < 4; ++q) atomicAdd(&hist[(v[q] >> kEcFusedShift) & kFusedMask], 1);
    }
  } else {
    for (int t = threadIdx.x; t < T; t += kEcThreads) {
      const uint32_t v = __float_as_uint(row[t]);
      key[t] = v;
      kand &= v;
      kor |= v;
      atomicAdd(&hist[(v >> kEcFusedShift) & kFusedMask], 1);
    }
  }
  // block-wide AND / OR (exact in any order)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kand &= static_cast<uint32_t>(__shfl_xor(static_cast<int>(kand), o, kWave));
    kor |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(kor), o, kWave));
  }
  if (lane_id() == 0) {
    red[0][wave_id()] = kand;
    red[1][wave_id()] = kor;
  }
  __syncthreads();
  kand = ~0u;
  kor = 0u;
  for (int i = 0; i < nw; ++i) {
    kand &= red[0][i];
    kor |= red[1][i];
  }
  const uint32_t diff = kand ^ kor;  // bits where keys differ
  // bits at and above `pos` are shared by every key (and already in `prefix`)
  int pos = diff ? 32 - __clz(static_cast<int>(diff)) : 0;
  const bool fused = (kor >> (kEcFusedShift + kEcDigitBits)) == 0 && pos > kEcFusedShift + 3;
  if (fused) pos = kEcFusedShift + kEcDigitBits;
  uint32_t prefix = pos >= 32 ? 0u : (kand >> pos) << pos;
  int need = C;  // rank (1-based, from the top) of the wanted key among those matching the prefix
  if (!fused) {
    for (int i = threadIdx.x; i < kEcBins; i += kEcThreads) hist[i] = 0;
    __syncthreads();
  }
  // first pass over every key (its histogram already taken when fused)
  if (pos > 0) {
    const int wbits = pos < kEcDigitBits ? pos : kEcDigitBits;
    const int shift = pos - wbits;
    const uint32_t dmask = (1u << wbits) - 1u;
    if (!fused) {
      for (int i = threadIdx.x; i < T; i += kEcThreads) atomicAdd(&hist[(key[i] >> shift) & dmask], 1);
      __syncthreads();
    }
    if (wave_id() == 0) {
      int digit, rank;
      ec_find_digit(hist, need, &digit, &rank);
      if (lane_id() == 0) {
        sel_state[0] = static_cast<uint32_t>(digit);
        sel_state[1] = static_cast<uint32_t>(rank);
      }
    }
    __syncthreads();
    const uint32_t digit = sel_state[0];
    need = static_cast<int>(sel_state[1]);
    prefix |= digit << shift;
    for (int i = threadIdx.x; i < kEcBins; i += kEcThreads) hist[i] = 0;
    if (shift > 0) {
      // the keys of the threshold digit become the candidates, in any order
      // (the later passes only count them): each wave appends its kept keys
      // at a place taken with one LDS atomic
      for (int i0 = 0; i0 < T; i0 += kEcThreads) {
        const int i = i0 + static_cast<int>(threadIdx.x);
        const uint32_t kv = i < T ? key[i] : 0u;
        const bool keep = i < T && ((kv >> shift) & dmask) == digit;
        const uint64_t b = __ballot(keep);
        if (b) {
          int base = 0;
          if (lane_id() == 0) base = atomicAdd(&ncand, __popcll(b));
          base = __shfl(base, 0, kWave);
          if (keep) cand[base + __popcll(b & lanemask_lt())] = kv;
        }
      }
    }
    pos = shift;
    __syncthreads();
  }
  // later passes over the candidates
  const int n0 = ncand;
  if (pos > 0 && n0 <= kEcWaveCand) {
    // wave 0 alone: LDS histogram, digit search and in-place compaction
    // (chunks of 64 in order: a chunk's writes land at or below its reads)
    if (wave_id() == 0) {
      const int l = lane_id();
      int n = n0;
      while (pos > 0) {
        const int wbits = pos < kEcDigitBits ? pos : kEcDigitBits;
        const int shift = pos - wbits;
        const uint32_t dmask = (1u << wbits) - 1u;
        for (int i = l; i < n; i += kWave) atomicAdd(&hist[(cand[i] >> shift) & dmask], 1);
        wave_lds_sync();
        int digit, rank;
        ec_find_digit(hist, need, &digit, &rank);
        need = rank;
        prefix |= static_cast<uint32_t>(digit) << shift;
        wave_lds_sync();
        for (int i = l; i < n; i += kWave) hist[(cand[i] >> shift) & dmask] = 0;  // only the bins used
        if (shift > 0) {
          int o = 0;
          for (int i0 = 0; i0 < n; i0 += kWave) {
            const int i = i0 + l;
            const uint32_t kv = i < n ? cand[i] : 0u;
            const bool keep = i < n && ((kv >> shift) & dmask) == static_cast<uint32_t>(digit);
            const uint64_t b = __ballot(keep);
            wave_lds_sync();  // every lane has read its entry before any writes
            if (keep) cand[o + __popcll(b & lanemask_lt())] = kv;
            o += __popcll(b);
          }
          n = o;
        }
        wave_lds_sync();
        pos = shift;
      }
      if (l == 0) {
        sel_state[1] = static_cast<uint32_t>(need);
        sel_state[2] = prefix;
      }
    }
    __syncthreads();
    need = static_cast<int>(sel_state[1]);
    prefix = sel_state[2];
  } else {
    bool first = true;
    while (pos > 0) {
      const int wbits = pos < kEcDigitBits ? pos : kEcDigitBits;
      const int shift = pos - wbits;
      const uint32_t dmask = (1u << wbits) - 1u;
      const int n = first ? n0 : ncand;
      for (int i = threadIdx.x; i < n; i += kEcThreads) atomicAdd(&hist[(cand[i] >> shift) & dmask], 1);
      __syncthreads();
      if (wave_id() == 0) {
        int digit, rank;
        ec_find_digit(hist, need, &digit, &rank);
        if (lane_id() == 0) {
          sel_state[0] = static_cast<uint32_t>(digit);
          sel_state[1] = static_cast<uint32_t>(rank);
        }
      }
      __syncthreads();
      const uint32_t digit = sel_state[0];
      need = static_cast<int>(sel_state[1]);
      prefix |= digit << shift;
      for (int i = threadIdx.x; i < kEcBins; i += kEcThreads) hist[i] = 0;
      if (shift > 0) {
        // in place: the scan's barriers put every read before any write
        uint32_t mine[kEcPer];
        int b0, b1;
        load_run(cand, n, mine, &b0, &b1);
        int kept = 0;
#pragma unroll
        for (int q = 0; q < kEcPer; ++q) kept += (b0 + q < b1 && ((mine[q] >> shift) & dmask) == digit);
        int total;
        int o = block_excl_scan(kept, scan_tmp, &total);
#pragma unroll
        for (int q = 0; q < kEcPer; ++q)
          if (b0 + q < b1 && ((mine[q] >> shift) & dmask) == digit) cand[o++] = mine[q];
        if (threadIdx.x == 0) ncand = total;
      }
      first = false;
      pos = shift;
      __syncthreads();
    }
  }
  // prefix is the C-th largest key; `need` of the keys equal to it are taken
  // (the lowest tokens), every key above it is taken.  Each thread takes a
  // run of consecutive tokens; one block scan of the packed pair (keys above,
  // keys equal) gives every selected token its position: the keys above
  // before it plus min(keys equal before it, need).
  uint32_t mine[kEcPer];
  int b0, b1;
  load_run(key, T, mine, &b0, &b1);
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int q = 0; q < kEcPer; ++q) {
    n_gt += b0 + q < b1 && mine[q] > prefix;
    n_eq += b0 + q < b1 && mine[q] == prefix;
  }
  int tot;
  const int packed = block_excl_scan((n_gt << 16) | n_eq, scan_tmp, &tot);  // T <= 16384 < 2^16
  int gt = packed >> 16, eq = packed & 0xffff;
#pragma unroll
  for (int q = 0; q < kEcPer; ++q) {
    if (b0 + q >= b1) break;
    const uint32_t kv = mine[q];
    if (kv > prefix) {
      const int p = gt + min(eq, need);
      ec_token[(int64_t)e * C + p] = b0 + q;
      ec_w[(int64_t)e * C + p] = __uint_as_float(kv);
      ++gt;
    } else if (kv == prefix) {
      if (eq < need) {
        const int p = gt + eq;
        ec_token[(int64_t)e * C + p] = b0 + q;
        ec_w[(int64_t)e * C + p] = __uint_as_float(kv);
      }
      ++eq;
    }
  }
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  int nt = 1;
  while (nt * 16 < a.E) nt <<= 1;
  if (a.x == nullptr) {
    const int blocks = (a.T + kF32Rows - 1) / kF32Rows;
#define MOE_GATE_CASE(NT_)                                                                                  \
  if (nt == NT_)                                                                                           \
    gate_only_kernel<NT_><<<blocks, kRouteThreads, 0, st>>>(a.logits, a.T, a.E, a.k, a.routing, a.topk_idx, \
                                                             a.topk_w, a.scores);
    MOE_GATE_CASE(1) MOE_GATE_CASE(2) MOE_GATE_CASE(4) MOE_GATE_CASE(8) MOE_GATE_CASE(16)
#undef MOE_GATE_CASE
  } else if (a.dtype == 0) {
    const int blocks = (a.T + kF32Rows - 1) / kF32Rows;
#define MOE_F32_CASE(NT_)                                                                              \
  if (nt == NT_)                                                                                      \
    route_f32_kernel<NT_><<<blocks, kRouteThreads, 0, st>>>(                                          \
        static_cast<const float *>(a.x), static_cast<const float *>(a.wr), a.bias, a.bias_stride, a.T, \
        a.d, a.E, a.k, a.routing, a.logits, a.topk_idx, a.topk_w, a.scores);
    MOE_F32_CASE(1) MOE_F32_CASE(2) MOE_F32_CASE(4) MOE_F32_CASE(8) MOE_F32_CASE(16)
#undef MOE_F32_CASE
  } else {
    // 16*mt tokens per workgroup; 64 when that still gives a workgroup to
    // every CU, since each workgroup streams all of W_r once
    int mt = nt == 1 ? 1 : 2;
    if (nt >= 2 && nt <= 8 && (a.T + 63) / 64 >= 256) mt = 4;
    const int blocks = (a.T + 16 * mt - 1) / (16 * mt);
    const uint16_t *x = static_cast<const uint16_t *>(a.x);
    const uint16_t *wr = static_cast<const uint16_t *>(a.wr);
    // 8 waves, 256-B staged rows (measured on the 8-, 64- and 128-expert
    // workloads: 12.7 / 12.1 / 14.7 us against 15.2 / 17.2 / 18.0 us with 4
    // waves and 128-B rows); 64-token tiles over 128 experts keep 128-B rows,
    // whose deeper ring measured faster there (14.0 us); the ring holds
    // 128-144 KB of LDS (one workgroup per CU)
#define MOE_ROUTE_CASE(MT_, NT_, NS_, KB_)                                                                   \
  if (mt == MT_ && nt == NT_) {                                                                             \
    route_bf16_kernel<MT_, NT_, NS_, 8, KB_><<<blocks, 8 * kWave, 0, st>>>(                                 \
        x, wr, a.bias, a.bias_stride, a.T, a.d, a.E, a.k, a.routing, a.logits, a.topk_idx, a.topk_w, a.scores); \
  }
    MOE_ROUTE_CASE(1, 1, 16, 256) MOE_ROUTE_CASE(2, 2, 8, 256) MOE_ROUTE_CASE(2, 4, 6, 256)
    MOE_ROUTE_CASE(2, 8, 3, 256) MOE_ROUTE_CASE(2, 16, 2, 256) MOE_ROUTE_CASE(4, 2, 6, 256)
    MOE_ROUTE_CASE(4, 4, 4, 256) MOE_ROUTE_CASE(4, 8, 6, 128)
#undef MOE_ROUTE_CASE
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.routing != 2) return err;
  ec_select_kernel<<<a.E, kEcThreads, 0, st>>>(a.scores, a.T, a.E, a.C, a.ec_token, a.ec_w);
  return hipGetLastError();
}

}  // namespace moe
