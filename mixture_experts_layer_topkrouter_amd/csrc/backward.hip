// Backward pass of the MoE block: everything except the fast grouped GEMMs
// (those are in gemm.hip).
//
// "How MegaDLMs Implements Mixture of Experts (MoE) Architectures", section
// "Activation Checkpointing and Constraints": the layer is trained, and its
// recompute mode re-runs the forward inside the backward pass.  Here the
// expert pre-activations are recomputed from the permuted tokens rather than
// kept from the forward.  The choice of experts (top-k, ExpertChoice
// selection, capacity drops) is held fixed; gradients flow through the gate
// weights (section "Routing Mechanisms": softmax over the router logits), the
// expert FFNs and the router's linear layer.
//
// Layout.  The backward keeps the routed rows expert-major like the forward,
// but each expert's block starts on a multiple of 32 rows (padded offsets
// poff) and its pad rows are zero.  The weight-gradient GEMMs contract over an
// expert's rows, so with the padding every expert's contraction is a whole
// number of 32-row K stages and needs no masking; pad rows add exact zeros.
//
// gfx950 design of the kernels here: every pass over token rows is one wave
// per token with 16-byte accesses (HBM streams, as in the forward's combine);
// reductions over a row are wave butterflies in a fixed order, so results are
// deterministic.  The generic grouped GEMM covers the layouts and dtypes the
// direct-to-LDS MFMA kernels do not (fp32, or contraction lengths that are
// not a multiple of 32): a plain 64 x 64 LDS-tiled FMA kernel.
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kTokens = kThreads / kWave;  // kThreads: gemm_common.h

template <bool BF16>
__device__ __forceinline__ void unpack(const u32x4 &v, float (&f)[BF16 ? 8 : 4]) {
  if (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
}

template <bool BF16>
__device__ __forceinline__ u32x4 pack(const float (&f)[BF16 ? 8 : 4]) {
  u32x4 o;
  if (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = static_cast<uint32_t>(f32_to_bf16(f[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(f[2 * i + 1])) << 16);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(f[i]);
  }
  return o;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Slots of token t: [t*k, t*k+k) for top-k, [tok_ptr[t], tok_ptr[t+1]) for
// ExpertChoice (clamped to the slot arrays).
__device__ __forceinline__ void token_slots(const int32_t *tok_ptr, int t, int k, int64_t nslots, int64_t *s0,
                                            int64_t *s1) {
  if (tok_ptr) {
    const int64_t a = min(max(static_cast<int64_t>(tok_ptr[t]), static_cast<int64_t>(0)), nslots);
    *s0 = uniform64(a);
    *s1 = uniform64(min(max(static_cast<int64_t>(tok_ptr[t + 1]), a), nslots));
  } else {
    *s0 = uniform64(static_cast<int64_t>(t) * k);
    *s1 = uniform64(static_cast<int64_t>(t) * k + k);
  }
}

// Padded offsets: poff[e+1] = poff[e] + (count_e rounded up to 32).
__global__ __launch_bounds__(kThreads) void bwd_offsets_kernel(const int32_t *__restrict__ count, int E,
                                                               int64_t max_rows, int32_t *__restrict__ poff,
                                                               const int32_t *__restrict__ stamp,
                                                               int32_t *__restrict__ roff) {
  __shared__ int tmp[kThreads / kWave + 1];
  const bool none = roff && *stamp == kStampTrain;  // saved pre-activations: nothing to recompute
  int carry = 0;
  for (int e0 = 0; e0 < E; e0 += kThreads) {
    const int e = e0 + threadIdx.x;
    int c = 0;
    if (e < E) c = static_cast<int>(min(max(static_cast<int64_t>(count[e]), static_cast<int64_t>(0)), max_rows));
    const int v = (c + kPadRows - 1) / kPadRows * kPadRows;
    int total;
    const int ex = block_excl_scan(v, tmp, &total);
    if (e < E) poff[e] = carry + ex;
    if (roff && e < E) roff[e] = none ? 0 : carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) poff[E] = carry;
  if (roff && threadIdx.x == 0) roff[E] = none ? 0 : carry;
}

// Backward of the combine (token_unpermutation), one wave per token.  For
// each kept slot s of token t (row r of expert e, gate weight w):
//   d_slot_w[s] = <dy[t], y_perm[r]>        (dL/dw, fp32, fixed order)
//   dyp[p]      = w * dy[t]                  (the expert's output gradient)
//   xp[p]       = x[t]                       (the expert's input, for the
//                                             recomputed forward)
// with p = r - offset[e] + poff[e]; slot_prow[s] = p, or -1 (and
// d_slot_w = 0) for a dropped slot.
template <bool BF16, int CPL>
__global__ __launch_bounds__(kThreads) void unpermute_bwd_kernel(BwdUnpermuteArgs a) {
  constexpr int kElems = BF16 ? 8 : 4;
  const int t = blockIdx.x * kTokens + wave_id();
  if (t >= a.T) return;
  const int l = lane_id();
  int64_t s0, s1;
  token_slots(a.tok_ptr, t, a.k, a.nslots, &s0, &s1);
  const size_t row_bytes = static_cast<size_t>(a.d) * (BF16 ? 2 : 4);
  const int nchunk = a.d / kElems;
  const uint8_t *dy = static_cast<const uint8_t *>(a.dy) + static_cast<size_t>(t) * row_bytes;
  const uint8_t *x = static_cast<const uint8_t *>(a.x) + static_cast<size_t>(t) * row_bytes;
  for (int64_t s = s0; s < s1; ++s) {
    const int r = __builtin_amdgcn_readfirstlane(a.slot_row[s]);
    int e = -1;
    if (r >= 0 && r < a.rows) e = a.ec_capacity > 0 ? r / a.ec_capacity : a.topk_idx[s];
    e = __builtin_amdgcn_readfirstlane(e);
    int p = -1;
    if (e >= 0 && e < a.E) p = r - a.offs[e] + a.poff[e];
    p = __builtin_amdgcn_readfirstlane(p);
    if (p < 0 || p >= a.prows) {
      if (l == 0) {
        a.d_slot_w[s] = 0.f;
        a.slot_prow[s] = -1;
      }
      continue;
    }
    const float w = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.slot_w[s])));
    const uint8_t *yp = static_cast<const uint8_t *>(a.y_perm) + static_cast<size_t>(r) * row_bytes;
    uint8_t *dyp = static_cast<uint8_t *>(a.dyp) + static_cast<size_t>(p) * row_bytes;
    uint8_t *xp = static_cast<uint8_t *>(a.xp) + static_cast<size_t>(p) * row_bytes;
    float dot = 0.f;
    for (int c0 = 0; c0 < nchunk; c0 += CPL * kWave) {
      u32x4 vd[CPL], vy[CPL], vx[CPL];
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = c0 + u * kWave + l;
        const bool in = c < nchunk;
        vd[u] = in ? ld16(dy + static_cast<size_t>(c) * 16) : u32x4{0u, 0u, 0u, 0u};
        vy[u] = in ? ld16(yp + static_cast<size_t>(c) * 16) : u32x4{0u, 0u, 0u, 0u};
        vx[u] = in ? ld16(x + static_cast<size_t>(c) * 16) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = c0 + u * kWave + l;
        if (c >= nchunk) continue;
        float fd[kElems], fy[kElems];
        unpack<BF16>(vd[u], fd);
        unpack<BF16>(vy[u], fy);
#pragma unroll
        for (int i = 0; i < kElems; ++i) {
          dot = fmaf(fd[i], fy[i], dot);
          fd[i] *= w;
        }
        st16(dyp + static_cast<size_t>(c) * 16, pack<BF16>(fd));
        st16(xp + static_cast<size_t>(c) * 16, vx[u]);
      }
    }
    dot = wave_sum(dot);
    if (l == 0) {
      a.d_slot_w[s] = dot;
      a.slot_prow[s] = p;
      if (a.prow_src) a.prow_src[p] = r;
    }
  }
}

// Zero the pad rows [poff[e] + count_e, poff[e+1]) of each expert's block in
// up to two row buffers (one workgroup per expert).
__global__ __launch_bounds__(kThreads) void pad_zero_kernel(const int32_t *__restrict__ poff,
                                                            const int32_t *__restrict__ count, int64_t prows,
                                                            size_t row_bytes, void *b0, void *b1,
                                                            int32_t *__restrict__ prow_src) {
  const int e = blockIdx.x;
  const int64_t p0 = min(max(static_cast<int64_t>(poff[e]), static_cast<int64_t>(0)), prows);
  const int64_t p1 = min(max(static_cast<int64_t>(poff[e + 1]), p0), prows);
  const int64_t first = min(p0 + max(count[e], 0), p1);
  if (prow_src)
    for (int64_t r = first + threadIdx.x; r < p1; r += blockDim.x) prow_src[r] = -1;
  const int64_t nch = static_cast<int64_t>(row_bytes / 16);
  const int64_t n = (p1 - first) * nch;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const size_t off = static_cast<size_t>(first) * row_bytes + static_cast<size_t>(i) * 16;
    if (b0) st16(static_cast<uint8_t *>(b0) + off, u32x4{0u, 0u, 0u, 0u});
    if (b1) st16(static_cast<uint8_t *>(b1) + off, u32x4{0u, 0u, 0u, 0u});
  }
}

// dst[r] = src[r] for r < rows, 0 for rows <= r < prows (row_bytes each).
__global__ __launch_bounds__(kThreads) void pad_copy_kernel(const void *__restrict__ src, void *__restrict__ dst,
                                                            int64_t rows, int64_t prows, size_t row_bytes) {
  const int64_t nch = static_cast<int64_t>(row_bytes / 16);
  const int64_t n = prows * nch, live = rows * nch;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const u32x4 v = i < live ? ld16(static_cast<const uint8_t *>(src) + i * 16) : u32x4{0u, 0u, 0u, 0u};
    st16(static_cast<uint8_t *>(dst) + i * 16, v);
  }
}

// dL/dlogits for one token per wave ("Routing Mechanisms": softmax over the
// router logits; the choice of experts held fixed).  Lane l owns experts l,
// l+64, l+128, l+192.
//   SOFTMAX_ALL:  w_j = p[idx_j], p = softmax(l): g_e = sum of dL/dw_j over
//                 the slots choosing e; dl_e = p_e (g_e - sum_i p_i g_i).
//   SOFTMAX_TOPK: w = softmax over the chosen logits (the forward's weights):
//                 dl[idx_j] = w_j (dL/dw_j - sum_i w_i dL/dw_i), others 0.
//   ExpertChoice: S = softmax(l) (the forward's scores), g_e = dL/dw of the
//                 row expert e took for this token, dl_e = S_e (g_e - sum S g).
__global__ __launch_bounds__(kThreads) void router_bwd_kernel(RouterBwdArgs a) {
  const int t = blockIdx.x * kTokens + wave_id();
  if (t >= a.T) return;
  const int l = lane_id();
  const int E = a.E;
  float v[4], g[4];
  bool in[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = l + kWave * q;
    in[q] = e < E;
    g[q] = 0.f;
    v[q] = 0.f;
  }
  int64_t s0, s1;
  token_slots(a.tok_ptr, t, a.k, a.nslots, &s0, &s1);
  if (a.routing == 1) {  // SOFTMAX_TOPK
    float s = 0.f;
    for (int64_t j = s0; j < s1; ++j) s += a.topk_w[j] * a.d_slot_w[j];
    for (int64_t j = s0; j < s1; ++j) {
      const int e = a.topk_idx[j];
      const float d = a.topk_w[j] * (a.d_slot_w[j] - s);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (e == l + kWave * q) g[q] += d;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (in[q]) a.dlogits[static_cast<int64_t>(t) * E + l + kWave * q] = g[q];
    return;
  }
  // the per-expert gradient of the weights g_e
  for (int64_t j = s0; j < s1; ++j) {
    int e;
    if (a.routing == 2) {
      const int r = a.slot_row[j];
      e = (r >= 0 && a.ec_capacity > 0) ? r / a.ec_capacity : -1;
    } else {
      e = a.topk_idx[j];
    }
    const float d = a.d_slot_w[j];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (e == l + kWave * q) g[q] += d;
  }
  // the probabilities: softmax of the logits (SOFTMAX_ALL) or the forward's
  // scores (ExpertChoice)
  if (a.routing == 2) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (in[q]) v[q] = a.scores[static_cast<int64_t>(l + kWave * q) * a.T + t];  // expert-major
  } else {
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (in[q]) {
        v[q] = a.logits[static_cast<int64_t>(t) * E + l + kWave * q];
        m = fmaxf(m, v[q]);
      }
    m = wave_max(m);
    float z = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (in[q]) {
        v[q] = expf(v[q] - m);
        z += v[q];
      }
    z = wave_sum(z);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = in[q] ? v[q] / z : 0.f;
  }
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) s += v[q] * g[q];
  s = wave_sum(s);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (in[q]) a.dlogits[static_cast<int64_t>(t) * E + l + kWave * q] = v[q] * (g[q] - s);
}

__device__ __forceinline__ float gelu_f(float z) { return 0.5f * z * (1.f + erff(z * 0.70710678118654752f)); }
// d/dz [z Phi(z)] = Phi(z) + z phi(z)
__device__ __forceinline__ float gelu_grad_f(float z) {
  return 0.5f * (1.f + erff(z * 0.70710678118654752f)) + z * 0.39894228040143268f * expf(-0.5f * z * z);
}
// bf16 data: the sigmoid from the hardware base-2 exponential and reciprocal
// (about 1 ulp each, far below bf16 rounding; measured on the Mixtral slice:
// act_fwd 131 -> 122 us, act_bwd unchanged at ~255 us, which is HBM-bound).
// fp32 data keeps expf and an IEEE divide.
template <bool FAST>
__device__ __forceinline__ float sigmoid_t(float z) {
  if constexpr (FAST) return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(z * -1.44269504088896341f));
  else return 1.f / (1.f + expf(-z));
}

// Activation backward on rows [0, rows_of) of the padded layout:
//   GELU:   z -> dz = dh * gelu'(z),         dh -> h = gelu(z)
//   SwiGLU: (a, b) -> (dh * b * silu'(a), dh * silu(a)),  dh -> h = silu(a) b
// z is [rows, n_up*dff] (SwiGLU: gate columns, then up columns), dh [rows, dff].
// The pre-activations are read from z itself (in place), or, when z_src is
// given, from row src_row(p) of z_src (the forward's saved z): src[p] when a
// map is given (-1: a pad row, whose z is 0), else p itself for p < src_rows.
// With `stamp` given, z_src is used only when *stamp == kStampTrain (the
// forward that filled it was a training forward); otherwise z holds the
// recomputed pre-activations and is read in place.
template <bool BF16, int ACT>
__global__ __launch_bounds__(kThreads) void act_bwd_kernel(void *__restrict__ z, void *__restrict__ dh,
                                                           const int32_t *__restrict__ rows_of, int64_t prows,
                                                           int dff, const void *__restrict__ z_src,
                                                           const int32_t *__restrict__ src, int64_t src_rows,
                                                           const int32_t *__restrict__ stamp) {
  constexpr int kElems = BF16 ? 8 : 4;
  if (z_src && stamp && *stamp != kStampTrain) z_src = nullptr;
  const int64_t rows = min(max(static_cast<int64_t>(*rows_of), static_cast<int64_t>(0)), prows);
  const int nch = dff / kElems;
  const int64_t n = rows * nch;
  const int n_up = ACT == ACT_SWIGLU ? 2 : 1;
  const size_t es = BF16 ? 2 : 4;
  const size_t zrow = static_cast<size_t>(n_up) * dff * es;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = i / nch;
    const int c = static_cast<int>(i - r * nch);
    uint8_t *zr = static_cast<uint8_t *>(z) + static_cast<size_t>(r) * zrow;
    uint8_t *dr = static_cast<uint8_t *>(dh) + static_cast<size_t>(r) * dff * es;
    const uint8_t *zin = zr;
    bool live = true;
    if (z_src) {
      const int64_t q = src ? static_cast<int64_t>(src[r]) : (r < src_rows ? r : -1);
      live = q >= 0 && q < src_rows;
      zin = static_cast<const uint8_t *>(z_src) + static_cast<size_t>(live ? q : 0) * zrow;
    }
    float fa[kElems], fg[kElems];
    unpack<BF16>(live ? ld16(zin + static_cast<size_t>(c) * 16) : u32x4{0u, 0u, 0u, 0u}, fa);
    unpack<BF16>(ld16(dr + static_cast<size_t>(c) * 16), fg);
    if (ACT == ACT_SWIGLU) {
      float fb[kElems], da[kElems], db[kElems], h[kElems];
      unpack<BF16>(live ? ld16(zin + static_cast<size_t>(dff) * es + static_cast<size_t>(c) * 16)
                        : u32x4{0u, 0u, 0u, 0u},
                   fb);
#pragma unroll
      for (int q = 0; q < kElems; ++q) {
        const float sg = sigmoid_t<BF16>(fa[q]);
        const float si = fa[q] * sg;
        da[q] = fg[q] * fb[q] * (sg + fa[q] * sg * (1.f - sg));
        db[q] = fg[q] * si;
        h[q] = si * fb[q];
      }
      st16(zr + static_cast<size_t>(c) * 16, pack<BF16>(da));
      st16(zr + static_cast<size_t>(dff) * es + static_cast<size_t>(c) * 16, pack<BF16>(db));
      st16(dr + static_cast<size_t>(c) * 16, pack<BF16>(h));
    } else {
      float dz[kElems], h[kElems];
#pragma unroll
      for (int q = 0; q < kElems; ++q) {
        dz[q] = fg[q] * gelu_grad_f(fa[q]);
        h[q] = gelu_f(fa[q]);
      }
      st16(zr + static_cast<size_t>(c) * 16, pack<BF16>(dz));
      st16(dr + static_cast<size_t>(c) * 16, pack<BF16>(h));
    }
  }
}

// Activation of a training forward (the expert GEMM1 wrote its raw
// pre-activations z, which the backward reuses): rows [0, rows_of),
//   GELU: h = gelu(z);  SwiGLU: h = silu(a) * b  (z = [a | b]).
template <bool BF16, int ACT>
__global__ __launch_bounds__(kThreads) void act_fwd_kernel(const void *__restrict__ z, void *__restrict__ h,
                                                           const int32_t *__restrict__ rows_of, int64_t max_rows,
                                                           int dff) {
  constexpr int kElems = BF16 ? 8 : 4;
  const int64_t rows = min(max(static_cast<int64_t>(*rows_of), static_cast<int64_t>(0)), max_rows);
  const int nch = dff / kElems;
  const int64_t n = rows * nch;
  const int n_up = ACT == ACT_SWIGLU ? 2 : 1;
  const size_t es = BF16 ? 2 : 4;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = i / nch;
    const int c = static_cast<int>(i - r * nch);
    const uint8_t *zr = static_cast<const uint8_t *>(z) + static_cast<size_t>(r) * n_up * dff * es;
    float fa[kElems], out[kElems];
    unpack<BF16>(ld16(zr + static_cast<size_t>(c) * 16), fa);
    if (ACT == ACT_SWIGLU) {
      float fb[kElems];
      unpack<BF16>(ld16(zr + static_cast<size_t>(dff) * es + static_cast<size_t>(c) * 16), fb);
#pragma unroll
      for (int q = 0; q < kElems; ++q) out[q] = fa[q] * sigmoid_t<BF16>(fa[q]) * fb[q];
    } else {
#pragma unroll
      for (int q = 0; q < kElems; ++q) out[q] = gelu_f(fa[q]);
    }
    st16(static_cast<uint8_t *>(h) + (static_cast<size_t>(r) * dff + static_cast<size_t>(c) * kElems) * es,
         pack<BF16>(out));
  }
}

// dx[t] = sum over t's kept slots, in slot order, of dxp[slot_prow[s]]
//         (+ dx_router[t], fp32) (+ dx_shared[t]); fp32 accumulation, one
// rounding.  One wave per token (the backward of the permutation: each
// token gathers back the gradients of its copies).
template <bool BF16, int CPL>
__global__ __launch_bounds__(kThreads) void gather_dx_kernel(GatherDxArgs a) {
  constexpr int kElems = BF16 ? 8 : 4;
  const int t = blockIdx.x * kTokens + wave_id();
  if (t >= a.T) return;
  const int l = lane_id();
  int64_t s0, s1;
  token_slots(a.tok_ptr, t, a.k, a.nslots, &s0, &s1);
  const size_t row_bytes = static_cast<size_t>(a.d) * (BF16 ? 2 : 4);
  const int nchunk = a.d / kElems;
  for (int c0 = 0; c0 < nchunk; c0 += CPL * kWave) {
    float acc[CPL][kElems];
#pragma unroll
    for (int u = 0; u < CPL; ++u)
#pragma unroll
      for (int i = 0; i < kElems; ++i) acc[u][i] = 0.f;
    for (int64_t s = s0; s < s1; ++s) {
      const int p = __builtin_amdgcn_readfirstlane(a.slot_prow[s]);
      if (p < 0 || p >= a.prows) continue;
      const uint8_t *src = static_cast<const uint8_t *>(a.dxp) + static_cast<size_t>(p) * row_bytes;
      u32x4 v[CPL];
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = c0 + u * kWave + l;
        v[u] = c < nchunk ? ld16(src + static_cast<size_t>(c) * 16) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        float f[kElems];
        unpack<BF16>(v[u], f);
#pragma unroll
        for (int i = 0; i < kElems; ++i) acc[u][i] += f[i];
      }
    }
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = c0 + u * kWave + l;
      if (c >= nchunk) continue;
      if (a.dx_router) {
        const float *rr = a.dx_router + static_cast<size_t>(t) * a.d + static_cast<size_t>(c) * kElems;
#pragma unroll
        for (int i = 0; i < kElems; i += 4) {
          const u32x4 v = ld16(rr + i);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[u][i + q] += __uint_as_float(v[q]);
        }
      }
      if (a.dx_shared) {
        float f[kElems];
        unpack<BF16>(ld16(static_cast<const uint8_t *>(a.dx_shared) + static_cast<size_t>(t) * row_bytes +
                          static_cast<size_t>(c) * 16),
                     f);
#pragma unroll
        for (int i = 0; i < kElems; ++i) acc[u][i] += f[i];
      }
      st16(static_cast<uint8_t *>(a.dx) + static_cast<size_t>(t) * row_bytes + static_cast<size_t>(c) * 16,
           pack<BF16>(acc[u]));
    }
  }
}

// out[j] = sum over g < groups of part[g * n + j] (fixed order), in dtype.
template <typename TC>
__global__ __launch_bounds__(kThreads) void sum_partials_kernel(const float *__restrict__ part, int groups, int64_t n,
                                                                void *__restrict__ out) {
  for (int64_t j = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; j < n;
       j += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float s = 0.f;
    for (int g = 0; g < groups; ++g) s += part[static_cast<int64_t>(g) * n + j];
    if constexpr (sizeof(TC) == 2) static_cast<uint16_t *>(out)[j] = f32_to_bf16(s);
    else static_cast<float *>(out)[j] = s;
  }
}

__global__ __launch_bounds__(kThreads) void zero_kernel(void *__restrict__ p, int64_t n16) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n16;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    st16(static_cast<uint8_t *>(p) + i * 16, u32x4{0u, 0u, 0u, 0u});
}

// ---------------------------------------------------------------------------
// Generic grouped GEMM: C(r, c) = sum_k A(r, k) B(k, c) with arbitrary element
// strides, fp32 FMA on 64 x 64 tiles (256 threads, 4 x 4 outputs each) over
// K steps of 16 staged in LDS.  Mode 0: groups of rows (rows of expert e are
// [offs[e], offs[e+1]), B per expert); mode 1: groups of K (expert e
// contracts over [offs[e], offs[e+1]), C per expert).
constexpr int GT = 64, GK = 16;

template <typename T>
__device__ __forceinline__ float load_el(const void *p, int64_t i) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
  else return static_cast<const float *>(p)[i];
}

template <typename TA, typename TB, typename TC>
__global__ __launch_bounds__(kThreads) void gemm_generic_kernel(GenGemmArgs g) {
  __shared__ float sA[GK][GT + 4], sB[GK][GT + 4];
  int e, row0, rows, nt, k0, k1;
  int64_t c_base = 0;
  if (g.mode == 0) {
    if (!map_tile<GT>(g.offs, g.E, g.max_rows, g.n_tiles, &e, &row0, &rows, &nt)) return;
    k0 = 0;
    k1 = g.K;
  } else {
    const int per = g.m_tiles * g.n_tiles;
    const int bid = blockIdx.x;
    e = bid / per;
    if (e >= g.E) return;
    const int q = bid - e * per;
    const int mt = q / g.n_tiles;
    nt = q - mt * g.n_tiles;
    row0 = mt * GT;
    rows = min(GT, g.M - row0);
    if (g.offs) {
      int me;
      expert_rows(g.offs, e, g.max_rows, &k0, &me);
      k1 = k0 + me;
    } else {  // uniform chunks of kchunk contraction rows
      k0 = static_cast<int>(min(static_cast<int64_t>(e) * g.kchunk, g.max_rows));
      k1 = static_cast<int>(min(static_cast<int64_t>(k0) + g.kchunk, g.max_rows));
    }
    c_base = static_cast<int64_t>(e) * g.c_es;
  }
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int col0 = nt * GT;
  const int64_t b_base = g.mode == 0 ? static_cast<int64_t>(e) * g.b_es : 0;
  float acc[4][4] = {};
  for (int kb = k0; kb < k1; kb += GK) {
    // stage A (GT rows x GK) and B (GK x GT columns)
    for (int i = tid; i < GT * GK; i += kThreads) {
      const int r = i / GK, kk = i % GK;
      const int k = kb + kk;
      float va = 0.f;
      if (r < rows && k < k1) va = load_el<TA>(g.A, static_cast<int64_t>(row0 + r) * g.a_rs + static_cast<int64_t>(k) * g.a_ks);
      sA[kk][r] = va;
      const int c = i % GT, kk2 = i / GT;
      const int k2 = kb + kk2;
      float vb = 0.f;
      if (col0 + c < g.N && k2 < k1)
        vb = load_el<TB>(g.B, b_base + static_cast<int64_t>(k2) * g.b_ks + static_cast<int64_t>(col0 + c) * g.b_cs);
      sB[kk2][c] = vb;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < GK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    if (r >= rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = col0 + tx * 4 + j;
      if (c >= g.N) continue;
      const int64_t o = c_base + static_cast<int64_t>(row0 + r) * g.c_rs + c;
      if constexpr (sizeof(TC) == 2) static_cast<uint16_t *>(g.C)[o] = f32_to_bf16(acc[i][j]);
      else static_cast<float *>(g.C)[o] = acc[i][j];
    }
  }
}

template <bool BF16>
void launch_unpermute_bwd(const BwdUnpermuteArgs &a, int blocks, hipStream_t st) {
  const int nchunk = a.d / (BF16 ? 8 : 4);
  const int per_lane = (nchunk + kWave - 1) / kWave;
  if (per_lane <= 1) unpermute_bwd_kernel<BF16, 1><<<blocks, kThreads, 0, st>>>(a);
  else if (per_lane <= 2) unpermute_bwd_kernel<BF16, 2><<<blocks, kThreads, 0, st>>>(a);
  else unpermute_bwd_kernel<BF16, 4><<<blocks, kThreads, 0, st>>>(a);
}

template <bool BF16>
void launch_gather_dx(const GatherDxArgs &a, int blocks, hipStream_t st) {
  const int nchunk = a.d / (BF16 ? 8 : 4);
  const int per_lane = (nchunk + kWave - 1) / kWave;
  if (per_lane <= 1) gather_dx_kernel<BF16, 1><<<blocks, kThreads, 0, st>>>(a);
  else if (per_lane <= 2) gather_dx_kernel<BF16, 2><<<blocks, kThreads, 0, st>>>(a);
  else if (per_lane <= 4) gather_dx_kernel<BF16, 4><<<blocks, kThreads, 0, st>>>(a);
  else gather_dx_kernel<BF16, 8><<<blocks, kThreads, 0, st>>>(a);
}

int stream_blocks(int64_t items) {
  const int64_t b = (items + kThreads - 1) / kThreads;
  return static_cast<int>(max(static_cast<int64_t>(1), min(b, static_cast<int64_t>(4096))));
}

}  // namespace

hipError_t launch_bwd_offsets(const int32_t *count, int E, int64_t max_rows, int32_t *poff, hipStream_t st,
                              const int32_t *stamp, int32_t *roff) {
  bwd_offsets_kernel<<<1, kThreads, 0, st>>>(count, E, max_rows, poff, stamp, stamp ? roff : nullptr);
  return hipGetLastError();
}

hipError_t launch_unpermute_bwd(const BwdUnpermuteArgs &a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const int blocks = (a.T + kTokens - 1) / kTokens;
  if (a.dtype == 1) launch_unpermute_bwd<true>(a, blocks, st);
  else launch_unpermute_bwd<false>(a, blocks, st);
  return hipGetLastError();
}

hipError_t launch_pad_zero(const int32_t *poff, const int32_t *count, int E, int64_t prows, size_t row_bytes,
                           void *b0, void *b1, int32_t *prow_src, hipStream_t st) {
  pad_zero_kernel<<<E, kThreads, 0, st>>>(poff, count, prows, row_bytes, b0, b1, prow_src);
  return hipGetLastError();
}

hipError_t launch_pad_copy(const void *src, void *dst, int64_t rows, int64_t prows, size_t row_bytes,
                           hipStream_t st) {
  if (prows == 0) return hipSuccess;
  pad_copy_kernel<<<stream_blocks(prows * static_cast<int64_t>(row_bytes / 16)), kThreads, 0, st>>>(
      src, dst, rows, prows, row_bytes);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const RouterBwdArgs &a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  router_bwd_kernel<<<(a.T + kTokens - 1) / kTokens, kThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_act_bwd(int dtype, int act, void *z, void *dh, const int32_t *rows_of, int64_t prows, int dff,
                          const void *z_src, const int32_t *src, int64_t src_rows, hipStream_t st,
                          const int32_t *stamp) {
  if (prows == 0) return hipSuccess;
  const int blocks = stream_blocks(prows * (dff / (dtype == 1 ? 8 : 4)));
#define MOE_ACTB(B, A) act_bwd_kernel<B, A><<<blocks, kThreads, 0, st>>>(z, dh, rows_of, prows, dff, z_src, src, src_rows, stamp)
  if (dtype == 1) {
    if (act == ACT_SWIGLU) MOE_ACTB(true, ACT_SWIGLU);
    else MOE_ACTB(true, ACT_GELU);
  } else {
    if (act == ACT_SWIGLU) MOE_ACTB(false, ACT_SWIGLU);
    else MOE_ACTB(false, ACT_GELU);
  }
#undef MOE_ACTB
  return hipGetLastError();
}

hipError_t launch_act_fwd(int dtype, int act, const void *z, void *h, const int32_t *rows_of, int64_t max_rows,
                          int dff, hipStream_t st) {
  if (max_rows == 0) return hipSuccess;
  const int blocks = stream_blocks(max_rows * (dff / (dtype == 1 ? 8 : 4)));
#define MOE_ACTF(B, A) act_fwd_kernel<B, A><<<blocks, kThreads, 0, st>>>(z, h, rows_of, max_rows, dff)
  if (dtype == 1) {
    if (act == ACT_SWIGLU) MOE_ACTF(true, ACT_SWIGLU);
    else MOE_ACTF(true, ACT_GELU);
  } else {
    if (act == ACT_SWIGLU) MOE_ACTF(false, ACT_SWIGLU);
    else MOE_ACTF(false, ACT_GELU);
  }
#undef MOE_ACTF
  return hipGetLastError();
}

hipError_t launch_gather_dx(const GatherDxArgs &a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const int blocks = (a.T + kTokens - 1) / kTokens;
  if (a.dtype == 1) launch_gather_dx<true>(a, blocks, st);
  else launch_gather_dx<false>(a, blocks, st);
  return hipGetLastError();
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  zero_kernel<<<stream_blocks(n16), kThreads, 0, st>>>(p, n16);
  return hipGetLastError();
}

int64_t gen_gemm_blocks(const GenGemmArgs &g) {
  if (g.mode == 0) {
    const int64_t mt = (g.max_rows + GT - 1) / GT + g.E;
    return mt * g.n_tiles;
  }
  return static_cast<int64_t>(g.E) * g.m_tiles * g.n_tiles;
}

hipError_t launch_gemm_generic(GenGemmArgs g, int a_dt, int b_dt, int c_dt, hipStream_t st) {
  if (g.N <= 0 || (g.mode == 1 && g.M <= 0)) return hipSuccess;
  g.n_tiles = (g.N + GT - 1) / GT;
  g.m_tiles = g.mode == 1 ? (g.M + GT - 1) / GT : 0;
  const int64_t blocks = gen_gemm_blocks(g);
  if (blocks <= 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
#define MOE_GEN(TA, TB, TC) gemm_generic_kernel<TA, TB, TC><<<grid, kThreads, 0, st>>>(g)
  if (a_dt == 1 && b_dt == 1 && c_dt == 1) MOE_GEN(uint16_t, uint16_t, uint16_t);
  else if (a_dt == 0 && b_dt == 0 && c_dt == 0) MOE_GEN(float, float, float);
  else if (a_dt == 0 && b_dt == 1 && c_dt == 0) MOE_GEN(float, uint16_t, float);
  else if (a_dt == 0 && b_dt == 1 && c_dt == 1) MOE_GEN(float, uint16_t, uint16_t);
  else if (a_dt == 0 && b_dt == 0 && c_dt == 1) MOE_GEN(float, float, uint16_t);
  else return hipErrorInvalidValue;
#undef MOE_GEN
  return hipGetLastError();
}

hipError_t launch_sum_partials(const float *part, int groups, int64_t n, int c_dt, void *out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (c_dt == 1) sum_partials_kernel<uint16_t><<<stream_blocks(n), kThreads, 0, st>>>(part, groups, n, out);
  else sum_partials_kernel<float><<<stream_blocks(n), kThreads, 0, st>>>(part, groups, n, out);
  return hipGetLastError();
}

}  // namespace moe
