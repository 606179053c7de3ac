// token_unpermutation: gather each token's expert outputs and take their
// gate-weighted sum (plus the shared expert's output).
//
// "How MegaDLMs Implements Mixture of Experts (MoE) Architectures", sections
// "Core MoE Layer Architecture" (MoELayer step 3: unpermutation rebuilds the
// sequence from the expert outputs) and "Token Dispatching and
// Communication" (token_unpermutation); "Expert Parallelism > Key
// Parameters", capacity_factor paragraph (a dropped assignment adds nothing).
//
// gfx950 design: one wave per token; each lane owns 16-byte column chunks of
// the output row, accumulates w * y_perm[row] in fp32 over the token's slots
// in slot order (a fixed order, so the result is deterministic), adds the
// shared expert's row and rounds once.  Every load and store is a 16-byte
// vector access to a contiguous row, so the pass is a pure HBM stream.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokens = kThreads / kWave;

template <bool BF16>
__global__ __launch_bounds__(kThreads) void combine_kernel(const void *__restrict__ y_perm_,
                                                           const int32_t *__restrict__ tok_ptr,
                                                           const int32_t *__restrict__ slot_row,
                                                           const float *__restrict__ slot_w,
                                                           const void *__restrict__ y_shared_,
                                                           void *__restrict__ y_, int T, int d, int k,
                                                           int64_t rows, int64_t nslots) {
  constexpr int kElems = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int t = blockIdx.x * kTokens + wave_id();
  if (t >= T) return;
  const int l = lane_id();
  // slot ranges and rows come from device memory: clamp them to the buffers
  const int64_t s0 = tok_ptr ? min(max(static_cast<int64_t>(tok_ptr[t]), static_cast<int64_t>(0)), nslots)
                             : static_cast<int64_t>(t) * k;
  const int64_t s1 = tok_ptr ? min(max(static_cast<int64_t>(tok_ptr[t + 1]), s0), nslots)
                             : static_cast<int64_t>(t) * k + k;
  const size_t row_bytes = static_cast<size_t>(d) * (BF16 ? 2 : 4);
  const uint8_t *y_perm = static_cast<const uint8_t *>(y_perm_);
  const uint8_t *y_shared = static_cast<const uint8_t *>(y_shared_);
  uint8_t *y = static_cast<uint8_t *>(y_);
  const int nchunk = d / kElems;
  for (int c = l; c < nchunk; c += kWave) {
    float acc[kElems];
#pragma unroll
    for (int i = 0; i < kElems; ++i) acc[i] = 0.f;
    for (int64_t s = s0; s < s1; ++s) {
      const int row = slot_row[s];
      if (row < 0 || row >= rows) continue;
      const float w = slot_w[s];
      const u32x4 v = ld16(y_perm + static_cast<size_t>(row) * row_bytes + static_cast<size_t>(c) * 16);
      if (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(w, __uint_as_float(v[i] << 16), acc[2 * i]);
          acc[2 * i + 1] = fmaf(w, __uint_as_float(v[i] & 0xffff0000u), acc[2 * i + 1]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, __uint_as_float(v[i]), acc[i]);
      }
    }
    const size_t off = static_cast<size_t>(t) * row_bytes + static_cast<size_t>(c) * 16;
    if (y_shared) {
      const u32x4 v = ld16(y_shared + off);
      if (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += __uint_as_float(v[i] << 16);
          acc[2 * i + 1] += __uint_as_float(v[i] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += __uint_as_float(v[i]);
      }
    }
    u32x4 o;
    if (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = static_cast<uint32_t>(f32_to_bf16(acc[2 * i])) |
               (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1])) << 16);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(acc[i]);
    }
    st16(y + off, o);
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const int blocks = (a.T + kTokens - 1) / kTokens;
  if (a.dtype == 1)
    combine_kernel<true><<<blocks, kThreads, 0, st>>>(a.y_perm, a.tok_ptr, a.slot_row, a.slot_w, a.y_shared,
                                                      a.y, a.T, a.d, a.k, a.rows, a.nslots);
  else
    combine_kernel<false><<<blocks, kThreads, 0, st>>>(a.y_perm, a.tok_ptr, a.slot_row, a.slot_w, a.y_shared,
                                                       a.y, a.T, a.d, a.k, a.rows, a.nslots);
  return hipGetLastError();
}

}  // namespace moe
