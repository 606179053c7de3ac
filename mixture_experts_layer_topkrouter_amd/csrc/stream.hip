// Measurement kernels (include/moe_probe.h).
//
// HBM stream kernels: a plain read, write and copy of a device buffer.  They
// measure the rates the device sustains for the access patterns of the
// HBM-bound stages (route, permute and combine are reads, writes or both of
// contiguous rows), which those stages are read against, and they are the
// known-size copy that calibrates the HBM byte counters.
//
// gfx950 design: 16-byte accesses, four in flight per thread; one workgroup
// per 16 KB of buffer, so the grid is large and each wave streams contiguous
// bytes.  Non-temporal accesses are an option (streaming data that is not
// reused); measured on one MI355X over 1 GiB: read 7.0, write 6.1, copy 6.1
// TB/s (non-temporal read and copy, plain write).
#include "../../include/moe_probe.h"
#include "common.h"

namespace moe {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;

template <bool NT>
__device__ __forceinline__ u32x4 sload(const u32x4 *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__device__ __forceinline__ void sstore(u32x4 *p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// KIND 0: read src (an XOR of every word is kept so the loads are not dead;
// it is written to sink only if it equals a value random data never gives);
// 1: write a pattern to dst; 2: copy src to dst.  Each workgroup takes one
// 16-KB run of the buffer (256 threads x 4 x 16 B, consecutive lanes on
// consecutive 16-B pieces), so every wave streams whole contiguous KB: a
// grid-stride loop over the whole buffer measured 15-25 % slower here.
template <int KIND, bool NT>
__global__ __launch_bounds__(kStreamThreads) void stream_kernel(const u32x4 *__restrict__ src,
                                                                u32x4 *__restrict__ dst, size_t n16,
                                                                uint32_t *__restrict__ sink) {
  const size_t i = static_cast<size_t>(blockIdx.x) * kStreamThreads * kStreamUnroll + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  const u32x4 pat = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, static_cast<uint32_t>(i)};
  u32x4 v[kStreamUnroll];
#pragma unroll
  for (int u = 0; u < kStreamUnroll; ++u)
    if (KIND != 1 && i + u * kStreamThreads < n16) v[u] = sload<NT>(src + i + u * kStreamThreads);
#pragma unroll
  for (int u = 0; u < kStreamUnroll; ++u) {
    const size_t j = i + u * kStreamThreads;
    if (j >= n16) break;
    if (KIND == 0) acc ^= v[u];
    else if (KIND == 1) sstore<NT>(dst + j, pat);
    else sstore<NT>(dst + j, v[u]);
  }
  if (KIND == 0 && acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u && sink) sink[0] = acc[2];
}

// Register-only matrix-core loop: wave w of workgroup b loads 8 fragments
// (16 B per lane each) from operands, then runs iters rounds of 8 MFMAs into
// 8 independent accumulators (a 128 x 64 block of 32 x 32 tiles; each
// accumulator is reused every 8 MFMAs, far past the MFMA's latency).
__global__ __launch_bounds__(256) void mfma_probe_kernel(const u32x4 *__restrict__ ops, int iters,
                                                         float *__restrict__ sink) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  const u32x4 *src = ops + static_cast<size_t>(wave) * 8 * kWave + l;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 va = src[i * kWave], vb = src[(4 + i) * kWave];
    a[i] = __builtin_bit_cast(bf16x8, va);
    b[i] = __builtin_bit_cast(bf16x8, vb);
  }
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  // two rounds per trip, the second on the other two B fragments
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[2 + j], acc[i][j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[i][j][v];
  if (s == 1234.5678f && sink) sink[wave] = s;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_mfma_probe(int32_t blocks, int32_t iters, const void *operands, void *sink,
                                     void *stream) {
  if (blocks <= 0 || iters <= 0 || !operands || (reinterpret_cast<uintptr_t>(operands) & 15))
    return MOE_ERR_INVALID_ARG;
  moe::mfma_probe_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const moe::u32x4 *>(operands), iters, static_cast<float *>(sink));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" moe_status moe_stream_probe(int32_t kind, int32_t nontemporal, const void *src, void *dst,
                                       size_t bytes, void *sink, void *stream) {
  if (kind < 0 || kind > 2 || (bytes & 15) != 0) return MOE_ERR_INVALID_ARG;
  if ((kind != 1 && !src) || (kind != 0 && !dst)) return MOE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15)) return MOE_ERR_INVALID_ARG;
  if (bytes == 0) return MOE_OK;
  using namespace moe;
  const size_t n16 = bytes / 16;
  const size_t per_block = static_cast<size_t>(kStreamThreads) * kStreamUnroll;
  const size_t nblk = (n16 + per_block - 1) / per_block;
  if (nblk > 0x7fffffffu) return MOE_ERR_UNSUPPORTED;
  const int blocks = static_cast<int>(nblk);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4 *s = static_cast<const u32x4 *>(src);
  u32x4 *d = static_cast<u32x4 *>(dst);
  uint32_t *k = static_cast<uint32_t *>(sink);
#define MOE_STREAM(K, N) stream_kernel<K, N><<<blocks, kStreamThreads, 0, st>>>(s, d, n16, k)
  if (kind == 0) { if (nontemporal) MOE_STREAM(0, true); else MOE_STREAM(0, false); }
  else if (kind == 1) { if (nontemporal) MOE_STREAM(1, true); else MOE_STREAM(1, false); }
  else { if (nontemporal) MOE_STREAM(2, true); else MOE_STREAM(2, false); }
#undef MOE_STREAM
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
