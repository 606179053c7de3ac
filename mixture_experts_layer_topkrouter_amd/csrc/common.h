// Internal helpers shared by the gfx950 kernels of the MoE library.
// Not part of the C ABI (that is include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// A value every lane holds the same copy of, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  return (static_cast<uint64_t>(1) << lane_id()) - 1;
}

// Inclusive prefix sum over the 64 lanes of a wave (integer, exact).
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int n = __shfl_up(v, o, kWave);
    if (l >= o) v += n;
  }
  return v;
}

// Exclusive prefix sum over a whole block (blockDim.x threads, multiple of 64,
// at most 1024).  `tmp` needs blockDim.x/64 + 1 ints of LDS.  Returns the
// exclusive prefix; *total gets the block sum.
__device__ __forceinline__ int block_excl_scan(int v, int *tmp, int *total) {
  const int nw = blockDim.x / kWave;
  int inc = wave_incl_scan(v);
  if (lane_id() == kWave - 1) tmp[wave_id()] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      int c = tmp[w];
      tmp[w] = run;
      run += c;
    }
    tmp[nw] = run;
  }
  __syncthreads();
  int r = tmp[wave_id()] + inc - v;
  *total = tmp[nw];
  __syncthreads();
  return r;
}

// 16-byte global load/store helpers.
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

}  // namespace moe
