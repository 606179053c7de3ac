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

// DPP lane moves (gfx9 encodings): row_shr:n (0x110 + n) shifts inside rows
// of 16 lanes; row_bcast:15 carries lane 15 of rows 0 and 2 into rows 1 and
// 3, row_bcast:31 carries lane 31 into rows 2 and 3.  A lane whose source
// lane does not exist, or whose row is outside ROWS, keeps its own value.
// A few cycles each, where a cross-lane shuffle is an LDS-crossbar round trip.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp_move(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes of a wave (integer, exact; every
// lane of the wave must be active): prefix sums inside each row of 16 by
// row shifts 1, 2, 4, 8, then the row totals carried up by the broadcasts.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = lane_id() & 15, row = lane_id() >> 4;
  int o = dpp_move<kDppRowShr1>(v);
  if (l >= 1) v += o;
  o = dpp_move<kDppRowShr2>(v);
  if (l >= 2) v += o;
  o = dpp_move<kDppRowShr4>(v);
  if (l >= 4) v += o;
  o = dpp_move<kDppRowShr8>(v);
  if (l >= 8) v += o;
  o = dpp_move<kDppRowBcast15, 0xa>(v);
  if (row & 1) v += o;
  o = dpp_move<kDppRowBcast31, 0xc>(v);
  if (row >= 2) v += o;
  return v;
}

// Sum over the 64 lanes (integer, exact), the same in every lane.
__device__ __forceinline__ int wave_sum_int(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), kWave - 1);
}

// Exclusive prefix sum over a whole block (blockDim.x threads, multiple of 64,
// at most 1024).  `tmp` needs blockDim.x/64 + 1 ints of LDS.  Returns the
// exclusive prefix; *total gets the block sum.
__device__ __forceinline__ int block_excl_scan(int v, int *tmp, int *total) {
  const int nw = blockDim.x / kWave;
  const int inc = wave_incl_scan(v);
  if (lane_id() == kWave - 1) tmp[wave_id()] = inc;
  __syncthreads();
  // every wave scans the per-wave totals itself (lane w holds wave w's)
  const int l = lane_id();
  const int wt = l < nw ? tmp[l] : 0;
  const int wi = wave_incl_scan(wt);
  const int before = __builtin_amdgcn_readlane(wi - wt, __builtin_amdgcn_readfirstlane(wave_id()));
  *total = __builtin_amdgcn_readlane(wi, nw - 1);
  __syncthreads();  // tmp may be reused at once
  return before + inc - v;
}

// the direct-to-LDS loads name M0, which the compiler reserves (it uses M0
// nowhere else in these kernels)
#pragma clang diagnostic ignored "-Winline-asm"

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from global memory straight into LDS at
// lds_addr + 16 * lane.  Written as inline asm so the compiler's wait-count
// pass does not see it: that pass cannot always tell which ring slot an LDS
// read touches and would then drain every load in flight before the read.
// The kernel orders these loads itself (explicit vmcnt waits + barriers).
// The instruction has no register result; M0 carries the LDS address and
// needs one wait state after it is written.  The global address is a
// wave-uniform base in SGPRs plus a 32-bit per-lane byte offset, so advancing
// a stage is scalar arithmetic and each lane keeps one VGPR per load stream.
__device__ __forceinline__ void dma16(uint32_t voff, const void *sbase, uint32_t lds_addr) {
  // the LDS address is wave-uniform; readfirstlane puts it in an SGPR for M0
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0v)
               : "memory", "m0");
}

// The same with the non-temporal hint: for a stream read once (expert
// weights no other workgroup shares), which then does not push reused data
// out of the caches.
__device__ __forceinline__ void dma16_nt(uint32_t voff, const void *sbase, uint32_t lds_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(m0v)
               : "memory", "m0");
}

// The same 16-byte direct-to-LDS load issued as a range-checked buffer load
// (MUBUF, raw: stride 0, num_records = kDmaRange bytes from sbase): a lane
// whose offset is kDmaSkip reads no memory and its 16 LDS bytes are written
// as zeros.  Rows a GEMM tile holds past its last real row load this way, so
// they multiply as zeros instead of as copies of a real row: the results of
// the real rows are the same, but a matrix core fed zeros draws less power,
// and this power-limited card then runs a higher clock.  Every real offset
// must stay below kDmaRange (the host bounds the widths accordingly).
constexpr uint32_t kDmaRange = 0x80000000u;
constexpr uint32_t kDmaSkip = 0x80000000u;
__device__ __forceinline__ void dma16_zp(uint32_t voff, const void *sbase, uint32_t lds_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  const uint64_t b = reinterpret_cast<uint64_t>(sbase);
  // words: base[31:0]; base[47:32] with stride 0; num_records; the gfx9
  // raw-buffer format word (32-bit data format, no swizzle, no index add)
  const u32x4 rsrc = {static_cast<uint32_t>(b), static_cast<uint32_t>(b >> 32), kDmaRange, 0x00020000u};
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "s"(m0v)
               : "memory", "m0");
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr_of(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t *)p));
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace

// 16-byte global load/store helpers.
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

}  // namespace moe
