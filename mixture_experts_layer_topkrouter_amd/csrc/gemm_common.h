// Internal to the grouped expert GEMM kernels (gemm.hip, gemm_skinny.hip):
// their parameter block, activations, the device-side block -> tile mapping
// and the direct-to-LDS load helpers.  Not part of the C ABI.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kThreads = 256;
constexpr int BK = 64;
constexpr int BN = 256;  // B rows per tile
constexpr int kGroupM = 8;  // most row tiles per group (see find_tile)

enum { ACT_NONE = 0, ACT_GELU = 1, ACT_SWIGLU = 2 };

struct GemmParams {
  const void *A;
  int64_t lda;  // A: [rows, K]
  const void *B;
  int64_t ldb, b_stride;  // B: per expert [Nb, K]
  void *C;
  int64_t ldc;  // C: [rows, n_out]
  const int32_t *offs;
  int E, K, n_out, up_off;
  int64_t max_rows;
  int m_tiles, n_tiles;
  // bf16 kernels: `units` workgroups make one round (one per CU); a K split
  // needs max_split > 1 and room for the fp32 partial tiles of every piece
  // (`slots` of them at part: 256 x 256 for the main kernel, bm x 256 for
  // the skinny one).
  float *part;
  int units, slots, max_split;
  // backward layouts of the 256-row kernel: C of group e starts c_stride
  // elements after group e-1's and has m_rows rows (groups of K)
  int64_t c_stride;
  int m_rows;
  // forward (NT) only: B is in the packed tile-major order of
  // launch_pack_weights (b_stride then counts the packed elements of one
  // expert; ldb and up_off are not used)
  int packed;
  // forward (NT) only, bf16: A is read / C is written K-blocked (row r,
  // column k at ((k / 32) * max_rows + r) * 32 + k % 32; lda / ldc unused)
  int a_kb, c_kb;
};

// Element index of (row, col) in an output: row-major with pitch ldc, or
// K-blocked over max_rows rows.
__device__ __forceinline__ int64_t c_index(const GemmParams &p, int64_t row, int col) {
  return p.c_kb ? (static_cast<int64_t>(col >> 5) * p.max_rows + row) * 32 + (col & 31) : row * p.ldc + col;
}

// K-blocked activations ([K/32][rows][32] bf16): the 32-wide K slice of
// consecutive rows is contiguous, so a tile's K stage is one contiguous run
// of 64-B row pieces whatever row the tile starts on.
constexpr int kKbRowBytes = 64;

// Packed weights: per expert, per column tile of BN weight rows (SwiGLU: the
// tile's BN/2 gate rows, then the matching BN/2 up rows), per 32-wide slice
// of K, one block of BN x 32 bf16 = 16 KB in the order the 256-row kernel's
// LDS stage holds it (16-B chunk q: row q/4, K chunk (q%4) ^ ((q/16)%4)).
// Rows past n_out are zero.
constexpr int kPackK = 32;
constexpr int kPackBlockBytes = BN * kPackK * 2;

namespace {

__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.f + erff(z * 0.70710678118654752f)); }
__device__ __forceinline__ float silu(float z) { return z / (1.f + expf(-z)); }
// The bf16 epilogues' SiLU: sigmoid from the hardware base-2 exponential and
// reciprocal (about 1 ulp each, far below bf16 rounding), a fraction of the
// cost of expf and an IEEE divide.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(z * -1.44269504088896341f));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed bf16 (round to nearest even; gfx950's
// v_cvt_pk_bf16_f32), lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Accumulator values of a 32x32 MFMA tile reach memory as rows.  Value
// 4g+t of lane l sits at row 8g + 4(l/32) + t, column l%32, so for each g a
// lane holds a 4-row slice of one column.  quad_rows() transposes these 4x4
// blocks inside each lane quad: lane s of a quad returns row 4(..)+s of its
// group at the quad's four columns, as 4 packed bf16 (8 bytes, memory order).
// Two exchanges with neighbour lanes (DPP quad permutations) and byte
// permutes; every lane of the wave must execute it.
__device__ __forceinline__ u32x2 quad_rows(float f0, float f1, float f2, float f3) {
  const int l = static_cast<int>(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
  // pairs: lanes 2m, 2m+1 (columns c, c+1) swap so that the even lane keeps
  // rows t = 0, 2 and the odd lane rows 1, 3, each at both columns
  const uint32_t p0 = pack_bf16x2(f0, f1), p1 = pack_bf16x2(f2, f3);
  const uint32_t q0 = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(p0), 0xB1, 0xF, 0xF, false));
  const uint32_t q1 = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(p1), 0xB1, 0xF, 0xF, false));
  const uint32_t sel = (l & 1) ? 0x03020706u : 0x05040100u;  // odd: (q.hi, p.hi); even: (p.lo, q.lo)
  const uint32_t r0 = __builtin_amdgcn_perm(q0, p0, sel);
  const uint32_t r1 = __builtin_amdgcn_perm(q1, p1, sel);
  // lanes s, s^2 (column pairs 0-1 and 2-3) swap one row each
  const bool upper = (l & 2) != 0;
  const uint32_t send = upper ? r0 : r1;
  const uint32_t recv = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(send), 0x4E, 0xF, 0xF, false));
  return upper ? u32x2{recv, r1} : u32x2{r0, recv};
}

// Block -> tile for the grouped GEMMs is done by every wave on its own (no
// LDS): the grid is an upper bound on the tile count and the real count
// follows from the device-side expert offsets.
//
// Rows of expert e, clamped to the buffer so a bad offset cannot address
// outside it.
__device__ __forceinline__ void expert_rows(const int32_t *__restrict__ offs, int e, int64_t max_rows, int *o0,
                                            int *me) {
  const int64_t a0 = min(max(static_cast<int64_t>(offs[e]), static_cast<int64_t>(0)), max_rows);
  const int64_t a1 = min(max(static_cast<int64_t>(offs[e + 1]), a0), max_rows);
  *o0 = static_cast<int>(a0);
  *me = static_cast<int>(a1 - a0);
}

// Real row tiles over all experts (every lane gets the same count).
template <int BM>
__device__ __forceinline__ int count_mtiles(const int32_t *__restrict__ offs, int E, int64_t max_rows) {
  const int l = lane_id();
  int m_tiles = 0;
  for (int e0 = 0; e0 < E; e0 += kWave) {
    int o0 = 0, me = 0;
    if (e0 + l < E) expert_rows(offs, e0 + l, max_rows, &o0, &me);
    m_tiles += wave_sum_int((me + BM - 1) / BM);
  }
  // the same in every lane; readfirstlane lets the compiler treat everything
  // derived from it (and the branches on it) as wave-uniform
  return __builtin_amdgcn_readfirstlane(m_tiles);
}

// Block ids are dispatched to the 8 XCDs round-robin; this remaps id b of
// [0, n) so that each XCD walks a contiguous run of tile indices.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int xcd = b & 7, slot = b >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd * per + min(xcd, rem) + slot;
}

// Tile index q -> (expert, rows, column tile).  Tiles are ordered expert by
// expert; inside an expert its row tiles form groups of at most kGroupM (as
// even as possible) and a group walks all column tiles with its row tiles
// innermost, so neighbouring tiles share either their weight tile (same
// expert, same column tile) or their rows.  Groups never straddle two
// experts, whose weights differ.
template <int BM>
__device__ __forceinline__ bool find_tile(const int32_t *__restrict__ offs, int E, int64_t max_rows, int n_tiles,
                                          int q, int *e_out, int *row0_out, int *rows_out, int *nt_out) {
  const int l = lane_id();
  int carry = 0, fe = -1, fo0 = 0, fme = 0, fexcl = 0, ftiles = 0;
  for (int e0 = 0; e0 < E; e0 += kWave) {
    const int e = e0 + l;
    int o0 = 0, me = 0;
    if (e < E) expert_rows(offs, e, max_rows, &o0, &me);
    const int tiles = (me + BM - 1) / BM;
    const int incl = wave_incl_scan(tiles) + carry;
    const int excl = incl - tiles;
    const uint64_t hit = __ballot(e < E && q >= excl * n_tiles && q < incl * n_tiles);
    if (hit) {
      const int src = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<unsigned long long>(hit)) - 1);
      fe = __builtin_amdgcn_readlane(e, src);
      fo0 = __builtin_amdgcn_readlane(o0, src);
      fme = __builtin_amdgcn_readlane(me, src);
      fexcl = __builtin_amdgcn_readlane(excl, src);
      ftiles = __builtin_amdgcn_readlane(tiles, src);
      break;
    }
    carry = __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  fe = __builtin_amdgcn_readfirstlane(fe);
  if (fe < 0) return false;
  fo0 = __builtin_amdgcn_readfirstlane(fo0);
  fme = __builtin_amdgcn_readfirstlane(fme);
  fexcl = __builtin_amdgcn_readfirstlane(fexcl);
  ftiles = __builtin_amdgcn_readfirstlane(ftiles);
  // ng groups: the first `big` hold base+1 row tiles, the others base
  const int ql = q - fexcl * n_tiles;
  const int ng = (ftiles + kGroupM - 1) / kGroupM;
  const int base = ftiles / ng, big = ftiles - base * ng;
  const int span_big = big * (base + 1) * n_tiles;
  int m0, gsz, in_g;
  if (ql < span_big) {
    const int g = ql / ((base + 1) * n_tiles);
    gsz = base + 1;
    m0 = g * gsz;
    in_g = ql - g * gsz * n_tiles;
  } else {
    const int g = (ql - span_big) / (base * n_tiles);
    gsz = base;
    m0 = big * (base + 1) + g * base;
    in_g = ql - span_big - g * base * n_tiles;
  }
  const int lmt = m0 + in_g % gsz;
  *nt_out = in_g / gsz;
  *e_out = fe;
  *row0_out = fo0 + lmt * BM;
  *rows_out = min(BM, fme - lmt * BM);
  return true;
}

// Block -> tile: one block per real tile, ids past the real count exit.
template <int BM>
__device__ __forceinline__ bool map_tile(const int32_t *__restrict__ offs, int E, int64_t max_rows, int n_tiles,
                                         int *e_out, int *row0_out, int *rows_out, int *nt_out) {
  const int m_tiles = count_mtiles<BM>(offs, E, max_rows);
  const int total = m_tiles * n_tiles;
  const int bid = blockIdx.x;
  if (bid >= total) return false;
  return find_tile<BM>(offs, E, max_rows, n_tiles, xcd_remap(bid, total), e_out, row0_out, rows_out, nt_out);
}

template <int S>
struct Slot {
  static constexpr int value = S;
};

}  // namespace

// Small-row-count expert GEMMs (gemm_skinny.hip): bm = 64 rows per tile, K
// a multiple of 64; p.part / p.slots / p.max_split as for the
// 256-row kernel (slots counted in bm x 256 fp32 partial tiles).
hipError_t run_bf16_skinny(GemmParams p, int act, int bm, hipStream_t st);
// fp32 partial-tile bytes of one K piece of a bm-row skinny tile, and the
// pieces a skinny GEMM splits into at most
size_t skinny_part_tile_bytes(int bm);
constexpr int kSkinnyMaxPieces = 512;
constexpr int kSkinnyMaxSplit = 8;  // pieces per tile at most

}  // namespace moe
