// Grouped expert FFN: for every local expert, its block of permuted rows goes
// through GEMM1 (+ GELU or SwiGLU) and GEMM2.
//
// "How MegaDLMs Implements Mixture of Experts (MoE) Architectures", section
// "Core MoE Layer Architecture" (MoELayer step 2: the local experts process
// the tokens dispatched to them).  The pages do not define the expert MLP;
// GELU (exact erf form) and SwiGLU (gate rows, then up rows, of W1) without
// biases are the forms used here.
//
// gfx950 design (bf16):
// * one launch per GEMM covers every expert: the grid is an upper bound on
//   the number of (expert, row tile, column tile) tiles, and each workgroup
//   finds its tile from the device-side expert offsets (a 64-lane prefix sum
//   over per-expert tile counts), so the host never reads how many rows each
//   expert received.  Surplus workgroups exit at once.
// * tiles are ordered expert by expert, and inside an expert its row tiles
//   form groups of at most 8 that walk the column tiles together; workgroup
//   ids are remapped so each of the 8 XCDs takes a contiguous run of that
//   order.  Tiles running together on one XCD then share weight tiles or
//   rows in its L2, and no group mixes two experts' weights.
// * main kernel (gemm_bf16_dma_kernel, K a multiple of 32, >= 192 rows per
//   expert on average): 256 x 256 tiles, 4 waves of 128 x 128
//   v_mfma_f32_32x32x16_bf16 results, operands loaded straight into a 5-deep
//   LDS ring by direct-to-LDS loads (its own comment has the details).  The
//   tiles left over after the last whole round of one workgroup per CU are
//   cut along K when K >= 8192; split_reduce_kernel adds the pieces.
// * small-expert kernel (gemm_bf16_kernel, BM = 128 or 256): tile BM x 256
//   x 64 with 4 waves in a 2 x 2 grid of v_mfma_f32_16x16x32_bf16 results,
//   operands staged global -> registers -> LDS, double-buffered; LDS rows are
//   128 B with the 16-B chunk c of row r stored at chunk c ^ ((r >> 1) & 7),
//   so a 16-lane fragment read hits distinct 16-B slots of the 64 banks.
// * both operands are K-contiguous ([rows, K] activations, [out, in]
//   weights), so each lane's MFMA fragment is one 16-byte LDS read.
// * SwiGLU: the B tile holds 128 gate rows and the 128 matching up rows, and
//   every wave computes the same output columns for both, so the epilogue
//   silu(gate) * up is lane-local.  GELU is applied in the epilogue as well:
//   the hidden activation is written once, in bf16.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "gemm_common.h"

namespace moe {
namespace {

template <int BM, int ACT>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmParams p) {
  constexpr int WM = BM / 2;   // rows per wave
  constexpr int MI = WM / 16;  // 16-row MFMA tiles per wave
  constexpr int NJ = 8;        // 16-col MFMA tiles per wave (128 B rows)
  constexpr int A_CH = BM * 8 / kThreads;
  constexpr int B_CH = BN * 8 / kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];

  int e, row0, rows, nt;
  if (!map_tile<BM>(p.offs, p.E, p.max_rows, p.n_tiles, &e, &row0, &rows, &nt)) return;

  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  const int wm = w >> 1, wn = w & 1;
  const uint16_t *A = static_cast<const uint16_t *>(p.A);
  const uint16_t *B = static_cast<const uint16_t *>(p.B) + static_cast<int64_t>(e) * p.b_stride;

  // this thread's 16-B chunk column and the rows it stages
  const int cc = tid & 7;
  const int rbase = tid >> 3;  // + 32*i
  int a_off[A_CH], b_off[B_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int r = rbase + 32 * i;
    a_off[i] = static_cast<int>((row0 + min(r, rows - 1)) * p.lda);
  }
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int r = rbase + 32 * i;
    int br;
    if (ACT == ACT_SWIGLU) {
      const int col = nt * (BN / 2) + (r & (BN / 2 - 1));
      br = (col < p.n_out ? col : 0) + (r >= BN / 2 ? p.up_off : 0);
    } else {
      const int col = nt * BN + r;
      br = col < p.n_out ? col : 0;
    }
    b_off[i] = static_cast<int>(br * p.ldb);
  }

  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[A_CH], rb[B_CH];
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto gload = [&](int k0) {
    const int kk = k0 + cc * 8;
    const bool kin = kk < p.K;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) ra[i] = kin ? ld16(A + a_off[i] + kk) : zero;
#pragma unroll
    for (int i = 0; i < B_CH; ++i) rb[i] = kin ? ld16(B + b_off[i] + kk) : zero;
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int r = rbase + 32 * i;
      *reinterpret_cast<u32x4 *>(&sA[buf][r * BK + ((cc ^ ((r >> 1) & 7)) * 8)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int r = rbase + 32 * i;
      *reinterpret_cast<u32x4 *>(&sB[buf][r * BK + ((cc ^ ((r >> 1) & 7)) * 8)]) = rb[i];
    }
  };

  const int nk = (p.K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int chunk = ((ks * 4 + (l >> 4)) ^ ((l >> 1) & 7)) * 8;
      bf16x8 a[MI], b[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        a[i] = *reinterpret_cast<const bf16x8 *>(&sA[cur][(wm * WM + i * 16 + (l & 15)) * BK + chunk]);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        int br;
        if (ACT == ACT_SWIGLU) br = (j < NJ / 2) ? wn * 64 + j * 16 : BN / 2 + wn * 64 + (j - NJ / 2) * 16;
        else br = wn * 128 + j * 16;
        b[j] = *reinterpret_cast<const bf16x8 *>(&sB[cur][(br + (l & 15)) * BK + chunk]);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  uint16_t *C = static_cast<uint16_t *>(p.C);
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lr = wm * WM + i * 16 + (l >> 4) * 4 + r;
      if (lr >= rows) continue;
      uint16_t *crow = C + static_cast<int64_t>(row0 + lr) * p.ldc;
      if (ACT == ACT_SWIGLU) {
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j) {
          const int col = nt * (BN / 2) + wn * 64 + j * 16 + (l & 15);
          if (col < p.n_out) crow[col] = f32_to_bf16(silu_fast(acc[i][j][r]) * acc[i][j + NJ / 2][r]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int col = nt * BN + wn * 128 + j * 16 + (l & 15);
          if (col < p.n_out) {
            const float v = acc[i][j][r];
            crow[col] = f32_to_bf16(ACT == ACT_GELU ? gelu_erf(v) : v);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Main bf16 kernel (K a multiple of 32): 256 x 256 tile, 32-wide K stages in a
// 5-deep LDS ring (5 x 32 KB = the whole 160 KB LDS) filled by
// global_load_lds_dwordx4 (gfx950 direct-to-LDS loads: no VGPR staging, each
// wave instruction writes 1 KB of LDS).  Stage kt+4 is requested right after
// the barrier that opens stage kt, so each load has four stages of MFMA work
// (about 1.7 us at full rate) to land.  The ring slots are distinct LDS arrays
// and the K loop is unrolled by five, so every slot index is static.
// LDS rows are 64 B (four 16-B chunks); chunk c of row r is stored at
// c ^ ((r >> 2) & 3).  gfx950 serves a 16-byte-per-lane LDS read 16 lanes at a
// time over 64 banks (256 B); the 16 rows one such group reads then land on 16
// distinct 16-B bank slots, so fragment reads are conflict-free.
constexpr int DK = 32;   // K per stage
constexpr int NST = 5;   // stages in the LDS ring
constexpr int DBM = 256; // tile rows
constexpr int kDmaWaves = 4;  // waves per workgroup of gemm_bf16_dma_kernel (4 or 8)
// The 256-row kernel runs when the experts average at least this many rows
// (measured: with 256 rows per expert it is 25-28 % faster than the 128-row
// kernel; with at most 128 it is slower, its tiles being mostly padding).
constexpr int64_t kDmaMinAvgRows = 192;
constexpr int DSTAGE = DBM * DK;  // elements per operand per stage

// K-split of the last round: only GEMMs with at least kSplitMinStages K
// stages split (measured on gfx950: with K = 14336 the split saves a sixth of
// the down projection, with K = 4096 it saves nothing: a short tail tile
// costs less than the pieces' prologues and the extra reduction pass); a
// piece keeps at least kPieceMinStages stages, and a tile splits into at
// most kMaxSplit pieces.
constexpr int kSplitMinStages = 256;
constexpr int kPieceMinStages = 32;
constexpr int kMaxSplit = 16;

// One workgroup's share of a 256 x 256 grouped GEMM.  The tiles that fill
// whole rounds of `units` workgroups run one per workgroup (XCD-remapped as in
// map_tile).  The remaining tiles, fewer than one round, would leave most of
// the chip idle during the last round; when the GEMM may split (max_split >
// 1), each of them is cut along K into
// nseg = min(units / remaining, stages / kPieceMinStages, max_split) pieces,
// so the last round takes about 1/nseg of a tile's time.  A piece stores its fp32 partial tile;
// split_reduce_kernel then adds the pieces in K order (so the result does not
// depend on which piece finished first) and applies the epilogue.
struct Split {
  int m_tiles, total, full, rest, nseg;
};

__device__ __forceinline__ Split split_plan(const GemmParams &p, int nk) {
  Split sp;
  sp.m_tiles = count_mtiles<DBM>(p.offs, p.E, p.max_rows);
  sp.total = sp.m_tiles * p.n_tiles;
  sp.full = sp.total / p.units * p.units;
  sp.rest = sp.total - sp.full;
  sp.nseg = 1;
  if (sp.rest > 0)
    sp.nseg = max(1, min(min(min(p.units, p.slots) / sp.rest, nk / kPieceMinStages), p.max_split));
  return sp;
}

struct Job {
  int e, row0, rows, nt;
  int kb, ke;           // K stages [kb, ke) of this piece
  int tail, seg, nseg;  // split tile index (-1 if whole), piece, pieces
  int k0;               // first contraction row of the group (groups of K)
};

__device__ __forceinline__ bool map_job(const GemmParams &p, int nk, Job *j) {
  const Split sp = split_plan(p, nk);
  const int bid = blockIdx.x;
  int q;
  j->kb = 0;
  j->ke = nk;
  j->tail = -1;
  j->seg = 0;
  j->nseg = 1;
  j->k0 = 0;
  if (bid < sp.full) {
    q = xcd_remap(bid, sp.full);
  } else {
    const int n = sp.rest * sp.nseg;
    if (bid - sp.full >= n) return false;
    // pieces walk piece-major (all tiles' first K piece, then the second,
    // ...) in XCD-contiguous runs, so the pieces one XCD runs together read
    // the same K slice of neighbouring tiles and share it in its L2
    const int u = xcd_remap(bid - sp.full, n);
    const int seg = u / sp.rest, t = u - seg * sp.rest;
    q = sp.full + t;
    if (sp.nseg > 1) {
      // wave-uniform: keep them in scalar registers across the K loop
      j->kb = __builtin_amdgcn_readfirstlane(seg * nk / sp.nseg);
      j->ke = __builtin_amdgcn_readfirstlane((seg + 1) * nk / sp.nseg);
      j->tail = __builtin_amdgcn_readfirstlane(t);
      j->seg = __builtin_amdgcn_readfirstlane(seg);
      j->nseg = __builtin_amdgcn_readfirstlane(sp.nseg);
    }
  }
  return find_tile<DBM>(p.offs, p.E, p.max_rows, p.n_tiles, q, &j->e, &j->row0, &j->rows, &j->nt);
}

// Operand layouts of the 256-row kernel.  NT (the forward): A [rows, K] and
// B [N, K], both contiguous along K.  NN (data gradients): B [K, N], N
// contiguous.  TN (weight gradients): A [K, M] and B [K, N] over the rows of
// a group, C_e = A_e^T B_e.  A [K, ...] operand is staged in LDS as 32 rows of
// 256 elements (512 B) per stage; chunk c (8 elements) of row kk is stored at
// c ^ (4 * (kk & 3)), and its MFMA fragments are read with gfx950's LDS
// transpose read (ds_read_b64_tr_b16): in each 16-lane group, lane i reads
// 4 elements of row i/4 at columns 4*(i%4)..+3 and receives column i of the
// group's 4 rows.  Two such reads give a lane the 8 consecutive K values of
// one column that a 32x32x16 operand needs.  The 32 lanes served together
// read rows kk..kk+3 at the same 64-B column range, which the swizzle puts in
// 4 distinct bank groups.
enum { LAY_NT = 0, LAY_NN = 1, LAY_TN = 2 };

__device__ __forceinline__ int tr_swz(int kk) { return 4 * (kk & 3); }

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x4 lds_read_tr16(const uint16_t *p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)((lds_u16 *)p));
}

// Groups of K (TN): one workgroup per (group, row tile, column tile), dense;
// row tiles innermost, so neighbouring workgroups of one XCD share the B
// panel of a column tile.  The group's contraction rows are
// [offs[e], offs[e+1]), whole 32-row stages.
__device__ __forceinline__ bool map_kgroup_job(const GemmParams &p, Job *j) {
  const int per = p.m_tiles * p.n_tiles;
  const int total = per * p.E;
  const int bid = blockIdx.x;
  if (bid >= total) return false;
  const int q = xcd_remap(bid, total);
  const int e = q / per, r = q - e * per;
  const int nt = r / p.m_tiles, mt = r - nt * p.m_tiles;
  int k0, me;
  expert_rows(p.offs, e, p.max_rows, &k0, &me);
  j->e = __builtin_amdgcn_readfirstlane(e);
  j->row0 = __builtin_amdgcn_readfirstlane(mt * DBM);
  j->rows = __builtin_amdgcn_readfirstlane(min(DBM, p.m_rows - mt * DBM));
  j->nt = __builtin_amdgcn_readfirstlane(nt);
  j->k0 = __builtin_amdgcn_readfirstlane(k0);
  j->kb = 0;
  j->ke = __builtin_amdgcn_readfirstlane(me / DK);
  j->tail = -1;
  j->seg = 0;
  j->nseg = 1;
  return true;
}

// An empty asm "use" at the end of an iteration keeps that iteration's
// fragment set live until then, so the register allocator cannot hand its
// registers to the next stage's LDS reads while queued MFMAs still have to
// read them (the hardware would hold the LDS read until they did).
template <int SET, int MI, int NJ>
__device__ __forceinline__ void keep_live(bf16x8 (&fa)[2][2][MI], bf16x8 (&fb)[2][2][NJ]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int i = 0; i < MI; ++i) asm volatile("" ::"v"(fa[SET][ks][i]));
#pragma unroll
    for (int j = 0; j < NJ; ++j) asm volatile("" ::"v"(fb[SET][ks][j]));
  }
}

template <int ACT, int WAVES, int LAY = LAY_NT>
__global__ __launch_bounds__(WAVES * 64) void gemm_bf16_dma_kernel(GemmParams p) {
  // v_mfma_f32_32x32x16_bf16 (the 16x16x32 form does not keep the matrix core
  // full from one wave per SIMD).  WAVES = 4: one wave per SIMD, each owning
  // 128 x 128 = 4 x 4 tiles of 32 x 32; WAVES = 8: two waves per SIMD, each
  // owning 64 x 128 = 2 x 4 tiles, so one wave's memory instructions can wait
  // while the other feeds the matrix core.  Per 16-wide K step a wave reads
  // MI A and NJ B fragments (16 B per lane: row l%32, K chunk l/32) and issues
  // MI * NJ MFMAs.
  static_assert(WAVES == 4 || WAVES == 8, "4 or 8 waves");
  constexpr int NTH = WAVES * kWave;
  constexpr int MI = WAVES == 4 ? 4 : 2, NJ = 4;
  constexpr int RW = 32 * MI;           // rows per wave
  constexpr int ND = 32 / WAVES;        // load instructions per wave per stage
  constexpr int NR = 2 * (MI + NJ);     // fragment reads per wave per stage
  constexpr int NM = 2 * MI * NJ;       // MFMAs per wave per stage
  static_assert((WAVES == 4 ? NM / 2 : 3 * NM / 4) == NR && NM / 4 == ND, "interleave covers every read and load");
  static_assert(LAY == LAY_NT || (ACT == ACT_NONE && WAVES == 4), "backward layouts: plain output, 4 waves");
  constexpr bool AT = LAY == LAY_TN;  // A staged as [K][M]
  constexpr bool BT = LAY != LAY_NT;  // B staged as [K][N]
  // one array per ring slot: A stage at [0, DSTAGE), B stage at [DSTAGE, 2*DSTAGE)
  __shared__ __attribute__((aligned(1024))) uint16_t s0[2 * DSTAGE], s1[2 * DSTAGE], s2[2 * DSTAGE],
      s3[2 * DSTAGE], s4[2 * DSTAGE];

  Job job;
  if constexpr (LAY == LAY_TN) {
    if (!map_kgroup_job(p, &job)) return;
    if (job.ke == 0) {
      // a group with no rows: its gradient tile is zero (coalesced 16-B stores)
      uint8_t *C = static_cast<uint8_t *>(p.C) + static_cast<int64_t>(job.e) * p.c_stride * 2;
      const int c0 = job.nt * BN, ncol = min(BN, p.n_out - c0);
      for (int q = threadIdx.x; q < job.rows * (BN / 8); q += NTH) {
        const int r = q / (BN / 8), c = (q - r * (BN / 8)) * 8;
        if (c < ncol) st16(C + (static_cast<int64_t>(job.row0 + r) * p.ldc + c0 + c) * 2, u32x4{0u, 0u, 0u, 0u});
      }
      return;
    }
  } else {
    if (!map_job(p, p.K / DK, &job)) return;
  }
  const int e = job.e, row0 = job.row0, rows = job.rows, nt = job.nt;
  const int l = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
  const int wm = w >> 1, wn = w & 1;
  // wave-uniform bases of this piece's K range: A at the tile's first row
  // (TN: its first column), B at the expert's weights (TN: the column
  // tile's first column); a stage advances them by a_step / b_step bytes
  const int64_t kfirst = static_cast<int64_t>(job.k0) + static_cast<int64_t>(job.kb) * DK;
  // K-blocked A: the tile's K stage is the 256 row pieces starting at row0
  // of the stage's 32-wide slice
  static_assert(kKbRowBytes == DK * 2, "a K-blocked row piece is one stage of one row");
  const bool a_kb = LAY == LAY_NT && p.a_kb;
  const char *A = static_cast<const char *>(p.A) +
                  (a_kb ? (static_cast<int64_t>(job.kb) * p.max_rows + row0) * kKbRowBytes
                        : (AT ? kfirst * p.lda + row0 : static_cast<int64_t>(row0) * p.lda + job.kb * DK) * 2);
  // packed B: the stage blocks of column tile nt follow each other, 16 KB
  // apart, and a stage is read as one contiguous block
  static_assert(kPackK == DK && kPackBlockBytes == DSTAGE * 2, "a packed block is one B stage");
  const bool packed = LAY == LAY_NT && p.packed;
  const char *B = static_cast<const char *>(p.B) +
                  (packed ? static_cast<int64_t>(e) * p.b_stride * 2 +
                                (static_cast<int64_t>(nt) * (p.K / DK) + job.kb) * kPackBlockBytes
                          : (BT ? (LAY == LAY_TN ? 0 : static_cast<int64_t>(e) * p.b_stride) + kfirst * p.ldb +
                                      static_cast<int64_t>(nt) * BN
                                : static_cast<int64_t>(e) * p.b_stride + job.kb * DK) * 2);
  const int64_t a_step = a_kb ? p.max_rows * kKbRowBytes : AT ? static_cast<int64_t>(DK) * p.lda * 2 : DK * 2;
  const int64_t b_step = packed ? kPackBlockBytes : BT ? static_cast<int64_t>(DK) * p.ldb * 2 : DK * 2;

  auto slot = [&](auto S) -> uint16_t * {
    constexpr int s = decltype(S)::value;
    if constexpr (s == 0) return s0;
    else if constexpr (s == 1) return s1;
    else if constexpr (s == 2) return s2;
    else if constexpr (s == 3) return s3;
    else return s4;
  };

  // DMA sources: wave w, instruction i of an operand fills LDS chunks
  // [(WAVES*i+w)*64, +64), i.e. rows (WAVES*i+w)*16 .. +16; lane l -> row
  // r = q/4, stored chunk q%4, which holds logical chunk (q%4) ^ ((r>>2)&3).
  // Per-lane byte offsets from A / B (they fit 32 bits: the host limits every
  // operand to 2^31 elements, and the widths below 2^22, so that a row-major
  // A tile's offsets stay below kDmaRange).
  // [K][.] operands: LDS chunk slot q is row kk = q/32, stored chunk q%32,
  // which holds logical chunk (q%32) ^ tr_swz(kk); columns past the operand's
  // width (partial tiles) read its last valid 8 columns instead.
  uint32_t a_off[ND / 2], b_off[ND / 2];
#pragma unroll
  for (int i = 0; i < ND / 2; ++i) {
    const int q = (WAVES * i + w) * 64 + l;
    const int r = q >> 2;
    const int c = (q & 3) ^ ((r >> 2) & 3);
    const int kk = q >> 5;
    const int tc = (q & 31) ^ tr_swz(kk);
    if constexpr (AT) {
      const int col = min(tc * 8, p.m_rows - row0 - 8);
      a_off[i] = static_cast<uint32_t>((static_cast<int64_t>(kk) * p.lda + col) * 2);
    } else {
      // rows past the tile's last real row load as zeros (dma16_zp)
      a_off[i] = r >= rows ? kDmaSkip
                 : a_kb    ? static_cast<uint32_t>(r * kKbRowBytes + c * 16)
                           : static_cast<uint32_t>((static_cast<int64_t>(r) * p.lda + c * 8) * 2);
    }
    if constexpr (BT) {
      const int col = min(tc * 8, p.n_out - nt * BN - 8);
      b_off[i] = static_cast<uint32_t>((static_cast<int64_t>(kk) * p.ldb + col) * 2);
    } else {
      int br;
      if (ACT == ACT_SWIGLU) {
        const int col = nt * (BN / 2) + (r & (BN / 2 - 1));
        br = (col < p.n_out ? col : 0) + (r >= BN / 2 ? p.up_off : 0);
      } else {
        const int col = nt * BN + r;
        br = col < p.n_out ? col : 0;
      }
      b_off[i] = packed ? static_cast<uint32_t>(q * 16)
                        : static_cast<uint32_t>((static_cast<int64_t>(br) * p.ldb + c * 8) * 2);
    }
  }
  // A loads: range-checked for the row-major layouts, so pad rows land as
  // zeros; the [K][M] layout clamps its columns instead
  auto dma_a = [&](uint32_t off, const char *src, uint32_t lds) {
    if constexpr (AT) dma16(off, src, lds);
    else dma16_zp(off, src, lds);
  };
  // stage st of this piece: K elements [st*DK, st*DK + DK) past A / B
  auto issue = [&](auto S, int st) {
    const uint32_t base = lds_addr_of(slot(S));
#pragma unroll
    for (int i = 0; i < ND / 2; ++i) {
      dma_a(a_off[i], A + st * a_step, base + (WAVES * i + w) * 64 * 16);
      dma16(b_off[i], B + st * b_step, base + DSTAGE * 2 + (WAVES * i + w) * 64 * 16);
    }
  };

  // fragment offsets inside a stage (elements), for the two 16-wide K steps
  const int frow = l & 31;
  const int fsw = (frow >> 2) & 3;
  const int fch0 = ((l >> 5) ^ fsw) * 8;        // K step 0: chunks 0,1
  const int fch1 = (((l >> 5) + 2) ^ fsw) * 8;  // K step 1: chunks 2,3
  const int a_row = (wm * RW + frow) * DK;      // + i*32*DK
  int b_row[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    int br;
    if (ACT == ACT_SWIGLU) br = (j < NJ / 2) ? wn * 64 + j * 32 : BN / 2 + wn * 64 + (j - NJ / 2) * 32;
    else br = wn * 128 + j * 32;
    b_row[j] = DSTAGE + (br + frow) * DK;
  }
  // transpose reads of a [K][.] operand: lane l (group g = l/16, i = l%16)
  // reads row 16*ks + 8*(g/2) + 4*r + i/4 at logical column
  // base + 16*(g%2) + 4*(i%4); a 32-column fragment starting at column 32*j
  // of the wave's half sits at stored chunk ((4j) ^ swizzle) + (column/8)%4
  const int tg = l >> 4, ti = l & 15;
  const int tr_row = (8 * (tg >> 1) + (ti >> 2)) * BN;
  const int tr_col = 16 * (tg & 1) + 4 * (ti & 3);
  const int tr_sw = tr_swz(ti >> 2);
  const int tr_base_a = tr_row + wm * RW + ((tr_col >> 3) << 3) + (tr_col & 7);
  const int tr_base_b = DSTAGE + tr_row + wn * 128 + ((tr_col >> 3) << 3) + (tr_col & 7);
  auto tr_frag = [&](const uint16_t *ls, int base, int tile, int ks) -> bf16x8 {
    const int off = base + (((4 * tile) ^ tr_sw) << 3) + ks * 16 * BN;
    const bf16x4 lo = lds_read_tr16(ls + off);
    const bf16x4 hi = lds_read_tr16(ls + off + 4 * BN);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto frag_a = [&](const uint16_t *ls, int ks, int i) -> bf16x8 {
    if constexpr (AT) return tr_frag(ls, tr_base_a, i, ks);
    else return *reinterpret_cast<const bf16x8 *>(ls + a_row + i * 32 * DK + (ks ? fch1 : fch0));
  };
  auto frag_b = [&](const uint16_t *ls, int ks, int j) -> bf16x8 {
    if constexpr (BT) return tr_frag(ls, tr_base_b, j, ks);
    else return *reinterpret_cast<const bf16x8 *>(ls + b_row[j] + (ks ? fch1 : fch0));
  };

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Fragments are double-buffered in registers: the reads of stage kt+1 go to
  // the set the MFMAs of stage kt do not use, and they are issued half-way
  // through stage kt's MFMAs (after the barrier that publishes stage kt+1), so
  // the matrix core never waits for an LDS read or for a register a queued
  // MFMA has yet to consume.
  bf16x8 fa[2][2][MI], fb[2][2][NJ];  // [set][16-wide K step][tile]
  auto read_frags = [&](auto SET, auto S) {
    constexpr int set = decltype(SET)::value;
    const uint16_t *ls = slot(S);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < MI; ++i) fa[set][ks][i] = frag_a(ls, ks, i);
#pragma unroll
      for (int j = 0; j < NJ; ++j) fb[set][ks][j] = frag_b(ls, ks, j);
    }
  };
  auto mma = [&](auto SET, int ks) {
    constexpr int set = decltype(SET)::value;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][ks][i], fb[set][ks][j], acc[i][j], 0, 0, 0);
  };
  // wait until stage `st` has landed given the stages issued so far, then a
  // plain barrier (this wave's LDS reads have returned; no fence, which would
  // also wait for the DMA still in flight)
  auto wait_stage = [&](int st, int issued_last) {
    const int ahead = issued_last - st;
    if (ahead >= 4) wait_vm<4 * ND>();
    else if (ahead == 3) wait_vm<3 * ND>();
    else if (ahead == 2) wait_vm<2 * ND>();
    else if (ahead == 1) wait_vm<ND>();
    else wait_vm<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  const int nk = job.ke - job.kb;  // stages of this piece (A / B start at its first)
  // prologue: stages 0..4 in flight, stage 0's fragments in set 0
  if (0 < nk) issue(Slot<0>{}, 0);
  if (1 < nk) issue(Slot<1>{}, 1);
  if (2 < nk) issue(Slot<2>{}, 2);
  if (3 < nk) issue(Slot<3>{}, 3);
  if (4 < nk) issue(Slot<4>{}, 4);
  wait_stage(0, min(nk - 1, 4));
  read_frags(Slot<0>{}, Slot<0>{});

  // iteration kt: stage kt sits in slot kt%5 and fragment set kt%2.
  // After the barrier that publishes stage kt+1, stage kt's NM MFMAs are
  // interleaved with the NR fragment reads of stage kt+1 (into the other
  // register set) and the ND DMA instructions that refill stage kt's slot
  // with stage kt+5; sched_barrier pins this order, so the LDS reads and the
  // loads issue in the shadow of the matrix core.  A steady iteration (at
  // least 5 stages after it) has every read and refill and waits with three
  // stages still in flight: all of that is known at compile time, so its
  // loads and wait carry no branches (a branch per load and a branch tree
  // per wait gave 185 instructions and 14 branches per stage; without them
  // 95 and none, and the Mixtral-slice FFN went from 2.79 to 2.75 ms).
  auto iter = [&](auto S, auto SET, int kt, auto STEADY) {
    constexpr int s = decltype(S)::value;
    constexpr int set = decltype(SET)::value;
    constexpr bool steady = decltype(STEADY)::value;
    const bool more = steady || kt + 1 < nk;
    const bool refill = steady || kt + 5 < nk;
    if constexpr (steady) {
      wait_vm<3 * ND>();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      if (more) wait_stage(kt + 1, min(nk - 1, kt + 4));
    }
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t *ls = slot(Slot<(s + 1) % NST>{});
    const uint32_t dbase = lds_addr_of(slot(S));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][ks][i], fb[set][ks][j], acc[i][j], 0, 0, 0);
          // every 4 MFMAs one load (t%4 == 1 for 4 waves, 3 for 8 waves) and
          // the fragment reads in the other slots (4 waves: t even; 8 waves:
          // t%4 != 3), spread out so the per-CU load path drains between
          // load issues instead of stalling the wave that issues them
          const int t = ks * (MI * NJ) + i * NJ + j;
          constexpr int kLoadSlot = WAVES == 4 ? 1 : 3;
          const bool is_read = WAVES == 4 ? (t & 1) == 0 : (t & 3) != 3;
          if (is_read) {
            if (more) {  // read rd: K step rd / (MI+NJ), A tiles then B tiles
              const int rd = WAVES == 4 ? t >> 1 : (t >> 2) * 3 + (t & 3);
              const int rks = rd / (MI + NJ), r = rd % (MI + NJ);
              if (r < MI) fa[set ^ 1][rks][r] = frag_a(ls, rks, r);
              else fb[set ^ 1][rks][r - MI] = frag_b(ls, rks, r - MI);
            }
          } else if ((t & 3) == kLoadSlot) {
            if (refill) {
              const int dd = t >> 2, ii = dd >> 1;
              if ((dd & 1) == 0) dma_a(a_off[ii], A + (kt + 5) * a_step, dbase + (WAVES * ii + w) * 64 * 16);
              else dma16(b_off[ii], B + (kt + 5) * b_step, dbase + DSTAGE * 2 + (WAVES * ii + w) * 64 * 16);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    keep_live<set>(fa, fb);
    __builtin_amdgcn_sched_barrier(0);
  };
  using Steady = std::integral_constant<bool, true>;
  using Edge = std::integral_constant<bool, false>;
  int kt = 0;
  // ten steady iterations while at least 15 stages remain (the last of them
  // still refills stage kt + 14)
  for (; kt + 14 < nk; kt += 10) {
    iter(Slot<0>{}, Slot<0>{}, kt, Steady{});
    iter(Slot<1>{}, Slot<1>{}, kt + 1, Steady{});
    iter(Slot<2>{}, Slot<0>{}, kt + 2, Steady{});
    iter(Slot<3>{}, Slot<1>{}, kt + 3, Steady{});
    iter(Slot<4>{}, Slot<0>{}, kt + 4, Steady{});
    iter(Slot<0>{}, Slot<1>{}, kt + 5, Steady{});
    iter(Slot<1>{}, Slot<0>{}, kt + 6, Steady{});
    iter(Slot<2>{}, Slot<1>{}, kt + 7, Steady{});
    iter(Slot<3>{}, Slot<0>{}, kt + 8, Steady{});
    iter(Slot<4>{}, Slot<1>{}, kt + 9, Steady{});
  }
  for (; kt + 9 < nk; kt += 10) {
    iter(Slot<0>{}, Slot<0>{}, kt, Edge{});
    iter(Slot<1>{}, Slot<1>{}, kt + 1, Edge{});
    iter(Slot<2>{}, Slot<0>{}, kt + 2, Edge{});
    iter(Slot<3>{}, Slot<1>{}, kt + 3, Edge{});
    iter(Slot<4>{}, Slot<0>{}, kt + 4, Edge{});
    iter(Slot<0>{}, Slot<1>{}, kt + 5, Edge{});
    iter(Slot<1>{}, Slot<0>{}, kt + 6, Edge{});
    iter(Slot<2>{}, Slot<1>{}, kt + 7, Edge{});
    iter(Slot<3>{}, Slot<0>{}, kt + 8, Edge{});
    iter(Slot<4>{}, Slot<1>{}, kt + 9, Edge{});
  }
  if (kt < nk) iter(Slot<0>{}, Slot<0>{}, kt, Edge{});
  if (kt + 1 < nk) iter(Slot<1>{}, Slot<1>{}, kt + 1, Edge{});
  if (kt + 2 < nk) iter(Slot<2>{}, Slot<0>{}, kt + 2, Edge{});
  if (kt + 3 < nk) iter(Slot<3>{}, Slot<1>{}, kt + 3, Edge{});
  if (kt + 4 < nk) iter(Slot<4>{}, Slot<0>{}, kt + 4, Edge{});
  if (kt + 5 < nk) iter(Slot<0>{}, Slot<1>{}, kt + 5, Edge{});
  if (kt + 6 < nk) iter(Slot<1>{}, Slot<0>{}, kt + 6, Edge{});
  if (kt + 7 < nk) iter(Slot<2>{}, Slot<1>{}, kt + 7, Edge{});
  if (kt + 8 < nk) iter(Slot<3>{}, Slot<0>{}, kt + 8, Edge{});

  if (job.nseg > 1) {
    // K-split piece: store the fp32 partial in accumulator order (lane l of
    // wave w, tile (i, j), values 4*v4..4*v4+3 at float4 index
    // ((w*MI + i)*NJ + j)*4*64 + v4*64 + l), so every store is a coalesced
    // 1 KB wave store; split_reduce_kernel finishes the tile.  The stores
    // take the accumulators straight from the AGPRs (inline asm with an
    // SGPR base and immediate offsets): through VGPRs, this path and the
    // epilogue together overflow the register file.  The compiler cannot see
    // inside the asm, so each block first waits out the MFMA / AGPR-write
    // read hazard itself (21 wait states).
    constexpr int kTileF = DBM * BN;
    const char *mine = reinterpret_cast<const char *>(p.part) +
                       (static_cast<int64_t>(job.tail * job.nseg + job.seg) * kTileF + w * (MI * NJ * 4 * kWave * 4)) * 4;
    const uint32_t voff = l * 16;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const char *sb = mine + (i * NJ + j) * 4 * kWave * 16;
        const f32x4 v0 = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
        const f32x4 v1 = {acc[i][j][4], acc[i][j][5], acc[i][j][6], acc[i][j][7]};
        const f32x4 v2 = {acc[i][j][8], acc[i][j][9], acc[i][j][10], acc[i][j][11]};
        const f32x4 v3 = {acc[i][j][12], acc[i][j][13], acc[i][j][14], acc[i][j][15]};
        asm volatile(
            "s_nop 7\n\ts_nop 7\n\ts_nop 4\n\t"
            "global_store_dwordx4 %0, %1, %5\n\t"
            "global_store_dwordx4 %0, %2, %5 offset:1024\n\t"
            "global_store_dwordx4 %0, %3, %5 offset:2048\n\t"
            "global_store_dwordx4 %0, %4, %5 offset:3072" ::"v"(voff),
            "a"(v0), "a"(v1), "a"(v2), "a"(v3), "s"(sb)
            : "memory");
      }
    }
    return;
  }

  // Epilogue: activation, then quad_rows() turns each 4-row column slice of a
  // lane into one 8-byte row piece, written to LDS (the ring is free by now);
  // then the block stores whole rows with 16-byte coalesced writes.  Row pitch
  // = row bytes + 64: the 8 rows one ds_write_b64 covers (8 x 64 B) fall on
  // the 4 distinct 64-B bank quarters twice, the minimum for 512 B.
  constexpr int OUT_COLS = (ACT == ACT_SWIGLU) ? BN / 2 : BN;  // output columns of the tile
  constexpr int NJO = (ACT == ACT_SWIGLU) ? NJ / 2 : NJ;      // output tiles per wave row
  constexpr int PITCH = OUT_COLS * 2 + 64;                     // bytes per LDS row
  static_assert(DBM * PITCH <= NST * 2 * DSTAGE * 2, "epilogue tile must fit in the ring");
  // The five slot arrays fill the 160 KB exactly, so they are contiguous; the
  // epilogue tile starts at whichever of them has the lowest LDS address.
  uint16_t *lo = s0;
  if (lds_addr_of(s1) < lds_addr_of(lo)) lo = s1;
  if (lds_addr_of(s2) < lds_addr_of(lo)) lo = s2;
  if (lds_addr_of(s3) < lds_addr_of(lo)) lo = s3;
  if (lds_addr_of(s4) < lds_addr_of(lo)) lo = s4;
  uint8_t *ep = reinterpret_cast<uint8_t *>(lo);
  const int lr0 = wm * RW + 4 * (l >> 5) + (l & 3);                // + 32 i + 8 g
  const int lc0 = wn * (OUT_COLS / 2) + 4 * ((l & 31) >> 2);       // + 32 j
  __syncthreads();  // every wave is done with the ring
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int j = 0; j < NJO; ++j) {
        float f[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float x = acc[i][j][4 * g + t];
          if (ACT == ACT_SWIGLU) f[t] = silu_fast(x) * acc[i][j + NJ / 2][4 * g + t];
          else if (ACT == ACT_GELU) f[t] = gelu_erf(x);
          else f[t] = x;
        }
        const u32x2 v = quad_rows(f[0], f[1], f[2], f[3]);
        *reinterpret_cast<u32x2 *>(ep + (lr0 + 32 * i + 8 * g) * PITCH + (lc0 + 32 * j) * 2) = v;
      }
    }
  }
  __syncthreads();
  constexpr int CHUNKS = OUT_COLS / 8;  // 16-byte chunks per row
  const int col0 = nt * OUT_COLS;
  uint8_t *C = static_cast<uint8_t *>(p.C) + (LAY == LAY_TN ? static_cast<int64_t>(e) * p.c_stride * 2 : 0);
  // non-temporal stores: the tile is not read again by this kernel, and its
  // lines would push the operands that the tiles running beside it share out
  // of L2 (correlated workloads: FFN 4-9 % faster; the others unchanged)
  if (LAY == LAY_NT && p.c_kb) {
    // K-blocked output: thread q takes chunk q%4 of row (q/4)%DBM in the
    // tile's 32-column slice q/(4 DBM), so a wave stores 16 whole row pieces,
    // 1 KB contiguous
    for (int q = threadIdx.x; q < DBM * CHUNKS; q += NTH) {
      const int c4 = q & 3, r = (q >> 2) & (DBM - 1), kbl = q / (4 * DBM);
      const int col = col0 + kbl * 32 + c4 * 8;
      if (r >= rows || col >= p.n_out) continue;
      const u32x4 val = *reinterpret_cast<const u32x4 *>(ep + r * PITCH + (kbl * 4 + c4) * 16);
      __builtin_nontemporal_store(val, reinterpret_cast<u32x4 *>(C + c_index(p, row0 + r, col) * 2));
    }
    return;
  }
  for (int q = threadIdx.x; q < DBM * CHUNKS; q += NTH) {
    const int r = q / CHUNKS, c = q - (q / CHUNKS) * CHUNKS;
    if (r >= rows || col0 + c * 8 >= p.n_out) continue;
    const u32x4 val = *reinterpret_cast<const u32x4 *>(ep + r * PITCH + c * 16);
    __builtin_nontemporal_store(val, reinterpret_cast<u32x4 *>(C + (static_cast<int64_t>(row0 + r) * p.ldc + col0 + c * 8) * 2));
  }
}

// Finishes the K-split tiles of gemm_bf16_dma_kernel: for each split tile,
// adds its pieces' fp32 partials in K order and applies the epilogue.  One
// thread per float4 of the accumulator layout (SwiGLU: per gate float4, which
// also reads its up partner, two column tiles further), grid-stride over
// (tile, block-of-work) pairs.
template <int ACT, int WAVES>
__global__ __launch_bounds__(kThreads) void split_reduce_kernel(GemmParams p) {
  constexpr int MI = WAVES == 4 ? 4 : 2, NJ = 4, RW = 32 * MI;  // as in gemm_bf16_dma_kernel
  constexpr int NJE = ACT == ACT_SWIGLU ? NJ / 2 : NJ;         // tiles a thread starts from
  constexpr int kTileF = DBM * BN;
  constexpr int kGroups = WAVES * MI * NJE * 4 * kWave;          // float4 groups per tile
  constexpr int kWork = kGroups / kThreads;                      // blocks of work per tile
  static_assert(kGroups * 4 == (ACT == ACT_SWIGLU ? kTileF / 2 : kTileF), "one float4 per thread");
  const Split sp = split_plan(p, p.K / DK);
  if (sp.nseg <= 1) return;
  uint16_t *C = static_cast<uint16_t *>(p.C);
  for (int b = blockIdx.x; b < sp.rest * kWork; b += gridDim.x) {
    const int t = b / kWork;
    int e, row0, rows, nt;
    if (!find_tile<DBM>(p.offs, p.E, p.max_rows, p.n_tiles, sp.full + t, &e, &row0, &rows, &nt)) continue;
    const int gi = (b - t * kWork) * kThreads + threadIdx.x;
    // gi -> (wave, i, j, v4, lane); SwiGLU threads start from the gate tiles
    const int lane = gi & 63, v4 = (gi >> 6) & 3;
    const int rest = gi >> 8;
    const int j = rest % NJE, i = (rest / NJE) % MI, w = rest / (NJE * MI);
    const int64_t off = static_cast<int64_t>((((w * MI + i) * NJ + j) * 4 + v4) * kWave + lane);
    const f32x4 *src = reinterpret_cast<const f32x4 *>(p.part + static_cast<int64_t>(t) * sp.nseg * kTileF) + off;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < sp.nseg; ++g) {
      a += src[static_cast<int64_t>(g) * (kTileF / 4)];
      if (ACT == ACT_SWIGLU) u += src[static_cast<int64_t>(g) * (kTileF / 4) + (NJ / 2) * 4 * kWave];
    }
    const int wm = w >> 1, wn = w & 1;
    const int r0 = wm * RW + i * 32 + 8 * v4 + 4 * (lane >> 5);
    const int col = ACT == ACT_SWIGLU ? nt * (BN / 2) + wn * 64 + j * 32 + (lane & 31)
                                      : nt * BN + wn * 128 + j * 32 + (lane & 31);
    if (col >= p.n_out) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r0 + r >= rows) continue;
      const float v = ACT == ACT_SWIGLU ? silu_fast(a[r]) * u[r] : (ACT == ACT_GELU ? gelu_erf(a[r]) : a[r]);
      C[c_index(p, row0 + r0 + r, col)] = f32_to_bf16(v);
    }
  }
}

// fp32 path: plain FMA tiles (32 rows x 32 B rows), 2x2 outputs per thread,
// K in 64-wide chunks staged through LDS, the next chunk loaded into
// registers while the current one is multiplied.  The fp32 workloads are
// small: memory round trips (one per chunk) and each workgroup's own work,
// not bandwidth, set their time, hence small tiles and wide chunks.  Each
// output still sums its products in K order.
constexpr int F_BM = 32, F_BN = 32, F_BK = 64;
constexpr int F_TM = F_BM / 16;  // outputs per thread along each tile side (16 x 16 threads)
constexpr int F_LD = F_BM * F_BK / kThreads;  // elements of A (and of B) a thread stages per chunk

template <int ACT>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmParams p) {
  __shared__ float sA[F_BK][F_BM + 4];
  __shared__ float sB[F_BK][F_BN + 4];
  int e, row0, rows, nt;
  if (!map_tile<F_BM>(p.offs, p.E, p.max_rows, p.n_tiles, &e, &row0, &rows, &nt)) return;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const float *A = static_cast<const float *>(p.A);
  const float *B = static_cast<const float *>(p.B) + static_cast<int64_t>(e) * p.b_stride;
  float acc[F_TM][F_TM];
#pragma unroll
  for (int i = 0; i < F_TM; ++i)
#pragma unroll
    for (int j = 0; j < F_TM; ++j) acc[i][j] = 0.f;
  // element i of this thread's share: row r = q / F_BK, K offset kk = q % F_BK
  // of the chunk (q = tid + i * kThreads), so a wave reads whole 256-B runs
  float ra[F_LD], rb[F_LD];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < F_LD; ++i) {
      const int q = tid + i * kThreads;
      const int r = q / F_BK, kk = q % F_BK;
      const int gk = k0 + kk;
      const int64_t ar = row0 + min(r, rows - 1);
      ra[i] = gk < p.K ? A[ar * p.lda + gk] : 0.f;
      int br;
      if (ACT == ACT_SWIGLU) {
        const int col = nt * (F_BN / 2) + (r & (F_BN / 2 - 1));
        br = (col < p.n_out ? col : 0) + (r >= F_BN / 2 ? p.up_off : 0);
      } else {
        const int col = nt * F_BN + r;
        br = col < p.n_out ? col : 0;
      }
      rb[i] = gk < p.K ? B[static_cast<int64_t>(br) * p.ldb + gk] : 0.f;
    }
  };
  load(0);
  for (int k0 = 0; k0 < p.K; k0 += F_BK) {
#pragma unroll
    for (int i = 0; i < F_LD; ++i) {
      const int q = tid + i * kThreads;
      sA[q % F_BK][q / F_BK] = ra[i];
      sB[q % F_BK][q / F_BK] = rb[i];
    }
    __syncthreads();
    if (k0 + F_BK < p.K) load(k0 + F_BK);
#pragma unroll
    for (int kk = 0; kk < F_BK; ++kk) {
      float a[F_TM], b[F_TM];
#pragma unroll
      for (int i = 0; i < F_TM; ++i) a[i] = sA[kk][ty * F_TM + i];
#pragma unroll
      for (int j = 0; j < F_TM; ++j) {
        // SwiGLU: the first half of a thread's columns are gates, the second
        // half the matching up columns, F_BN / 2 further
        constexpr int H = F_TM / 2;
        const int bc = (ACT == ACT_SWIGLU) ? ((j < H) ? tx * H + j : F_BN / 2 + tx * H + (j - H)) : tx * F_TM + j;
        b[j] = sB[kk][bc];
      }
#pragma unroll
      for (int i = 0; i < F_TM; ++i)
#pragma unroll
        for (int j = 0; j < F_TM; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float *C = static_cast<float *>(p.C);
#pragma unroll
  for (int i = 0; i < F_TM; ++i) {
    const int lr = ty * F_TM + i;
    if (lr >= rows) continue;
    float *crow = C + static_cast<int64_t>(row0 + lr) * p.ldc;
    if (ACT == ACT_SWIGLU) {
#pragma unroll
      for (int j = 0; j < F_TM / 2; ++j) {
        const int col = nt * (F_BN / 2) + tx * (F_TM / 2) + j;
        if (col < p.n_out) crow[col] = silu(acc[i][j]) * acc[i][j + F_TM / 2];
      }
    } else {
#pragma unroll
      for (int j = 0; j < F_TM; ++j) {
        const int col = nt * F_BN + tx * F_TM + j;
        if (col < p.n_out) crow[col] = (ACT == ACT_GELU) ? gelu_erf(acc[i][j]) : acc[i][j];
      }
    }
  }
}

int64_t mtile_bound(int64_t rows, int E, int bm) { return rows / bm + std::min<int64_t>(E, rows); }

template <int BM>
hipError_t run_bf16(GemmParams p, int act, hipStream_t st) {
  p.m_tiles = static_cast<int>(mtile_bound(p.max_rows, p.E, BM));
  const int bn_out = act == ACT_SWIGLU ? BN / 2 : BN;
  p.n_tiles = (p.n_out + bn_out - 1) / bn_out;
  const int64_t blocks = static_cast<int64_t>(p.m_tiles) * p.n_tiles;
  if (blocks <= 0) return hipSuccess;
  if (act == ACT_SWIGLU) gemm_bf16_kernel<BM, ACT_SWIGLU><<<blocks, kThreads, 0, st>>>(p);
  else if (act == ACT_GELU) gemm_bf16_kernel<BM, ACT_GELU><<<blocks, kThreads, 0, st>>>(p);
  else gemm_bf16_kernel<BM, ACT_NONE><<<blocks, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t run_f32(GemmParams p, int act, hipStream_t st) {
  p.m_tiles = static_cast<int>(mtile_bound(p.max_rows, p.E, F_BM));
  const int bn_out = act == ACT_SWIGLU ? F_BN / 2 : F_BN;
  p.n_tiles = (p.n_out + bn_out - 1) / bn_out;
  const int64_t blocks = static_cast<int64_t>(p.m_tiles) * p.n_tiles;
  if (blocks <= 0) return hipSuccess;
  if (act == ACT_SWIGLU) gemm_f32_kernel<ACT_SWIGLU><<<blocks, kThreads, 0, st>>>(p);
  else if (act == ACT_GELU) gemm_f32_kernel<ACT_GELU><<<blocks, kThreads, 0, st>>>(p);
  else gemm_f32_kernel<ACT_NONE><<<blocks, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t run_bf16_dma(GemmParams p, int act, hipStream_t st) {
  p.m_tiles = static_cast<int>(mtile_bound(p.max_rows, p.E, DBM));
  const int bn_out = act == ACT_SWIGLU ? BN / 2 : BN;
  p.n_tiles = (p.n_out + bn_out - 1) / bn_out;
  const int64_t tiles = static_cast<int64_t>(p.m_tiles) * p.n_tiles;
  if (tiles <= 0) return hipSuccess;
  // whole-round tiles + at most one round of K-split pieces, then (when this
  // GEMM may split) the reduction of the split tiles, whose workgroups exit
  // at once when the device-side counts left nothing to split
  const int64_t blocks = tiles + p.units;
  const int rblocks = 1024;
  const bool reduce = p.max_split > 1 && p.slots > 1;
  constexpr int W = kDmaWaves;
  if (act == ACT_SWIGLU) {
    gemm_bf16_dma_kernel<ACT_SWIGLU, W><<<blocks, W * kWave, 0, st>>>(p);
    if (reduce) split_reduce_kernel<ACT_SWIGLU, W><<<rblocks, kThreads, 0, st>>>(p);
  } else if (act == ACT_GELU) {
    gemm_bf16_dma_kernel<ACT_GELU, W><<<blocks, W * kWave, 0, st>>>(p);
    if (reduce) split_reduce_kernel<ACT_GELU, W><<<rblocks, kThreads, 0, st>>>(p);
  } else {
    gemm_bf16_dma_kernel<ACT_NONE, W><<<blocks, W * kWave, 0, st>>>(p);
    if (reduce) split_reduce_kernel<ACT_NONE, W><<<rblocks, kThreads, 0, st>>>(p);
  }
  return hipGetLastError();
}

// Which kernel each GEMM of the FFN runs (the host never sees the per-expert
// row counts, so the choice follows the average rows per expert), and which
// of them may split their last round along K.
struct FfnPlan {
  int bm;
  bool dma1, dma2;      // GEMM1 / GEMM2 on the 256 x 256 direct-to-LDS kernel
  bool split1, split2;  // ... with enough K stages to split
  int sk1, sk2;         // GEMM1 / GEMM2 on the skinny kernel with this tile height (0: not)
};

// Experts averaging at most this many rows run the skinny (weight-streaming)
// kernel when K is a multiple of 64.
constexpr int64_t kSkinnyMaxAvgRows = 128;

FfnPlan plan_ffn(int dtype, int E, int d, int d_ff, int64_t max_rows, bool packed) {
  FfnPlan f{};
  const int64_t avg_rows = max_rows / E;
  if (packed) {
    // packed weights (bf16, d and d_ff multiples of 64) are read by the two
    // kernels that know the packed order: the skinny one up to
    // kSkinnyMaxAvgRows rows per expert, the 256-row one above
    f.bm = 256;
    f.sk1 = f.sk2 = avg_rows <= kSkinnyMaxAvgRows ? 64 : 0;
    f.dma1 = f.dma2 = f.sk1 == 0;
    f.split1 = f.dma1 && d / DK >= kSplitMinStages;
    f.split2 = f.dma2 && d_ff / DK >= kSplitMinStages;
    return f;
  }
  f.bm = avg_rows >= kDmaMinAvgRows ? 256 : 128;
  f.dma1 = dtype == 1 && f.bm == 256 && d % DK == 0;
  f.dma2 = dtype == 1 && f.bm == 256 && d_ff % DK == 0;
  f.split1 = f.dma1 && d / DK >= kSplitMinStages;
  f.split2 = f.dma2 && d_ff / DK >= kSplitMinStages;
  const int sk = 64;  // tile height (measured: 64 beats 32 even for decode batches)
  f.sk1 = dtype == 1 && avg_rows <= kSkinnyMaxAvgRows && d % 64 == 0 ? sk : 0;
  f.sk2 = dtype == 1 && avg_rows <= kSkinnyMaxAvgRows && d_ff % 64 == 0 ? sk : 0;
  return f;
}

// Scratch: the fp32 partial tiles of the K-split pieces (the two GEMMs run
// one after the other and share it).
constexpr size_t kPartTileBytes = static_cast<size_t>(DBM) * BN * sizeof(float);

// Workgroups in one round: one per CU (the kernel's 160 KB of LDS allows one
// per CU), at most kSplitUnits.
int round_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = kSplitUnits;
  n = std::max(8, std::min(n, kSplitUnits));
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}


}  // namespace

size_t ffn_scratch_bytes(int dtype, int E, int d, int d_ff, int64_t max_rows, bool packed) {
  if (max_rows == 0) return 0;
  const FfnPlan f = plan_ffn(dtype, E, d, d_ff, max_rows, packed);
  size_t need = 0;
  if (f.split1 || f.split2) {
    // the pieces of one round: at most kSplitUnits, and at most kMaxSplit per
    // tile of the larger GEMM
    const int64_t mt = mtile_bound(max_rows, E, DBM);
    const int64_t nt = std::max<int64_t>((d_ff + BN / 2 - 1) / (BN / 2), (d + BN - 1) / BN);
    const int64_t pieces = std::min<int64_t>(kSplitUnits, mt * nt * kMaxSplit);
    need = static_cast<size_t>(pieces) * kPartTileBytes;
  }
  const int sk = std::max(f.sk1, f.sk2);
  if (sk) need = std::max(need, static_cast<size_t>(kSkinnyMaxPieces) * skinny_part_tile_bytes(sk));
  return need;
}

hipError_t launch_expert_ffn(const FfnArgs &a, hipStream_t st) {
  if (a.max_rows == 0) return hipSuccess;
  const int n_up = a.act == 1 ? 2 : 1;
  const FfnPlan f = plan_ffn(a.dtype, a.E, a.d, a.d_ff, a.max_rows, a.packed);
  const size_t need = ffn_scratch_bytes(a.dtype, a.E, a.d, a.d_ff, a.max_rows, a.packed);
  if (a.scratch_bytes < need || (need > 0 && a.scratch == nullptr)) return hipErrorInvalidValue;
  // packed weights: bf16 only, no kept pre-activations, both GEMMs on a
  // kernel that reads the packed order
  if (a.packed && (a.dtype != 1 || a.z || a.d % 64 || a.d_ff % 64 || !(f.dma1 || f.sk1) || !(f.dma2 || f.sk2)))
    return hipErrorInvalidValue;
  if (a.x_kb && !a.packed) return hipErrorInvalidValue;
  float *part = static_cast<float *>(a.scratch);
  const int units = round_units();
  const int slots = static_cast<int>(std::min<size_t>(kSplitUnits, need / kPartTileBytes));
  const int sk_slots = std::max(f.sk1, f.sk2)
                           ? static_cast<int>(std::min<size_t>(kSkinnyMaxPieces,
                                                               need / skinny_part_tile_bytes(std::max(f.sk1, f.sk2))))
                           : 0;
  GemmParams g1{};
  g1.A = a.x_perm;
  g1.lda = a.d;
  g1.B = a.w1;
  g1.ldb = a.d;
  g1.b_stride = a.packed ? static_cast<int64_t>(packed_weight_bytes(1, a.d_ff, a.d, a.act == 1) / 2)
                         : static_cast<int64_t>(n_up) * a.d_ff * a.d;
  g1.packed = a.packed;
  g1.a_kb = a.x_kb;
  g1.c_kb = a.packed;  // h K-blocked: GEMM2 reads its stages contiguously
  g1.C = a.h;
  g1.ldc = a.d_ff;
  g1.offs = a.expert_offset;
  g1.E = a.E;
  g1.K = a.d;
  g1.n_out = a.d_ff;
  g1.up_off = a.d_ff;
  g1.max_rows = a.max_rows;
  g1.part = part;
  g1.units = units;
  g1.slots = slots;
  g1.max_split = f.split1 ? kMaxSplit : 1;
  // training forward: GEMM1 keeps its raw pre-activations z (both SwiGLU
  // halves), a second pass applies the activation
  int act1 = a.act == 1 ? ACT_SWIGLU : ACT_GELU;
  if (a.z) {
    g1.C = a.z;
    g1.ldc = static_cast<int64_t>(n_up) * a.d_ff;
    g1.n_out = n_up * a.d_ff;
    act1 = ACT_NONE;
  }
  hipError_t err;
  if (a.dtype == 0) {
    err = run_f32(g1, act1, st);
  } else if (f.dma1) {
    err = run_bf16_dma(g1, act1, st);
  } else if (f.sk1) {
    g1.slots = sk_slots;
    g1.max_split = sk_slots > 0 ? kSkinnyMaxSplit : 1;
    err = run_bf16_skinny(g1, act1, f.sk1, st);
  } else {
    err = f.bm == 256 ? run_bf16<256>(g1, act1, st) : run_bf16<128>(g1, act1, st);
  }
  if (err != hipSuccess) return err;
  if (a.z && (err = launch_act_fwd(a.dtype, a.act == 1 ? ACT_SWIGLU : ACT_GELU, a.z, a.h, a.expert_offset + a.E,
                                   a.max_rows, a.d_ff, st)) != hipSuccess)
    return err;
  GemmParams g2{};
  g2.A = a.h;
  g2.lda = a.d_ff;
  g2.B = a.w2;
  g2.ldb = a.d_ff;
  g2.b_stride = a.packed ? static_cast<int64_t>(packed_weight_bytes(1, a.d, a.d_ff, false) / 2)
                         : static_cast<int64_t>(a.d) * a.d_ff;
  g2.packed = a.packed;
  g2.a_kb = a.packed;
  g2.C = a.y_perm;
  g2.ldc = a.d;
  g2.offs = a.expert_offset;
  g2.E = a.E;
  g2.K = a.d_ff;
  g2.n_out = a.d;
  g2.up_off = 0;
  g2.max_rows = a.max_rows;
  g2.part = part;
  g2.units = units;
  g2.slots = slots;
  g2.max_split = f.split2 ? kMaxSplit : 1;
  if (a.dtype == 0) return run_f32(g2, ACT_NONE, st);
  if (f.dma2) return run_bf16_dma(g2, ACT_NONE, st);
  if (f.sk2) {
    g2.slots = sk_slots;
    g2.max_split = sk_slots > 0 ? kSkinnyMaxSplit : 1;
    return run_bf16_skinny(g2, ACT_NONE, f.sk2, st);
  }
  return f.bm == 256 ? run_bf16<256>(g2, ACT_NONE, st) : run_bf16<128>(g2, ACT_NONE, st);
}

__global__ void fill_offsets_kernel(int32_t *dst, int32_t t, const int32_t *stamp) {
  if (threadIdx.x == 0) {
    dst[0] = 0;
    dst[1] = (stamp && *stamp == kStampTrain) ? 0 : t;
  }
}

hipError_t launch_fill_offsets(int32_t *dst, int32_t t, hipStream_t st, const int32_t *stamp) {
  fill_offsets_kernel<<<1, 64, 0, st>>>(dst, t, stamp);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weight packing (the order is described beside kPackBlockBytes): one thread
// per 16-B chunk of the packed buffer, grid-stride.  Four neighbouring
// threads read one row's 64 B of a 32-wide K slice; the writes are
// contiguous.  A one-off transform, run when the weights are loaded.
namespace {

__global__ __launch_bounds__(256) void pack_weights_kernel(PackArgs a, int64_t chunks, int nk, int n_tiles) {
  const char *src = static_cast<const char *>(a.src);
  char *dst = static_cast<char *>(a.dst);
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; g < chunks;
       g += static_cast<int64_t>(gridDim.x) * 256) {
    const int q = static_cast<int>(g & 1023);
    const int64_t blk = g >> 10;  // (e * n_tiles + nt) * nk + kb
    const int kb = static_cast<int>(blk % nk);
    const int64_t et = blk / nk;
    const int nt = static_cast<int>(et % n_tiles);
    const int64_t e = et / n_tiles;
    const int r = q >> 2, c = (q & 3) ^ ((r >> 2) & 3);
    int col, row;
    if (a.swiglu) {
      col = nt * (BN / 2) + (r & (BN / 2 - 1));
      row = col + (r >= BN / 2 ? a.n_out : 0);
    } else {
      col = nt * BN + r;
      row = col;
    }
    u32x4 v = {0u, 0u, 0u, 0u};
    if (col < a.n_out)
      v = *reinterpret_cast<const u32x4 *>(
          src + ((e * a.n_rows + row) * static_cast<int64_t>(a.K) + kb * kPackK + c * 8) * 2);
    *reinterpret_cast<u32x4 *>(dst + g * 16) = v;
  }
}

}  // namespace

size_t packed_weight_bytes(int E, int n_out, int K, bool swiglu) {
  const int64_t n_tiles = swiglu ? (n_out + BN / 2 - 1) / (BN / 2) : (n_out + BN - 1) / BN;
  return static_cast<size_t>(E) * static_cast<size_t>(n_tiles) * static_cast<size_t>(K / kPackK) * kPackBlockBytes;
}

hipError_t launch_pack_weights(const PackArgs &a, hipStream_t st) {
  if (a.E <= 0 || a.n_out <= 0 || a.K <= 0 || a.K % kPackK) return hipErrorInvalidValue;
  const int n_tiles = a.swiglu ? (a.n_out + BN / 2 - 1) / (BN / 2) : (a.n_out + BN - 1) / BN;
  const int64_t chunks = static_cast<int64_t>(packed_weight_bytes(a.E, a.n_out, a.K, a.swiglu) / 16);
  const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, 16384);
  pack_weights_kernel<<<static_cast<unsigned>(blocks), 256, 0, st>>>(a, chunks, a.K / kPackK, n_tiles);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped GEMMs of the backward pass.  bf16: the recomputed forward GEMM
// (NT) takes the kernel the forward would (256-row direct-to-LDS, skinny or
// 128-row); the data-gradient GEMMs (NN) run the 256-row kernel with its B
// operand staged as [K][N] when K is a multiple of 32; the weight-gradient
// GEMMs (TN) run it with both operands staged as [K][.] over each group's
// rows (multiples of 32 by construction).  Everything else (fp32, other K)
// runs the generic kernel.
namespace {

enum { BP_GENERIC = 0, BP_DMA = 1, BP_SKINNY = 2, BP_V1 = 3 };

struct BwdPlan {
  int path;
  bool split;
};

BwdPlan plan_bwd(const BwdGemm &g) {
  BwdPlan b{BP_GENERIC, false};
  if (g.dtype != 1 || g.E <= 0) return b;
  const int64_t avg = g.max_rows / g.E;
  if (g.kind == BWD_TN) {
    b.path = BP_DMA;
  } else if (g.kind == BWD_NN) {
    if (g.K % DK == 0) {
      b.path = BP_DMA;
      b.split = g.K / DK >= kSplitMinStages;
    }
  } else {
    if (avg >= kDmaMinAvgRows && g.K % DK == 0) {
      b.path = BP_DMA;
      b.split = g.K / DK >= kSplitMinStages;
    } else if (avg <= kSkinnyMaxAvgRows && g.K % 64 == 0) {
      b.path = BP_SKINNY;
    } else {
      b.path = BP_V1;
    }
  }
  return b;
}

GemmParams bwd_params(const BwdGemm &g) {
  GemmParams p{};
  p.A = g.A;
  p.lda = g.lda;
  p.B = g.B;
  p.ldb = g.ldb;
  p.b_stride = g.b_stride;
  p.C = g.C;
  p.ldc = g.ldc;
  p.offs = g.offs;
  p.E = g.E;
  p.K = g.K;
  p.n_out = g.N;
  p.up_off = 0;
  p.max_rows = g.max_rows;
  p.c_stride = g.c_stride;
  p.m_rows = g.M;
  p.units = round_units();
  p.max_split = 1;
  return p;
}

hipError_t run_bwd_dma(GemmParams p, int kind, hipStream_t st) {
  constexpr int W = kDmaWaves;
  if (kind == BWD_TN) {
    p.m_tiles = (p.m_rows + DBM - 1) / DBM;
    p.n_tiles = (p.n_out + BN - 1) / BN;
    const int64_t blocks = static_cast<int64_t>(p.E) * p.m_tiles * p.n_tiles;
    if (blocks <= 0) return hipSuccess;
    gemm_bf16_dma_kernel<ACT_NONE, W, LAY_TN><<<blocks, W * kWave, 0, st>>>(p);
    return hipGetLastError();
  }
  p.m_tiles = static_cast<int>(mtile_bound(p.max_rows, p.E, DBM));
  p.n_tiles = (p.n_out + BN - 1) / BN;
  const int64_t tiles = static_cast<int64_t>(p.m_tiles) * p.n_tiles;
  if (tiles <= 0) return hipSuccess;
  const int64_t blocks = tiles + p.units;
  const bool reduce = p.max_split > 1 && p.slots > 1;
  if (kind == BWD_NN) gemm_bf16_dma_kernel<ACT_NONE, W, LAY_NN><<<blocks, W * kWave, 0, st>>>(p);
  else gemm_bf16_dma_kernel<ACT_NONE, W, LAY_NT><<<blocks, W * kWave, 0, st>>>(p);
  if (reduce) split_reduce_kernel<ACT_NONE, W><<<1024, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

size_t bwd_gemm_scratch_bytes(const BwdGemm &g) {
  if (g.max_rows <= 0) return 0;
  const BwdPlan b = plan_bwd(g);
  if (b.path == BP_DMA && b.split) {
    const int64_t mt = mtile_bound(g.max_rows, g.E, DBM);
    const int64_t nt = (g.N + BN - 1) / BN;
    return static_cast<size_t>(std::min<int64_t>(kSplitUnits, mt * nt * kMaxSplit)) * kPartTileBytes;
  }
  if (b.path == BP_SKINNY) return static_cast<size_t>(kSkinnyMaxPieces) * skinny_part_tile_bytes(64);
  return 0;
}

hipError_t launch_bwd_gemm(const BwdGemm &g, hipStream_t st) {
  const BwdPlan b = plan_bwd(g);
  const size_t need = bwd_gemm_scratch_bytes(g);
  if (need > 0 && (g.scratch == nullptr || g.scratch_bytes < need)) return hipErrorInvalidValue;
  if (b.path == BP_DMA) {
    GemmParams p = bwd_params(g);
    if (b.split) {
      p.part = static_cast<float *>(g.scratch);
      p.slots = static_cast<int>(std::min<size_t>(kSplitUnits, need / kPartTileBytes));
      p.max_split = kMaxSplit;
    }
    return run_bwd_dma(p, g.kind, st);
  }
  if (b.path == BP_SKINNY) {
    GemmParams p = bwd_params(g);
    p.part = static_cast<float *>(g.scratch);
    p.slots = static_cast<int>(std::min<size_t>(kSkinnyMaxPieces, need / skinny_part_tile_bytes(64)));
    p.max_split = p.slots > 0 ? kSkinnyMaxSplit : 1;
    return run_bf16_skinny(p, ACT_NONE, 64, st);
  }
  if (b.path == BP_V1) {
    GemmParams p = bwd_params(g);
    return g.max_rows / g.E >= kDmaMinAvgRows ? run_bf16<256>(p, ACT_NONE, st) : run_bf16<128>(p, ACT_NONE, st);
  }
  GenGemmArgs a{};
  a.A = g.A;
  a.B = g.B;
  a.C = g.C;
  a.offs = g.offs;
  a.E = g.E;
  a.max_rows = g.max_rows;
  a.N = g.N;
  a.K = g.K;
  a.M = g.M;
  a.c_rs = g.ldc;
  if (g.kind == BWD_TN) {
    a.mode = 1;
    a.a_rs = 1;
    a.a_ks = g.lda;
    a.b_ks = g.ldb;
    a.b_cs = 1;
    a.c_es = g.c_stride;
  } else {
    a.mode = 0;
    a.a_rs = g.lda;
    a.a_ks = 1;
    a.b_es = g.b_stride;
    if (g.kind == BWD_NT) {
      a.b_ks = 1;
      a.b_cs = g.ldb;
    } else {
      a.b_ks = g.ldb;
      a.b_cs = 1;
    }
  }
  return launch_gemm_generic(a, g.dtype, g.dtype, g.dtype, st);
}

}  // namespace moe
