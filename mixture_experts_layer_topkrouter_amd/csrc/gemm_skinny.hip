// Grouped expert GEMM for experts that receive few rows (tens, or a handful
// when decoding): the same computation as gemm.hip (MoELayer step 2 of
// "How MegaDLMs Implements Mixture of Experts (MoE) Architectures", section
// "Core MoE Layer Architecture"), laid out for the regime where streaming the
// expert weights from HBM, not the matrix core, bounds the time.
//
// gfx950 design (bf16, K a multiple of 64):
// * tile BM (64; 32 also compiles) rows x 256 weight rows; 4 waves side by side, each
//   owning BM x 64 outputs (BM/32 x 2 tiles of v_mfma_f32_32x32x16_bf16;
//   SwiGLU: 32 gate and the 32 matching up columns, so the epilogue stays
//   lane-local).
// * K advances in 64-wide stages, so every operand row of a stage is one
//   whole 128-byte line (a 64-byte half line costs a CU the same request
//   slot as a whole one), loaded straight into LDS.  The ring holds two
//   stages (80 KB), so two workgroups share a CU and each streams the next
//   stage while it multiplies the current one; measured against a 4-deep
//   ring with one workgroup per CU this is 25 % faster on the Switch-style
//   experts (all 288 tiles of the up projection run at once) and no slower
//   on decode batches.  LDS rows are 128 B with 16-B chunk c of row r at
//   c ^ ((r >> 1) & 7): the 16 rows of a 16-lane fragment read hit distinct
//   bank groups.
// * few experts x few row tiles leave most CUs idle, so when the real tile
//   count is below kSkinnyTarget each tile is cut along K into pieces (at
//   least kPieceStages stages each); pieces store fp32 partials and
//   skinny_reduce_kernel adds them in K order and applies the epilogue, so
//   results do not depend on timing.
#include "gemm_common.h"

namespace moe {
namespace {

constexpr int SK = 64;                // K per stage
constexpr int SBN = 256;              // weight rows per tile
constexpr int kSkinnyTarget = 512;    // workgroups the K split aims for
constexpr int kPieceStages = 4;       // a K piece keeps at least this many stages
constexpr int kSkinnyStages = 2;      // LDS ring depth: 2 stages (80 KB), two workgroups per CU
// Weight loads carry the non-temporal hint when K is at least this long
// (each weight tile is read by one workgroup only).
constexpr int kSkinnyNtMinK = 4096;
static_assert(kSkinnyTarget <= kSkinnyMaxPieces, "partial buffer holds every piece");

template <int BM>
struct Sk {
  static constexpr int MI = BM / 32, NJ = 2;
  static constexpr int A_ELEMS = BM * SK, STAGE = (BM + SBN) * SK;  // uint16 elements
  static constexpr int A_INSTR = BM / 32;   // A loads per wave per stage (8 rows x 128 B each)
  static constexpr int B_INSTR = SBN / 32;  // B loads per wave per stage
  static constexpr int ND = A_INSTR + B_INSTR;
  static constexpr int TILE_F = BM * SBN;   // floats of a partial tile
};

struct SkJob {
  int e, row0, rows, nt;
  int kb, ke;           // K stages [kb, ke)
  int slot, nseg;       // partial slot (tile * nseg + piece) and pieces per tile
};

// Pieces per tile: enough to give about kSkinnyTarget workgroups, limited
// by the stages of K and by the partial buffer.
__device__ __forceinline__ int skinny_nseg(const GemmParams &p, int total, int nk) {
  if (p.max_split <= 1 || total <= 0 || total >= kSkinnyTarget) return 1;
  int n = min(min(kSkinnyTarget / total, nk / kPieceStages), p.max_split);
  n = min(n, p.slots / total);
  return max(n, 1);
}

template <int BM>
__device__ __forceinline__ bool skinny_job(const GemmParams &p, int nk, SkJob *j) {
  const int total = count_mtiles<BM>(p.offs, p.E, p.max_rows) * p.n_tiles;
  const int nseg = skinny_nseg(p, total, nk);
  const int n = total * nseg;
  if (static_cast<int>(blockIdx.x) >= n) return false;
  // piece-major in XCD-contiguous runs: the pieces one XCD runs together
  // read the same K slice of neighbouring tiles
  const int u = xcd_remap(blockIdx.x, n);
  const int seg = u / total, t = u - seg * total;
  j->kb = __builtin_amdgcn_readfirstlane(seg * nk / nseg);
  j->ke = __builtin_amdgcn_readfirstlane((seg + 1) * nk / nseg);
  j->slot = __builtin_amdgcn_readfirstlane(t * nseg + seg);
  j->nseg = __builtin_amdgcn_readfirstlane(nseg);
  return find_tile<BM>(p.offs, p.E, p.max_rows, p.n_tiles, t, &j->e, &j->row0, &j->rows, &j->nt);
}

// LDS row of 128 B: element offset of logical chunk c of row r
__device__ __forceinline__ int sk_chunk(int r, int c) { return r * SK + ((c ^ ((r >> 1) & 7)) << 3); }

template <int ACT, int BM, int SST, bool BNT>
__global__ __launch_bounds__(kThreads) void gemm_bf16_skinny_kernel(GemmParams p) {
  using C = Sk<BM>;
  constexpr int MI = C::MI, NJ = C::NJ;
  static_assert(SST >= 2 && SST <= 4, "ring of 2 to 4 stages");
  __shared__ __attribute__((aligned(1024))) uint16_t ring[SST][C::STAGE];
  SkJob job;
  if (!skinny_job<BM>(p, p.K / SK, &job)) return;
  const int rows = job.rows, nt = job.nt;
  const int l = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
  // K-blocked A: a 64-wide stage is two 32-wide slices, max_rows row pieces
  // apart
  static_assert(SK * 2 == 2 * kKbRowBytes, "a stage row is two K-blocked row pieces");
  const bool a_kb = p.a_kb != 0;
  const int64_t kb_slice = p.max_rows * kKbRowBytes;  // bytes between consecutive 32-wide slices
  const char *A = static_cast<const char *>(p.A) +
                  (a_kb ? 2 * job.kb * kb_slice + static_cast<int64_t>(job.row0) * kKbRowBytes
                        : (static_cast<int64_t>(job.row0) * p.lda + job.kb * SK) * 2);
  const int64_t a_step = a_kb ? 2 * kb_slice : SK * 2;
  // packed B: a 64-wide stage is the column tile's two consecutive 32-wide
  // blocks, 32 KB contiguous
  static_assert(SK == 2 * kPackK && SBN == BN, "a stage is two packed blocks of one column tile");
  const bool packed = p.packed != 0;
  const char *B = static_cast<const char *>(p.B) +
                  (packed ? static_cast<int64_t>(job.e) * p.b_stride * 2 +
                                (static_cast<int64_t>(nt) * (p.K / kPackK) + 2 * job.kb) * kPackBlockBytes
                          : (static_cast<int64_t>(job.e) * p.b_stride + job.kb * SK) * 2);
  const int64_t b_step = packed ? 2 * kPackBlockBytes : SK * 2;

  auto slot = [&](auto S) -> uint16_t * { return ring[decltype(S)::value]; };

  // load instruction g of an operand fills LDS rows 8g .. 8g+7 (1 KB); lane q
  // -> row 8g + q/8, stored chunk q%8, which holds logical chunk
  // (q%8) ^ ((row >> 1) & 7).  Wave w issues g = w, w+4, ...
  uint32_t a_off[C::A_INSTR], b_off[C::B_INSTR];
#pragma unroll
  for (int i = 0; i < C::A_INSTR; ++i) {
    const int r = 8 * (w + 4 * i) + (l >> 3);
    const int c = (l & 7) ^ ((r >> 1) & 7);
    // rows past the tile's last real row load as zeros (dma16_zp)
    a_off[i] = r >= rows ? kDmaSkip
               : a_kb    ? static_cast<uint32_t>((c >> 2) * kb_slice + r * kKbRowBytes + (c & 3) * 16)
                         : static_cast<uint32_t>((static_cast<int64_t>(r) * p.lda + c * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < C::B_INSTR; ++i) {
    const int r = 8 * (w + 4 * i) + (l >> 3);
    const int c = (l & 7) ^ ((r >> 1) & 7);
    int br;
    if (ACT == ACT_SWIGLU) {
      const int col = nt * (SBN / 2) + (r & (SBN / 2 - 1));
      br = (col < p.n_out ? col : 0) + (r >= SBN / 2 ? p.up_off : 0);
    } else {
      const int col = nt * SBN + r;
      br = col < p.n_out ? col : 0;
    }
    // packed: logical chunk c of row r sits in block c/4 at chunk
    // 4r + ((c%4) ^ ((r/4)%4))
    b_off[i] = packed ? static_cast<uint32_t>((c >> 2) * kPackBlockBytes + (4 * r + ((c & 3) ^ ((r >> 2) & 3))) * 16)
                      : static_cast<uint32_t>((static_cast<int64_t>(br) * p.ldb + c * 8) * 2);
  }
  auto issue = [&](auto S, int st) {
    const uint32_t base = lds_addr_of(slot(S));
#pragma unroll
    for (int i = 0; i < C::A_INSTR; ++i) dma16_zp(a_off[i], A + st * a_step, base + (w + 4 * i) * 1024);
#pragma unroll
    for (int i = 0; i < C::B_INSTR; ++i)
      if constexpr (BNT) dma16_nt(b_off[i], B + st * b_step, base + C::A_ELEMS * 2 + (w + 4 * i) * 1024);
      else dma16(b_off[i], B + st * b_step, base + C::A_ELEMS * 2 + (w + 4 * i) * 1024);
  };

  // fragment rows: A tile i rows i*32 + l%32; B tile j rows brow[j] + l%32
  int brow[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) brow[j] = ACT == ACT_SWIGLU ? j * (SBN / 2) + w * 32 : w * 64 + j * 32;

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = job.ke - job.kb;
  // stage st lives in slot st % SST; stages 0 .. SST-2 go out first
  if (0 < nk) issue(Slot<0>{}, 0);
  if (SST > 2 && 1 < nk) issue(Slot<1 % SST>{}, 1);
  if (SST > 3 && 2 < nk) issue(Slot<2 % SST>{}, 2);

  // iteration kt: wait for stage kt (stages up to kt+SST-2 issued), barrier
  // (it also tells that every wave is done with stage kt-1), refill stage
  // kt-1's slot with stage kt+SST-1, multiply stage kt
  auto iter = [&](auto S, int kt) {
    constexpr int s = decltype(S)::value;
    const int ahead = min(nk - 1, kt + SST - 2) - kt;
    if (ahead >= 2) wait_vm<2 * C::ND>();
    else if (ahead == 1) wait_vm<C::ND>();
    else wait_vm<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (kt + SST - 1 < nk) issue(Slot<(s + SST - 1) % SST>{}, kt + SST - 1);
    const uint16_t *ls = slot(S);
#pragma unroll
    for (int ks = 0; ks < SK / 16; ++ks) {
      bf16x8 fa[MI], fb[NJ];
      const int ch = 2 * ks + (l >> 5);
#pragma unroll
      for (int i = 0; i < MI; ++i)
        fa[i] = *reinterpret_cast<const bf16x8 *>(ls + sk_chunk(i * 32 + (l & 31), ch));
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        fb[j] = *reinterpret_cast<const bf16x8 *>(ls + C::A_ELEMS + sk_chunk(brow[j] + (l & 31), ch));
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };
  int kt = 0;
  for (; kt + SST - 1 < nk; kt += SST) {
    iter(Slot<0>{}, kt);
    iter(Slot<1>{}, kt + 1);
    if constexpr (SST > 2) iter(Slot<2 % SST>{}, kt + 2);
    if constexpr (SST > 3) iter(Slot<3 % SST>{}, kt + 3);
  }
  if (kt < nk) iter(Slot<0>{}, kt);
  if (SST > 2 && kt + 1 < nk) iter(Slot<1 % SST>{}, kt + 1);
  if (SST > 3 && kt + 2 < nk) iter(Slot<2 % SST>{}, kt + 2);

  // value v of lane l in a 32x32 result: row 8*(v/4) + 4*(l/32) + v%4,
  // column l%32
  if (job.nseg > 1) {
    // K piece: fp32 partial in accumulator order (float4 index
    // ((w*MI + i)*NJ + j)*4*64 + v4*64 + l); rows past the tile's rows are
    // neither stored nor read back
    f32x4 *dst = reinterpret_cast<f32x4 *>(p.part + static_cast<int64_t>(job.slot) * C::TILE_F) +
                 w * (MI * NJ * 4 * kWave) + l;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
          if (i * 32 + 8 * v4 + 4 * (l >> 5) < rows)
            dst[((i * NJ + j) * 4 + v4) * kWave] =
                f32x4{acc[i][j][4 * v4], acc[i][j][4 * v4 + 1], acc[i][j][4 * v4 + 2], acc[i][j][4 * v4 + 3]};
    return;
  }
  uint16_t *Cp = static_cast<uint16_t *>(p.C);
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = i * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
      if (r >= rows) continue;
      const int64_t grow = job.row0 + r;
      if (ACT == ACT_SWIGLU) {
        const int col = nt * (SBN / 2) + w * 32 + (l & 31);
        if (col < p.n_out) Cp[c_index(p, grow, col)] = f32_to_bf16(silu_fast(acc[i][0][v]) * acc[i][1][v]);
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int col = nt * SBN + w * 64 + j * 32 + (l & 31);
          const float x = acc[i][j][v];
          if (col < p.n_out) Cp[c_index(p, grow, col)] = f32_to_bf16(ACT == ACT_GELU ? gelu_erf(x) : x);
        }
      }
    }
  }
}

// Adds the K pieces of every split tile in piece order and applies the
// epilogue: one thread per float4 of the accumulator layout (SwiGLU: per
// gate float4, which also reads its up partner), grid-stride.
template <int ACT, int BM>
__global__ __launch_bounds__(kThreads) void skinny_reduce_kernel(GemmParams p) {
  using C = Sk<BM>;
  constexpr int MI = C::MI, NJ = C::NJ;
  constexpr int NJE = ACT == ACT_SWIGLU ? 1 : NJ;
  constexpr int kGroups = 4 * MI * NJE * 4 * kWave;  // float4 groups a tile hands out
  constexpr int kWork = kGroups / kThreads;
  const int nk = p.K / SK;
  const int total = count_mtiles<BM>(p.offs, p.E, p.max_rows) * p.n_tiles;
  const int nseg = skinny_nseg(p, total, nk);
  if (nseg <= 1) return;
  uint16_t *Cp = static_cast<uint16_t *>(p.C);
  for (int b = blockIdx.x; b < total * kWork; b += gridDim.x) {
    const int t = b / kWork;
    int e, row0, rows, nt;
    if (!find_tile<BM>(p.offs, p.E, p.max_rows, p.n_tiles, t, &e, &row0, &rows, &nt)) continue;
    const int gi = (b - t * kWork) * kThreads + threadIdx.x;
    const int lane = gi & 63, v4 = (gi >> 6) & 3;
    const int rest = gi >> 8;
    const int j = rest % NJE, i = (rest / NJE) % MI, w = rest / (NJE * MI);
    const int r0 = i * 32 + 8 * v4 + 4 * (lane >> 5);
    if (r0 >= rows) continue;
    const int64_t off = static_cast<int64_t>((((w * MI + i) * NJ + j) * 4 + v4) * kWave + lane);
    const f32x4 *src = reinterpret_cast<const f32x4 *>(p.part + static_cast<int64_t>(t) * nseg * C::TILE_F) + off;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < nseg; ++g) {
      a += src[static_cast<int64_t>(g) * (C::TILE_F / 4)];
      if (ACT == ACT_SWIGLU) u += src[static_cast<int64_t>(g) * (C::TILE_F / 4) + 4 * kWave];
    }
    const int col = ACT == ACT_SWIGLU ? nt * (SBN / 2) + w * 32 + (lane & 31) : nt * SBN + w * 64 + j * 32 + (lane & 31);
    if (col >= p.n_out) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r0 + r >= rows) continue;
      const float v = ACT == ACT_SWIGLU ? silu_fast(a[r]) * u[r] : (ACT == ACT_GELU ? gelu_erf(a[r]) : a[r]);
      Cp[c_index(p, row0 + r0 + r, col)] = f32_to_bf16(v);
    }
  }
}

int64_t sk_mtile_bound(int64_t rows, int E, int bm) { return rows / bm + std::min<int64_t>(E, rows); }

template <int ACT, int BM>
void launch_skinny(const GemmParams &p, int64_t blocks, bool reduce, hipStream_t st) {
  if (p.K >= kSkinnyNtMinK) gemm_bf16_skinny_kernel<ACT, BM, kSkinnyStages, true><<<blocks, kThreads, 0, st>>>(p);
  else gemm_bf16_skinny_kernel<ACT, BM, kSkinnyStages, false><<<blocks, kThreads, 0, st>>>(p);
  if (reduce) skinny_reduce_kernel<ACT, BM><<<1024, kThreads, 0, st>>>(p);
}

}  // namespace

size_t skinny_part_tile_bytes(int bm) { return static_cast<size_t>(bm) * SBN * sizeof(float); }

hipError_t run_bf16_skinny(GemmParams p, int act, int bm, hipStream_t st) {
  p.m_tiles = static_cast<int>(sk_mtile_bound(p.max_rows, p.E, bm));
  const int bn_out = act == ACT_SWIGLU ? SBN / 2 : SBN;
  p.n_tiles = (p.n_out + bn_out - 1) / bn_out;
  const int64_t tiles = static_cast<int64_t>(p.m_tiles) * p.n_tiles;
  if (tiles <= 0) return hipSuccess;
  // whole tiles, or at most kSkinnyTarget pieces when the K split applies
  const int64_t blocks = std::max<int64_t>(tiles, kSkinnyTarget);
  const bool reduce = p.max_split > 1 && p.slots > 1;
  if (bm != 64) return hipErrorInvalidValue;  // the only height instantiated
  if (act == ACT_SWIGLU) launch_skinny<ACT_SWIGLU, 64>(p, blocks, reduce, st);
  else if (act == ACT_GELU) launch_skinny<ACT_GELU, 64>(p, blocks, reduce, st);
  else launch_skinny<ACT_NONE, 64>(p, blocks, reduce, st);
  return hipGetLastError();
}

}  // namespace moe
