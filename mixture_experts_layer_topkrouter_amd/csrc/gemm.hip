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
//   the number of (expert, 256- or 128-row) tiles times the column tiles, and
//   each workgroup finds its expert from the device-side expert offsets (a
//   64-lane prefix sum over per-expert tile counts), so the host never reads
//   how many rows each expert received.  Surplus workgroups exit at once.
// * tile BM x 256 x 64 with 4 waves in a 2 x 2 grid; each wave owns a
//   BM/2 x 128 sub-tile of v_mfma_f32_16x16x32_bf16 results (fp32 accumulators).
//   Both operands are K-contiguous ([rows, K] activations, [out, in] weights),
//   so each lane's MFMA fragment is one 16-byte LDS read.
// * operands are staged global -> registers -> LDS, double-buffered: the
//   next K slice is in flight while the current one feeds the MFMAs.  LDS
//   rows are 128 B; the 16-B chunk c of row r is stored at chunk c ^ (r & 7),
//   so the 16 rows a fragment read touches hit distinct banks.
// * SwiGLU: the B tile holds 128 gate rows and the 128 matching up rows, and
//   every wave computes the same output columns for both, so the epilogue
//   silu(gate) * up is lane-local.  GELU is applied in the epilogue as well:
//   the hidden activation is written once, in bf16.
// * workgroup ids are remapped so the 8 XCDs each take a contiguous range of
//   tiles, walked in groups of 4 row tiles, so tiles that share weights or
//   rows run together on one XCD and hit its L2.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int BK = 64;
constexpr int BN = 256;  // B rows per tile
constexpr int kGroupM = 4;

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
};

__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.f + erff(z * 0.70710678118654752f)); }
__device__ __forceinline__ float silu(float z) { return z / (1.f + expf(-z)); }

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = nblocks >> 3, rem = nblocks & 7;
  return xcd * per + min(xcd, rem) + slot;
}

// Global m-tile index -> (expert, first row, valid rows).  Wave 0 scans the
// per-expert tile counts; the result is broadcast through LDS.
template <int BM>
__device__ __forceinline__ void find_tile(const int32_t *__restrict__ offs, int E, int64_t max_rows, int mt,
                                          int *info) {
  if (wave_id() == 0) {
    const int l = lane_id();
    int carry = 0;
    bool found = false;
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int e = e0 + l;
      int o0 = 0, me = 0;
      if (e < E) {  // offsets are clamped to the buffer, so a bad offset cannot address outside it
        const int64_t a0 = min(max(static_cast<int64_t>(offs[e]), static_cast<int64_t>(0)), max_rows);
        const int64_t a1 = min(max(static_cast<int64_t>(offs[e + 1]), a0), max_rows);
        o0 = static_cast<int>(a0);
        me = static_cast<int>(a1 - a0);
      }
      const int tiles = (me + BM - 1) / BM;
      const int incl = wave_incl_scan(tiles) + carry;
      const int excl = incl - tiles;
      const uint64_t hit = __ballot(e < E && mt >= excl && mt < incl);
      if (hit) {
        if (l == __ffsll(static_cast<unsigned long long>(hit)) - 1) {
          const int lt = mt - excl;
          info[0] = e;
          info[1] = o0 + lt * BM;
          info[2] = min(BM, me - lt * BM);
        }
        found = true;
        break;
      }
      carry = __shfl(incl, kWave - 1, kWave);
    }
    if (!found && l == 0) info[0] = -1;
  }
  __syncthreads();
}

__device__ __forceinline__ void tile_coords(const GemmParams &p, int *mt, int *nt) {
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = kGroupM * p.n_tiles;
  const int group = bid / per_group;
  const int first_m = group * kGroupM;
  const int gsz = min(p.m_tiles - first_m, kGroupM);
  const int in_g = bid - group * per_group;
  *mt = first_m + in_g % gsz;
  *nt = in_g / gsz;
}

template <int BM, int ACT>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmParams p) {
  constexpr int WM = BM / 2;   // rows per wave
  constexpr int MI = WM / 16;  // 16-row MFMA tiles per wave
  constexpr int NJ = 8;        // 16-col MFMA tiles per wave (128 B rows)
  constexpr int A_CH = BM * 8 / kThreads;
  constexpr int B_CH = BN * 8 / kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];
  __shared__ int info[3];

  int mt, nt;
  tile_coords(p, &mt, &nt);
  find_tile<BM>(p.offs, p.E, p.max_rows, mt, info);
  const int e = info[0];
  if (e < 0) return;
  const int row0 = info[1], rows = info[2];

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
      *reinterpret_cast<u32x4 *>(&sA[buf][r * BK + ((cc ^ (r & 7)) * 8)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int r = rbase + 32 * i;
      *reinterpret_cast<u32x4 *>(&sB[buf][r * BK + ((cc ^ (r & 7)) * 8)]) = rb[i];
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
      const int chunk = ((ks * 4 + (l >> 4)) ^ (l & 7)) * 8;
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
          if (col < p.n_out) crow[col] = f32_to_bf16(silu(acc[i][j][r]) * acc[i][j + NJ / 2][r]);
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

// fp32 path: plain FMA tiles (64 rows x 64 B rows x 16), 4x4 per thread.
constexpr int F_BM = 64, F_BN = 64, F_BK = 16;

template <int ACT>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmParams p) {
  __shared__ float sA[F_BK][F_BM + 4];
  __shared__ float sB[F_BK][F_BN + 4];
  __shared__ int info[3];
  int mt, nt;
  tile_coords(p, &mt, &nt);
  find_tile<F_BM>(p.offs, p.E, p.max_rows, mt, info);
  const int e = info[0];
  if (e < 0) return;
  const int row0 = info[1], rows = info[2];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const float *A = static_cast<const float *>(p.A);
  const float *B = static_cast<const float *>(p.B) + static_cast<int64_t>(e) * p.b_stride;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < p.K; k0 += F_BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + i * kThreads;
      const int r = q / F_BK, kk = q % F_BK;
      const int gk = k0 + kk;
      const int64_t ar = row0 + min(r, rows - 1);
      sA[kk][r] = gk < p.K ? A[ar * p.lda + gk] : 0.f;
      int br;
      if (ACT == ACT_SWIGLU) {
        const int col = nt * (F_BN / 2) + (r & (F_BN / 2 - 1));
        br = (col < p.n_out ? col : 0) + (r >= F_BN / 2 ? p.up_off : 0);
      } else {
        const int col = nt * F_BN + r;
        br = col < p.n_out ? col : 0;
      }
      sB[kk][r] = gk < p.K ? B[static_cast<int64_t>(br) * p.ldb + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < F_BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int bc = (ACT == ACT_SWIGLU) ? ((j < 2) ? tx * 2 + j : F_BN / 2 + tx * 2 + (j - 2)) : tx * 4 + j;
        b[j] = sB[kk][bc];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float *C = static_cast<float *>(p.C);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = ty * 4 + i;
    if (lr >= rows) continue;
    float *crow = C + static_cast<int64_t>(row0 + lr) * p.ldc;
    if (ACT == ACT_SWIGLU) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = nt * (F_BN / 2) + tx * 2 + j;
        if (col < p.n_out) crow[col] = silu(acc[i][j]) * acc[i][j + 2];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = nt * F_BN + tx * 4 + j;
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

hipError_t run_gemm(int dtype, int bm, const GemmParams &p, int act, hipStream_t st) {
  if (dtype == 0) return run_f32(p, act, st);
  return bm == 256 ? run_bf16<256>(p, act, st) : run_bf16<128>(p, act, st);
}

}  // namespace

hipError_t launch_expert_ffn(const FfnArgs &a, hipStream_t st) {
  if (a.max_rows == 0) return hipSuccess;
  const int n_up = a.act == 1 ? 2 : 1;
  const int64_t avg_rows = a.max_rows / a.E;
  const int bm = avg_rows >= 384 ? 256 : 128;
  GemmParams g1{};
  g1.A = a.x_perm;
  g1.lda = a.d;
  g1.B = a.w1;
  g1.ldb = a.d;
  g1.b_stride = static_cast<int64_t>(n_up) * a.d_ff * a.d;
  g1.C = a.h;
  g1.ldc = a.d_ff;
  g1.offs = a.expert_offset;
  g1.E = a.E;
  g1.K = a.d;
  g1.n_out = a.d_ff;
  g1.up_off = a.d_ff;
  g1.max_rows = a.max_rows;
  hipError_t err = run_gemm(a.dtype, bm, g1, a.act == 1 ? ACT_SWIGLU : ACT_GELU, st);
  if (err != hipSuccess) return err;
  GemmParams g2{};
  g2.A = a.h;
  g2.lda = a.d_ff;
  g2.B = a.w2;
  g2.ldb = a.d_ff;
  g2.b_stride = static_cast<int64_t>(a.d) * a.d_ff;
  g2.C = a.y_perm;
  g2.ldc = a.d;
  g2.offs = a.expert_offset;
  g2.E = a.E;
  g2.K = a.d_ff;
  g2.n_out = a.d;
  g2.up_off = 0;
  g2.max_rows = a.max_rows;
  return run_gemm(a.dtype, bm, g2, ACT_NONE, st);
}

__global__ void fill_offsets_kernel(int32_t *dst, int32_t t) {
  if (threadIdx.x == 0) {
    dst[0] = 0;
    dst[1] = t;
  }
}

hipError_t launch_fill_offsets(int32_t *dst, int32_t t, hipStream_t st) {
  fill_offsets_kernel<<<1, 64, 0, st>>>(dst, t);
  return hipGetLastError();
}

}  // namespace moe
