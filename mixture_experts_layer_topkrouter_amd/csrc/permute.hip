// token_permutation on one GPU: per-expert histogram, stable ranks, capacity
// dropping, prefix-sum offsets and the row scatter into expert-major order.
//
// "How MegaDLMs Implements Mixture of Experts (MoE) Architectures", section
// "Token Dispatching and Communication" (token_permutation moves tokens to
// their experts) and "Expert Parallelism > Key Parameters", capacity_factor
// paragraph (assignments beyond an expert's capacity are dropped and add
// nothing to the output).
//
// gfx950 design (two or three launches, no floating point, no global
// atomics, so the result is bit-reproducible):
// 1. count: a block takes 1024 consecutive assignments (token-major order).
//    Each wave labels 64 of them at a time: a lane finds the lanes holding the
//    same expert with one ballot per bit of the expert id, so its rank inside
//    the 64 is a popcount and the lowest such lane writes the group size to a
//    private LDS slot.  A per-expert scan over the 16 groups gives block-local
//    ranks and the block's histogram row.
// 2. scan: the [blocks x E] histogram becomes per-block bases (exclusive
//    over blocks), the loads, the kept counts min(load, C) and the exclusive
//    expert offsets.
// 3. scatter: one wave per token computes its k rows (or -1 when the rank is
//    at or above the capacity), loads the token row once with 16-B loads and
//    stores it to each kept row.
// When the histogram table is small (the usual case) every scatter
// workgroup does step 2 itself in LDS, which saves the single-workgroup
// scan launch.  With at most kSelfCount assignments (a few tens of KB of
// expert ids) there is a single launch: every scatter workgroup counts all
// assignments itself (steps 1 and 2 on its own, the ids read from L2 by all
// but the first workgroups), which removes the counting launch and the gap
// between the two.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Token rows are read once here: non-temporal loads keep them from
// displacing other lines in L2 (measured: the median after an
// L2/MALL-evicting write drops from 31 to 25 us on the Mixtral slice, the
// warm time is unchanged; non-temporal stores of x_perm, which the expert
// GEMM reads next, were slower).
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
constexpr int kGroups = kPermuteBlock / kWave;  // 16 groups of 64 per block

// Address of 16-B chunk c of permuted row `row`: row-major rows of row_bytes,
// or (kb_rows > 0, bf16) K-blocked over kb_rows rows, where the four chunks
// c = 4 s .. 4 s + 3 of every row (its 32-wide K slice s) lie together and
// the slices of consecutive rows follow each other.
__device__ __forceinline__ uint8_t *xp_chunk(uint8_t *x_perm, size_t row_bytes, int64_t kb_rows, int64_t row,
                                             int c) {
  return kb_rows > 0 ? x_perm + ((static_cast<int64_t>(c >> 2) * kb_rows + row) * 4 + (c & 3)) * 16
                     : x_perm + static_cast<size_t>(row) * row_bytes + static_cast<size_t>(c) * 16;
}

__global__ __launch_bounds__(kThreads) void count_kernel(const int32_t *__restrict__ idx, int64_t A, int E,
                                                         int ebits, int32_t *__restrict__ blk,
                                                         int32_t *__restrict__ rank) {
  __shared__ int grp[kGroups][kMaxExperts];
  const int l = lane_id(), w = wave_id();
  for (int i = threadIdx.x; i < kGroups * E; i += blockDim.x) grp[i / E][i % E] = 0;
  __syncthreads();
  constexpr int per_wave = kGroups / (kThreads / kWave);
  int e_reg[per_wave], r_reg[per_wave];
#pragma unroll
  for (int i = 0; i < per_wave; ++i) {
    const int g = w * per_wave + i;
    const int64_t a = static_cast<int64_t>(blockIdx.x) * kPermuteBlock + g * kWave + l;
    bool valid = a < A;
    int e = valid ? idx[a] : E;  // E marks an empty lane
    if (e < 0 || e > E) e = E;     // an id outside [0,E) is never counted
    uint64_t peers = ~static_cast<uint64_t>(0);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int r = __popcll(peers & lanemask_lt());
    valid = valid && e < E;
    if (valid && r == 0) grp[g][e] = __popcll(peers);
    e_reg[i] = e;
    r_reg[i] = r;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int g = 0; g < kGroups; ++g) {
      const int c = grp[g][e];
      grp[g][e] = run;
      run += c;
    }
    blk[static_cast<int64_t>(blockIdx.x) * E + e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < per_wave; ++i) {
    const int g = w * per_wave + i;
    const int64_t a = static_cast<int64_t>(blockIdx.x) * kPermuteBlock + g * kWave + l;
    if (a < A && e_reg[i] < E) rank[a] = grp[g][e_reg[i]] + r_reg[i];
  }
}

constexpr int kScanThreads = 256;

__global__ __launch_bounds__(kScanThreads) void scan_kernel(int32_t *__restrict__ blk, int nblk, int E,
                                                            int64_t cap, int32_t *__restrict__ expert_count,
                                                            int32_t *__restrict__ expert_load,
                                                            int32_t *__restrict__ expert_offset) {
  __shared__ int tmp[kScanThreads / kWave + 1];
  const int e = threadIdx.x;  // E <= 256 = blockDim.x
  int cnt = 0;
  if (e < E) {
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
      const int c = blk[static_cast<int64_t>(b) * E + e];
      blk[static_cast<int64_t>(b) * E + e] = run;
      run += c;
    }
    cnt = (cap >= 0 && run > cap) ? static_cast<int>(cap) : run;
    expert_load[e] = run;
    expert_count[e] = cnt;
  }
  int total;
  const int off = block_excl_scan(cnt, tmp, &total);
  if (e < E) expert_offset[e] = off;
  if (e == 0) expert_offset[E] = total;
}

constexpr int kScatterTokens = kThreads / kWave;  // one wave per token

// Loads the token row (CPL 16-B chunks per lane per pass) and stores it to
// each of the token's kept rows (row of slot j in lane j).
template <int CPL>
__device__ __forceinline__ void copy_row(const uint8_t *__restrict__ x, size_t row_bytes, int t, int k, int row,
                                         uint8_t *__restrict__ x_perm, int64_t kb_rows, int c_begin = 0) {
  const int l = lane_id();
  if (__ballot(row >= 0) == 0) return;  // every slot dropped: the row is not read
  const int nchunk = static_cast<int>(row_bytes / 16);
  const uint8_t *src = x + static_cast<size_t>(t) * row_bytes;
  for (int c0 = c_begin; c0 < nchunk; c0 += CPL * kWave) {
    u32x4 v[CPL];
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = c0 + u * kWave + l;
      if (c < nchunk) v[u] = ld16_stream(src + static_cast<size_t>(c) * 16);
    }
    for (int j = 0; j < k; ++j) {
      const int rj = __shfl(row, j, kWave);
      if (rj < 0) continue;
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = c0 + u * kWave + l;
        if (c < nchunk) st16(xp_chunk(x_perm, row_bytes, kb_rows, rj, c), v[u]);
      }
    }
  }
}

template <int CPL>
__global__ __launch_bounds__(kThreads) void scatter_kernel(
    const uint8_t *__restrict__ x, size_t row_bytes, const int32_t *__restrict__ idx, int T, int k, int E,
    int64_t cap, const int32_t *__restrict__ blk, const int32_t *__restrict__ rank,
    const int32_t *__restrict__ expert_offset, uint8_t *__restrict__ x_perm, int32_t *__restrict__ row_token,
    int32_t *__restrict__ slot_row, int64_t kb_rows) {
  const int t = blockIdx.x * kScatterTokens + wave_id();
  if (t >= T) return;
  const int l = lane_id();
  int row = -1;
  if (l < k) {
    const int64_t a = static_cast<int64_t>(t) * k + l;
    const int e = idx[a];
    const int r = (e >= 0 && e < E) ? blk[(a / kPermuteBlock) * E + e] + rank[a] : -1;
    if (r >= 0 && (cap < 0 || r < cap)) {
      row = expert_offset[e] + r;
      row_token[row] = t;
    }
    slot_row[a] = row;
  }
  copy_row<CPL>(x, row_bytes, t, k, row, x_perm, kb_rows);
}

// Scan and scatter in one launch, for histogram tables of at most
// kFusedTable entries: every workgroup loads the [blocks x E] histogram into
// LDS and computes the per-block bases (exclusive over blocks), the loads,
// the kept counts and the expert offsets itself (workgroup 0 also stores
// them), then copies its 16 tokens' rows.
constexpr int kFusedThreads = 1024;
constexpr int kFusedTokens = kFusedThreads / kWave;
constexpr int kFusedTable = 8192;

template <int CPL>
__global__ __launch_bounds__(kFusedThreads) void scan_scatter_kernel(
    const uint8_t *__restrict__ x, size_t row_bytes, const int32_t *__restrict__ idx, int T, int k, int E,
    int64_t cap, const int32_t *__restrict__ blk, int nblk, const int32_t *__restrict__ rank,
    int32_t *__restrict__ expert_count, int32_t *__restrict__ expert_load, int32_t *__restrict__ expert_offset,
    uint8_t *__restrict__ x_perm, int32_t *__restrict__ row_token, int32_t *__restrict__ slot_row,
    int64_t kb_rows) {
  __shared__ int tab[kFusedTable];
  __shared__ int offs[kMaxExperts + 1];
  __shared__ int tmp[kFusedThreads / kWave + 1];
  const int tid = threadIdx.x;
  const int n = nblk * E;
  for (int i = tid; i < n; i += kFusedThreads) tab[i] = blk[i];
  __syncthreads();
  int cnt = 0, load = 0;
  if (tid < E) {
    for (int b = 0; b < nblk; ++b) {
      const int c = tab[b * E + tid];
      tab[b * E + tid] = load;
      load += c;
    }
    cnt = (cap >= 0 && load > cap) ? static_cast<int>(cap) : load;
  }
  int total;
  const int off = block_excl_scan(cnt, tmp, &total);
  if (tid < E) offs[tid] = off;
  if (tid == 0) offs[E] = total;
  if (blockIdx.x == 0) {
    if (tid < E) {
      expert_load[tid] = load;
      expert_count[tid] = cnt;
      expert_offset[tid] = off;
    }
    if (tid == 0) expert_offset[E] = total;
  }
  __syncthreads();
  const int t = blockIdx.x * kFusedTokens + wave_id();
  if (t >= T) return;
  const int l = lane_id();
  int row = -1;
  if (l < k) {
    const int64_t a = static_cast<int64_t>(t) * k + l;
    const int e = idx[a];
    const int r = (e >= 0 && e < E) ? tab[static_cast<int>(a / kPermuteBlock) * E + e] + rank[a] : -1;
    if (r >= 0 && (cap < 0 || r < cap)) {
      row = offs[e] + r;
      row_token[row] = t;
    }
    slot_row[a] = row;
  }
  copy_row<CPL>(x, row_bytes, t, k, row, x_perm, kb_rows);
}

// One launch for at most kSelfCount assignments: each workgroup (16 tokens,
// one wave per token for the copy) first counts every assignment.  Waves take
// 64-assignment chunks; per chunk one ballot per bit of the expert id finds
// each lane's peers, and the lowest lane of each peer group adds the group's
// size to the expert's total, and (for the part of the chunk before the
// workgroup's first assignment) to the expert's base.  LDS integer adds, so
// the counts do not depend on their order.  The workgroup's own assignments
// (at most 16 k) keep their ids in LDS; an assignment's rank is its expert's
// base plus the earlier own assignments with the same expert.  The first
// pass of each token's row is loaded before the counting starts, so the
// counting runs in the shadow of those loads.
constexpr int kSelfCount = 8192;
constexpr int kSelfPerLane = kSelfCount / kFusedThreads;

template <int CPL>
__global__ __launch_bounds__(kFusedThreads) void count_scatter_kernel(
    const uint8_t *__restrict__ x, size_t row_bytes, const int32_t *__restrict__ idx, int T, int k, int E,
    int ebits, int64_t cap, int32_t *__restrict__ expert_count, int32_t *__restrict__ expert_load,
    int32_t *__restrict__ expert_offset, uint8_t *__restrict__ x_perm, int32_t *__restrict__ row_token,
    int32_t *__restrict__ slot_row, int64_t kb_rows) {
  __shared__ int base[kMaxExperts], total[kMaxExperts], offs[kMaxExperts + 1];
  __shared__ int tmp[kFusedThreads / kWave + 1];
  __shared__ int own[kFusedTokens * kMaxTopK];
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  const int A = T * k;  // <= kSelfCount
  const int a0 = blockIdx.x * kFusedTokens * k;
  const int a1 = min(A, a0 + kFusedTokens * k);
  const int t = blockIdx.x * kFusedTokens + w;
  const bool has_t = t < T;
  const int nchunk = static_cast<int>(row_bytes / 16);
  // dropless: every token's row is written, so it is requested before the
  // counting; with a capacity the row is read only if a slot is kept
  const bool pre = cap < 0;
  u32x4 v[CPL];
  auto load_first = [&]() {
    const uint8_t *src = x + static_cast<size_t>(has_t ? t : 0) * row_bytes;
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = u * kWave + l;
      v[u] = (has_t && c < nchunk) ? ld16_stream(src + static_cast<size_t>(c) * 16) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  if (pre) load_first();
  for (int e = tid; e < E; e += kFusedThreads) {
    base[e] = 0;
    total[e] = 0;
  }
  // every id this lane counts, loaded up front (chunk c = w + 16 i)
  int ev[kSelfPerLane];
#pragma unroll
  for (int i = 0; i < kSelfPerLane; ++i) {
    const int a = (w + i * (kFusedThreads / kWave)) * kWave + l;
    int e = a < A ? idx[a] : E;
    ev[i] = (e < 0 || e > E) ? E : e;  // an id outside [0,E) is never counted
  }
  __syncthreads();
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int i = 0; i < kSelfPerLane; ++i) {
    const int c0 = (w + i * (kFusedThreads / kWave)) * kWave;
    if (c0 >= A) break;  // wave-uniform
    const int a = c0 + l;
    const int e = ev[i];
    uint64_t peers = ~static_cast<uint64_t>(0);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const bool valid = e < E;
    if (valid && (peers & lt) == 0) atomicAdd(&total[e], __popcll(peers));
    const uint64_t pre = peers & __ballot(a < a0);
    if (valid && a < a0 && (pre & lt) == 0) atomicAdd(&base[e], __popcll(pre));
    if (a >= a0 && a < a1) own[a - a0] = e;
  }
  __syncthreads();
  int cnt = 0, load = 0;
  if (tid < E) {
    load = total[tid];
    cnt = (cap >= 0 && load > cap) ? static_cast<int>(cap) : load;
  }
  int tot;
  const int off = block_excl_scan(cnt, tmp, &tot);
  if (tid < E) offs[tid] = off;
  if (tid == 0) offs[E] = tot;
  if (blockIdx.x == 0) {
    if (tid < E) {
      expert_load[tid] = load;
      expert_count[tid] = cnt;
      expert_offset[tid] = off;
    }
    if (tid == 0) expert_offset[E] = tot;
  }
  __syncthreads();
  if (!has_t) return;
  int row = -1;
  if (l < k) {
    const int j = w * k + l;  // own index
    const int e = own[j];
    if (e < E) {
      int r = base[e];
      for (int q = 0; q < j; ++q) r += own[q] == e;
      if (cap < 0 || r < cap) {
        row = offs[e] + r;
        row_token[row] = t;
      }
    }
    slot_row[static_cast<int64_t>(t) * k + l] = row;
  }
  if (__ballot(row >= 0) == 0) return;  // every slot dropped: the row is not read
  if (!pre) load_first();
  for (int j = 0; j < k; ++j) {
    const int rj = __shfl(row, j, kWave);
    if (rj < 0) continue;
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = u * kWave + l;
      if (c < nchunk) st16(xp_chunk(x_perm, row_bytes, kb_rows, rj, c), v[u]);
    }
  }
  if (nchunk > CPL * kWave) copy_row<CPL>(x, row_bytes, t, k, row, x_perm, kb_rows, CPL * kWave);
}

// ---------------------------------------------------------------- ExpertChoice

// ExpertChoice permutation in one launch, token-major.  Row e*C + i holds
// token ec_token[e, i]; each expert's list ascends, so a workgroup that owns
// tokens [t0, t0 + 16) finds, per expert, the run of list entries that fall in
// its range by two binary searches (lower bounds of t0 and t0 + 16), and the
// number of selections before t0 (the CSR base of its first token) is the sum
// of the first lower bounds over the experts.  A per-token bit mask of the
// experts holding it (LDS integer ORs, order-independent) gives each entry
// its place in its token's list (ascending expert); then every token's row is
// read once and written to each of its rows.
constexpr int kEcPermTokens = kFusedTokens;  // 16 tokens, one wave each for the copy
constexpr int kEcMaskWords = kMaxExperts / 32;

__device__ __forceinline__ int ec_lower_bound(const int32_t *__restrict__ list, int C, int t) {
  int lo = 0, hi = C;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (list[mid] < t) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

template <int CPL>
__global__ __launch_bounds__(kFusedThreads) void ec_permute_kernel(
    const uint8_t *__restrict__ x, size_t row_bytes, const int32_t *__restrict__ ec_token,
    const float *__restrict__ ec_w, int T, int E, int C, uint8_t *__restrict__ x_perm,
    int32_t *__restrict__ row_token, int32_t *__restrict__ slot_row, float *__restrict__ slot_w,
    int32_t *__restrict__ tok_ptr, int32_t *__restrict__ expert_count, int32_t *__restrict__ expert_load,
    int32_t *__restrict__ expert_offset, int64_t kb_rows) {
  __shared__ int p0[kMaxExperts], p1[kMaxExperts];
  __shared__ uint32_t mask[kEcPermTokens][kEcMaskWords];
  __shared__ int tok_off[kEcPermTokens + 1];
  __shared__ int rows_of[kEcPermTokens][kMaxExperts];
  __shared__ int tmp[kFusedThreads / kWave + 1];
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  const int t0 = blockIdx.x * kEcPermTokens;
  const int t1 = min(T, t0 + kEcPermTokens);
  if (blockIdx.x == 0) {
    for (int e = tid; e <= E; e += kFusedThreads) {
      if (e < E) {
        expert_count[e] = C;
        expert_load[e] = C;
      }
      expert_offset[e] = e * C;
    }
  }
  // the first pass of this wave's token row is requested before the searches
  const int t = t0 + w;
  const bool has_t = t < T;
  const int nchunk = static_cast<int>(row_bytes / 16);
  u32x4 v[CPL];
  {
    const uint8_t *src = x + static_cast<size_t>(has_t ? t : 0) * row_bytes;
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = u * kWave + l;
      v[u] = (has_t && c < nchunk) ? ld16_stream(src + static_cast<size_t>(c) * 16) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  for (int i = tid; i < kEcPermTokens * kEcMaskWords; i += kFusedThreads) (&mask[0][0])[i] = 0u;
  int before = 0;  // selections of expert `tid` before t0
  if (tid < E) {
    const int32_t *list = ec_token + static_cast<int64_t>(tid) * C;
    p0[tid] = before = ec_lower_bound(list, C, t0);
    p1[tid] = ec_lower_bound(list, C, t1);
  }
  int base_total;
  block_excl_scan(before, tmp, &base_total);  // base_total = selections before t0
  // (block_excl_scan ends with a barrier: p0, p1 and the cleared masks are visible)
  for (int e = tid; e < E; e += kFusedThreads)
    for (int p = p0[e]; p < p1[e]; ++p) {
      const int tl = ec_token[static_cast<int64_t>(e) * C + p] - t0;
      if (tl >= 0 && tl < kEcPermTokens) atomicOr(&mask[tl][e >> 5], 1u << (e & 31));
    }
  __syncthreads();
  if (w == 0) {  // per-token counts, their scan, the CSR pointers
    int cnt = 0;
    if (l < kEcPermTokens)
      for (int q = 0; q < kEcMaskWords; ++q) cnt += __popc(mask[l][q]);
    const int incl = wave_incl_scan(cnt);
    if (l < kEcPermTokens) {
      tok_off[l] = base_total + incl - cnt;
      if (t0 + l < T) tok_ptr[t0 + l] = base_total + incl - cnt;
      if (t0 + l == T - 1) tok_ptr[T] = base_total + incl;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kFusedThreads)
    for (int p = p0[e]; p < p1[e]; ++p) {
      const int64_t r = static_cast<int64_t>(e) * C + p;
      const int tl = ec_token[r] - t0;
      if (tl < 0 || tl >= kEcPermTokens) continue;  // only an unsorted list gets here
      int rank = 0;  // experts below e that hold this token
      for (int q = 0; q < (e >> 5); ++q) rank += __popc(mask[tl][q]);
      rank += __popc(mask[tl][e >> 5] & ((1u << (e & 31)) - 1u));
      const int slot = tok_off[tl] + rank;
      slot_row[slot] = static_cast<int32_t>(r);
      slot_w[slot] = ec_w[r];
      row_token[r] = t0 + tl;
      rows_of[tl][rank] = static_cast<int32_t>(r);
    }
  __syncthreads();
  if (!has_t) return;
  int cnt = 0;
  for (int q = 0; q < kEcMaskWords; ++q) cnt += __popc(mask[w][q]);
  for (int j = 0; j < cnt; ++j) {
    const int rj = rows_of[w][j];
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = u * kWave + l;
      if (c < nchunk) st16(xp_chunk(x_perm, row_bytes, kb_rows, rj, c), v[u]);
    }
  }
  if (nchunk > CPL * kWave) {
    // rows longer than one pass: the rest, read once per pass
    const uint8_t *src = x + static_cast<size_t>(t) * row_bytes;
    for (int c0 = CPL * kWave; c0 < nchunk; c0 += CPL * kWave) {
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = c0 + u * kWave + l;
        if (c < nchunk) v[u] = ld16_stream(src + static_cast<size_t>(c) * 16);
      }
      for (int j = 0; j < cnt; ++j) {
        const int rj = rows_of[w][j];
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
          const int c = c0 + u * kWave + l;
          if (c < nchunk) st16(xp_chunk(x_perm, row_bytes, kb_rows, rj, c), v[u]);
        }
      }
    }
  }
}

}  // namespace

size_t permute_scratch_bytes(int T, int k, int E) {
  const int64_t A = static_cast<int64_t>(T) * k;
  const int64_t nblk = (A + kPermuteBlock - 1) / kPermuteBlock;
  size_t b = static_cast<size_t>(nblk * E) * 4;
  b = (b + 255) & ~static_cast<size_t>(255);
  b += static_cast<size_t>(A) * 4;
  return (b + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_permute_topk(const PermuteArgs &a, hipStream_t st) {
  const int64_t A = static_cast<int64_t>(a.T) * a.k;
  const int nblk = static_cast<int>((A + kPermuteBlock - 1) / kPermuteBlock);
  int ebits = 0;
  while ((1 << ebits) <= a.E) ++ebits;  // ids 0..E (E marks an empty lane)
  const int per_lane = static_cast<int>((a.row_bytes / 16 + kWave - 1) / kWave);  // 16-B chunks per lane
  const uint8_t *x = static_cast<const uint8_t *>(a.x);
  uint8_t *xp = static_cast<uint8_t *>(a.x_perm);
  if (a.T > 0 && A <= kSelfCount) {
    const int blocks = (a.T + kFusedTokens - 1) / kFusedTokens;
#define MOE_COUNT_SCATTER(CPL)                                                                                 \
  count_scatter_kernel<CPL><<<blocks, kFusedThreads, 0, st>>>(x, a.row_bytes, a.topk_idx, a.T, a.k, a.E, ebits, \
                                                              a.cap, a.expert_count, a.expert_load,             \
                                                              a.expert_offset, xp, a.row_token, a.slot_row,     \
                                                              a.kb_rows)
    if (per_lane <= 2) MOE_COUNT_SCATTER(2);
    else if (per_lane <= 4) MOE_COUNT_SCATTER(4);
    else MOE_COUNT_SCATTER(8);
#undef MOE_COUNT_SCATTER
    return hipGetLastError();
  }
  if (nblk > 0) count_kernel<<<nblk, kThreads, 0, st>>>(a.topk_idx, A, a.E, ebits, a.blk, a.rank);
  if (a.T > 0 && static_cast<int64_t>(nblk) * a.E <= kFusedTable) {
    const int blocks = (a.T + kFusedTokens - 1) / kFusedTokens;
#define MOE_SCAN_SCATTER(CPL)                                                                                  \
  scan_scatter_kernel<CPL><<<blocks, kFusedThreads, 0, st>>>(x, a.row_bytes, a.topk_idx, a.T, a.k, a.E, a.cap, \
                                                             a.blk, nblk, a.rank, a.expert_count,              \
                                                             a.expert_load, a.expert_offset, xp, a.row_token,  \
                                                             a.slot_row, a.kb_rows)
    if (per_lane <= 2) MOE_SCAN_SCATTER(2);
    else if (per_lane <= 4) MOE_SCAN_SCATTER(4);
    else MOE_SCAN_SCATTER(8);
#undef MOE_SCAN_SCATTER
    return hipGetLastError();
  }
  scan_kernel<<<1, kScanThreads, 0, st>>>(a.blk, nblk, a.E, a.cap, a.expert_count, a.expert_load,
                                          a.expert_offset);
  if (a.T > 0) {
    const int blocks = (a.T + kScatterTokens - 1) / kScatterTokens;
#define MOE_SCATTER(CPL)                                                                                      \
  scatter_kernel<CPL><<<blocks, kThreads, 0, st>>>(x, a.row_bytes, a.topk_idx, a.T, a.k, a.E, a.cap, a.blk,   \
                                                   a.rank, a.expert_offset, xp, a.row_token, a.slot_row,       \
                                                   a.kb_rows)
    if (per_lane <= 2) MOE_SCATTER(2);
    else if (per_lane <= 4) MOE_SCATTER(4);
    else MOE_SCATTER(8);
#undef MOE_SCATTER
  }
  return hipGetLastError();
}

hipError_t launch_permute_ec(const PermuteEcArgs &a, hipStream_t st) {
  const int blocks = (a.T + kEcPermTokens - 1) / kEcPermTokens;
  const int per_lane = static_cast<int>((a.row_bytes / 16 + kWave - 1) / kWave);  // 16-B chunks per lane
  const uint8_t *x = static_cast<const uint8_t *>(a.x);
  uint8_t *xp = static_cast<uint8_t *>(a.x_perm);
#define MOE_EC_PERMUTE(CPL)                                                                                     \
  ec_permute_kernel<CPL><<<blocks > 0 ? blocks : 1, kFusedThreads, 0, st>>>(                                   \
      x, a.row_bytes, a.ec_token, a.ec_w, a.T, a.E, a.C, xp, a.row_token, a.slot_row, a.slot_w, a.tok_ptr,     \
      a.expert_count, a.expert_load, a.expert_offset, a.kb_rows)
  if (per_lane <= 2) MOE_EC_PERMUTE(2);
  else if (per_lane <= 4) MOE_EC_PERMUTE(4);
  else MOE_EC_PERMUTE(8);
#undef MOE_EC_PERMUTE
  return hipGetLastError();
}

}  // namespace moe
