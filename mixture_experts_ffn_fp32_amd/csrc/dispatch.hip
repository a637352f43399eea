// Dispatch kernels for gfx950: group the (token, k) pairs by expert, stably.
//
// Each token is computed only by the K experts it selected (DeepSeekMoE
// paper summary, papercache.org, sec. A3: gate sparsity).  The expert GEMMs
// want each expert's tokens contiguous, so the pairs p = t*K + k are sorted
// by expert, ascending p within an expert (a stable counting sort):
//
//  1. tile_rank: per tile of kRankTile (32) tokens, a lane mask per expert
//     in LDS gives each pair its rank among the tile's pairs of the same
//     expert (popcount of the lower lanes) and each expert's count in the
//     tile.  Integer only, no global atomics, deterministic.  The tiled
//     router does the same for its 32-token blocks in its own epilogue, and
//     the layer forward then skips this launch.
//  2. dispatch_scan: one block turns tile counts into per-expert totals,
//     offsets (exclusive scan over experts) and per-(tile, expert) bases.
//  3. scatter: sorted_pair[base + rank] = p.
// A batch of at most 64 tokens (decode) does all three in one launch.
#include <algorithm>

#include "dispatch_wave.h"
#include "moe_internal.h"

namespace moe {
namespace {

// One wavefront per tile of kRankTile tokens; lane = token (lanes past the
// tile idle).
__global__ __launch_bounds__(64) void tile_rank_kernel(const int32_t* __restrict__ idx, int T,
                                                       int N, int K,
                                                       int32_t* __restrict__ tile_counts,
                                                       int32_t* __restrict__ rank) {
  __shared__ unsigned long long mask[256];
  static_assert(kRankTile <= 64, "one lane per token");
  const int lane = threadIdx.x;
  const int tile = blockIdx.x;
  const int t = lane < kRankTile ? tile * kRankTile + lane : T;
  for (int e = lane; e < N; e += 64) mask[e] = 0ull;
  __syncthreads();
  const unsigned long long bit = 1ull << lane;
  int ev[kKReg];
  if (t < T) load_ids(idx, t, K, ev);
  // ids outside [0, N) are ignored (the router never produces them)
  if (t < T)
    for_ids(idx, t, K, ev, [&](int, int e) {
      if ((unsigned)e < (unsigned)N) atomicOr(&mask[e], bit);
    });
  __syncthreads();
  if (t < T) {
    const unsigned long long below = bit - 1ull;
    for_ids(idx, t, K, ev, [&](int k, int e) {
      rank[(size_t)t * K + k] = ((unsigned)e < (unsigned)N) ? __popcll(mask[e] & below) : 0;
    });
  }
  const int row = rank_row((int)gridDim.x);
  for (int e = lane; e < N; e += 64) tile_counts[(size_t)e * row + tile] = __popcll(mask[e]);
}

// Inclusive scan over segments of G lanes (G a power of two, at most 64).
__device__ __forceinline__ int seg_inclusive_scan(int x, int g, int G) {
  for (int o = 1; o < G; o <<= 1) {
    const int y = __shfl_up(x, o, G);
    if (g >= o) x += y;
  }
  return x;
}

// One block of 1024 threads.  Expert e's row of tile counts is read in
// rounds of G 16-byte groups (4 tiles each) by G consecutive lanes (G =
// 1024 / NP2 capped at 64, NP2 = N rounded up to a power of two), so each
// round is one coalesced run and its prefix a segmented lane scan; up to R
// rounds stay in registers between the totals and the bases, longer rows
// are read again.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const int32_t* __restrict__ tile_counts,
                                                             int ntiles, int N, int NP2,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ tile_base,
                                                             TileTableOut tt) {
  __shared__ int s_off[257];
  const int tid = threadIdx.x;
  const int G = min(1024 / NP2, 64);
  const int g = tid % G, e = tid / G;
  const bool live = e < N;
  const int row = rank_row(ntiles), nq = row / 4;  // 16-byte groups per row
  const int rounds = (nq + G - 1) / G;
  const u32x4* src = (const u32x4*)(tile_counts + (size_t)(live ? e : 0) * row);
  // group q of the row, the counts past the last tile (row padding, and
  // groups past the row) as 0.  The load itself is unconditional (an
  // in-range group): a load under a lane-dependent branch would be waited
  // for before the branch joins, one round trip per group.
  auto group = [&](int q) {
    u32x4 v = src[min(q, nq - 1)];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * q + j >= ntiles) v[j] = 0u;
    return v;
  };
  auto sum4 = [](u32x4 v) { return (int)(v[0] + v[1] + v[2] + v[3]); };

  constexpr int R = 16;
  const bool in_regs = rounds <= R;
  u32x4 cr[R];
  int s = 0;
  // (lanes of experts past N read row 0 and their sums go unused)
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < R; ++i) cr[i] = group(i * G + g);
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first is used
#pragma unroll
    for (int i = 0; i < R; ++i) s += sum4(cr[i]);
  } else {
    for (int i0 = 0; i0 < rounds; i0 += R) {
      u32x4 c[R];
#pragma unroll
      for (int i = 0; i < R; ++i) c[i] = group((i0 + i) * G + g);
#pragma unroll
      for (int i = 0; i < R; ++i) s += sum4(c[i]);
    }
  }
  // the expert's total: the last lane of its segment
  const int tot = __shfl(seg_inclusive_scan(s, g, G), G - 1, G);
  if (live && g == 0) s_off[e] = tot;
  __syncthreads();
  // exclusive scan of the totals over experts (first wavefront, 64 at a time)
  if (tid < 64) {
    int carry = 0;
    for (int b = 0; b < N; b += 64) {
      const int v = (b + tid < N) ? s_off[b + tid] : 0;
      const int incv = wave_inclusive_scan(v);
      const int total = __shfl(incv, 63);
      if (b + tid < N) {
        counts[b + tid] = v;
        s_off[b + tid] = carry + incv - v;
      }
      carry += total;
    }
    if (tid == 0) s_off[N] = carry;
  }
  __syncthreads();
  for (int i = tid; i <= N; i += 1024) offsets[i] = s_off[i];
  if (tid < 64 && tt.tiles1 != nullptr) tile_tables_wave(s_off, N, s_off[N], tt);
  // each tile's base: the expert's offset plus the counts of the row's
  // earlier tiles, round by round (every lane of a segment takes part in
  // each round's scan)
  u32x4* dstb = (u32x4*)(tile_base + (size_t)(live ? e : 0) * row);
  int run = live ? s_off[e] : 0;
  auto round_bases = [&](int q, u32x4 c) {
    const int gs = sum4(c);
    const int inc = seg_inclusive_scan(gs, g, G);
    uint32_t b = (uint32_t)(run + inc - gs);
    u32x4 out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[j] = b;
      b += c[j];
    }
    if (live && q < nq) dstb[q] = out;
    run += __shfl(inc, G - 1, G);
  };
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (i < rounds) round_bases(i * G + g, cr[i]);
  } else {
    for (int i = 0; i < rounds; ++i) round_bases(i * G + g, group(i * G + g));
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ rank,
                                                      const int32_t* __restrict__ tile_base,
                                                      int T, int N, int K,
                                                      int32_t* __restrict__ sorted_pair) {
  const long long p = (long long)blockIdx.x * 256 + threadIdx.x;
  if (p >= (long long)T * K) return;
  const int t = (int)(p / K);
  const int e = idx[p];
  if ((unsigned)e >= (unsigned)N) return;
  const int row = rank_row((T + kRankTile - 1) / kRankTile);
  sorted_pair[tile_base[(size_t)e * row + t / kRankTile] + rank[p]] = (int32_t)p;
}

// Steps 2 and 3 in one launch, for batches whose tile counts are small
// enough to read whole in every block (N * rank_row(ntiles) <= kScanScatterMax
// ints): block b owns RT consecutive tiles.  Each block derives what its
// scatter needs from the counts — every expert's total and its count in the
// tiles before the block's own (thread (e, g) sums groups g, g + P, ... of
// expert e's row, P threads per expert), the totals' exclusive scan (the
// offsets) and the bases of its own tiles — then writes the sorted pairs of
// its tokens.  Block 0 also writes counts, offsets and the tile tables.
constexpr int kScanScatterRT = 16;           // most tiles per block
constexpr int kScanScatterMax = 16 * 1024;   // most tile counts a block reads (64 KB)

__global__ __launch_bounds__(256) void scan_scatter_kernel(const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ rank,
                                                           const int32_t* __restrict__ tile_counts,
                                                           int T, int N, int K, int NP2, int ntiles,
                                                           int RT, int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_pair,
                                                           TileTableOut tt) {
  __shared__ int s_tot[256], s_below[256], s_off[257];
  __shared__ int s_base[kScanScatterRT][256];  // the block's tiles: counts, then bases
  const int tid = threadIdx.x;
  const int P = min(max(256 / NP2, 1), 64);  // threads per expert (one wavefront at most)
  const int e = tid / P, g = tid % P;
  const bool live = e < N;
  const int row = rank_row(ntiles), nq = row / 4;
  const int j0 = blockIdx.x * RT, j1 = min(j0 + RT, ntiles);
  const u32x4* src = (const u32x4*)(tile_counts + (size_t)(live ? e : 0) * row);
  // group q's counts: the total, the part before tile j0, the block's own
  int tot = 0, below = 0;
  auto take = [&](int q, u32x4 c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * q + i;
      const int v = j < ntiles ? (int)c[i] : 0;  // (row padding)
      tot += v;
      if (j < j0) below += v;
      else if (j < j1 && live) s_base[j - j0][e] = v;
    }
  };
  constexpr int B = 16;
  for (int q0 = g; q0 < nq; q0 += B * P) {
    u32x4 c[B];
#pragma unroll
    for (int i = 0; i < B; ++i) c[i] = src[min(q0 + i * P, nq - 1)];  // unconditional, in range
#pragma unroll
    for (int i = 0; i < B; ++i)
      if (q0 + i * P < nq) take(q0 + i * P, c[i]);
  }
  // the P partial sums of an expert (consecutive lanes)
  for (int o = 1; o < P; o <<= 1) {
    tot += __shfl_xor(tot, o, P);
    below += __shfl_xor(below, o, P);
  }
  if (live && g == 0) {
    s_tot[e] = tot;
    s_below[e] = below;
  }
  __syncthreads();
  // exclusive scan of the totals over experts (first wavefront, 64 at a time)
  if (tid < 64) {
    int carry = 0;
    for (int b = 0; b < N; b += 64) {
      const int v = (b + tid < N) ? s_tot[b + tid] : 0;
      const int incv = wave_inclusive_scan(v);
      const int total = __shfl(incv, 63);
      if (b + tid < N) {
        s_off[b + tid] = carry + incv - v;
        if (blockIdx.x == 0) {
          counts[b + tid] = v;
          offsets[b + tid] = carry + incv - v;
        }
      }
      carry += total;
    }
    if (tid == 0) {
      s_off[N] = carry;
      if (blockIdx.x == 0) offsets[N] = carry;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid < 64 && tt.tiles1 != nullptr) tile_tables_wave(s_off, N, s_off[N], tt);
  // the bases of the block's tiles
  for (int x = tid; x < N; x += 256) {
    int run = s_off[x] + s_below[x];
    for (int r = 0; r < j1 - j0; ++r) {
      const int c = s_base[r][x];
      s_base[r][x] = run;
      run += c;
    }
  }
  __syncthreads();
  const long long p0 = (long long)j0 * kRankTile * K;
  const long long p1 = (long long)min(j1 * kRankTile, T) * K;
  for (long long p = p0 + tid; p < p1; p += 256) {
    const int t = (int)(p / K);
    const int x = idx[p];
    if ((unsigned)x >= (unsigned)N) continue;
    sorted_pair[s_base[t / kRankTile - j0][x] + rank[p]] = (int32_t)p;
  }
}

// A batch of at most 64 tokens in one launch (one wavefront, lane = token):
// the ranks, counts, offsets and sorted pairs of dispatch_wave, and the tile
// tables -- the same ranks and order as steps 1-3.
__global__ __launch_bounds__(64) void dispatch_small_kernel(const int32_t* __restrict__ idx,
                                                            int T, int N, int K,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_pair,
                                                            TileTableOut tt) {
  __shared__ unsigned long long mask[256];
  __shared__ int s_off[257];
  dispatch_wave(idx, T, N, K, mask, s_off, nullptr, counts, offsets, sorted_pair);
  if (tt.tiles1 != nullptr) tile_tables_wave(s_off, N, s_off[N], tt);
}

}  // namespace

hipError_t launch_dispatch_small(const int32_t* idx, int T, int N, int K, int32_t* counts,
                                 int32_t* offsets, int32_t* sorted_pair, const TileTableOut& tt,
                                 hipStream_t stream) {
  return launch_kernel(dispatch_small_kernel, dim3(1), dim3(64), stream, idx, T, N, K, counts,
                       offsets, sorted_pair, tt);
}

hipError_t launch_tile_rank(const int32_t* idx, int T, int N, int K, int32_t* tile_counts,
                            int32_t* rank, hipStream_t stream) {
  const int ntiles = (T + kRankTile - 1) / kRankTile;
  return launch_kernel(tile_rank_kernel, dim3(ntiles), dim3(64), stream, idx, T, N, K,
                       tile_counts, rank);
}

hipError_t launch_dispatch_scan(const int32_t* tile_counts, int ntiles, int N, int32_t* counts,
                                int32_t* offsets, int32_t* tile_base, const TileTableOut& tt,
                                hipStream_t stream) {
  int np2 = 1;
  while (np2 < N) np2 <<= 1;
  return launch_kernel(dispatch_scan_kernel, dim3(1), dim3(1024), stream, tile_counts, ntiles, N,
                       np2, counts, offsets, tile_base, tt);
}

bool scan_scatter_fits(int T, int N) {
  const int ntiles = (T + kRankTile - 1) / kRankTile;
  int np2 = 1;
  while (np2 < N) np2 <<= 1;
  const int RT = std::max(2, (ntiles + 127) / 128);
  return RT <= kScanScatterRT && (long long)N * rank_row(ntiles) <= kScanScatterMax;
}

hipError_t launch_scan_scatter(const int32_t* idx, const int32_t* rank, const int32_t* tile_counts,
                               int T, int N, int K, int32_t* counts, int32_t* offsets,
                               int32_t* sorted_pair, const TileTableOut& tt, hipStream_t stream) {
  const int ntiles = (T + kRankTile - 1) / kRankTile;
  int np2 = 1;
  while (np2 < N) np2 <<= 1;
  const int RT = std::max(2, (ntiles + 127) / 128);  // about 128 blocks
  const int blocks = (ntiles + RT - 1) / RT;
  return launch_kernel(scan_scatter_kernel, dim3(blocks), dim3(256), stream, idx, rank, tile_counts,
                       T, N, K, np2, ntiles, RT, counts, offsets, sorted_pair, tt);
}

hipError_t launch_scatter(const int32_t* idx, const int32_t* rank, const int32_t* tile_base,
                          int T, int N, int K, int32_t* sorted_pair, hipStream_t stream) {
  const long long pairs = (long long)T * K;
  const int blocks = (int)((pairs + 255) / 256);
  return launch_kernel(scatter_kernel, dim3(blocks), dim3(256), stream, idx, rank, tile_base, T, N,
                       K, sorted_pair);
}

}  // namespace moe
