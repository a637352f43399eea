// Dispatch kernels for gfx950: group the (token, k) pairs by expert, stably.
//
// Each token is computed only by the K experts it selected (DeepSeekMoE
// paper summary, papercache.org, sec. A3: gate sparsity).  The expert GEMMs
// want each expert's tokens contiguous, so the pairs p = t*K + k are sorted
// by expert, ascending p within an expert (a stable counting sort):
//
//  1. tile_rank: per 64-token tile, a 64-bit lane mask per expert in LDS
//     gives each pair its rank among the tile's pairs of the same expert
//     (popcount of the lower lanes) and each expert's count in the tile.
//     Integer only, no global atomics, deterministic.
//  2. dispatch_scan: one block turns tile counts into per-expert totals,
//     offsets (exclusive scan over experts) and per-(tile, expert) bases.
//  3. scatter: sorted_pair[base + rank] = p.
// A batch of at most 64 tokens (decode) does all three in one launch.
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Expert ids of token t's K pairs, all requested before any is used (up to
// kKReg of them in registers; more are read again where needed).
constexpr int kKReg = 16;
__device__ __forceinline__ void load_ids(const int32_t* __restrict__ idx, int t, int K,
                                         int (&ev)[kKReg]) {
#pragma unroll
  for (int k = 0; k < kKReg; ++k)
    if (k < K) ev[k] = idx[(size_t)t * K + k];
}
// f(k, e) for each of token t's pairs in order k = 0 .. K-1 (register
// indices fixed at compile time, so the ids stay in registers).
template <class F>
__device__ __forceinline__ void for_ids(const int32_t* __restrict__ idx, int t, int K,
                                        const int (&ev)[kKReg], F f) {
#pragma unroll
  for (int k = 0; k < kKReg; ++k)
    if (k < K) f(k, ev[k]);
  for (int k = kKReg; k < K; ++k) f(k, idx[(size_t)t * K + k]);
}

// One wavefront per tile of 64 tokens; lane = token.
__global__ __launch_bounds__(64) void tile_rank_kernel(const int32_t* __restrict__ idx, int T,
                                                       int N, int K,
                                                       int32_t* __restrict__ tile_counts,
                                                       int32_t* __restrict__ rank) {
  __shared__ unsigned long long mask[256];
  const int lane = threadIdx.x;
  const int tile = blockIdx.x;
  const int t = tile * kRankTile + lane;
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
  for (int e = lane; e < N; e += 64) tile_counts[(size_t)tile * N + e] = __popcll(mask[e]);
}

// One block of 1024 threads.  Thread (e, g) owns expert e and the contiguous
// chunk g of the tiles; G = 1024 / NP2 chunks per expert (NP2 = N rounded up
// to a power of two).
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const int32_t* __restrict__ tile_counts,
                                                             int ntiles, int N, int NP2,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ tile_base,
                                                             TileTableOut tt) {
  __shared__ int csum[1024];     // [g][e] chunk sums, later chunk bases
  __shared__ int s_off[257];
  const int tid = threadIdx.x;
  const int e = tid % NP2, g = tid / NP2;
  const int G = 1024 / NP2;
  const int C = (ntiles + G - 1) / G;
  const int lo = min(g * C, ntiles), hi = min(lo + C, ntiles);

  // the chunk's counts, eight requested at a time before any is added
  constexpr int B = 8;
  int s = 0;
  if (e < N)
    for (int t0 = lo; t0 < hi; t0 += B) {
      int c[B];
#pragma unroll
      for (int i = 0; i < B; ++i) c[i] = t0 + i < hi ? tile_counts[(size_t)(t0 + i) * N + e] : 0;
#pragma unroll
      for (int i = 0; i < B; ++i) s += c[i];
    }
  csum[tid] = s;
  __syncthreads();
  // per-expert exclusive scan over the G chunks, and the expert totals
  if (tid < NP2) {
    int run = 0;
    for (int gg = 0; gg < G; ++gg) {
      const int v = csum[gg * NP2 + tid];
      csum[gg * NP2 + tid] = run;
      run += v;
    }
    if (tid < N) {
      counts[tid] = run;
      s_off[tid] = run;
    }
  }
  __syncthreads();
  // exclusive scan of the totals over experts (first wavefront, 64 at a time)
  if (tid < 64) {
    int carry = 0;
    for (int b = 0; b < N; b += 64) {
      const int v = (b + tid < N) ? s_off[b + tid] : 0;
      const int inc = wave_inclusive_scan(v);
      const int total = __shfl(inc, 63);
      if (b + tid < N) s_off[b + tid] = carry + inc - v;
      carry += total;
    }
    if (tid == 0) s_off[N] = carry;
  }
  __syncthreads();
  for (int i = tid; i <= N; i += 1024) offsets[i] = s_off[i];
  if (tid < 64 && tt.tiles1 != nullptr) tile_tables_wave(s_off, N, s_off[N], tt);
  if (e < N) {
    int run = s_off[e] + csum[tid];
    for (int t0 = lo; t0 < hi; t0 += B) {
      int c[B];
#pragma unroll
      for (int i = 0; i < B; ++i) c[i] = t0 + i < hi ? tile_counts[(size_t)(t0 + i) * N + e] : 0;
#pragma unroll
      for (int i = 0; i < B; ++i)
        if (t0 + i < hi) {
          tile_base[(size_t)(t0 + i) * N + e] = run;
          run += c[i];
        }
    }
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
  sorted_pair[tile_base[(size_t)(t / kRankTile) * N + e] + rank[p]] = (int32_t)p;
}

// A batch of at most 64 tokens in one launch (one wavefront, lane = token):
// the lane masks of step 1 for the single tile, then the expert counts, their
// exclusive scan and the scatter -- the same ranks and order as steps 1-3.
__global__ __launch_bounds__(64) void dispatch_small_kernel(const int32_t* __restrict__ idx,
                                                            int T, int N, int K,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_pair,
                                                            TileTableOut tt) {
  __shared__ unsigned long long mask[256];
  __shared__ int s_off[257];
  const int lane = threadIdx.x;
  for (int e = lane; e < N; e += 64) mask[e] = 0ull;
  __syncthreads();
  const unsigned long long bit = 1ull << lane;
  int ev[kKReg];
  if (lane < T) load_ids(idx, lane, K, ev);
  if (lane < T)
    for_ids(idx, lane, K, ev, [&](int, int e) {
      if ((unsigned)e < (unsigned)N) atomicOr(&mask[e], bit);
    });
  __syncthreads();
  int carry = 0;
  for (int b = 0; b < N; b += 64) {
    const int e = b + lane;
    const int c = e < N ? __popcll(mask[e]) : 0;
    const int inc = wave_inclusive_scan(c);
    if (e < N) {
      counts[e] = c;
      s_off[e] = carry + inc - c;
      offsets[e] = carry + inc - c;
    }
    carry += __shfl(inc, 63);
  }
  if (lane == 0) {
    offsets[N] = carry;
    s_off[N] = carry;
  }
  __syncthreads();
  if (tt.tiles1 != nullptr) tile_tables_wave(s_off, N, carry, tt);
  if (lane < T) {
    const unsigned long long below = bit - 1ull;
    for_ids(idx, lane, K, ev, [&](int k, int e) {
      if ((unsigned)e < (unsigned)N)
        sorted_pair[s_off[e] + __popcll(mask[e] & below)] = lane * K + k;
    });
  }
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

hipError_t launch_scatter(const int32_t* idx, const int32_t* rank, const int32_t* tile_base,
                          int T, int N, int K, int32_t* sorted_pair, hipStream_t stream) {
  const long long pairs = (long long)T * K;
  const int blocks = (int)((pairs + 255) / 256);
  return launch_kernel(scatter_kernel, dim3(blocks), dim3(256), stream, idx, rank, tile_base, T, N,
                       K, sorted_pair);
}

}  // namespace moe
