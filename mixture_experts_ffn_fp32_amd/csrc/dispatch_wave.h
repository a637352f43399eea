// The dispatch of a small batch by one wavefront (gfx950): shared by the
// one-launch dispatch kernel and the decode GEMM1, whose blocks each derive
// the dispatch of a batch of at most 64 tokens themselves.
//
// Each token is computed only by the K experts it selected (DeepSeekMoE paper
// summary, papercache.org, sec. A3: gate sparsity), so the pairs p = t*K + k
// are grouped by expert, ascending p within an expert (a stable counting
// sort): lane t sets bit t of a 64-bit mask per expert in LDS for each of its
// pairs; a pair's rank among its expert's pairs is the popcount of the lower
// lanes' bits, an expert's count the popcount of its mask, and the counts'
// exclusive scan gives the offsets.
#pragma once

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

// This wavefront's LDS accesses are complete (one wavefront: no barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

// One wavefront (all 64 lanes call it; lane = token, T <= 64).  LDS: mask[N]
// (scratch), s_off[N + 1] (the offsets, kept), s_sp[T*K] (the sorted pairs,
// when set).  Global outputs where the pointers are set: counts[N],
// offsets[N + 1], sorted_pair[T*K].  Expert ids outside [0, N) are ignored.
__device__ __forceinline__ void dispatch_wave(const int32_t* __restrict__ idx, int T, int N, int K,
                                              unsigned long long* mask, int* s_off, int* s_sp,
                                              int32_t* counts, int32_t* offsets,
                                              int32_t* sorted_pair) {
  const int lane = threadIdx.x & 63;
  for (int e = lane; e < N; e += 64) mask[e] = 0ull;
  wave_lds_sync();
  const unsigned long long bit = 1ull << lane;
  int ev[kKReg];
  if (lane < T) load_ids(idx, lane, K, ev);
  if (lane < T)
    for_ids(idx, lane, K, ev, [&](int, int e) {
      if ((unsigned)e < (unsigned)N) atomicOr(&mask[e], bit);
    });
  wave_lds_sync();
  int carry = 0;
  for (int b = 0; b < N; b += 64) {
    const int e = b + lane;
    const int c = e < N ? __popcll(mask[e]) : 0;
    const int inc = wave_inclusive_scan(c);
    if (e < N) {
      s_off[e] = carry + inc - c;
      if (counts != nullptr) counts[e] = c;
      if (offsets != nullptr) offsets[e] = carry + inc - c;
    }
    carry += __shfl(inc, 63);
  }
  if (lane == 0) {
    s_off[N] = carry;
    if (offsets != nullptr) offsets[N] = carry;
  }
  wave_lds_sync();
  if (lane < T) {
    const unsigned long long below = bit - 1ull;
    for_ids(idx, lane, K, ev, [&](int k, int e) {
      if ((unsigned)e < (unsigned)N) {
        const int pos = s_off[e] + __popcll(mask[e] & below);
        if (s_sp != nullptr) s_sp[pos] = lane * K + k;
        if (sorted_pair != nullptr) sorted_pair[pos] = lane * K + k;
      }
    });
  }
  wave_lds_sync();
}

// Exclusive prefix of bm-row m-tiles per virtual expert into out[0..V]
// (experts 0..N-1 routed, with off[0..N] their slot offsets; N..V-1 shared,
// T rows each), one wavefront (all lanes call it) -- the table a grouped GEMM
// walks, as tile_tables_wave writes it.
__device__ __forceinline__ void mtile_prefix_wave(const int* off, int N, int V, int T, int TK,
                                                  int bm, int* out) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int b = 0; b < V; b += 64) {
    const int v = b + lane;
    int mt = 0;
    if (v < V) {
      int rows = T;
      if (v < N) {
        const int lo = min(max(off[v], 0), TK), hi = min(max(off[v + 1], lo), TK);
        rows = hi - lo;
      }
      mt = (rows + bm - 1) / bm;
    }
    const int inc = wave_inclusive_scan(mt);
    if (v < V) out[v] = carry + inc - mt;
    carry += __shfl(inc, 63);
  }
  if (lane == 0) out[V] = carry;
  wave_lds_sync();
}

}  // namespace
}  // namespace moe
