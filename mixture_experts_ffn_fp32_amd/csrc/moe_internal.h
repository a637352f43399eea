// Internal declarations shared by the gfx950 kernels and the C-ABI host code.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Timing of the stage being enqueued (the C ABI's stage scopes, when timing is
// on): the next launch's start / stop events (null when the stage is not
// timed; the start only on the stage's first launch, the stop on each, so the
// pair spans all of the stage's kernels).  They ride on the kernel dispatch
// itself (hipExtLaunchKernel), so timing puts no marker packets between
// kernels.
struct LaunchEvents {
  hipEvent_t start, stop;
};
LaunchEvents stage_launch_events();

template <class... P, class... A>
inline hipError_t launch_kernel(void (*k)(P...), dim3 grid, dim3 block, hipStream_t st,
                                A... args) {
  const LaunchEvents ev = stage_launch_events();
  hipExtLaunchKernelGGL(k, grid, block, 0, st, ev.start, ev.stop, 0, args...);
  return hipGetLastError();
}

// ---------------------------------------------------------------- types
using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
using f32x4 = float __attribute__((ext_vector_type(4)));
using f32x16 = float __attribute__((ext_vector_type(16)));
using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using bf16x2 = __bf16 __attribute__((ext_vector_type(2)));

// Element traits: storage type and how many elements one 16-byte chunk holds.
struct ElemF32 {
  using T = float;
  static constexpr int kPerChunk = 4;
};
struct ElemBF16 {
  using T = uint16_t;  // bfloat16 bit pattern
  static constexpr int kPerChunk = 8;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}
// float -> bfloat16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t x = __float_as_uint(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return uint16_t((x >> 16) | 0x40u);
  x += 0x7fffu + ((x >> 16) & 1u);
  return uint16_t(x >> 16);
}

template <class E>
__device__ __forceinline__ float load_as_f32(const typename E::T* p);
template <>
__device__ __forceinline__ float load_as_f32<ElemF32>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_as_f32<ElemBF16>(const uint16_t* p) {
  return bf16_to_f32(*p);
}

template <class E>
__device__ __forceinline__ void store_from_f32(typename E::T* p, float v);
template <>
__device__ __forceinline__ void store_from_f32<ElemF32>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_from_f32<ElemBF16>(uint16_t* p, float v) {
  *p = f32_to_bf16(v);
}

// ---------------------------------------------------------------- LDS tiles
// A tile row holds 128 bytes of the contraction dimension as 8 chunks of 16
// bytes.  Chunk c of row r lives at chunk slot c ^ ((r >> 1) & 7): 16 lanes
// reading 16 consecutive rows at one chunk index then touch 16 distinct
// 16-byte bank groups (two rows span the 256-byte bank width).
__device__ __forceinline__ int lds_chunk_offset(int r, int c) {
  return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}
// The same for 64-byte rows (4 chunks): four rows share a 256-byte bank
// window, so chunk c of row r lives at slot c ^ ((r >> 2) & 3).
template <int ROW_BYTES>
__device__ __forceinline__ int lds_chunk_offset_t(int r, int c) {
  if (ROW_BYTES == 128) return lds_chunk_offset(r, c);
  return r * 64 + ((c ^ ((r >> 2) & 3)) << 4);
}

// ---------------------------------------------------------------- launchers
// Router: logits, softmax, top-K.  Returns hipError_t of the launch.  With
// `rank` and `tile_counts` set, the tiled router (batches of more than 128
// tokens, or any batch with MOE_ROUTER_SMALL=0) also writes step 1 of the
// dispatch for its kRankTile-token blocks (what tile_rank below writes) and
// sets *ranked; the one-block-per-token router leaves *ranked false.
hipError_t launch_router(int dtype, const void* u, const void* E_gate, const float* bias, int T,
                         int d, int N, int K, int32_t* idx, float* gate, float* scores,
                         hipStream_t stream, int32_t* rank = nullptr,
                         int32_t* tile_counts = nullptr, bool* ranked = nullptr);

// Tile tables of the grouped GEMMs: per virtual expert (routed experts, then
// the shared ones) an exclusive prefix of m-tiles of bm rows, and the
// persistent GEMMs' 16 tile-claim counters zeroed.  GEMM1 has N + K_s virtual
// experts of bm1 rows (a shared expert has T rows), GEMM2 N + (K_s > 0) of
// bm2 rows (the shared experts are one virtual expert).  Either dispatch
// launch writes them when `tiles1` is set (the forward then needs no launch
// of its own for them).
struct TileTableOut {
  int32_t* tiles1;    // [N + K_s + 1]
  int32_t* tiles2;    // [N + 2]
  int32_t* counters;  // [16]
  int K_s, T, bm1, bm2;
};
// Lanes 0..63 of one wavefront; off[0..N] are the dispatch offsets (each
// expert's slot range clamped into [0, TK] exactly as the GEMMs clamp it).
__device__ __forceinline__ void tile_tables_wave(const int* off, int N, int TK,
                                                 const TileTableOut& o) {
  const int lane = threadIdx.x & 63;
  if (lane < 16) o.counters[lane] = 0;
  for (int which = 0; which < 2; ++which) {
    const int V = which == 0 ? N + o.K_s : N + (o.K_s > 0 ? 1 : 0);
    const int bm = which == 0 ? o.bm1 : o.bm2;
    int32_t* out = which == 0 ? o.tiles1 : o.tiles2;
    int carry = 0;
    for (int b = 0; b < V; b += 64) {
      const int v = b + lane;
      int mt = 0;
      if (v < V) {
        int rows = o.T;
        if (v < N) {
          const int lo = min(max(off[v], 0), TK), hi = min(max(off[v + 1], lo), TK);
          rows = hi - lo;
        }
        mt = (rows + bm - 1) / bm;
      }
      int inc = mt;
#pragma unroll
      for (int k = 1; k < 64; k <<= 1) {
        const int y = __shfl_up(inc, k);
        if (lane >= k) inc += y;
      }
      if (v < V) out[v] = carry + inc - mt;
      carry += __shfl(inc, 63);
    }
    if (lane == 0) out[V] = carry;
  }
}

// Dispatch: per-tile ranks (tiles of kRankTile tokens, the tiled router's
// block), global scan, scatter; batches of at most kSmallDispatchT tokens in
// one launch.
constexpr int kRankTile = 32;
constexpr int kSmallDispatchT = 64;
// tile_counts and tile_base are [N][rank_row(ntiles)]: one row of tiles per
// expert, its length rounded up to whole 16-byte groups.
__host__ __device__ inline int rank_row(int ntiles) { return (ntiles + 3) & ~3; }
hipError_t launch_tile_rank(const int32_t* idx, int T, int N, int K, int32_t* tile_counts,
                            int32_t* rank, hipStream_t stream);
// tt.tiles1 == NULL: no tile tables.
hipError_t launch_dispatch_scan(const int32_t* tile_counts, int ntiles, int N, int32_t* counts,
                                int32_t* offsets, int32_t* tile_base, const TileTableOut& tt,
                                hipStream_t stream);
hipError_t launch_dispatch_small(const int32_t* idx, int T, int N, int K, int32_t* counts,
                                 int32_t* offsets, int32_t* sorted_pair, const TileTableOut& tt,
                                 hipStream_t stream);
// Steps 2 and 3 in one launch (every block re-derives the scan it needs),
// where the tile counts are small enough: scan_scatter_fits(T, N).
bool scan_scatter_fits(int T, int N);
hipError_t launch_scan_scatter(const int32_t* idx, const int32_t* rank, const int32_t* tile_counts,
                               int T, int N, int K, int32_t* counts, int32_t* offsets,
                               int32_t* sorted_pair, const TileTableOut& tt, hipStream_t stream);
hipError_t launch_scatter(const int32_t* idx, const int32_t* rank, const int32_t* tile_base,
                          int T, int N, int K, int32_t* sorted_pair, hipStream_t stream);

// Expert GEMMs.
struct ExpertArgs {
  const void* u;
  const void* W_routed;
  const void* W_shared;
  const int32_t* offsets;      // [N+1]
  const int32_t* sorted_pair;  // [T*K]
  const float* gate;           // [T*K]
  void* H_routed;              // [T*K][I]
  void* H_shared;              // [T][K_s*I]
  void* Y;                     // [T*K][d]
  void* Y_shared;              // [T][d]
  int32_t* tiles1;             // [N+K_s+1] m-tile prefix for GEMM1
  int32_t* tiles2;             // [N+2]     m-tile prefix for GEMM2
  int32_t* counters;           // [16]      tile claims per XCD (GEMM1, GEMM2), zeroed per launch
  int T, d, I, N, K, K_s;
  // N that picks the kernels (0: N).  A launch over the shared experts alone
  // (N = 0) keeps the choice the whole layer would make.
  int sel_N;
  // A decode batch's dispatch derived inside GEMM1 (idx set; only where
  // gemm1_derives_dispatch says so): every block computes it from the
  // routing, block 0 also writes its outputs and the tile tables for the
  // launches after it.
  struct {
    const int32_t* idx;     // [T][K]
    int32_t* counts;        // [N]
    int32_t* offsets;       // [N+1] (the array `offsets` above then points to)
    int32_t* sorted_pair;   // [T*K] (likewise)
    TileTableOut tt;
  } fd;
};
// Most (token, expert) pairs a GEMM1 launch derives the dispatch of itself.
constexpr int kFusedDispatchPairs = 1024;
// Whether the GEMM1 launch of these shapes derives the dispatch itself when
// given the routing (a bf16 batch of at most kSmallDispatchT tokens on the
// long-run streaming kernel, at most kFusedDispatchPairs pairs).
bool gemm1_derives_dispatch(int dtype, const ExpertArgs& a);
// Weight streaming with 512-byte runs per weight row (expert_stream.hip):
// whether a launch of GEMM `mode` fits it, its m-tile height, and the launch.
bool stream_long_ok(int mode, const ExpertArgs& a);
int stream_long_rows();
hipError_t launch_stream_long(int mode, const ExpertArgs& a, int cus, hipStream_t st);
int expert_tile_table_ints(int N, int K_s);
// The tables' outputs and m-tile heights for these shapes (a.offsets unused).
TileTableOut expert_tile_tables(int dtype, const ExpertArgs& a);
hipError_t launch_tile_table(int dtype, const ExpertArgs& a, hipStream_t stream);
hipError_t launch_gemm1(int dtype, const ExpertArgs& a, hipStream_t stream);
hipError_t launch_gemm2(int dtype, const ExpertArgs& a, hipStream_t stream);

// Balance statistics: per-chunk partial sums, then one block.  groups.of[i]
// is the device group of routed expert i (D = 0: no device groups).
constexpr int kBalRows = 128;
struct BalanceGroups {
  int D;
  int32_t of[256];
};
size_t balance_workspace_bytes(int T, int N);
hipError_t launch_balance(const float* scores, const int32_t* idx, int T, int N, int K,
                          const BalanceGroups& groups, float alpha1, float alpha2, float* f,
                          float* P, float* f_dev, float* P_dev, float* losses, void* workspace,
                          hipStream_t stream);

// Backward pass (csrc/backward.hip).  Slot-ordered buffers follow the
// dispatch order of the forward (routed slots), shared ones are per token.
struct BwdArgs {
  const void* u;
  const void* dh;
  const void* E_gate;
  const void* W_routed;
  const void* W_shared;
  const int32_t* offsets;      // [N+1]
  const int32_t* sorted_pair;  // [T*K]
  float* AC;                   // [T*K][2I]      a = W_gate x, c = W_up x (routed slots)
  float* ACs;                  // [T][K_s*2I]    the same for the shared experts
  float* dP;                   // [T*K][I]       W_down^T dh (routed slots)
  float* dPs;                  // [T][K_s*I]
  void* dAC;                   // [T*K][2I] dtype  [da, dc]
  void* dACs;                  // [T][K_s*2I]
  void* P;                     // [T*K][I] dtype   p = SiLU(a) c (bf16 path: g p)
  void* Ps;                    // [T][K_s*I]
  void* dY;                    // [T*K][d] dtype   g * dh rows
  float* dX;                   // [T*K][d]       W_gate^T da + W_up^T dc (routed slots)
  float* dXs;                  // [K_s][T][d]
  void* dzE;                   // [T][NP] dtype  softmax gradient, rows padded to NP
  float* dE_part;              // [chunks][N][d] partial router gradients
  float* dE_gate;              // [N][d]
  float* dW_routed;            // N weight blocks (float32)
  float* dW_shared;            // K_s weight blocks (float32)
  int T, d, I, N, K, K_s, NP;
  // bfloat16 path (every product a grouped GEMM on the LDS-DMA pipeline; V = N + K_s)
  const float* gate;           // [T*K] kept gates by pair
  void* XT;                    // [d][ldx]    u^T over the padded slot columns
  void* dhT;                   // [d][ldx]    dh^T over the same columns
  float* dsp;                  // [T*K][ceil(I/128)] partial gate gradients per 128 columns
  int32_t* pcol;               // [N+1] padded first column of each routed expert
  long long ldx;               // row pitch (elements) of XT and dhT
  int Tp;                      // T rounded up to 64: the shared experts' column count
};
int backward_de_chunks(int T);
// Padded slot columns: every virtual expert's slots rounded up to 64.
inline long long bt_routed_cols(int T, int K, int N) {
  return (((long long)T * K + 63LL * N) + 63) / 64 * 64;
}
__host__ __device__ inline int bt_pad64(int x) { return (x + 63) & ~63; }
int bt_tables_ints(int N, int K_s);
hipError_t launch_bt_prep(const BwdArgs& a, int32_t* tabs, hipStream_t st);
hipError_t launch_bt_gemm(int G, const BwdArgs& a, int32_t* tabs, hipStream_t st);
hipError_t launch_bt_ds(const BwdArgs& a, const int32_t* slot_of, float* ds_pair, hipStream_t st);
// tabs: the pipelined bfloat16 path's tables (bt_tables_ints + N + 1 ints for
// the padded columns), or NULL for the generic path.
hipError_t launch_backward(int dtype, const BwdArgs& a, const float* gate, const float* scores,
                           const int32_t* idx, float* ds_pair, int32_t* slot_of, float* dz,
                           float* dgate_bias, void* du, int32_t* tab,
                           int32_t* tabs, hipStream_t stream);

hipError_t launch_combine(int dtype, const void* u, const void* Y, const void* Y_shared, int T,
                          int d, int K, int K_s, void* h, hipStream_t stream);

}  // namespace moe
