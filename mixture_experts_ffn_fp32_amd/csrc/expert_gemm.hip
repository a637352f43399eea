// Grouped expert GEMMs for gfx950 (MFMA 32x32, LDS-staged, double-buffered).
//
// Each expert is a SwiGLU FFN, FFN(x) = W_down (SiLU(W_gate x) * (W_up x))
// (an expert has the structure of a standard FFN: DeepSeekMoE paper summary,
// papercache.org, sec. A3; SwiGLU per the dtcms.com notes on DeepSeek LLM's
// model structure).  Routed expert i sees only the tokens that selected it
// and its output is scaled by the gate g_{i,t}; shared experts see every
// token with coefficient 1 (sec. 3.2 layer equation).
//
//  GEMM1: H = SiLU(X W_gate^T) * (X W_up^T), X = the expert's rows of u
//         (gathered through sorted_pair), gate and up tiles of the same
//         columns computed by the same wavefront so the SwiGLU is in-register.
//  GEMM2: Y = g * (H W_down^T), written to the token-major row t*K+k so the
//         combine reads each token's K rows contiguously.  The K_s shared
//         experts are one FFN of intermediate K_s*I (their H columns side by
//         side), so their down projections sum inside one contraction.
//
// Routed experts and shared experts are "virtual experts" of one launch: a
// tile table (exclusive prefix of m-tiles per virtual expert) maps the linear
// tile id to (expert, m-tile, n-tile), m fastest so concurrent tiles share
// the expert's weight tile, and the block id is remapped so that each XCD
// (workgroups are dealt round-robin over the 8 XCDs) owns a contiguous range
// of tiles and its L2 holds that expert's weights and tokens.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "lds_dma.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxV = 256 + 16;  // routed + shared virtual experts

__device__ __forceinline__ f32x16 mfma32(ElemBF16, u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// float32: a 16-byte chunk holds 4 k values; step i takes element i from every lane.
__device__ __forceinline__ f32x16 mfma32(ElemF32, u32x4 a, u32x4 b, f32x16 c) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i]), __uint_as_float(b[i]), c, 0,
                                             0, 0);
  return c;
}

__device__ __forceinline__ int xcd_swizzle(int b, int G) {
  const int x = b & 7, q = G >> 3, r = G & 7;
  return x * q + min(x, r) + (b >> 3);
}

// Tile tables of both GEMMs from caller-given dispatch offsets (one wavefront).
__global__ __launch_bounds__(64) void tile_table_kernel(const int32_t* __restrict__ offsets,
                                                        int N, int TK, TileTableOut o) {
  tile_tables_wave(offsets, N, TK, o);
}

// ---------------------------------------------------------------- shared pieces
// The tile of one block: virtual expert v, its first output column n0, first
// row m0, and the expert's slot range.
// (All int: a bool member leaves padding bytes that a struct copy moves
// through per-thread memory, which the compiler may place in LDS and then
// wait for every direct-to-LDS load in flight before touching.)
struct Tile {
  int v, n0, m0, row_base, rows;
  int routed;  // 0 or 1
};

// Maps the block to its tile through the tile table (m fastest within an
// expert).  Returns false if the block has no tile (grids are sized for the
// worst case, so the highest block ids may find none).  Every thread of the
// block gets the same answer.
template <int BM, int BNO, int MODE>
__device__ __forceinline__ bool find_tile(const ExpertArgs& a, int* s_tab, int* s_v, Tile& ti) {
  const int tid = threadIdx.x;
  const int V = MODE == 1 ? a.N + a.K_s : a.N + (a.K_s > 0 ? 1 : 0);
  const int32_t* tab = MODE == 1 ? a.tiles1 : a.tiles2;
  const int nt = (MODE == 1 ? a.I : a.d) / BNO;
  for (int i = tid; i <= V; i += blockDim.x) s_tab[i] = tab[i];
  __syncthreads();
  // blocks past the real tile count leave; the rest are dealt over the XCDs
  const int total = s_tab[V] * nt;
  if ((int)blockIdx.x >= total) return false;
  const int L = xcd_swizzle(blockIdx.x, total);
  for (int i = tid; i < V; i += blockDim.x)
    if (s_tab[i] * nt <= L && L < s_tab[i + 1] * nt) *s_v = i;
  __syncthreads();
  const int v = *s_v;
  const int mt_v = s_tab[v + 1] - s_tab[v];
  const int local = L - s_tab[v] * nt;
  ti.v = v;
  ti.n0 = (local / mt_v) * BNO;
  ti.m0 = (local % mt_v) * BM;
  ti.routed = v < a.N ? 1 : 0;
  const int TK = a.T * a.K;
  ti.row_base = 0;
  ti.rows = a.T;
  if (ti.routed) {
    ti.row_base = min(max(a.offsets[v], 0), TK);
    ti.rows = min(max(a.offsets[v + 1], ti.row_base), TK) - ti.row_base;
  }
  return true;
}

// Persistent kernels: load the tile table once, then map any tile id.
template <int MODE>
__device__ __forceinline__ int load_tile_table(const ExpertArgs& a, int* s_tab) {
  const int V = MODE == 1 ? a.N + a.K_s : a.N + (a.K_s > 0 ? 1 : 0);
  const int32_t* tab = MODE == 1 ? a.tiles1 : a.tiles2;
  for (int i = threadIdx.x; i <= V; i += blockDim.x) s_tab[i] = tab[i];
  __syncthreads();
  return V;
}

// Tile L of the table in LDS (every thread searches the same entries: no barrier).
// kLdsOff: the dispatch offsets are read from an LDS copy `s_off` (no global
// load, whose wait would also wait for every load in flight).
template <int BM, int BNO, int MODE, bool kLdsOff = false>
__device__ __forceinline__ Tile tile_of(const ExpertArgs& a, const int* s_tab, int V, int L,
                                        const int* s_off = nullptr) {
  const int nt = ((MODE == 1 ? a.I : a.d) + BNO - 1) / BNO;  // the last n-tile may be partial
  int lo = 0, hi = V - 1;  // largest v with s_tab[v] * nt <= L
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_tab[mid] * nt <= L) lo = mid; else hi = mid - 1;
  }
  // empty experts share their start with the next one: move to the first that owns L
  while (lo + 1 <= V && s_tab[lo + 1] * nt <= L) ++lo;
  Tile ti;
  const int v = lo;
  const int mt_v = s_tab[v + 1] - s_tab[v];
  const int local = L - s_tab[v] * nt;
  ti.v = v;
  ti.n0 = (local / mt_v) * BNO;
  ti.m0 = (local % mt_v) * BM;
  ti.routed = v < a.N ? 1 : 0;
  const int TK = a.T * a.K;
  ti.row_base = 0;
  ti.rows = a.T;
  if (ti.routed) {
    const int o0 = kLdsOff ? s_off[v] : a.offsets[v];
    const int o1 = kLdsOff ? s_off[v + 1] : a.offsets[v + 1];
    ti.row_base = min(max(o0, 0), TK);
    ti.rows = min(max(o1, ti.row_base), TK) - ti.row_base;
  }
  return ti;
}

// Start of tile row r (A rows 0..BM-1, then B rows) at contraction index 0.
// A rows past the expert's last slot repeat its last row (never stored).
template <class E, int MODE, int BM, int BNB>
__device__ __forceinline__ const typename E::T* tile_row_ptr(const ExpertArgs& a, const Tile& ti,
                                                             int r) {
  using Tp = typename E::T;
  const size_t Id = (size_t)a.I * a.d;
  if (r < BM) {
    const int p = min(ti.m0 + r, ti.rows - 1);
    if (MODE == 1) {
      int tok = p;
      if (ti.routed) {
        const int TK = a.T * a.K;
        const int pair = a.sorted_pair[ti.row_base + p];
        tok = ((unsigned)pair < (unsigned)TK) ? pair / a.K : 0;
      }
      return (const Tp*)a.u + (size_t)tok * a.d;
    }
    return ti.routed ? (const Tp*)a.H_routed + (size_t)(ti.row_base + p) * a.I
                     : (const Tp*)a.H_shared + (size_t)p * a.K_s * a.I;
  }
  const int rb = r - BM;
  const Tp* W = ti.routed ? (const Tp*)a.W_routed + (size_t)ti.v * 3 * Id
                          : (const Tp*)a.W_shared + (size_t)(MODE == 1 ? ti.v - a.N : 0) * 3 * Id;
  // columns past the last one (a partial last n-tile) reread the last row
  if (MODE == 1)
    return rb < BNB / 2 ? W + (size_t)min(ti.n0 + rb, a.I - 1) * a.d
                        : W + Id + (size_t)min(ti.n0 + rb - BNB / 2, a.I - 1) * a.d;
  return W + 2 * Id + (size_t)min(ti.n0 + rb, a.d - 1) * a.I;
}

// Element offset of contraction index k0 in a B row.  The shared experts'
// down projections are one contraction over K_s*I: index k0 lies in expert
// k0 / I's W_down block.
template <int MODE>
__device__ __forceinline__ size_t b_offset(const ExpertArgs& a, const Tile& ti, size_t k0) {
  if (MODE == 2 && !ti.routed) {
    // 32-bit quotient (k0 < K_s * I < 2^31): a 64-bit one is a long scalar
    // sequence, and this runs at every k-step of a shared tile
    const uint32_t kb = (uint32_t)k0 / (uint32_t)a.I;
    return k0 + (size_t)kb * (3 * (size_t)a.I * a.d - a.I);
  }
  return k0;
}

// B tile row of wavefront column wn's fragment fn.  GEMM1 puts the gate rows
// in the first half of the B tile and the up rows of the same columns in the
// second half; a wavefront takes matching gate and up fragments.
template <int MODE, int FN, int BNB>
__device__ __forceinline__ int b_frag_row(int wn, int fn) {
  if (MODE == 1)
    return fn < FN / 2 ? (wn * (FN / 2) + fn) * 32
                       : BNB / 2 + (wn * (FN / 2) + fn - FN / 2) * 32;
  return (wn * FN + fn) * 32;
}

// Epilogue.  acc[fm][fn][r] holds tile row (wm*FM + fm)*32 + 8*(r/4) + 4*(lane/32) + r%4,
// column lane%32 of fragment fn.
template <class E, int MODE, int FM, int FN>
__device__ __forceinline__ void store_tile(const ExpertArgs& a, const Tile& ti, int wm, int wn,
                                           f32x16 (&acc)[FM][FN]) {
  using Tp = typename E::T;
  const int lane = threadIdx.x & 63;
  const int lc = lane & 31, lh = lane >> 5;
  const int TK = a.T * a.K;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int p = ti.m0 + (wm * FM + fm) * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (p >= ti.rows) continue;
      if (MODE == 1) {
#pragma unroll
        for (int fn = 0; fn < FN / 2; ++fn) {
          const float gt = acc[fm][fn][r], up = acc[fm][fn + FN / 2][r];
          const float hv = gt / (1.f + expf(-gt)) * up;   // SiLU(gate) * up
          const int col = ti.n0 + (wn * (FN / 2) + fn) * 32 + lc;
          if (col >= a.I) continue;  // partial last n-tile
          Tp* dst = ti.routed
                        ? (Tp*)a.H_routed + (size_t)(ti.row_base + p) * a.I + col
                        : (Tp*)a.H_shared + (size_t)p * a.K_s * a.I + (size_t)(ti.v - a.N) * a.I + col;
          store_from_f32<E>(dst, hv);
        }
      } else {
        float g = 1.f;
        Tp* dst;
        if (ti.routed) {
          int pair = a.sorted_pair[ti.row_base + p];
          pair = ((unsigned)pair < (unsigned)TK) ? pair : 0;
          g = a.gate[pair];
          dst = (Tp*)a.Y + (size_t)pair * a.d;
        } else {
          dst = (Tp*)a.Y_shared + (size_t)p * a.d;
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int col = ti.n0 + (wn * FN + fn) * 32 + lc;
          if (col < a.d) store_from_f32<E>(dst + col, acc[fm][fn][r] * g);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- register-staged kernel
// Any d, I that are multiples of 64: tiles staged global -> registers -> LDS,
// two LDS buffers, up to two blocks per CU.
template <class E, int WM, int WN, int FM, int FN, int MODE>
__global__ __launch_bounds__(256) void expert_gemm_kernel(ExpertArgs a) {
  using Tp = typename E::T;
  constexpr int BM = WM * FM * 32;
  constexpr int BNB = WN * FN * 32;               // B rows per tile
  constexpr int BNO = MODE == 1 ? BNB / 2 : BNB;  // output columns per tile
  constexpr int ROWS = BM + BNB;
  constexpr int PASSES = ROWS / 32;
  constexpr int PASSES_A = BM / 32;
  constexpr int kStep = 128 / (int)sizeof(Tp);
  static_assert(WM * WN == 4, "four wavefronts");
  static_assert(MODE == 2 || FN % 2 == 0, "GEMM1 pairs gate and up fragments");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][ROWS * 128];
  __shared__ int s_tab[kMaxV + 1];
  __shared__ int s_v;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  Tile ti;
  if (!find_tile<BM, BNO, MODE>(a, s_tab, &s_v, ti)) return;
  const int Kc = MODE == 1 ? a.d : (ti.routed ? a.I : a.K_s * a.I);  // contraction length
  const int nsteps = Kc / kStep;

  // each thread moves chunk c of rows tid/8 + 32 i
  const int c = tid & 7;
  const Tp* rowp[PASSES];
#pragma unroll
  for (int i = 0; i < PASSES; ++i) rowp[i] = tile_row_ptr<E, MODE, BM, BNB>(a, ti, (tid >> 3) + 32 * i);
  u32x4 stage[PASSES];
  auto gload = [&](int s) {
    const size_t k0 = (size_t)s * kStep;
    const size_t kb = b_offset<MODE>(a, ti, k0);
#pragma unroll
    for (int i = 0; i < PASSES; ++i)
      stage[i] = *(const u32x4*)(rowp[i] + (i < PASSES_A ? k0 : kb) + c * E::kPerChunk);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PASSES; ++i)
      *(u32x4*)(lds[buf] + lds_chunk_offset((tid >> 3) + 32 * i, c)) = stage[i];
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) gload(s + 1);
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {  // a 128-byte row = four k-groups of 2 chunks
      const int ch = kg * 2 + (lane >> 5);
      u32x4 af[FM], bfr[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = *(const u32x4*)(lds[buf] + lds_chunk_offset((wm * FM + fm) * 32 + (lane & 31), ch));
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        bfr[fn] = *(const u32x4*)(lds[buf] +
                                  lds_chunk_offset(BM + b_frag_row<MODE, FN, BNB>(wn, fn) + (lane & 31), ch));
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma32(E{}, af[fm], bfr[fn], acc[fm][fn]);
    }
    if (s + 1 < nsteps) lstore(buf ^ 1);
    __syncthreads();
  }
  store_tile<E, MODE, FM, FN>(a, ti, wm, wn, acc);
}

// ---------------------------------------------------------------- LDS-DMA helpers
// Direct-to-LDS loads of one k-step of this lane's rows into `wr` (every row
// of a wavefront belongs to the same operand, so `base` is wavefront-uniform
// and each load is a scalar base plus a 32-bit lane offset).  The restrict
// qualifier gives the compiler an alias scope, so it never makes LDS reads of
// the other ring slot wait for these loads (the kernel orders the refill of a
// slot after its last reads with its own waits and barrier).
template <int NINST>
__device__ __forceinline__ void dma_fill(uint8_t* __restrict__ wr, const uint8_t* base,
                                         const uint32_t (&off)[NINST], int nrec = 0x7fffffff) {
#pragma unroll
  for (int i = 0; i < NINST; ++i) dma16(base, off[i], wr + i * 1024, nrec);
}

template <int FM, int FN, int RB, int BM, int BNB, int MODE>
__device__ __forceinline__ void load_frags(const uint8_t* __restrict__ rd, int kg, int wm, int wn,
                                           int lane, u32x4 (&af)[FM], u32x4 (&bfr)[FN]) {
  const int ch = kg * 2 + (lane >> 5);
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
    af[fm] = *(const u32x4*)(rd + lds_chunk_offset_t<RB>((wm * FM + fm) * 32 + (lane & 31), ch));
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
    bfr[fn] = *(const u32x4*)(rd + lds_chunk_offset_t<RB>(
                                       BM + b_frag_row<MODE, FN, BNB>(wn, fn) + (lane & 31), ch));
}

// ---------------------------------------------------------------- pipelined LDS-DMA kernel
// Tiles of 256 rows x 256 B rows (GEMM1: 128 gate + 128 up rows of the same
// columns; GEMM2: 256 output columns), W wavefronts in (W/2) x 2, each owning
// 512/W rows x 128 columns (FM x 4 fragments of 32 x 32; W = 8, two
// wavefronts per SIMD).  Operands reach LDS by
// direct-to-LDS loads (buffer_load_dwordx4 ... lds: lane L of a wavefront writes
// 16 bytes at the wavefront's LDS address + 16 L), one 128-byte k-step per
// row, in a two-slot ring: k-step s + 1 lands while k-step s is multiplied.
// The LDS swizzle is applied on the global side (lane L fetches the chunk that
// belongs in LDS slot L).  The kernel is persistent and the next tile's
// first k-step loads during a tile's last one.  bf16 results leave straight
// from the accumulators (16-byte runs after lane exchanges) once the next
// tile's first k-step has landed and its second k-step's loads are issued;
// float32 results are written at the end of their tile (store_tile).  One
// block per CU.
constexpr int kPipeBM = 256, kPipeBNB = 256, kPipeRB = 128;
constexpr int kPipeSlot = (kPipeBM + kPipeBNB) * kPipeRB;  // 64 KB
template <int W>
struct PipeCfg {
  static constexpr int kThreads = 64 * W;
  static constexpr int kNinst = (kPipeBM + kPipeBNB) / (8 * W);  // loads per wavefront per k-step
  static constexpr int FM = kPipeBM / (32 * (W / 2));            // row fragments per wavefront
  static constexpr int FN = 4;
};

// Per-tile load state of one lane: operand bases and 32-bit byte offsets.
template <int NI>
struct PipeLoads {
  const uint8_t* a_base;  // u (GEMM1) or H (GEMM2) at contraction index 0
  const uint8_t* b_row0;  // the tile's first B row at contraction index 0
  uint32_t off[NI];       // this lane's chunk of each of its rows
};

__device__ __forceinline__ Tile uni(const Tile& t) {
  Tile u;
  u.v = uni(t.v);
  u.n0 = uni(t.n0);
  u.m0 = uni(t.m0);
  u.row_base = uni(t.row_base);
  u.rows = uni(t.rows);
  u.routed = uni(t.routed);
  return u;
}

template <class E, int MODE, int NI>
__device__ __forceinline__ void pipe_prepare(const ExpertArgs& a, const Tile& ti, int wave,
                                             int lane, bool is_a, PipeLoads<NI>& ld) {
  ld.b_row0 = uni((const uint8_t*)tile_row_ptr<E, MODE, kPipeBM, kPipeBNB>(a, ti, kPipeBM));
  ld.a_base = uni(MODE == 1 ? (const uint8_t*)a.u
                            : (const uint8_t*)(ti.routed ? a.H_routed : a.H_shared));
  if (MODE == 1 && ti.routed && is_a) {
    // gathered token rows: every row's pair index is requested before any
    // is used, so the lookups cost one round trip, not one each
    const int TK = a.T * a.K;
    int pr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (wave * NI + i) * 8 + (lane >> 3);
      pr[i] = a.sorted_pair[ti.row_base + min(ti.m0 + r, ti.rows - 1)];
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (wave * NI + i) * 8 + (lane >> 3);
      const uint32_t tok = (unsigned)pr[i] < (unsigned)TK ? (unsigned)pr[i] / (unsigned)a.K : 0u;
      const int chunk = (lane & 7) ^ ((r >> 1) & 7);
      ld.off[i] = tok * (uint32_t)a.d * (uint32_t)sizeof(typename E::T) + chunk * 16;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = (wave * NI + i) * 8 + (lane >> 3);
    const uint8_t* rp = (const uint8_t*)tile_row_ptr<E, MODE, kPipeBM, kPipeBNB>(a, ti, r);
    const int chunk = (lane & 7) ^ ((r >> 1) & 7);
    ld.off[i] = (uint32_t)(rp - (r < kPipeBM ? ld.a_base : ld.b_row0)) + chunk * 16;
  }
}

// Wavefront-uniform global base of this wavefront's rows at k-step s.
template <class E, int MODE, int NI>
__device__ __forceinline__ const uint8_t* pipe_dma_base(const ExpertArgs& a, const Tile& ti,
                                                        const PipeLoads<NI>& ld, int s, bool is_a) {
  using Tp = typename E::T;
  constexpr int kStep = kPipeRB / (int)sizeof(Tp);
  const size_t k0 = (size_t)s * kStep;
  const uint8_t* ab = ld.a_base + k0 * sizeof(Tp);
  const uint8_t* bb = ld.b_row0 + b_offset<MODE>(a, ti, k0) * sizeof(Tp);
  return uni(is_a ? ab : bb);
}

template <class E, int MODE, int NI>
__device__ __forceinline__ void pipe_issue(const ExpertArgs& a, const Tile& ti,
                                           const PipeLoads<NI>& ld, int s, bool is_a,
                                           uint8_t* __restrict__ wr) {
  dma_fill<NI>(wr, pipe_dma_base<E, MODE>(a, ti, ld, s, is_a), ld.off);
}

// The k-groups of one k-step that also issue the other slot's loads.
constexpr int kDmaGroups = 2;

// Multiplies one k-step out of slot `rd` and issues the direct-to-LDS loads
// of the other slot (base `db`, lane offsets `off`, into `wr`).  The
// instruction stream is laid out explicitly: the fragments of k-group g + 1
// are read from LDS, and the loads issued, one instruction after each MFMA
// of group g, so neither the LDS latency nor a burst of loads holds the
// MFMAs back.  A wavefront whose rows are all padding (`active` false) only
// issues its loads.
// kIssue false: the loads were issued already (nothing is issued here).
template <class E, int MODE, int FM, int NI, bool kIssue = true>
__device__ __forceinline__ void pipe_mma(const uint8_t* __restrict__ rd, int wm, int wn, int lane,
                                         f32x16 (&acc)[FM][4], bool active,
                                         const uint8_t* db, const uint32_t (&off)[NI],
                                         uint8_t* __restrict__ wr, int nrec = 0x7fffffff) {
  constexpr int FN = 4, KG = kPipeRB / 32, PARTS = kIssue ? kDmaGroups : 0,
                PER = kIssue ? NI / kDmaGroups : 0;
  static_assert(!kIssue || (NI % kDmaGroups == 0 && kDmaGroups <= KG), "DMA parts");
  if (!active) {
    if (kIssue) {
#pragma unroll
      for (int i = 0; i < NI; ++i) dma16(db, off[i], wr + i * 1024, nrec);
    }
    return;
  }
  u32x4 af[2][FM], bfr[2][FN];
  load_frags<FM, FN, kPipeRB, kPipeBM, kPipeBNB, MODE>(rd, 0, wm, wn, lane, af[0], bfr[0]);
#pragma unroll
  for (int kg = 0; kg < KG; ++kg) {
    if (kg < PARTS) {
#pragma unroll
      for (int i = kg * PER; i < (kg + 1) * PER; ++i) dma16(db, off[i], wr + i * 1024, nrec);
    }
    if (kg + 1 < KG)
      load_frags<FM, FN, kPipeRB, kPipeBM, kPipeBNB, MODE>(rd, kg + 1, wm, wn, lane,
                                                            af[(kg + 1) & 1], bfr[(kg + 1) & 1]);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        // bf16: weights as the 32-row operand (the layout the epilogue wants)
        acc[fm][fn] = std::is_same<E, ElemBF16>::value
                          ? mfma32(E{}, bfr[kg & 1][fn], af[kg & 1][fm], acc[fm][fn])
                          : mfma32(E{}, af[kg & 1][fm], bfr[kg & 1][fn], acc[fm][fn]);
  }
  // the layout: group 0's fragment reads first, then per k-group g its MFMAs,
  // each followed by one of group g + 1's reads and one of its loads
  __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
#pragma unroll
  for (int kg = 0; kg < KG; ++kg) {
    const int nr = kg + 1 < KG ? FM + FN : 0, nd = kg < PARTS ? PER : 0;
#pragma unroll
    for (int m = 0; m < FM * FN; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m < nr) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (m < nd) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  }
}

// SiLU(g) * u with the hardware exp2 and reciprocal (a few float32 ulp).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}


// 16 float32 of one 32 x 32 fragment (MFMA operands swapped: lane l holds
// token row l % 32 and output columns 8g + 4(l / 32) + 0..3, g = 0..3) ->
// two 16-byte bf16 runs: after exchanging halves between lanes l and l + 32
// (v_permlane32_swap), lane l holds columns 0-7 and 16-23 (l < 32) or 8-15
// and 24-31 (l >= 32).
__device__ __forceinline__ void pack_runs16(const float (&v)[16], u32x4& r0, u32x4& r1) {
  uint32_t w[4][2];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    w[g][0] = pack_bf16x2(v[4 * g], v[4 * g + 1]);
    w[g][1] = pack_bf16x2(v[4 * g + 2], v[4 * g + 3]);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const auto s01 = __builtin_amdgcn_permlane32_swap(w[0][q], w[1][q], false, false);
    const auto s23 = __builtin_amdgcn_permlane32_swap(w[2][q], w[3][q], false, false);
    w[0][q] = s01[0];
    w[1][q] = s01[1];
    w[2][q] = s23[0];
    w[3][q] = s23[1];
  }
  r0 = u32x4{w[0][0], w[0][1], w[1][0], w[1][1]};
  r1 = u32x4{w[2][0], w[2][1], w[3][0], w[3][1]};
}

// Epilogue straight from the accumulators (no LDS, no barrier): each lane
// writes two 16-byte runs per fragment of its token rows; dst[fm] / g[fm]
// are the destination row (-1: past the expert's last slot) and gate of the
// lane's row (wm * FM + fm) * 32 + lane % 32.
template <int MODE, int FM>
__device__ __forceinline__ void pipe_store_direct(const ExpertArgs& a, const Tile& ti, int wm,
                                                  int wn, f32x16 (&acc)[FM][4],
                                                  const int (&dsts)[FM], const float (&gates)[FM]) {
  constexpr int NF = MODE == 1 ? 2 : 4;  // output column groups of 32 per wavefront
  const int lane = threadIdx.x & 63, hi = lane >> 5;
  const int lim = MODE == 1 ? a.I : a.d;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int dst = dsts[fm];
    uint16_t* rp;
    if (MODE == 1)
      rp = ti.routed ? (uint16_t*)a.H_routed + (size_t)max(dst, 0) * a.I
                     : (uint16_t*)a.H_shared + (size_t)max(dst, 0) * a.K_s * a.I +
                           (size_t)(ti.v - a.N) * a.I;
    else
      rp = (ti.routed ? (uint16_t*)a.Y : (uint16_t*)a.Y_shared) + (size_t)max(dst, 0) * a.d;
    const float g = MODE == 2 ? gates[fm] : 1.f;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      float v[16];
      if (MODE == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = silu_mul(acc[fm][f][r], acc[fm][f + 2][r]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = acc[fm][f][r] * g;
      }
      u32x4 r0, r1;
      pack_runs16(v, r0, r1);  // every lane takes part in the exchange
      const int col = ti.n0 + (wn * NF + f) * 32;
      if (dst >= 0 && col < lim) {
        *(u32x4*)(rp + col + 8 * hi) = r0;
        *(u32x4*)(rp + col + 16 + 8 * hi) = r1;
      }
    }
  }
}

// Destination row of tile row r (H slot / token, or -1 past the expert's
// last slot); for GEMM2's routed rows the raw pair index, looked up here and
// checked by pipe_row_gate after the next barrier (nothing waits for the
// load in between).
template <int MODE>
__device__ __forceinline__ int pipe_row_dest(const ExpertArgs& a, const Tile& ti, int r) {
  const int p = ti.m0 + r;
  if (p >= ti.rows) return -1;
  if (MODE == 1 || !ti.routed) return (MODE == 1 && ti.routed) ? ti.row_base + p : p;
  return a.sorted_pair[ti.row_base + p];
}

// GEMM2's routed rows: the pair index brought into range and its gate.
template <int MODE>
__device__ __forceinline__ void pipe_row_gate(const ExpertArgs& a, const Tile& ti, int r, int& dst,
                                              float& g) {
  g = 1.f;
  if (MODE == 1 || !ti.routed || ti.m0 + r >= ti.rows) return;
  const int TK = a.T * a.K;
  dst = ((unsigned)dst < (unsigned)TK) ? dst : 0;
  g = a.gate[dst];
}

// The claim of a tile from a share's counter, issued by one lane.  The
// address is made to look lane-varying so that the compiler does not turn
// the atomic into a wavefront reduction whose broadcast waits for the reply
// at once: the reply is awaited at the next barrier's wait instead.
__device__ __forceinline__ int claim_issue(int* ctr) {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return atomicAdd(ctr + z, 1);
}

template <class E, int MODE, int W>
__global__ __launch_bounds__(64 * W, 1) void expert_gemm_pipe_kernel(ExpertArgs a) {
  using Tp = typename E::T;
  using Cfg = PipeCfg<W>;
  constexpr int BNO = MODE == 1 ? kPipeBNB / 2 : kPipeBNB;
  constexpr int kStep = kPipeRB / (int)sizeof(Tp);
  constexpr int NINST = Cfg::kNinst, FM = Cfg::FM;
  constexpr bool kDirect = std::is_same<E, ElemBF16>::value;  // bf16: epilogue from registers
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kPipeSlot];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kPipeSlot];
  __shared__ int s_tab[kMaxV + 1];
  __shared__ int s_off[kMaxV + 1];
  __shared__ int s_claim;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // wavefronts 0 .. W/2-1 load the A rows, the others the B rows
  static_assert((kPipeBM / 8) % NINST == 0, "a wavefront loads rows of one operand");
  const bool is_a = wave * NINST < kPipeBM / 8;

  // Persistent: the blocks of XCD x (blockIdx % 8, workgroups are dealt
  // round-robin over the XCDs) walk that XCD's contiguous share of the tiles,
  // so concurrent tiles share an expert's weights and tokens in the XCD's L2.
  // A GEMM2 tile of the shared experts contracts over K_s * I and costs K_s
  // routed tiles: every XCD then takes an equal share of those first (the
  // long tiles start early) and an equal share of the routed tiles after
  // them.  Each block takes one tile by its index in its XCD's share, then
  // claims the next one from the share's counter; when its XCD has none
  // left it claims from the other XCDs' (the XCDs run at different clocks).
  for (int i = tid; i <= a.N; i += blockDim.x) s_off[i] = a.offsets[i];
  const int V = load_tile_table<MODE>(a, s_tab);  // (its barrier also covers s_off)
  const int nt = ((MODE == 1 ? a.I : a.d) + BNO - 1) / BNO;
  const int total = s_tab[V] * nt;
  const int Lr = MODE == 2 ? s_tab[a.N] * nt : total;  // tiles before the shared ones
  const int S = total - Lr;                            // GEMM2's shared tiles
  const bool split = MODE == 2 && a.K_s > 1 && S > 0;
  const int X = min(8, (int)gridDim.x);
  const int x = blockIdx.x % X, lb = blockIdx.x / X;
  // 32-bit arithmetic: the host's operand bounds keep n * 8 far below 2^32
  auto part = [&](int n, int y) { return (int)((unsigned)n * (unsigned)y / (unsigned)X); };
  auto n_of = [&](int y) -> int {  // tiles in XCD y's share
    return split ? (part(S, y + 1) - part(S, y)) + (part(Lr, y + 1) - part(Lr, y))
                 : part(total, y + 1) - part(total, y);
  };
  auto map = [&](int y, int p) -> int {  // position p of XCD y's share -> tile
    if (split) {
      const int ns = part(S, y + 1) - part(S, y);
      return p < ns ? Lr + part(S, y) + p : part(Lr, y) + (p - ns);
    }
    return part(total, y) + p;
  };
  int* const ctr = a.counters + (MODE - 1) * 8;
  // position p of XCD y's share given counter reply c (the first blocks took
  // their tiles by index)
  auto pos = [&](int y, int c) { return ((int)gridDim.x - y + X - 1) / X + c; };
  // the next tile from the other XCDs' counters (-1: none), replies awaited one by one
  auto claim_others = [&]() -> int {
    for (int k = 1; k < X; ++k) {
      const int y = x + k < X ? x + k : x + k - X;
      const int p = pos(y, atomicAdd(ctr + y, 1));
      if (p < n_of(y)) return map(y, p);
    }
    return -1;
  };
  // the tile of the own XCD's counter reply c, else one of the others'
  auto claim_resolve = [&](int c) -> int {
    const int p = pos(x, c);
    return p < n_of(x) ? map(x, p) : claim_others();
  };
  int L = lb < n_of(x) ? map(x, lb) : -1;
  if (L < 0) {
    if (tid == 0) s_claim = claim_resolve(atomicAdd(ctr + x, 1));
    __syncthreads();
    L = uni(s_claim);
    __syncthreads();  // read by all before the first tile's claim rewrites it
    if (L < 0) return;
  }

  Tile ti = uni(tile_of<kPipeBM, BNO, MODE, true>(a, s_tab, V, L, s_off));
  PipeLoads<NINST> ld;
  pipe_prepare<E, MODE>(a, ti, wave, lane, is_a, ld);
  pipe_issue<E, MODE>(a, ti, ld, 0, is_a, lds0 + wave * NINST * 1024);

  f32x16 acc[FM][4];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  };
  zero_acc();
  // Destination row and gate of this lane's rows (wm * FM + fm) * 32 +
  // lane % 32, in registers until the epilogue.  bf16: a tile's results are
  // written after the next tile's first barrier (its first k-step has
  // landed), so that the wait for that k-step's loads does not also wait for
  // the stores; until then they stay in acc, dst and gate.
  int dst[FM];
  float gate[FM];
  bool pending = false;
  Tile tp = ti;
  while (true) {
    const int Kc = MODE == 1 ? a.d : (ti.routed ? a.I : a.K_s * a.I);
    // an odd k-step count is padded with one k-step of zeros (loaded as out
    // of range), so that k-steps always come in (slot 0, slot 1) pairs
    const int nreal = Kc / kStep;
    const int nsteps = nreal + (nreal & 1);
    // A wavefront whose rows all lie past the expert's last slot skips its
    // MFMAs (the other wavefront on its SIMD gets the MFMA unit).
    const bool active = ti.m0 + wm * FM * 32 < ti.rows;
    // The block's next tile, needed at the last k-step, is claimed during
    // the first k-step (the counter's reply is awaited with the second
    // k-step's loads) and published in s_claim at the last pair; with only
    // two k-steps it is claimed at once.
    int claim = -1, reply = 0;
    if (nsteps == 2 && tid == 0) claim = claim_resolve(atomicAdd(ctr + x, 1));
    int Ln = -1;
    bool has_next = false;

    Tile tn = ti;
    for (int s = 0; s < nsteps; s += 2) {
      if (s + 2 >= nsteps && tid == 0) s_claim = claim;
      // even k-step: slot 0 holds k-step s; k-step s + 1 goes to slot 1
      pipe_sync();
      const uint8_t* db1 = pipe_dma_base<E, MODE>(a, ti, ld, s + 1 < nreal ? s + 1 : 0, is_a);
      const int nrec1 = s + 1 < nreal ? 0x7fffffff : 0;
      uint8_t* const wr1 = lds1 + wave * NINST * 1024;
      // the next k-step's loads go out first (ahead of the previous tile's
      // stores after a tile change, so they do not queue behind them)
      dma_fill<NINST>(wr1, db1, ld.off, nrec1);
      if (kDirect && s == 0 && pending) {  // the previous tile's results
        pipe_store_direct<MODE, FM>(a, tp, wm, wn, acc, dst, gate);
        zero_acc();
      }
      if (s == 0) {
        // this tile's rows (GEMM2: the pair index now, its gate after the
        // next barrier, which awaits the lookup with the k-step's loads)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) dst[fm] = pipe_row_dest<MODE>(a, ti, (wm * FM + fm) * 32 + (lane & 31));
        if (!kDirect) zero_acc();
      }
      pipe_mma<E, MODE, FM, NINST, false>(lds0, wm, wn, lane, acc, active, db1, ld.off, wr1, nrec1);
      if (s == 0 && nsteps > 2 && tid == 0) reply = claim_issue(ctr + x);
      // odd k-step: slot 1 holds k-step s + 1; slot 0 gets k-step s + 2, or
      // the next tile's first k-step after the last one
      if (s + 2 >= nsteps) {
        Ln = uni(s_claim);
        has_next = Ln >= 0;
      }
      if (s + 2 >= nsteps && has_next) {
        tn = uni(tile_of<kPipeBM, BNO, MODE, true>(a, s_tab, V, Ln, s_off));
        pipe_prepare<E, MODE>(a, tn, wave, lane, is_a, ld);  // this tile's loads are all issued
      }
      pipe_sync();
      if (s == 0) {
        if (nsteps > 2 && tid == 0) claim = claim_resolve(reply);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          pipe_row_gate<MODE>(a, ti, (wm * FM + fm) * 32 + (lane & 31), dst[fm], gate[fm]);
      }
      // after the last k-step: the next tile's first k-step, or (last tile)
      // the first k-step again into the slot nobody reads any more
      const uint8_t* db2 = s + 2 < nsteps ? pipe_dma_base<E, MODE>(a, ti, ld, s + 2, is_a)
                                          : pipe_dma_base<E, MODE>(a, tn, ld, 0, is_a);
      pipe_mma<E, MODE, FM>(lds1, wm, wn, lane, acc, active, uni(db2), ld.off,
                            lds0 + wave * NINST * 1024);
    }

    if constexpr (kDirect) {
      if (has_next) {
        pending = true;  // written after the next tile's first barrier
        tp = ti;
      } else {
        pipe_store_direct<MODE, FM>(a, ti, wm, wn, acc, dst, gate);
      }
    } else {
      lds_sync();
      store_tile<E, MODE, FM, 4>(a, ti, wm, wn, acc);
      __syncthreads();
    }
    if (!has_next) {
      MOE_WAIT_VMCNT(0);  // the spare reload into slot 0 lands before the block ends
      break;
    }
    L = Ln;
    ti = tn;
  }
}

// ---------------------------------------------------------------- weight-streaming kernel
// Decode-sized batches (a few tokens per expert) are bound by streaming the
// weights of every selected expert once, so this kernel keeps as many bytes
// in flight per CU as LDS allows.  Tiles are 32 rows (slots of one expert)
// x 128 B rows (GEMM1: gate and up rows of 64 columns, interleaved in runs
// of 32; GEMM2: 128 output columns), one 128-byte k-step of every row per
// ring slot, kStrS slots.  The block is persistent and walks its tiles as
// one sequence of k-steps.  Wavefronts 2..5 only load: they keep the next
// kStrS - 1 k-steps in flight with direct-to-LDS buffer loads, wait for the
// oldest with an exact vmcnt (they issue nothing else), and release it with a
// barrier (four loading wavefronts issue ~1% faster than two: the loads are
// accepted at the rate the memory system takes them, not issued late).
// Wavefronts 0 and 1 only compute: after each barrier they multiply the
// released slot (each owns 64 of the 128 B rows) and, at the end of a tile,
// write its rows.
constexpr int kStrBM = 32, kStrBR = 128, kStrS = 6, kStrLW = 4;
constexpr int kStrRows = kStrBM + kStrBR;
constexpr int kStrSlot = kStrRows * 128;
constexpr int kStrNI = kStrRows / 8 / kStrLW;  // loads per loading wavefront per k-step
constexpr int kStrThreads = 64 * (2 + kStrLW);
static_assert(kStrRows % (8 * kStrLW) == 0 && kStrBM % 8 == 0, "whole 8-row loads per wavefront");
static_assert((kStrS - 2) * kStrNI < 64, "vmcnt range");

template <int MODE>
__host__ __device__ __forceinline__ int str_nt(const ExpertArgs& a) {
  return MODE == 1 ? a.I / (kStrBR / 2) : a.d / kStrBR;
}

// Row r of a stream tile at contraction index 0: A rows 0..31, B rows after.
template <int MODE>
__device__ __forceinline__ const uint16_t* str_row_ptr(const ExpertArgs& a, const Tile& ti, int r) {
  if (r < kStrBM) return (const uint16_t*)tile_row_ptr<ElemBF16, MODE, kStrBM, kStrBR>(a, ti, r);
  const int rb = r - kStrBM;
  const size_t Id = (size_t)a.I * a.d;
  const uint16_t* W = ti.routed ? (const uint16_t*)a.W_routed + (size_t)ti.v * 3 * Id
                                : (const uint16_t*)a.W_shared +
                                      (size_t)(MODE == 1 ? ti.v - a.N : 0) * 3 * Id;
  if (MODE == 1) {
    const int q = rb >> 5, col = ti.n0 + (q >> 1) * 32 + (rb & 31);  // runs: gate, up, gate, up
    return W + ((q & 1) ? Id : 0) + (size_t)col * a.d;
  }
  return W + 2 * Id + (size_t)(ti.n0 + rb) * a.I;
}

// Steps of tile L and its geometry.
template <int MODE>
__device__ __forceinline__ int str_steps(const ExpertArgs& a, const Tile& ti) {
  return (MODE == 1 ? a.d : (ti.routed ? a.I : a.K_s * a.I)) / 64;
}

// Tiles are dealt to the blocks by stride (block b takes b, b + G, ...), so
// the first total % G blocks take one more tile than the rest.  GEMM2's shared
// tiles (the last of the table) contract over K_s * I and cost K_s routed
// tiles: they are moved to the positions just past those blocks, so a block
// that takes one does not also take the extra tile.
__device__ __forceinline__ int str_perm(int p, int total, int G, int E) {
  const int r = total % G;
  if (E == 0 || r + E > G || p < r) return p;
  if (p < r + E) return total - E + (p - r);
  return p - E;
}

template <int MODE>
__global__ __launch_bounds__(kStrThreads, 1) void expert_gemm_stream_kernel(ExpertArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kStrS * kStrSlot];
  __shared__ int s_tab[kMaxV + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int V = load_tile_table<MODE>(a, s_tab);
  const int nt = str_nt<MODE>(a);
  const int total = s_tab[V] * nt;
  const int G = gridDim.x;
  if ((int)blockIdx.x >= total) return;  // whole block: no barrier is left behind
  const int E = (MODE == 2 && a.K_s > 1) ? (s_tab[V] - s_tab[V - 1]) * nt : 0;
  // the block's k-steps, over its tiles blockIdx.x, + G, ...
  int nsteps_all = 0;
  for (int L = blockIdx.x; L < total; L += G)
    nsteps_all += str_steps<MODE>(a, tile_of<kStrBM, (MODE == 1 ? kStrBR / 2 : kStrBR), MODE>(a, s_tab, V, str_perm(L, total, G, E)));

  if (wave >= 2) {
    // ---- loading wavefronts: rows (wave - 2) * 8 kStrNI .. + 8 kStrNI - 1 of each slot
    const int w2 = wave - 2;
    int L = blockIdx.x, s = 0;
    Tile ti = uni(tile_of<kStrBM, (MODE == 1 ? kStrBR / 2 : kStrBR), MODE>(a, s_tab, V, str_perm(L, total, G, E)));
    int ns = str_steps<MODE>(a, ti);
    uint32_t off[kStrNI];
    const uint8_t* a_base = nullptr;
    const uint8_t* b_base = nullptr;
    auto prepare = [&]() {
      b_base = uni((const uint8_t*)str_row_ptr<MODE>(a, ti, kStrBM));
      a_base = uni(MODE == 1 ? (const uint8_t*)a.u
                             : (const uint8_t*)(ti.routed ? a.H_routed : a.H_shared));
#pragma unroll
      for (int i = 0; i < kStrNI; ++i) {
        const int r = (w2 * kStrNI + i) * 8 + (lane >> 3);
        const uint8_t* rp = (const uint8_t*)str_row_ptr<MODE>(a, ti, r);
        const int chunk = (lane & 7) ^ ((r >> 1) & 7);
        off[i] = (uint32_t)(rp - (r < kStrBM ? a_base : b_base)) + chunk * 16;
      }
    };
    prepare();
    // issue the loads of the cursor's k-step into slot `slot`, then advance
    // the cursor (past the block's last k-step it stays there: the spare
    // loads reread valid memory into slots nobody reads any more)
    auto issue = [&](int slot) {
      const size_t k0 = (size_t)s * 64;
      const uint8_t* ab = uni(a_base + k0 * 2);
      const uint8_t* bb = uni(b_base + b_offset<MODE>(a, ti, k0) * 2);
      uint8_t* wr = ring + slot * kStrSlot + w2 * kStrNI * 1024;
#pragma unroll
      for (int i = 0; i < kStrNI; ++i) {
        const bool is_a = (w2 * kStrNI + i) * 8 < kStrBM;  // whole instruction: 8 rows
        dma16(is_a ? ab : bb, off[i], wr + i * 1024);
      }
      if (s + 1 < ns) {
        ++s;
      } else if (L + G < total) {
        L += G;
        s = 0;
        ti = uni(tile_of<kStrBM, (MODE == 1 ? kStrBR / 2 : kStrBR), MODE>(a, s_tab, V, str_perm(L, total, G, E)));
        ns = str_steps<MODE>(a, ti);
        prepare();
      }
    };
#pragma unroll
    for (int j = 0; j < kStrS - 1; ++j) issue(j);
    int slot = kStrS - 1;
    for (int g = 0; g < nsteps_all; ++g) {
      MOE_WAIT_VMCNT((kStrS - 2) * kStrNI);  // k-step g has landed
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue(slot);  // k-step g + kStrS - 1 into the slot read at k-step g - 1
      slot = slot + 1 == kStrS ? 0 : slot + 1;
    }
    MOE_WAIT_VMCNT(0);
    return;
  }

  // ---- computing wavefronts: B rows wave * 64 .. + 63 (two 32-row fragments)
  const int lc = lane & 31, lh = lane >> 5;
  int L = blockIdx.x, s = 0, slot = 0;
  Tile ti = uni(tile_of<kStrBM, (MODE == 1 ? kStrBR / 2 : kStrBR), MODE>(a, s_tab, V, str_perm(L, total, G, E)));
  int ns = str_steps<MODE>(a, ti);
  f32x16 acc[2];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[f][r] = 0.f;
  for (int g = 0; g < nsteps_all; ++g) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const uint8_t* rd = ring + slot * kStrSlot;
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const int ch = kg * 2 + lh;
      const u32x4 af = *(const u32x4*)(rd + lds_chunk_offset(lc, ch));
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const u32x4 bf = *(const u32x4*)(rd + lds_chunk_offset(kStrBM + wave * 64 + f * 32 + lc, ch));
        acc[f] = mfma32(ElemBF16{}, bf, af, acc[f]);  // lane = token row
      }
    }
    MOE_WAIT_LGKMCNT0();  // this slot's reads are done before the next barrier
    slot = slot + 1 == kStrS ? 0 : slot + 1;
    if (++s < ns) continue;
    // ---- end of tile: lane holds row m0 + lc, columns 8j + 4 lh + 0..3 of each fragment
    const int p = ti.m0 + lc;
    if (p < ti.rows) {
      if (MODE == 1) {
        uint16_t* dst = ti.routed ? (uint16_t*)a.H_routed + (size_t)(ti.row_base + p) * a.I
                                  : (uint16_t*)a.H_shared + (size_t)p * a.K_s * a.I +
                                        (size_t)(ti.v - a.N) * a.I;
        dst += ti.n0 + wave * 32 + 4 * lh;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint2 w;
          w.x = pack_bf16x2(silu_mul(acc[0][4 * j], acc[1][4 * j]),
                            silu_mul(acc[0][4 * j + 1], acc[1][4 * j + 1]));
          w.y = pack_bf16x2(silu_mul(acc[0][4 * j + 2], acc[1][4 * j + 2]),
                            silu_mul(acc[0][4 * j + 3], acc[1][4 * j + 3]));
          *(uint2*)(dst + 8 * j) = w;
        }
      } else {
        float gt = 1.f;
        uint16_t* dst;
        if (ti.routed) {
          const int TK = a.T * a.K;
          int pair = a.sorted_pair[ti.row_base + p];
          pair = ((unsigned)pair < (unsigned)TK) ? pair : 0;
          gt = a.gate[pair];
          dst = (uint16_t*)a.Y + (size_t)pair * a.d;
        } else {
          dst = (uint16_t*)a.Y_shared + (size_t)p * a.d;
        }
        dst += ti.n0 + wave * 64 + 4 * lh;
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint2 w;
            w.x = pack_bf16x2(acc[f][4 * j] * gt, acc[f][4 * j + 1] * gt);
            w.y = pack_bf16x2(acc[f][4 * j + 2] * gt, acc[f][4 * j + 3] * gt);
            *(uint2*)(dst + f * 32 + 8 * j) = w;
          }
      }
    }
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[f][r] = 0.f;
    s = 0;
    L += G;
    if (L < total) {
      ti = uni(tile_of<kStrBM, (MODE == 1 ? kStrBR / 2 : kStrBR), MODE>(a, s_tab, V, str_perm(L, total, G, E)));
      ns = str_steps<MODE>(a, ti);
    }
  }
}

// Kernel choice.  kind 0: register-staged kernel with wavefronts WM x WN and
// 32x32 fragments FM x FN per wavefront; kind 1: the pipelined LDS-DMA
// kernel; kinds 2 and 3: the weight-streaming kernels (bf16, decode-sized
// batches; 3: 512-byte runs with the token rows held in LDS, where they fit).
struct Shape {
  int kind, WM, WN, FM, FN;
  int bm() const {
    return kind == 1 ? kPipeBM : kind == 2 ? kStrBM : kind == 3 ? stream_long_rows() : WM * FM * 32;
  }
};

// Few tokens per expert (decode-sized batches): short M tiles, wide N tiles,
// so every CU streams a large weight slab.
bool small_m(const ExpertArgs& a) {
  return (long long)a.T * a.K < 64LL * (a.sel_N > 0 ? a.sel_N : a.N);
}

// The pipelined kernel takes any shape the ABI admits (d and I multiples of
// 64: whole 128-byte k-steps; an odd k-step count gets one zero-filled
// k-step; partial last n-tiles are masked).
bool pipe_ok1(const ExpertArgs& a, int es) { return (a.d * es) % 128 == 0 && a.I % 64 == 0; }
bool pipe_ok2(const ExpertArgs& a, int es) { return (a.I * es) % 128 == 0 && a.d % 64 == 0; }

// MOE_STREAM=short keeps the 128-byte-run streaming kernel (read on every call).
bool stream_long(int mode, const ExpertArgs& a) {
  const char* e = getenv("MOE_STREAM");
  return !(e != nullptr && !strcmp(e, "short")) && stream_long_ok(mode, a);
}

Shape shape1(const ExpertArgs& a, int es) {
  if (small_m(a) && es == 2) return Shape{stream_long(1, a) ? 3 : 2, 0, 0, 0, 0};
  if (small_m(a)) return a.I % 128 == 0 ? Shape{0, 1, 4, 1, 2} : Shape{0, 2, 2, 1, 2};
  if (pipe_ok1(a, es)) return Shape{1, 4, 2, 2, 4};
  return Shape{0, 2, 2, 2, 2};
}
Shape shape2(const ExpertArgs& a, int es) {
  if (small_m(a) && es == 2 && stream_long(2, a)) return Shape{3, 0, 0, 0, 0};
  if (small_m(a) && es == 2 && a.d % kStrBR == 0) return Shape{2, 0, 0, 0, 0};
  if (small_m(a)) return a.d % 256 == 0 ? Shape{0, 1, 4, 1, 2} : Shape{0, 2, 2, 1, 1};
  if (pipe_ok2(a, es)) return Shape{1, 4, 2, 2, 4};
  return a.d % 128 == 0 ? Shape{0, 2, 2, 2, 2} : Shape{0, 2, 2, 2, 1};
}

long long grid_tiles(const ExpertArgs& a, int bm, int nt, int mode) {
  const long long routed = ((long long)a.T * a.K + (long long)a.N * (bm - 1)) / bm;
  const long long mtT = (a.T + bm - 1) / bm;
  const long long shared = mode == 1 ? a.K_s * mtT : (a.K_s > 0 ? mtT : 0);
  return (routed + shared) * nt;
}

template <class E, int WM, int WN, int FM, int FN, int MODE>
hipError_t launch_reg(const ExpertArgs& a, hipStream_t st) {
  constexpr int BM = WM * FM * 32;
  constexpr int BNO = MODE == 1 ? WN * FN * 16 : WN * FN * 32;
  const long long g = grid_tiles(a, BM, (MODE == 1 ? a.I : a.d) / BNO, MODE);
  if (g <= 0) return hipSuccess;
  if (g > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  return launch_kernel(expert_gemm_kernel<E, WM, WN, FM, FN, MODE>, dim3((unsigned)g), dim3(256),
                       st, a);
}

// Compute units of the current device (cached per device).
int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

template <class E, int MODE, int W>
hipError_t launch_pipe(const ExpertArgs& a, hipStream_t st) {
  constexpr int BNO = MODE == 1 ? kPipeBNB / 2 : kPipeBNB;
  long long g = grid_tiles(a, kPipeBM, ((MODE == 1 ? a.I : a.d) + BNO - 1) / BNO, MODE);
  if (g <= 0) return hipSuccess;
  g = std::min<long long>(g, (long long)cu_count());  // persistent: one block per CU
  return launch_kernel(expert_gemm_pipe_kernel<E, MODE, W>, dim3((unsigned)g),
                       dim3(PipeCfg<W>::kThreads), st, a);
}

template <int MODE>
hipError_t launch_stream(const ExpertArgs& a, hipStream_t st) {
  long long g = grid_tiles(a, kStrBM, str_nt<MODE>(a), MODE);
  if (g <= 0) return hipSuccess;
  g = std::min<long long>(g, (long long)cu_count());  // persistent: one block per CU
  return launch_kernel(expert_gemm_stream_kernel<MODE>, dim3((unsigned)g), dim3(kStrThreads), st,
                       a);
}

template <class E, int MODE>
hipError_t launch_mode(const ExpertArgs& a, hipStream_t st) {
  const int es = (int)sizeof(typename E::T);
  const Shape s = MODE == 1 ? shape1(a, es) : shape2(a, es);
  if constexpr (std::is_same<E, ElemBF16>::value) {
    if (s.kind == 2) return launch_stream<MODE>(a, st);
    if (s.kind == 3) return launch_stream_long(MODE, a, cu_count(), st);
  }
  if (s.kind == 1) return launch_pipe<E, MODE, 8>(a, st);
  if (MODE == 1) {
    if (s.WM == 1) return launch_reg<E, 1, 4, 1, 2, 1>(a, st);
    if (s.FM == 1) return launch_reg<E, 2, 2, 1, 2, 1>(a, st);
    return launch_reg<E, 2, 2, 2, 2, 1>(a, st);
  }
  if (s.WM == 1) return launch_reg<E, 1, 4, 1, 2, 2>(a, st);
  if (s.FM == 1) return launch_reg<E, 2, 2, 1, 1, 2>(a, st);
  if (s.FN == 2) return launch_reg<E, 2, 2, 2, 2, 2>(a, st);
  return launch_reg<E, 2, 2, 2, 1, 2>(a, st);
}

}  // namespace

bool gemm1_derives_dispatch(int dtype, const ExpertArgs& a) {
  return dtype == 1 && a.T <= kSmallDispatchT && (long long)a.T * a.K <= kFusedDispatchPairs &&
         shape1(a, 2).kind == 3;
}

int expert_tile_table_ints(int N, int K_s) { return (N + K_s + 1) + (N + 2) + 16; }

TileTableOut expert_tile_tables(int dtype, const ExpertArgs& a) {
  const int es = dtype == 1 ? 2 : 4;
  return TileTableOut{a.tiles1, a.tiles2, a.counters, a.K_s, a.T, shape1(a, es).bm(),
                      shape2(a, es).bm()};
}

hipError_t launch_tile_table(int dtype, const ExpertArgs& a, hipStream_t stream) {
  return launch_kernel(tile_table_kernel, dim3(1), dim3(64), stream, a.offsets, a.N, a.T * a.K,
                       expert_tile_tables(dtype, a));
}

hipError_t launch_gemm1(int dtype, const ExpertArgs& a, hipStream_t stream) {
  return dtype == 1 ? launch_mode<ElemBF16, 1>(a, stream) : launch_mode<ElemF32, 1>(a, stream);
}

hipError_t launch_gemm2(int dtype, const ExpertArgs& a, hipStream_t stream) {
  return dtype == 1 ? launch_mode<ElemBF16, 2>(a, stream) : launch_mode<ElemF32, 2>(a, stream);
}

}  // namespace moe
