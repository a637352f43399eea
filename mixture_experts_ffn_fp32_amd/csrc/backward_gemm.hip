// Pipelined bfloat16 backward of the DeepSeekMoE layer (DeepSeekMoE paper
// summary, papercache.org, sec. 3.2 layer equation, differentiated by the
// chain rule with each token's top-K set held fixed).
//
// Every expert-slot product of the backward runs as a grouped GEMM on one
// LDS-DMA MFMA pipeline: tiles of 256 x 256, eight wavefronts of 64 x 128,
// k-steps landing by direct-to-LDS loads in a two-slot ring while the other
// slot is multiplied.  An operand is either contiguous along the contraction
// ("k-major": 256 rows of 128 bytes per k-step) or read in its stored layout
// with rows along the contraction (64 rows of 256 columns per k-step; MFMA
// fragments through transposing LDS reads).  Only the token rows that a
// weight-gradient product contracts over are transposed beforehand:
//
//   XT, dhT = u^T, dh^T over padded slot columns (gathered by dispatch, each
//   expert's slots rounded up to 64, zeros in the padding)
//
// Products, per virtual expert v (routed: its slots; shared: every token):
//   DP   dP[slot][i]   = dh_tok . W_down[:, i]             (K = d)
//   AC   [a c][slot][i] = u_tok . [W_gate; W_up][i]         (K = d), fused epilogue:
//        p = SiLU(a) c, da = g dP c SiLU'(a), dc = g dP SiLU(a); writes
//        [da dc] and g p slot-major, and the partial gate gradients
//        sum_i dP p per 128 columns
//   DX   dx[slot][n]   = [da dc][slot] . [W_gate; W_up][:, n] (K = 2I), bfloat16 rows
//   DWD  dW_down[n][i] = dhT[n] . (g p)[:, i]              (K = the expert's slots)
//   DWGC dW_gu[j][n]   = [da dc][:, j] . XT[n]             (K = the same)
// Slot-major operands of the weight gradients stop at the expert's last slot
// by a bounded buffer range (the loads past it return zeros); XT and dhT
// hold zeros there.
#include <algorithm>

#include "lds_dma.h"
#include "moe_internal.h"

namespace moe {
namespace {

enum : int { BT_DP = 1, BT_AC = 2, BT_DX = 3, BT_DWD = 4, BT_DWGC = 5, BT_NG = 5 };
constexpr int kBtBM = 256, kBtBNB = 256, kBtRB = 128;  // A rows, B rows, k bytes per step
constexpr int kBtSlot = (kBtBM + kBtBNB) * kBtRB;      // 64 KB
constexpr int kBtThreads = 512, kBtNI = 8;             // DMA instructions per wavefront per step
constexpr int kBtMaxV = 256 + 16;

__host__ __device__ constexpr int bt_bn(int G) { return G == BT_AC ? kBtBNB / 2 : kBtBNB; }

struct BtGroup {  // (all int: a bool member's padding would be copied through memory)
  int M, Nc, steps, rows, base;
  int routed;  // 0 or 1
};

// Geometry of virtual expert v in product G.
template <int G>
__device__ __forceinline__ BtGroup bt_group(const BwdArgs& a, int v) {
  BtGroup g;
  const int TK = a.T * a.K;
  g.routed = v < a.N ? 1 : 0;
  if (g.routed) {
    g.base = min(max(a.offsets[v], 0), TK);
    g.rows = min(max(a.offsets[v + 1], g.base), TK) - g.base;
  } else {
    g.base = 0;
    g.rows = a.T;
  }
  const int kpad = (g.rows + 63) >> 6;
  switch (G) {
    case BT_DP: g.M = g.rows; g.Nc = a.I; g.steps = a.d >> 6; break;
    case BT_AC: g.M = g.rows; g.Nc = a.I; g.steps = a.d >> 6; break;
    case BT_DX: g.M = g.rows; g.Nc = a.d; g.steps = a.I >> 5; break;
    case BT_DWD: g.M = a.d; g.Nc = a.I; g.steps = kpad; break;
    default: g.M = 2 * a.I; g.Nc = a.d; g.steps = kpad; break;
  }
  return g;
}

template <int G>
__device__ __forceinline__ int bt_tiles(const BwdArgs& a, int v) {
  const BtGroup g = bt_group<G>(a, v);
  return g.M > 0 ? ((g.M + kBtBM - 1) / kBtBM) * ((g.Nc + bt_bn(G) - 1) / bt_bn(G)) : 0;
}

// First padded column of virtual expert v in XT / dhT (shared experts share one range).
__device__ __forceinline__ long long bt_colx(const BwdArgs& a, int v) {
  return v < a.N ? a.pcol[v] : a.pcol[a.N];
}

// Group order of product G's tile table.  The weight-gradient products
// contract over an expert's slots, so a shared expert's tiles (all T tokens)
// are many times longer than a routed expert's: they go first, so the long
// tiles start at once and the short ones fill in behind them.
template <int G>
__device__ __forceinline__ int bt_order(const BwdArgs& a, int k) {
  if (G == BT_DWD || G == BT_DWGC) return k < a.K_s ? a.N + k : k - a.K_s;
  return k;
}

template <int G>
__device__ __forceinline__ void bt_table_one(const BwdArgs& a, int lane, int V,
                                             int32_t* __restrict__ out) {
  int carry = 0;
  for (int b = 0; b < V; b += 64) {
    const int k = b + lane;
    const int t = k < V ? bt_tiles<G>(a, bt_order<G>(a, k)) : 0;
    int inc = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    if (k < V) out[k] = carry + inc - t;
    carry += __shfl(inc, 63);
  }
  if (lane == 0) out[V] = carry;
}

// Padded column offsets of the routed experts and the tile prefix of every
// product (one wavefront).
__global__ __launch_bounds__(64) void bt_table_kernel(BwdArgs a, int32_t* __restrict__ tabs) {
  const int lane = threadIdx.x, V = a.N + a.K_s;
  int carry = 0;
  for (int b = 0; b < a.N; b += 64) {
    const int v = b + lane;
    int c = 0;
    if (v < a.N) c = (bt_group<BT_DP>(a, v).rows + 63) & ~63;
    int inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    if (v < a.N) a.pcol[v] = carry + inc - c;
    carry += __shfl(inc, 63);
  }
  if (lane == 0) a.pcol[a.N] = carry;
  bt_table_one<BT_DP>(a, lane, V, tabs + 0 * (V + 1));
  bt_table_one<BT_AC>(a, lane, V, tabs + 1 * (V + 1));
  bt_table_one<BT_DX>(a, lane, V, tabs + 2 * (V + 1));
  bt_table_one<BT_DWD>(a, lane, V, tabs + 3 * (V + 1));
  bt_table_one<BT_DWGC>(a, lane, V, tabs + 4 * (V + 1));
  if (lane < BT_NG * 8) tabs[BT_NG * (V + 1) + lane] = 0;  // claim counters
}

// ---------------------------------------------------------------- transposes
// u^T (z = 0) and dh^T (z = 1) over the padded slot columns, 64 x 64 tiles
// through LDS: out[n][r] = the token row of padded column r at column n, zero
// in the padding.
__global__ __launch_bounds__(256) void bt_gather_t_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64, z = blockIdx.z;
  // the virtual range this 64-column block lies in
  int rv_lo, rv_rows, rv_slot0 = 0;
  bool rv_routed = false;
  const int R = a.pcol[a.N];
  if (r0 >= R + a.Tp) return;
  if (r0 >= R) {
    rv_lo = R;
    rv_rows = a.T;
  } else {
    int lo = 0, hi = a.N - 1;  // last routed expert whose range starts at or before r0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.pcol[mid] <= r0) lo = mid; else hi = mid - 1;
    }
    const int TK = a.T * a.K;
    rv_routed = true;
    rv_lo = a.pcol[lo];
    rv_slot0 = min(max(a.offsets[lo], 0), TK);
    rv_rows = min(max(a.offsets[lo + 1], rv_slot0), TK) - rv_slot0;
  }
  uint16_t* dst = (uint16_t*)(z == 0 ? a.XT : a.dhT);
  const size_t dst_ld = (size_t)a.ldx;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = tid + h * 256, r = q >> 3, ch = q & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    const int local = r0 + r - rv_lo;
    if (local < rv_rows) {
      int tok = local;
      if (rv_routed) {
        const int TK = a.T * a.K;
        const int p = a.sorted_pair[rv_slot0 + local];
        tok = ((unsigned)p < (unsigned)TK) ? p / a.K : 0;
      }
      const uint16_t* row = (const uint16_t*)(z == 0 ? a.u : a.dh) + (size_t)tok * a.d;
      v = *(const u32x4*)(row + c0 + ch * 8);
    }
    *(u32x4*)&tile[r][ch * 8] = v;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = tid + h * 256, c = q >> 3, rc = q & 7;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (uint32_t)tile[rc * 8 + 2 * k][c] | ((uint32_t)tile[rc * 8 + 2 * k + 1][c] << 16);
    *(u32x4*)(dst + (size_t)(c0 + c) * dst_ld + r0 + rc * 8) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// ---------------------------------------------------------------- operand rows
// Start (k = 0) of row m of A and row r of B's tile for group v; rows are
// clamped to the group's extent (the repeats are never stored).
template <int G>
__device__ __forceinline__ const uint8_t* bt_a_row(const BwdArgs& a, int v, const BtGroup& g,
                                                   int m) {
  const int j = v - a.N;
  switch (G) {
    case BT_DP:
    case BT_AC: {
      int tok = m;
      if (g.routed) {
        const int TK = a.T * a.K;
        const int p = a.sorted_pair[g.base + m];
        tok = ((unsigned)p < (unsigned)TK) ? p / a.K : 0;
      }
      return (const uint8_t*)((const uint16_t*)(G == BT_DP ? a.dh : a.u) + (size_t)tok * a.d);
    }
    case BT_DX:
      return (const uint8_t*)(g.routed
                                  ? (const uint16_t*)a.dAC + (size_t)(g.base + m) * 2 * a.I
                                  : (const uint16_t*)a.dACs + ((size_t)m * a.K_s + j) * 2 * a.I);
    default:  // BT_DWD (DWGC reads dAC in its stored layout)
      return (const uint8_t*)((const uint16_t*)a.dhT + (size_t)m * a.ldx + bt_colx(a, v));
  }
}

template <int G>
__device__ __forceinline__ const uint8_t* bt_b_row(const BwdArgs& a, int v, int n0, int r) {
  const size_t Id = (size_t)a.I * a.d;
  switch (G) {
    case BT_AC: {
      const uint16_t* W = v < a.N ? (const uint16_t*)a.W_routed + (size_t)v * 3 * Id
                                  : (const uint16_t*)a.W_shared + (size_t)(v - a.N) * 3 * Id;
      // the first half of the B tile: W_gate rows of the tile's columns; the
      // second half: W_up rows of the same columns
      const int half = kBtBNB / 2;
      const int i = r < half ? min(n0 + r, a.I - 1) : a.I + min(n0 + r - half, a.I - 1);
      return (const uint8_t*)(W + (size_t)i * a.d);
    }
    default:  // BT_DWGC (DWD reads g p in its stored layout)
      return (const uint8_t*)((const uint16_t*)a.XT + (size_t)min(n0 + r, a.d - 1) * a.ldx +
                              bt_colx(a, v));
  }
}

// B tile row of wavefront column wn's fragment fn: AC pairs gate fragment fn
// with the up fragment fn + 2 of the same columns.
template <int G>
__device__ __forceinline__ int bt_bcol(int wn, int fn) {
  if (G == BT_AC) return fn < 2 ? (wn * 2 + fn) * 32 : kBtBNB / 2 + (wn * 2 + fn - 2) * 32;
  return (wn * 4 + fn) * 32;
}

// Operands read in their stored layout (rows along the contraction): the
// tile of a k-step is 64 rows of 256 columns (512 bytes, 16-byte chunk c of
// row k at c ^ 2(k & 7)) in the operand's half of the ring slot.
//   A: DWGC's [da dc] (slot-major)
//   B: DP's W_down, DX's [W_gate; W_up], DWD's g p (slot-major)
__host__ __device__ constexpr bool bt_atr(int G) { return G == BT_DWGC; }
__host__ __device__ constexpr bool bt_btr(int G) {
  return G == BT_DP || G == BT_DX || G == BT_DWD;
}

__device__ __forceinline__ int bt_tr_off(int region, int k, int n) {
  return region + k * 512 + ((((n >> 3) ^ ((k & 7) << 1))) << 4) + (n & 7) * 2;
}

// Row 0 (contraction index 0) of a stored-layout operand of tile t, its row
// pitch and width (elements), and the number of contraction rows that exist
// (-1: all; a slot-major operand ends at the expert's last slot).
template <int G>
__device__ __forceinline__ const uint16_t* bt_tr_src(const BwdArgs& a, int v, const BtGroup& g,
                                                     int& pitch, int& width, int& rows) {
  const size_t Id = (size_t)a.I * a.d;
  const int j = v - a.N;
  rows = -1;
  if (G == BT_DWD) {  // g p [slot][I]
    rows = g.rows;
    width = a.I;
    pitch = g.routed ? a.I : a.K_s * a.I;
    return g.routed ? (const uint16_t*)a.P + (size_t)g.base * a.I : (const uint16_t*)a.Ps + (size_t)j * a.I;
  }
  if (G == BT_DWGC) {  // [da dc] [slot][2I]
    rows = g.rows;
    width = 2 * a.I;
    pitch = g.routed ? 2 * a.I : a.K_s * 2 * a.I;
    return g.routed ? (const uint16_t*)a.dAC + (size_t)g.base * 2 * a.I
                    : (const uint16_t*)a.dACs + (size_t)j * 2 * a.I;
  }
  const uint16_t* W = v < a.N ? (const uint16_t*)a.W_routed + (size_t)v * 3 * Id
                              : (const uint16_t*)a.W_shared + (size_t)j * 3 * Id;
  if (G == BT_DP) {  // W_down [d][I]: row n, columns i
    pitch = width = a.I;
    return W + 2 * Id;
  }
  pitch = width = a.d;  // [W_gate; W_up] [2I][d]: row j, columns n
  return W;
}

// Four consecutive contraction indices of one column through a transposing
// LDS read: within each 16-lane group, lane j names row (k0 + j / 4) at column
// (n0 + 4 (j % 4)), and lane i receives column n0 + i of rows k0 .. k0 + 3.
typedef short bt_v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 bt_read_tr(const uint8_t* p) {
  const bt_v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) bt_v4s*)(__attribute__((address_space(3))) const uint8_t*)p);
  return __builtin_bit_cast(uint2, v);
}

__host__ __device__ constexpr bool bt_swap(int G) { return G == BT_AC || G == BT_DX; }

__device__ __forceinline__ f32x16 bt_mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// MFMA fragments of k-group kg: 32 rows x 16 contraction indices, 8 per lane
// (lane l: row l % 32, indices 8(l / 32) ..).  Stored-layout operands: within
// each 16-lane group lane l names row kg*16 + 8(l / 32) + (l % 16) / 4 (+ 4 for
// the upper four) at column 16((l / 16) % 2) + 4(l % 4) of the fragment.
__device__ __forceinline__ u32x4 bt_frag_tr(const uint8_t* rd, int region, int kg, int col0,
                                            int lane) {
  const int k = kg * 16 + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int n = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint2 lo = bt_read_tr(rd + bt_tr_off(region, k, n));
  const uint2 hi = bt_read_tr(rd + bt_tr_off(region, k + 4, n));
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

template <int G>
__device__ __forceinline__ void bt_frags(const uint8_t* __restrict__ rd, int kg, int wm, int wn,
                                         int lane, u32x4 (&af)[2], u32x4 (&bfr)[4]) {
  const int ch = kg * 2 + (lane >> 5);
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
    af[fm] = bt_atr(G) ? bt_frag_tr(rd, 0, kg, wm * 64 + fm * 32, lane)
                       : *(const u32x4*)(rd + lds_chunk_offset(wm * 64 + fm * 32 + (lane & 31), ch));
#pragma unroll
  for (int fn = 0; fn < 4; ++fn)
    bfr[fn] = bt_btr(G) ? bt_frag_tr(rd, kBtBM * kBtRB, kg, bt_bcol<G>(wn, fn), lane)
                        : *(const u32x4*)(rd + lds_chunk_offset(kBtBM + bt_bcol<G>(wn, fn) + (lane & 31), ch));
}

// One k-step out of ring slot `rd`.  The next k-step's direct-to-LDS loads
// (base `db`, lane offsets `off`, into `wr`; `nrec` = 0 after the last k-step
// makes them return zeros without touching memory) are interleaved with the
// MFMAs of the first two k-groups, and the next k-group's fragments are read
// after each MFMA.  (One instance in the loop: a second, load-free copy for
// the last k-step doubles the live ranges and spills.)
template <int G, bool ISSUE = true>
__device__ __forceinline__ void bt_mma(const uint8_t* __restrict__ rd, int wm, int wn, int lane,
                                       f32x16 (&acc)[2][4], const uint8_t* db,
                                       const uint32_t (&off)[kBtNI], uint8_t* __restrict__ wr,
                                       int nrec) {
  constexpr int KG = kBtRB / 32, PARTS = 2, PER = kBtNI / PARTS;
  u32x4 af[2][2], bfr[2][4];
  bt_frags<G>(rd, 0, wm, wn, lane, af[0], bfr[0]);
#pragma unroll
  for (int kg = 0; kg < KG; ++kg) {
    if (ISSUE && kg < PARTS) {
#pragma unroll
      for (int i = kg * PER; i < (kg + 1) * PER; ++i) dma16(db, off[i], wr + i * 1024, nrec);
    }
    if (kg + 1 < KG) bt_frags<G>(rd, kg + 1, wm, wn, lane, af[(kg + 1) & 1], bfr[(kg + 1) & 1]);
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int fn = 0; fn < 4; ++fn)
        // AC, DX: weights as the 32-row operand, so a lane holds four
        // consecutive output columns of one slot row (8-byte bf16 stores)
        acc[fm][fn] = bt_swap(G) ? bt_mfma(bfr[kg & 1][fn], af[kg & 1][fm], acc[fm][fn])
                                 : bt_mfma(af[kg & 1][fm], bfr[kg & 1][fn], acc[fm][fn]);
  }
  constexpr int NR = (bt_atr(G) ? 4 : 2) + (bt_btr(G) ? 8 : 4);  // LDS reads per k-group
  __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
  for (int kg = 0; kg < KG; ++kg) {
    const int nr = kg + 1 < KG ? NR : 0, nd = (ISSUE && kg < PARTS) ? PER : 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m < nr) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (NR > 8 && m < NR - 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if (m < nd) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  }
}

__device__ __forceinline__ float bt_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

struct BtTile {
  BtGroup g;
  int v, m0, n0, steps;
};

// Tile L of product G: its group (through the table's order), m-tile and n-tile.
template <int G>
__device__ __forceinline__ BtTile bt_tile_of(const BwdArgs& a, const int* s_tab, int V, int L) {
  int lo = 0, hi = V - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_tab[mid] <= L) lo = mid; else hi = mid - 1;
  }
  BtTile t;
  t.v = uni(bt_order<G>(a, lo));
  t.g = bt_group<G>(a, t.v);
  t.g.M = uni(t.g.M);
  t.g.Nc = uni(t.g.Nc);
  t.g.rows = uni(t.g.rows);
  t.g.base = uni(t.g.base);
  const int nmt = (t.g.M + kBtBM - 1) / kBtBM;
  const int local = L - s_tab[lo];
  t.m0 = uni((local % nmt) * kBtBM);
  t.n0 = uni((local / nmt) * bt_bn(G));
  t.steps = uni(t.g.steps);
  return t;
}

// This lane's direct-to-LDS rows of tile t (wavefronts 0-3 the A rows, 4-7 the B
// rows): a wavefront-uniform base at k = 0 and 32-bit lane offsets.
// Loading state of one wavefront for a tile: its operand's base at the
// tile's first k-step, bytes per k-step, and for a slot-major operand the
// contraction rows that exist and the row pitch in bytes (to bound the range).
struct BtLoad {
  const uint8_t* base;
  uint32_t step;
  int rows;      // -1: no bound
  int pitch_b;
};

// Range (bytes) the loads of k-step s may touch: rows past the operand's
// last one read zeros.
__device__ __forceinline__ int bt_nrec(const BtLoad& l, int s) {
  if (l.rows < 0) return 0x7fffffff;
  return min(max(l.rows - 64 * s, 0), 64) * l.pitch_b;
}

// This lane's direct-to-LDS rows of tile t (wavefronts 0-3 the A operand,
// 4-7 the B operand): 32-bit lane offsets from the wavefront's base.
template <int G>
__device__ __forceinline__ BtLoad bt_prepare(const BwdArgs& a, const BtTile& t, int wave, int lane,
                                             uint32_t (&off)[kBtNI]) {
  BtLoad l;
  l.step = kBtRB;
  l.rows = -1;
  l.pitch_b = 0;
  const bool is_a = wave < 4;
  if (is_a ? bt_atr(G) : bt_btr(G)) {
    // stored layout: instruction i of the wavefront moves rows 2(8w + i) and
    // 2(8w + i) + 1 of the k-step (w = wave % 4); lane L the chunk at position L % 32
    int pitch, width, rows;
    const uint16_t* src = bt_tr_src<G>(a, t.v, t.g, pitch, width, rows);
    const int c0 = is_a ? t.m0 : t.n0;
    l.base = uni((const uint8_t*)src);
    l.step = uni(64 * pitch * 2);
    l.rows = uni(rows);
    l.pitch_b = uni(pitch * 2);
#pragma unroll
    for (int i = 0; i < kBtNI; ++i) {
      const int k = 2 * ((wave & 3) * kBtNI + i) + (lane >> 5);
      const int c = (lane & 31) ^ ((k & 7) << 1);
      // columns past the last one (a partial tile) reread the last chunk
      const int col = min(c0 + 8 * c, width - 8);
      off[i] = (uint32_t)(((size_t)k * pitch + col) * 2);
    }
  } else if (is_a) {
    constexpr bool gathered = G == BT_DP || G == BT_AC;
    l.base = uni(gathered ? (const uint8_t*)(G == BT_DP ? a.dh : a.u)
                          : bt_a_row<G>(a, t.v, t.g, min(t.m0, t.g.M - 1)));
#pragma unroll
    for (int i = 0; i < kBtNI; ++i) {
      const int r = (wave * kBtNI + i) * 8 + (lane >> 3);
      const uint8_t* rp = bt_a_row<G>(a, t.v, t.g, min(t.m0 + r, t.g.M - 1));
      off[i] = (uint32_t)(rp - l.base) + ((lane & 7) ^ ((r >> 1) & 7)) * 16;
    }
  } else {
    l.base = uni(bt_b_row<G>(a, t.v, t.n0, 0));
#pragma unroll
    for (int i = 0; i < kBtNI; ++i) {
      const int r = ((wave - 4) * kBtNI + i) * 8 + (lane >> 3);
      const uint8_t* rp = bt_b_row<G>(a, t.v, t.n0, r);
      off[i] = (uint32_t)(rp - l.base) + ((lane & 7) ^ ((r >> 1) & 7)) * 16;
    }
  }
  return l;
}

// AC: the gate of every tile row (rows past the expert's last slot: 0).
__device__ __forceinline__ void bt_fill_gate(const BwdArgs& a, const BtTile& t, float* s_gate) {
  const int tid = threadIdx.x;
  if (tid < kBtBM) {
    const int m = t.m0 + tid;
    float gv = 0.f;
    if (m < t.g.M) {
      if (t.g.routed) {
        const int TK = a.T * a.K;
        const int p = a.sorted_pair[t.g.base + m];
        gv = ((unsigned)p < (unsigned)TK) ? a.gate[p] : 0.f;
      } else {
        gv = 1.f;
      }
    }
    s_gate[tid] = gv;
  }
}

// Epilogue of tile t.
template <int G>
__device__ __forceinline__ void bt_epilogue(const BwdArgs& a, const BtTile& t, int wm, int wn,
                                            int lane, f32x16 (&acc)[2][4],
                                            uint8_t* __restrict__ lds0, uint8_t* __restrict__ lds1,
                                            const float* s_gate, float (*s_ds)[kBtBM]) {
  const int tid = threadIdx.x;
  const BtGroup& g = t.g;
  const int v = t.v, m0 = t.m0, n0 = t.n0;
  // acc[fm][fn][r]: tile row wm*64 + fm*32 + 8(r/4) + 4(lane/32) + r%4,
  // tile column bt_bcol(wn, fn) + lane%32
  const int lc = lane & 31, lh = lane >> 5;
  if constexpr (G == BT_DX) {
    // swapped operands: acc[fm][fn][4q + e] is slot row wm*64 + fm*32 + lane%32,
    // column bt_bcol(wn, fn) + 8q + 4(lane/32) + e; dx rows go out as bfloat16
    const int j = v - a.N;
#pragma unroll
    for (int fm = 0; fm < 2; ++fm) {
      const int m = m0 + wm * 64 + fm * 32 + lc;
      if (m >= g.M) continue;
      uint16_t* c = g.routed ? (uint16_t*)a.dX + (size_t)(g.base + m) * a.d
                             : (uint16_t*)a.dXs + ((size_t)j * a.T + m) * a.d;
#pragma unroll
      for (int fn = 0; fn < 4; ++fn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + bt_bcol<G>(wn, fn) + 8 * q + 4 * lh;
          if (n < g.Nc) {
            uint2 w;
            w.x = pack_bf16x2(acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1]);
            w.y = pack_bf16x2(acc[fm][fn][4 * q + 2], acc[fm][fn][4 * q + 3]);
            *(uint2*)(c + n) = w;
          }
        }
    }
    return;
  } else if constexpr (G != BT_AC) {
    const size_t Id = (size_t)a.I * a.d;
    const int j = v - a.N;
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + fm * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (m >= g.M) continue;
        float* c;
        switch (G) {
          case BT_DP:
            c = g.routed ? a.dP + (size_t)(g.base + m) * a.I
                         : a.dPs + ((size_t)m * a.K_s + j) * a.I;
            break;
          case BT_DWD:
            c = (g.routed ? a.dW_routed + (size_t)v * 3 * Id : a.dW_shared + (size_t)j * 3 * Id) +
                2 * Id + (size_t)m * a.I;
            break;
          default:
            c = (g.routed ? a.dW_routed + (size_t)v * 3 * Id : a.dW_shared + (size_t)j * 3 * Id) +
                (size_t)m * a.d;
            break;
        }
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) {
          const int n = n0 + bt_bcol<G>(wn, fn) + lc;
          if (n < g.Nc) c[n] = acc[fm][fn][r];
        }
      }
    return;
  }

  // ---- AC epilogue: the SwiGLU backward of the tile.  Swapped operands:
  // acc[fm][fn][4q + e] is slot row wm*64 + fm*32 + lane%32 and column
  // bt_bcol(wn, fn) + 8q + 4(lane/32) + e (gate fn < 2, up fn + 2, same
  // columns).  da and dc are staged row-major in the two ring slots ([256
  // rows][128 columns] bfloat16, chunk c of row r at c ^ (r & 15)), then g p
  // in the first, and go out as whole 16-byte row chunks.
  const int j = v - a.N;
  const float* dp_base = g.routed ? a.dP + (size_t)g.base * a.I : a.dPs + (size_t)j * a.I;
  const size_t dp_pitch = g.routed ? (size_t)a.I : (size_t)a.K_s * a.I;
  float dsr[2];
#pragma unroll
  for (int fm = 0; fm < 2; ++fm) {
    const int row = wm * 64 + fm * 32 + lc, m = m0 + row;
    const float gv = s_gate[row];
    // the row's 32 dP values (eight 16-byte loads) in flight at once
    f32x4 dpv[2][4];
#pragma unroll
    for (int fp = 0; fp < 2; ++fp)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = n0 + bt_bcol<BT_AC>(wn, fp) + 8 * q + 4 * lh;
        dpv[fp][q] = (m < g.M && i < a.I) ? *(const f32x4*)(dp_base + (size_t)m * dp_pitch + i)
                                          : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    dsr[fm] = 0.f;
#pragma unroll
    for (int fp = 0; fp < 2; ++fp)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float da[4], dc[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float dp = dpv[fp][q][e];
          const float av = acc[fm][fp][4 * q + e], cv = acc[fm][fp + 2][4 * q + e];
          const float sg = bt_sigmoid(av), sl = av * sg;
          const float dpg = gv * dp;
          da[e] = dpg * cv * sg * (1.f + av * (1.f - sg));
          dc[e] = dpg * sl;
          dsr[fm] += dp * (sl * cv);
        }
        const int col = bt_bcol<BT_AC>(wn, fp) + 8 * q + 4 * lh;  // 0 .. 127
        const int at = row * 256 + ((((col >> 3) ^ (row & 15))) << 4) + (col & 7) * 2;
        *(uint2*)(lds0 + at) = uint2{pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3])};
        *(uint2*)(lds1 + at) = uint2{pack_bf16x2(dc[0], dc[1]), pack_bf16x2(dc[2], dc[3])};
      }
    // this wavefront's 64 columns: the two lane halves, then the two column halves
    const float x = dsr[fm] + __shfl_xor(dsr[fm], 32);
    if (lh == 0) s_ds[wn][row] = x;
  }
  lds_sync();
  // slot-major copies: thread t moves chunk t % 16 of rows t / 16 + 32k
  const int ncols = min(kBtBNB / 2, a.I - n0);
  uint16_t* dac_base = g.routed ? (uint16_t*)a.dAC + (size_t)g.base * 2 * a.I
                                : (uint16_t*)a.dACs + (size_t)j * 2 * a.I;
  const size_t dac_pitch = g.routed ? 2 * (size_t)a.I : (size_t)a.K_s * 2 * a.I;
  uint16_t* gp_base = g.routed ? (uint16_t*)a.P + (size_t)g.base * a.I : (uint16_t*)a.Ps + (size_t)j * a.I;
  const size_t gp_pitch = g.routed ? (size_t)a.I : (size_t)a.K_s * a.I;
  const int cc = tid & 15;
  const bool col_ok = cc * 8 < ncols;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int row = (tid >> 4) + 32 * k, m = m0 + row;
    const int at = row * 256 + ((cc ^ (row & 15)) << 4);
    const u32x4 va = *(const u32x4*)(lds0 + at), vc = *(const u32x4*)(lds1 + at);
    if (m < g.M && col_ok) {
      uint16_t* r = dac_base + (size_t)m * dac_pitch + n0 + cc * 8;
      *(u32x4*)r = va;
      *(u32x4*)(r + a.I) = vc;
    }
  }
  if (g.routed && tid < kBtBM && m0 + tid < g.M) {
    const int NT = (a.I + kBtBNB / 2 - 1) / (kBtBNB / 2);
    a.dsp[(size_t)(g.base + m0 + tid) * NT + n0 / (kBtBNB / 2)] = s_ds[0][tid] + s_ds[1][tid];
  }
  lds_sync();
  // g p, recomputed from the accumulators
#pragma unroll
  for (int fm = 0; fm < 2; ++fm) {
    const int row = wm * 64 + fm * 32 + lc;
    const float gv = s_gate[row];
#pragma unroll
    for (int fp = 0; fp < 2; ++fp)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float gp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float av = acc[fm][fp][4 * q + e], cv = acc[fm][fp + 2][4 * q + e];
          gp[e] = gv * (av * bt_sigmoid(av) * cv);
        }
        const int col = bt_bcol<BT_AC>(wn, fp) + 8 * q + 4 * lh;
        const int at = row * 256 + ((((col >> 3) ^ (row & 15))) << 4) + (col & 7) * 2;
        *(uint2*)(lds0 + at) = uint2{pack_bf16x2(gp[0], gp[1]), pack_bf16x2(gp[2], gp[3])};
      }
  }
  lds_sync();
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int row = (tid >> 4) + 32 * k, m = m0 + row;
    const u32x4 vg = *(const u32x4*)(lds0 + row * 256 + ((cc ^ (row & 15)) << 4));
    if (m < g.M && col_ok) *(u32x4*)(gp_base + (size_t)m * gp_pitch + n0 + cc * 8) = vg;
  }
}

// Grouped GEMM C = A B^T for product G (bfloat16 operands, float32
// accumulation).  Persistent, one block per CU, 256 x bt_bn(G) tiles.
// Slot-row products: each XCD (blocks are dealt to the XCDs round-robin)
// owns a contiguous range of tiles (m fastest: the tiles of one weight tile
// share an L2) and its blocks claim them from the range's counter.  Weight-
// gradient products: one counter over the table's order (longest first).
// After a tile's last k-step the next tile's first k-step is already loading
// while the tile is written out (AC, whose epilogue stages through the ring,
// loads it afterwards).
template <int G>
__global__ __launch_bounds__(kBtThreads, 1) void bt_gemm_kernel(BwdArgs a,
                                                                const int32_t* __restrict__ tab,
                                                                int32_t* __restrict__ counters) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kBtSlot];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kBtSlot];
  __shared__ int s_tab[kBtMaxV + 1];
  __shared__ float s_gate[kBtBM];
  __shared__ float s_ds[2][kBtBM];
  __shared__ int s_claim[2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uni(tid >> 6), wm = wave >> 1, wn = wave & 1;
  const int V = a.N + a.K_s;
  for (int i = tid; i <= V; i += kBtThreads) s_tab[i] = tab[i];
  __syncthreads();
  const int total = s_tab[V];
  constexpr bool kWgrad = G == BT_DWD || G == BT_DWGC;
  int start, end, stride, x;
  if (kWgrad) {
    start = 0;
    end = total;
    stride = gridDim.x;
    x = 0;
  } else {
    const int X = min(8, (int)gridDim.x);
    x = blockIdx.x % X;
    start = (int)((long long)total * x / X);
    end = (int)((long long)total * (x + 1) / X);
    stride = ((int)gridDim.x - x + X - 1) / X;
  }
  const int L = start + (kWgrad ? (int)blockIdx.x : (int)blockIdx.x / min(8, (int)gridDim.x));
  if (L >= end) return;
  // the next tile (-1: none left): slot-row products claim from their XCD's
  // range first, then from the other XCDs' (which run at different clocks)
  auto claim_next = [&]() -> int {
    if (kWgrad) {
      const int p = stride + atomicAdd(counters, 1);
      return p < total ? p : -1;
    }
    const int X = min(8, (int)gridDim.x);
    for (int k = 0; k < X; ++k) {
      const int y = x + k < X ? x + k : x + k - X;
      const int s0 = (int)((long long)total * y / X), s1 = (int)((long long)total * (y + 1) / X);
      const int p = s0 + ((int)gridDim.x - y + X - 1) / X + atomicAdd(counters + y, 1);
      if (p < s1) return p;
    }
    return -1;
  };

  BtTile cur = bt_tile_of<G>(a, s_tab, V, L);
  uint32_t off[kBtNI];
  BtLoad ld = bt_prepare<G>(a, cur, wave, lane, off);
  if (G == BT_AC) bt_fill_gate(a, cur, s_gate);
  int ph = 0;  // ring slot of the current tile's k-step 0
  if (cur.steps > 0) {
    uint8_t* w = lds0 + wave * kBtNI * 1024;
    const int nrec = bt_nrec(ld, 0);
#pragma unroll
    for (int i = 0; i < kBtNI; ++i) dma16(ld.base, off[i], w + i * 1024, nrec);
  }
  for (int it = 0;; ++it) {
    if (tid == 0) s_claim[it & 1] = claim_next();
    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    int Ln = -1;
    BtTile nxt = cur;
    bool pre = false;  // the next tile's first k-step was issued under this tile
    if (cur.steps == 0) {
      // (the wait also lands the zero loads issued into this slot under the
      // previous tile before the slot is loaded again)
      pipe_sync();
      Ln = uni(s_claim[it & 1]);
      if (G != BT_AC && Ln >= 0) {
        nxt = bt_tile_of<G>(a, s_tab, V, Ln);
        ld = bt_prepare<G>(a, nxt, wave, lane, off);
        pre = true;
        uint8_t* w = ((ph & 1) ? lds1 : lds0) + wave * kBtNI * 1024;
        const int nrec = nxt.steps > 0 ? bt_nrec(ld, 0) : 0;
#pragma unroll
        for (int i = 0; i < kBtNI; ++i) dma16(ld.base, off[i], w + i * 1024, nrec);
      }
    }
    for (int s = 0; s < cur.steps; ++s) {
      pipe_sync();  // k-step s has landed; every wavefront is done with the other slot
      const int q = (ph + s) & 1;
      const uint8_t* rd = q ? lds1 : lds0;
      uint8_t* wr = (q ? lds0 : lds1) + wave * kBtNI * 1024;
      const uint8_t* db = ld.base + (size_t)(s + 1) * ld.step;
      int nrec = bt_nrec(ld, s + 1);
      if (s + 1 == cur.steps) {
        Ln = uni(s_claim[it & 1]);
        nrec = 0;
        db = ld.base;
        if (G != BT_AC && Ln >= 0) {
          nxt = bt_tile_of<G>(a, s_tab, V, Ln);
          ld = bt_prepare<G>(a, nxt, wave, lane, off);
          db = ld.base;
          pre = true;
          if (nxt.steps > 0) nrec = bt_nrec(ld, 0);
        }
      }
      bt_mma<G>(rd, wm, wn, lane, acc, uni(db), off, wr, uni(nrec));
    }
    if (G == BT_AC) pipe_sync();  // the ring is free for the staged epilogue
    bt_epilogue<G>(a, cur, wm, wn, lane, acc, lds0, lds1, s_gate, s_ds);
    ph += cur.steps;
    if (Ln < 0) break;
    if (!pre) {
      // AC: its epilogue staged through the ring, so the next tile's first
      // k-step is loaded only now (the zero loads of the last k-step landed
      // before the epilogue)
      __syncthreads();
      nxt = bt_tile_of<G>(a, s_tab, V, Ln);
      ld = bt_prepare<G>(a, nxt, wave, lane, off);
      if (G == BT_AC) bt_fill_gate(a, nxt, s_gate);
      if (nxt.steps > 0) {
        uint8_t* w = ((ph & 1) ? lds1 : lds0) + wave * kBtNI * 1024;
        const int nrec = bt_nrec(ld, 0);
#pragma unroll
        for (int i = 0; i < kBtNI; ++i) dma16(ld.base, off[i], w + i * 1024, nrec);
      }
    }
    cur = nxt;
  }
  MOE_WAIT_VMCNT(0);  // no direct-to-LDS load outlives the block
}

// ds_pair[p] = sum of the partial gate gradients of p's slot, in column order.
__global__ __launch_bounds__(256) void bt_ds_kernel(const float* __restrict__ dsp, int NT,
                                                    const int32_t* __restrict__ slot_of, int TK,
                                                    float* __restrict__ ds_pair) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= TK) return;
  const float* s = dsp + (size_t)slot_of[p] * NT;
  float x = 0.f;
  for (int t = 0; t < NT; ++t) x += s[t];
  ds_pair[p] = x;
}

long long bt_grid(int G, const BwdArgs& a) {
  auto ct = [](long long x, long long b) { return (x + b - 1) / b; };
  const long long TK = (long long)a.T * a.K, V = a.N + a.K_s;
  const long long mt = (TK + (long long)a.N * (kBtBM - 1)) / kBtBM + a.K_s * ct(a.T, kBtBM);
  switch (G) {
    case BT_DP: return mt * ct(a.I, kBtBNB);
    case BT_AC: return mt * ct(a.I, kBtBNB / 2);
    case BT_DX: return mt * ct(a.d, kBtBNB);
    case BT_DWD: return V * ct(a.d, kBtBM) * ct(a.I, kBtBNB);
    default: return V * ct(2LL * a.I, kBtBM) * ct(a.d, kBtBNB);
  }
}

int bt_cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus > 0)
      n = cus;
    else
      n = 256;
  }
  return n;
}

template <int G>
hipError_t bt_launch(const BwdArgs& a, int32_t* tabs, hipStream_t st) {
  const long long ub = bt_grid(G, a);
  if (ub <= 0) return hipSuccess;
  const int V = a.N + a.K_s;
  const long long grid = std::min<long long>(ub, bt_cu_count());
  bt_gemm_kernel<G><<<dim3((unsigned)grid), dim3(kBtThreads), 0, st>>>(
      a, tabs + (G - 1) * (V + 1), tabs + BT_NG * (V + 1) + (G - 1) * 8);
  return hipGetLastError();
}

}  // namespace

// tile tables of the five products, then 8 claim counters per product
int bt_tables_ints(int N, int K_s) { return BT_NG * (N + K_s + 1) + BT_NG * 8; }

hipError_t launch_bt_prep(const BwdArgs& a, int32_t* tabs, hipStream_t st) {
  bt_table_kernel<<<1, 64, 0, st>>>(a, tabs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bt_gather_t_kernel<<<dim3(a.d / 64, (unsigned)(a.ldx / 64), 2), 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_bt_gemm(int G, const BwdArgs& a, int32_t* tabs, hipStream_t st) {
  switch (G) {
    case BT_DP: return bt_launch<BT_DP>(a, tabs, st);
    case BT_AC: return bt_launch<BT_AC>(a, tabs, st);
    case BT_DX: return bt_launch<BT_DX>(a, tabs, st);
    case BT_DWD: return bt_launch<BT_DWD>(a, tabs, st);
    case BT_DWGC: return bt_launch<BT_DWGC>(a, tabs, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bt_ds(const BwdArgs& a, const int32_t* slot_of, float* ds_pair, hipStream_t st) {
  const int TK = a.T * a.K, NT = (a.I + kBtBNB / 2 - 1) / (kBtBNB / 2);
  bt_ds_kernel<<<(TK + 255) / 256, 256, 0, st>>>(a.dsp, NT, slot_of, TK, ds_pair);
  return hipGetLastError();
}

}  // namespace moe
