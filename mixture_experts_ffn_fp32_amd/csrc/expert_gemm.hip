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

// Tile tables of both GEMMs from the dispatch offsets (one wavefront).
__global__ __launch_bounds__(64) void tile_table_kernel(const int32_t* __restrict__ offsets,
                                                        int N, int K_s, int T, int TK, int bm1,
                                                        int bm2, int32_t* __restrict__ tiles1,
                                                        int32_t* __restrict__ tiles2) {
  const int lane = threadIdx.x;
  for (int which = 0; which < 2; ++which) {
    const int V = which == 0 ? N + K_s : N + (K_s > 0 ? 1 : 0);
    const int bm = which == 0 ? bm1 : bm2;
    int32_t* out = which == 0 ? tiles1 : tiles2;
    int carry = 0;
    for (int b = 0; b < V; b += 64) {
      const int v = b + lane;
      int mt = 0;
      if (v < V) {
        int rows;
        if (v < N) {
          const int lo = min(max(offsets[v], 0), TK), hi = min(max(offsets[v + 1], lo), TK);
          rows = hi - lo;
        } else {
          rows = T;
        }
        mt = (rows + bm - 1) / bm;
      }
      int inc = mt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
      }
      if (v < V) out[v] = carry + inc - mt;
      carry += __shfl(inc, 63);
    }
    if (lane == 0) out[V] = carry;
  }
}

template <class E, int WM, int WN, int FM, int FN, int MODE>
__global__ __launch_bounds__(256) void expert_gemm_kernel(ExpertArgs a) {
  using Tp = typename E::T;
  constexpr int BM = WM * FM * 32;
  constexpr int BNB = WN * FN * 32;          // B rows per tile
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
  const int N = a.N, K = a.K, d = a.d, I = a.I, K_s = a.K_s, T = a.T;

  // ---- which tile is this block's
  const int V = MODE == 1 ? N + K_s : N + (K_s > 0 ? 1 : 0);
  const int32_t* tab = MODE == 1 ? a.tiles1 : a.tiles2;
  const int nt = (MODE == 1 ? I : d) / BNO;
  for (int i = tid; i <= V; i += 256) s_tab[i] = tab[i];
  __syncthreads();
  const int L = xcd_swizzle(blockIdx.x, gridDim.x);
  if (L >= s_tab[V] * nt) return;  // same decision in every thread of the block
  for (int i = tid; i < V; i += 256)
    if (s_tab[i] * nt <= L && L < s_tab[i + 1] * nt) s_v = i;
  __syncthreads();
  const int v = s_v;
  const int mt_v = s_tab[v + 1] - s_tab[v];
  const int local = L - s_tab[v] * nt;
  const int n0 = (local / mt_v) * BNO;
  const int m0 = (local % mt_v) * BM;
  const bool routed = v < N;
  const int TK = T * K;
  int row_base = 0, rows = T;
  if (routed) {
    row_base = min(max(a.offsets[v], 0), TK);
    rows = min(max(a.offsets[v + 1], row_base), TK) - row_base;
  }
  const size_t Id = (size_t)I * d;
  const int Kc = MODE == 1 ? d : (routed ? I : K_s * I);  // contraction length
  const int nsteps = Kc / kStep;

  // ---- per-thread load rows (chunk c of rows tid/8 + 32 i)
  const int c = tid & 7;
  const Tp* rowp[PASSES];
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int r = (tid >> 3) + 32 * i;
    if (i < PASSES_A) {
      const int p = min(m0 + r, rows - 1);  // rows past the end repeat the last row
      if (MODE == 1) {
        int tok = p;
        if (routed) {
          const int pair = a.sorted_pair[row_base + p];
          tok = ((unsigned)pair < (unsigned)TK) ? pair / K : 0;
        }
        rowp[i] = (const Tp*)a.u + (size_t)tok * d;
      } else {
        rowp[i] = routed ? (const Tp*)a.H_routed + (size_t)(row_base + p) * I
                         : (const Tp*)a.H_shared + (size_t)p * K_s * I;
      }
    } else {
      const int rb = r - BM;
      const Tp* W = routed ? (const Tp*)a.W_routed + (size_t)v * 3 * Id
                           : (const Tp*)a.W_shared + (size_t)(MODE == 1 ? v - N : 0) * 3 * Id;
      if (MODE == 1) {
        rowp[i] = rb < BNB / 2 ? W + (size_t)(n0 + rb) * d : W + Id + (size_t)(n0 + rb - BNB / 2) * d;
      } else {
        rowp[i] = W + 2 * Id + (size_t)(n0 + rb) * I;
      }
    }
  }
  // shared down projection: the k-step at k0 reads expert k0 / I's W_down
  const bool shared_down = MODE == 2 && !routed;
  u32x4 stage[PASSES];
  auto gload = [&](int s) {
    const size_t k0 = (size_t)s * kStep;
    const size_t kb = shared_down ? k0 + (k0 / I) * (3 * Id - I) : k0;
#pragma unroll
    for (int i = 0; i < PASSES; ++i)
      stage[i] = *(const u32x4*)(rowp[i] + (i < PASSES_A ? k0 : kb) + c * E::kPerChunk);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PASSES; ++i)
      *(u32x4*)(lds[buf] + lds_chunk_offset((tid >> 3) + 32 * i, c)) = stage[i];
  };
  auto brow = [&](int fn) {
    if (MODE == 1)
      return fn < FN / 2 ? (wn * (FN / 2) + fn) * 32 : BNB / 2 + (wn * (FN / 2) + fn - FN / 2) * 32;
    return (wn * FN + fn) * 32;
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
        bfr[fn] = *(const u32x4*)(lds[buf] + lds_chunk_offset(BM + brow(fn) + (lane & 31), ch));
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma32(E{}, af[fm], bfr[fn], acc[fm][fn]);
    }
    if (s + 1 < nsteps) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  acc[fm][fn][r]: row 8*(r/4) + 4*(lane/32) + r%4, column lane%32.
  const int lc = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int p = m0 + (wm * FM + fm) * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (p >= rows) continue;
      if (MODE == 1) {
#pragma unroll
        for (int fn = 0; fn < FN / 2; ++fn) {
          const float gt = acc[fm][fn][r], up = acc[fm][fn + FN / 2][r];
          const float hv = gt / (1.f + expf(-gt)) * up;
          const int col = n0 + (wn * (FN / 2) + fn) * 32 + lc;
          Tp* dst = routed ? (Tp*)a.H_routed + (size_t)(row_base + p) * I + col
                           : (Tp*)a.H_shared + (size_t)p * K_s * I + (size_t)(v - N) * I + col;
          store_from_f32<E>(dst, hv);
        }
      } else {
        float g = 1.f;
        Tp* dst;
        if (routed) {
          int pair = a.sorted_pair[row_base + p];
          pair = ((unsigned)pair < (unsigned)TK) ? pair : 0;
          g = a.gate[pair];
          dst = (Tp*)a.Y + (size_t)pair * d;
        } else {
          dst = (Tp*)a.Y_shared + (size_t)p * d;
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int col = n0 + (wn * FN + fn) * 32 + lc;
          store_from_f32<E>(dst + col, acc[fm][fn][r] * g);
        }
      }
    }
  }
}

// Tile shapes (wavefronts WM x WN, 32x32 fragments FM x FN per wavefront).
struct Shape {
  int WM, WN, FM, FN;
  int bm() const { return WM * FM * 32; }
  int bnb() const { return WN * FN * 32; }
};

// Few tokens per expert (decode-sized batches): short M tiles, wide N tiles,
// so every CU streams a large weight slab.  Otherwise 128x128 tiles.
bool small_m(const ExpertArgs& a) { return (long long)a.T * a.K < 64LL * a.N; }

Shape shape1(const ExpertArgs& a) {
  if (small_m(a)) return a.I % 128 == 0 ? Shape{1, 4, 1, 2} : Shape{2, 2, 1, 2};
  return Shape{2, 2, 2, 2};
}
Shape shape2(const ExpertArgs& a) {
  if (small_m(a)) return a.d % 256 == 0 ? Shape{1, 4, 1, 2} : Shape{2, 2, 1, 1};
  return a.d % 128 == 0 ? Shape{2, 2, 2, 2} : Shape{2, 2, 2, 1};
}

long long grid_tiles(const ExpertArgs& a, int bm, int nt, int shared_mtiles) {
  const long long routed = ((long long)a.T * a.K + (long long)a.N * (bm - 1)) / bm;
  return (routed + shared_mtiles) * nt;
}

template <class E, int WM, int WN, int FM, int FN, int MODE>
hipError_t launch_one(const ExpertArgs& a, hipStream_t st) {
  constexpr int BM = WM * FM * 32;
  constexpr int BNO = MODE == 1 ? WN * FN * 16 : WN * FN * 32;
  const int nt = (MODE == 1 ? a.I : a.d) / BNO;
  const int mtT = (a.T + BM - 1) / BM;
  const int shared_mt = MODE == 1 ? a.K_s * mtT : (a.K_s > 0 ? mtT : 0);
  const long long g = grid_tiles(a, BM, nt, shared_mt);
  if (g <= 0) return hipSuccess;
  if (g > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  expert_gemm_kernel<E, WM, WN, FM, FN, MODE><<<dim3((unsigned)g), dim3(256), 0, st>>>(a);
  return hipGetLastError();
}

template <class E>
hipError_t launch_gemm1_t(const ExpertArgs& a, hipStream_t st) {
  const Shape s = shape1(a);
  if (s.WM == 1) return launch_one<E, 1, 4, 1, 2, 1>(a, st);
  if (s.FM == 1) return launch_one<E, 2, 2, 1, 2, 1>(a, st);
  return launch_one<E, 2, 2, 2, 2, 1>(a, st);
}

template <class E>
hipError_t launch_gemm2_t(const ExpertArgs& a, hipStream_t st) {
  const Shape s = shape2(a);
  if (s.WM == 1) return launch_one<E, 1, 4, 1, 2, 2>(a, st);
  if (s.FM == 1) return launch_one<E, 2, 2, 1, 1, 2>(a, st);
  if (s.FN == 2) return launch_one<E, 2, 2, 2, 2, 2>(a, st);
  return launch_one<E, 2, 2, 2, 1, 2>(a, st);
}

}  // namespace

int expert_tile_table_ints(int N, int K_s) { return (N + K_s + 1) + (N + 2); }

hipError_t launch_tile_table(int dtype, const ExpertArgs& a, hipStream_t stream) {
  (void)dtype;
  tile_table_kernel<<<1, 64, 0, stream>>>(a.offsets, a.N, a.K_s, a.T, a.T * a.K, shape1(a).bm(),
                                          shape2(a).bm(), a.tiles1, a.tiles2);
  return hipGetLastError();
}

hipError_t launch_gemm1(int dtype, const ExpertArgs& a, hipStream_t stream) {
  return dtype == 1 ? launch_gemm1_t<ElemBF16>(a, stream) : launch_gemm1_t<ElemF32>(a, stream);
}

hipError_t launch_gemm2(int dtype, const ExpertArgs& a, hipStream_t stream) {
  return dtype == 1 ? launch_gemm2_t<ElemBF16>(a, stream) : launch_gemm2_t<ElemF32>(a, stream);
}

}  // namespace moe
