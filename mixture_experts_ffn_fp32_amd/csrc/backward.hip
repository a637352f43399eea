// Backward pass of the DeepSeekMoE layer forward (DeepSeekMoE paper summary,
// papercache.org, sec. 3.2 layer equation with the router of sec. A3),
// differentiated by the chain rule with the top-K set held fixed:
//
//   FFN backward per (token, expert) slot, a = W_gate x, c = W_up x,
//   p = SiLU(a) c, y = W_down p, upstream dy (= g dh routed, dh shared):
//     dP_raw = W_down^T dh,  dp = g dP_raw,  ds = dP_raw . p  (= dh . y),
//     da = dp c SiLU'(a),  dc = dp SiLU(a),
//     dW_down += dy p^T,  dW_gate += da x^T,  dW_up += dc x^T,
//     dx = W_gate^T da + W_up^T dc;
//   softmax: dz_i = s_i (ds_i - sum_j s_j ds_j)  (ds_i = 0 off the top-K);
//   router: du += E_gate^T dz,  dE_gate = sum_t dz u^T,  db = sum_t dz;
//   du += dh (residual).
//
// Work layout: the forward's routing and dispatch are recomputed; every
// product over expert slots is one launch of a grouped MFMA GEMM whose
// groups are the routed experts (their slot ranges) and the shared experts
// (all tokens).  Operands are either contiguous along the contraction
// ("k-major": rows of 64-byte k-steps, staged as they are) or contiguous
// along the output dimension ("r-major": staged into LDS transposed); rows
// gathered through the dispatch order where the operand is a token row.
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

enum : int { BG_AC = 1, BG_DP = 2, BG_DX = 3, BG_DWD = 4, BG_DWGC = 5, BG_DE = 6 };

constexpr int kBgBM = 128, kBgBN = 128, kBgRB = 64;  // tile rows, cols, bytes of k per step
constexpr int kBgDeRows = 512;                        // tokens per partial dE_gate

__device__ __forceinline__ f32x16 bg_mfma(ElemBF16, u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 bg_mfma(ElemF32, u32x4 a, u32x4 b, f32x16 c) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i]), __uint_as_float(b[i]), c, 0,
                                             0, 0);
  return c;
}

// The token row of routed slot q of expert range [lo, hi) (clamped to valid memory).
__device__ __forceinline__ int bg_token(const BwdArgs& a, int slot) {
  const int TK = a.T * a.K;
  const int pair = a.sorted_pair[min(max(slot, 0), TK - 1)];
  return ((unsigned)pair < (unsigned)TK) ? pair / a.K : 0;
}

// Geometry of group g of product G: rows M, columns Nc, contraction Kc, slot base.
template <int G>
__device__ __forceinline__ void bg_geometry(const BwdArgs& a, int g, int& M, int& Nc, int& Kc,
                                            int& base, bool& routed) {
  routed = g < a.N;
  int rows;
  if (G == BG_DE) {  // token chunks, each giving a partial dE_gate
    routed = false;
    base = g * kBgDeRows;
    rows = min(kBgDeRows, a.T - base);
  } else if (routed) {
    const int TK = a.T * a.K;
    base = min(max(a.offsets[g], 0), TK);
    rows = min(max(a.offsets[g + 1], base), TK) - base;
  } else {
    base = 0;
    rows = a.T;
  }
  switch (G) {
    case BG_AC: M = rows; Nc = 2 * a.I; Kc = a.d; break;
    case BG_DP: M = rows; Nc = a.I; Kc = a.d; break;
    case BG_DX: M = rows; Nc = a.d; Kc = 2 * a.I; break;
    case BG_DWD: M = a.d; Nc = a.I; Kc = rows; break;
    case BG_DWGC: M = 2 * a.I; Nc = a.d; Kc = rows; break;
    default: M = a.N; Nc = a.d; Kc = rows; break;  // BG_DE
  }
}

template <int G>
__host__ __device__ __forceinline__ int bg_groups(const BwdArgs& a) {
  return G == BG_DE ? (a.T + kBgDeRows - 1) / kBgDeRows : a.N + a.K_s;
}

// Tile prefix of product G over its groups (one wavefront).
template <int G>
__global__ __launch_bounds__(64) void bg_tile_table_kernel(BwdArgs a, int32_t* __restrict__ out) {
  const int lane = threadIdx.x, NG = bg_groups<G>(a);
  int carry = 0;
  for (int b = 0; b < NG; b += 64) {
    const int g = b + lane;
    int t = 0;
    if (g < NG) {
      int M, Nc, Kc, base;
      bool routed;
      bg_geometry<G>(a, g, M, Nc, Kc, base, routed);
      t = M > 0 && (G == BG_DWD || G == BG_DWGC || G == BG_DE || Kc > 0)
              ? ((M + kBgBM - 1) / kBgBM) * ((Nc + kBgBN - 1) / kBgBN)
              : 0;
    }
    int inc = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    if (g < NG) out[g] = carry + inc - t;
    carry += __shfl(inc, 63);
  }
  if (lane == 0) out[NG] = carry;
}

// Operand element pointers.  A(m, k) and B(n, k) of group g.  For a k-major
// operand the returned pointer is the start of row m (n) at k = 0; for an
// r-major operand it is the start of contraction row k at m (n) = 0.
template <class E, int G>
struct BgOps {
  using Tp = typename E::T;
  static constexpr bool kAKMajor = G == BG_AC || G == BG_DP || G == BG_DX;
  static constexpr bool kBKMajor = G == BG_AC;
  __device__ static const Tp* wblock(const BwdArgs& a, int g, bool routed) {
    const size_t Id = (size_t)a.I * a.d;
    return routed ? (const Tp*)a.W_routed + (size_t)g * 3 * Id
                  : (const Tp*)a.W_shared + (size_t)(g - a.N) * 3 * Id;
  }
  // A: row m (k-major) or contraction row k (r-major)
  __device__ static const Tp* arow(const BwdArgs& a, int g, bool routed, int base, int idx) {
    const int j = g - a.N;
    switch (G) {
      case BG_AC:
        return (const Tp*)a.u + (size_t)(routed ? bg_token(a, base + idx) : idx) * a.d;
      case BG_DP:
        return (const Tp*)a.dh + (size_t)(routed ? bg_token(a, base + idx) : idx) * a.d;
      case BG_DX:
        return routed ? (const Tp*)a.dAC + (size_t)(base + idx) * 2 * a.I
                      : (const Tp*)a.dACs + (size_t)idx * a.K_s * 2 * a.I + (size_t)j * 2 * a.I;
      case BG_DWD:
        return routed ? (const Tp*)a.dY + (size_t)(base + idx) * a.d
                      : (const Tp*)a.dh + (size_t)idx * a.d;
      case BG_DWGC:
        return routed ? (const Tp*)a.dAC + (size_t)(base + idx) * 2 * a.I
                      : (const Tp*)a.dACs + (size_t)idx * a.K_s * 2 * a.I + (size_t)j * 2 * a.I;
      default:
        return (const Tp*)a.dzE + (size_t)(base + idx) * a.NP;
    }
  }
  // B: row n (k-major) or contraction row k (r-major)
  __device__ static const Tp* brow(const BwdArgs& a, int g, bool routed, int base, int idx) {
    const int j = g - a.N;
    switch (G) {
      case BG_AC: return wblock(a, g, routed) + (size_t)idx * a.d;          // [W_gate; W_up]
      case BG_DP: return wblock(a, g, routed) + 2 * (size_t)a.I * a.d + (size_t)idx * a.I;
      case BG_DX: return wblock(a, g, routed) + (size_t)idx * a.d;
      case BG_DWD:
        return routed ? (const Tp*)a.P + (size_t)(base + idx) * a.I
                      : (const Tp*)a.Ps + (size_t)idx * a.K_s * a.I + (size_t)j * a.I;
      case BG_DWGC:
        return (const Tp*)a.u + (size_t)(routed ? bg_token(a, base + idx) : idx) * a.d;
      default:
        return (const Tp*)a.u + (size_t)(base + idx) * a.d;
    }
  }
  __device__ static float* crow(const BwdArgs& a, int g, bool routed, int base, int m) {
    const int j = g - a.N;
    const size_t Id = (size_t)a.I * a.d;
    switch (G) {
      case BG_AC:
        return routed ? a.AC + (size_t)(base + m) * 2 * a.I
                      : a.ACs + (size_t)m * a.K_s * 2 * a.I + (size_t)j * 2 * a.I;
      case BG_DP:
        return routed ? a.dP + (size_t)(base + m) * a.I
                      : a.dPs + (size_t)m * a.K_s * a.I + (size_t)j * a.I;
      case BG_DX:
        return routed ? a.dX + (size_t)(base + m) * a.d
                      : a.dXs + ((size_t)j * a.T + m) * a.d;
      case BG_DWD:
        return (routed ? a.dW_routed + (size_t)g * 3 * Id : a.dW_shared + (size_t)j * 3 * Id) +
               2 * Id + (size_t)m * a.I;
      case BG_DWGC:
        return (routed ? a.dW_routed + (size_t)g * 3 * Id : a.dW_shared + (size_t)j * 3 * Id) +
               (size_t)m * a.d;
      default:
        return a.dE_part + ((size_t)g * a.N + m) * a.d;
    }
  }
};

// LDS: rows of 64 bytes (4 chunks of 16 B), chunk c of row r at c ^ ((r >> 2) & 3).
__device__ __forceinline__ int bg_off(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

// C_g = A_g B_g^T for every group g of product G (float32 out).  128 x 128
// tiles, 4 wavefronts of 64 x 64 (2 x 2 fragments of 32 x 32), 64 bytes of
// the contraction per k-step through two LDS buffers, next k-step staged in
// registers.  Rows and columns past the group's extent read a valid row and
// are not stored; contraction indices past its end (ragged slot counts) are
// staged as zeros.
template <class E, int G>
__global__ __launch_bounds__(256) void bg_gemm_kernel(BwdArgs a, const int32_t* __restrict__ tab) {
  using Tp = typename E::T;
  using Ops = BgOps<E, G>;
  constexpr int EPC = E::kPerChunk;               // elements per 16-byte chunk
  constexpr int KS = kBgRB / (int)sizeof(Tp);     // contraction elements per k-step
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kBgBM * kBgRB];  // [buf][A/B]
  __shared__ int s_g;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int NG = bg_groups<G>(a);
  const int L = blockIdx.x;
  if (L >= tab[NG]) return;
  if (tid == 0) {
    int lo = 0, hi = NG - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tab[mid] <= L) lo = mid; else hi = mid - 1;
    }
    while (lo + 1 < NG && tab[lo + 1] <= L) ++lo;
    s_g = lo;
  }
  __syncthreads();
  const int g = s_g;
  int M, Nc, Kc, base;
  bool routed;
  bg_geometry<G>(a, g, M, Nc, Kc, base, routed);
  const int nmt = (M + kBgBM - 1) / kBgBM;
  const int local = L - tab[g];
  const int m0 = (local % nmt) * kBgBM, n0 = (local / nmt) * kBgBN;
  const int nsteps = (Kc + KS - 1) / KS;

  // staging: thread t moves chunk t and t + 256 of each operand tile
  // k-major: chunk q = row q / 4, chunk column q % 4;  r-major: chunk q = 8 rows
  // (q % 16) * 8 .. + 7 at contraction index q / 16 (bf16: 8 rows per chunk;
  // float32: 4 rows per chunk, 32 row groups at 16 contraction indices)
  constexpr int RPC = EPC;                         // rows per r-major chunk
  constexpr int RGR = kBgBM / RPC;                 // row groups per contraction index
  u32x4 sa[2], sb[2];
  auto load = [&](int s) {
    const int k0 = s * KS;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = tid + h * 256;
      if (Ops::kAKMajor) {
        const int r = q >> 2, c = q & 3;
        const Tp* p = Ops::arow(a, g, routed, base, min(m0 + r, M - 1));
        sa[h] = *(const u32x4*)(p + k0 + c * EPC);
      } else {
        const int k = k0 + q / RGR, r = (q % RGR) * RPC;
        if (k < Kc) {
          const Tp* p = Ops::arow(a, g, routed, base, k);
          sa[h] = *(const u32x4*)(p + min(m0 + r, (G == BG_DE ? a.NP : M) - RPC));
        } else {
          sa[h] = u32x4{0u, 0u, 0u, 0u};
        }
      }
      if (Ops::kBKMajor) {
        const int r = q >> 2, c = q & 3;
        const Tp* p = Ops::brow(a, g, routed, base, min(n0 + r, Nc - 1));
        sb[h] = *(const u32x4*)(p + k0 + c * EPC);
      } else {
        const int k = k0 + q / RGR, r = (q % RGR) * RPC;
        if (k < Kc) {
          const Tp* p = Ops::brow(a, g, routed, base, k);
          sb[h] = *(const u32x4*)(p + min(n0 + r, Nc - RPC));
        } else {
          sb[h] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = tid + h * 256;
      if (Ops::kAKMajor) {
        *(u32x4*)(lds[buf][0] + bg_off(q >> 2, q & 3)) = sa[h];
      } else {
        const int kk = q / RGR, r = (q % RGR) * RPC;
        const Tp* v = (const Tp*)&sa[h];
#pragma unroll
        for (int e = 0; e < RPC; ++e)
          *(Tp*)(lds[buf][0] + bg_off(r + e, (kk * (int)sizeof(Tp)) >> 4) +
                 ((kk * (int)sizeof(Tp)) & 15)) = v[e];
      }
      if (Ops::kBKMajor) {
        *(u32x4*)(lds[buf][1] + bg_off(q >> 2, q & 3)) = sb[h];
      } else {
        const int kk = q / RGR, r = (q % RGR) * RPC;
        const Tp* v = (const Tp*)&sb[h];
#pragma unroll
        for (int e = 0; e < RPC; ++e)
          *(Tp*)(lds[buf][1] + bg_off(r + e, (kk * (int)sizeof(Tp)) >> 4) +
                 ((kk * (int)sizeof(Tp)) & 15)) = v[e];
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  load(0);
  store(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) load(s + 1);
    // k-major operands past Kc do not occur (their contraction is d, I or 2I);
    // r-major ones were staged as zeros
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
      const int ch = kg * 2 + (lane >> 5);
      u32x4 af[2], bfr[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        af[f] = *(const u32x4*)(lds[buf][0] + bg_off((wm * 2 + f) * 32 + (lane & 31), ch));
        bfr[f] = *(const u32x4*)(lds[buf][1] + bg_off((wn * 2 + f) * 32 + (lane & 31), ch));
      }
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn) acc[fm][fn] = bg_mfma(E{}, af[fm], bfr[fn], acc[fm][fn]);
    }
    if (s + 1 < nsteps) store(buf ^ 1);
    __syncthreads();
  }

  // acc[fm][fn][r]: row (wm*2+fm)*32 + 8*(r/4) + 4*(lane/32) + r%4, column (wn*2+fn)*32 + lane%32
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + (wm * 2 + fm) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m >= M) continue;
      float* c = Ops::crow(a, g, routed, base, m);
#pragma unroll
      for (int fn = 0; fn < 2; ++fn) {
        const int n = n0 + (wn * 2 + fn) * 32 + (lane & 31);
        if (n < Nc) c[n] = acc[fm][fn][r];
      }
    }
}

// ---------------------------------------------------------------- elementwise
__device__ __forceinline__ float bw_silu(float a) { return a / (1.f + __expf(-a)); }
__device__ __forceinline__ float bw_silu_grad(float a) {
  const float sg = 1.f / (1.f + __expf(-a));
  return sg * (1.f + a * (1.f - sg));
}

// One block per slot row (routed: slot q in expert order; shared: token t and
// expert j).  From a, c (AC) and dP_raw: p, dAC = [da, dc], and for routed
// rows dY = g dh and ds = dP_raw . p (stored by pair).
template <class E>
__global__ __launch_bounds__(256) void bw_slot_kernel(BwdArgs a, const float* __restrict__ gate,
                                                      float* __restrict__ ds_pair) {
  using Tp = typename E::T;
  __shared__ float red[256];
  const int TK = a.T * a.K;
  const int row = blockIdx.x, tid = threadIdx.x;
  const bool routed = row < TK;
  const float* ac;
  const float* dp;
  Tp* pout;
  Tp* dac;
  float g = 1.f;
  int pair = -1, tok = 0;
  if (routed) {
    pair = a.sorted_pair[row];
    pair = ((unsigned)pair < (unsigned)TK) ? pair : -1;
    tok = pair >= 0 ? pair / a.K : 0;
    g = pair >= 0 ? gate[pair] : 0.f;
    ac = a.AC + (size_t)row * 2 * a.I;
    dp = a.dP + (size_t)row * a.I;
    pout = (Tp*)a.P + (size_t)row * a.I;
    dac = (Tp*)a.dAC + (size_t)row * 2 * a.I;
  } else {
    const int r = row - TK, t = r / a.K_s, j = r % a.K_s;
    ac = a.ACs + (size_t)t * a.K_s * 2 * a.I + (size_t)j * 2 * a.I;
    dp = a.dPs + (size_t)t * a.K_s * a.I + (size_t)j * a.I;
    pout = (Tp*)a.Ps + (size_t)t * a.K_s * a.I + (size_t)j * a.I;
    dac = (Tp*)a.dACs + (size_t)t * a.K_s * 2 * a.I + (size_t)j * 2 * a.I;
  }
  float dsum = 0.f;
  for (int i = tid; i < a.I; i += 256) {
    const float av = ac[i], cv = ac[a.I + i], dpr = dp[i];
    const float sl = bw_silu(av);
    const float p = sl * cv;
    const float dpg = g * dpr;
    dsum += dpr * p;
    store_from_f32<E>(pout + i, p);
    store_from_f32<E>(dac + i, dpg * cv * bw_silu_grad(av));
    store_from_f32<E>(dac + a.I + i, dpg * sl);
  }
  if (!routed) return;
  const Tp* dhr = (const Tp*)a.dh + (size_t)tok * a.d;
  Tp* dy = (Tp*)a.dY + (size_t)row * a.d;
  for (int n = tid; n < a.d; n += 256) store_from_f32<E>(dy + n, g * load_as_f32<E>(dhr + n));
  red[tid] = dsum;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0 && pair >= 0) ds_pair[pair] = red[0];
}

// slot_of[pair] = slot (inverse of the dispatch order).
__global__ void bw_slot_of_kernel(const int32_t* __restrict__ sorted_pair, int TK,
                                  int32_t* __restrict__ slot_of) {
  const int q = blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= TK) return;
  const int p = sorted_pair[q];
  if ((unsigned)p < (unsigned)TK) slot_of[p] = q;
}

// Softmax backward per token (one 64-lane wavefront per token): dz from the
// scores and the K gate gradients; dz kept in float32 and in the storage type.
template <class E>
__global__ __launch_bounds__(256) void bw_softmax_kernel(BwdArgs a, const float* __restrict__ s,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ ds_pair,
                                                         float* __restrict__ dz) {
  using Tp = typename E::T;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= a.T) return;
  // sum_k s_{idx_k} ds_k (identical in every lane: a fixed-order loop)
  float dot = 0.f;
  for (int k = 0; k < a.K; ++k) {
    const int e = idx[(size_t)t * a.K + k];
    dot += s[(size_t)t * a.N + e] * ds_pair[(size_t)t * a.K + k];
  }
  for (int i = lane; i < a.NP; i += 64) {
    float v = 0.f;  // columns N .. NP-1 pad each row to whole 16-byte chunks
    if (i < a.N) {
      float dsi = 0.f;
      for (int k = 0; k < a.K; ++k)
        if (idx[(size_t)t * a.K + k] == i) dsi = ds_pair[(size_t)t * a.K + k];
      v = s[(size_t)t * a.N + i] * (dsi - dot);
      dz[(size_t)t * a.N + i] = v;
    }
    store_from_f32<E>((Tp*)a.dzE + (size_t)t * a.NP + i, v);
  }
}

// Eight consecutive elements of the storage type as float32, and back.
__device__ __forceinline__ void bw_load8(const uint16_t* p, float (&o)[8]) {
  const u32x4 v = *(const u32x4*)p;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[2 * e] = __uint_as_float(v[e] << 16);
    o[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
  }
}
__device__ __forceinline__ void bw_load8(const float* p, float (&o)[8]) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = a[e];
    o[4 + e] = b[e];
  }
}
__device__ __forceinline__ void bw_store8(uint16_t* p, const float (&v)[8]) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = (uint32_t)f32_to_bf16(v[2 * e]) | ((uint32_t)f32_to_bf16(v[2 * e + 1]) << 16);
  *(u32x4*)p = w;
}
__device__ __forceinline__ void bw_store8(float* p, const float (&v)[8]) {
  *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
  *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// du_t = dh_t + sum_k dX[slot_of(t, k)] + sum_j dXs[j][t] + E_gate^T dz_t, one
// float32 sum in that order, rounded once.  A block takes kDuTok tokens, a
// thread eight columns of each (every E_gate chunk is read once for all of
// them); the tokens' dz rows and slots are read once into LDS.  dX rows are
// bfloat16 (XB) or float32.
constexpr int kDuTok = 8;
template <class E, bool XB>
__global__ __launch_bounds__(256) void bw_du_kernel(BwdArgs a, const int32_t* __restrict__ slot_of,
                                                    const float* __restrict__ dz, void* du) {
  using Tp = typename E::T;
  using Xt = typename std::conditional<XB, uint16_t, float>::type;
  __shared__ float s_dz[kDuTok][256];
  __shared__ int s_slot[kDuTok][256];
  const int t0 = blockIdx.x * kDuTok, tid = threadIdx.x;
  const int nt = min(kDuTok, a.T - t0);
  for (int q = tid; q < nt * a.N; q += 256) s_dz[q / a.N][q % a.N] = dz[(size_t)t0 * a.N + q];
  for (int q = tid; q < nt * a.K; q += 256) s_slot[q / a.K][q % a.K] = slot_of[(size_t)t0 * a.K + q];
  for (int q = nt * 256 + tid; q < kDuTok * 256; q += 256) s_dz[q / 256][q % 256] = 0.f;
  __syncthreads();
  const Tp* Eg = (const Tp*)a.E_gate;
  const Xt* dX = (const Xt*)a.dX;
  const Xt* dXs = (const Xt*)a.dXs;
  for (int n = tid * 8; n < a.d; n += 256 * 8) {
    float acc[kDuTok][8], v[8];
#pragma unroll
    for (int tb = 0; tb < kDuTok; ++tb) {
      if (tb >= nt) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[tb][e] = 0.f;
        continue;
      }
      const int t = t0 + tb;
      bw_load8((const Tp*)a.dh + (size_t)t * a.d + n, acc[tb]);
      for (int k = 0; k < a.K; ++k) {
        bw_load8(dX + (size_t)s_slot[tb][k] * a.d + n, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[tb][e] += v[e];
      }
      for (int j = 0; j < a.K_s; ++j) {
        bw_load8(dXs + ((size_t)j * a.T + t) * a.d + n, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[tb][e] += v[e];
      }
    }
    for (int i = 0; i < a.N; ++i) {
      bw_load8(Eg + (size_t)i * a.d + n, v);
#pragma unroll
      for (int tb = 0; tb < kDuTok; ++tb) {
        const float z = s_dz[tb][i];  // rows past the batch are never stored
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[tb][e] += z * v[e];
      }
    }
#pragma unroll
    for (int tb = 0; tb < kDuTok; ++tb)
      if (tb < nt) bw_store8((Tp*)du + (size_t)(t0 + tb) * a.d + n, acc[tb]);
  }
}

// dE_gate = sum of the per-chunk partials, in chunk order.
__global__ __launch_bounds__(256) void bw_de_reduce_kernel(const float* __restrict__ part, int nch,
                                                           int Nd, float* __restrict__ dE) {
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= Nd) return;
  float acc = 0.f;
  for (int c = 0; c < nch; ++c) acc += part[(size_t)c * Nd + q];
  dE[q] = acc;
}

// db_i = sum_t dz[t][i]: one block per expert, float64 partial sums per
// thread over a fixed token stride, then a fixed-order tree.
__global__ __launch_bounds__(256) void bw_db_kernel(const float* __restrict__ dz, int T, int N,
                                                    float* __restrict__ db) {
  __shared__ double red[256];
  const int i = blockIdx.x, tid = threadIdx.x;
  double acc = 0.0;
  for (int t = tid; t < T; t += 256) acc += dz[(size_t)t * N + i];
  red[tid] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) db[i] = (float)red[0];
}

template <class E, int G>
hipError_t bg_launch(const BwdArgs& a, int32_t* tab, hipStream_t st) {
  bg_tile_table_kernel<G><<<1, 64, 0, st>>>(a, tab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // upper bound of the tile count; blocks past the table's total leave at once
  const long long TK = (long long)a.T * a.K;
  long long tiles;
  auto ct = [](long long x, long long b) { return (x + b - 1) / b; };
  switch (G) {
    case BG_AC:
    case BG_DP:
    case BG_DX: {
      const long long cols = G == BG_AC ? 2LL * a.I : G == BG_DP ? a.I : a.d;
      const long long mt = (TK + (long long)a.N * (kBgBM - 1)) / kBgBM + a.K_s * ct(a.T, kBgBM);
      tiles = mt * ct(cols, kBgBN);
      break;
    }
    case BG_DWD: tiles = (long long)(a.N + a.K_s) * ct(a.d, kBgBM) * ct(a.I, kBgBN); break;
    case BG_DWGC: tiles = (long long)(a.N + a.K_s) * ct(2LL * a.I, kBgBM) * ct(a.d, kBgBN); break;
    default: tiles = (long long)bg_groups<G>(a) * ct(a.N, kBgBM) * ct(a.d, kBgBN); break;
  }
  if (tiles <= 0) return hipSuccess;
  bg_gemm_kernel<E, G><<<dim3((unsigned)tiles), dim3(256), 0, st>>>(a, tab);
  return hipGetLastError();
}

template <class E>
hipError_t backward_t(const BwdArgs& a, const float* gate, const float* scores,
                      const int32_t* idx, float* ds_pair, int32_t* slot_of, float* dz,
                      float* dgate_bias, void* du, int32_t* tab,
                      hipStream_t st) {
  hipError_t e;
  const int TK = a.T * a.K;
  if ((e = bg_launch<E, BG_AC>(a, tab, st)) != hipSuccess) return e;
  if ((e = bg_launch<E, BG_DP>(a, tab, st)) != hipSuccess) return e;
  bw_slot_kernel<E><<<TK + a.T * a.K_s, 256, 0, st>>>(a, gate, ds_pair);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bw_slot_of_kernel<<<(TK + 255) / 256, 256, 0, st>>>(a.sorted_pair, TK, slot_of);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = bg_launch<E, BG_DX>(a, tab, st)) != hipSuccess) return e;
  if ((e = bg_launch<E, BG_DWD>(a, tab, st)) != hipSuccess) return e;
  if ((e = bg_launch<E, BG_DWGC>(a, tab, st)) != hipSuccess) return e;
  bw_softmax_kernel<E><<<(a.T + 3) / 4, 256, 0, st>>>(a, scores, idx, ds_pair, dz);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = bg_launch<E, BG_DE>(a, tab, st)) != hipSuccess) return e;
  {
    const int Nd = a.N * a.d;
    bw_de_reduce_kernel<<<(Nd + 255) / 256, 256, 0, st>>>(a.dE_part, bg_groups<BG_DE>(a), Nd,
                                                          a.dE_gate);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  bw_du_kernel<E, false><<<(a.T + kDuTok - 1) / kDuTok, 256, 0, st>>>(a, slot_of, dz, du);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (dgate_bias != nullptr) {
    bw_db_kernel<<<a.N, 256, 0, st>>>(dz, a.T, a.N, dgate_bias);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// bfloat16: every expert-slot product on the pipelined k-major GEMM
// (backward_gemm.hip); the router gradient and the sums here.
hipError_t backward_pipe_bf16(const BwdArgs& a, const float* scores, const int32_t* idx,
                              float* ds_pair, int32_t* slot_of, float* dz,
                              float* dgate_bias, void* du, int32_t* tab, int32_t* tabs,
                              hipStream_t st) {
  using E = ElemBF16;
  hipError_t e;
  const int TK = a.T * a.K;
  if ((e = launch_bt_prep(a, tabs, st)) != hipSuccess) return e;
  if ((e = launch_bt_gemm(1, a, tabs, st)) != hipSuccess) return e;  // dP
  if ((e = launch_bt_gemm(2, a, tabs, st)) != hipSuccess) return e;  // a, c and the SwiGLU backward
  bw_slot_of_kernel<<<(TK + 255) / 256, 256, 0, st>>>(a.sorted_pair, TK, slot_of);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_bt_ds(a, slot_of, ds_pair, st)) != hipSuccess) return e;
  bw_softmax_kernel<E><<<(a.T + 3) / 4, 256, 0, st>>>(a, scores, idx, ds_pair, dz);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = bg_launch<E, BG_DE>(a, tab, st)) != hipSuccess) return e;
  {
    const int Nd = a.N * a.d;
    bw_de_reduce_kernel<<<(Nd + 255) / 256, 256, 0, st>>>(a.dE_part, bg_groups<BG_DE>(a), Nd,
                                                          a.dE_gate);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = launch_bt_gemm(3, a, tabs, st)) != hipSuccess) return e;  // dx
  bw_du_kernel<E, true><<<(a.T + kDuTok - 1) / kDuTok, 256, 0, st>>>(a, slot_of, dz, du);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_bt_gemm(4, a, tabs, st)) != hipSuccess) return e;  // dW_down
  if ((e = launch_bt_gemm(5, a, tabs, st)) != hipSuccess) return e;  // dW_gate, dW_up
  if (dgate_bias != nullptr) {
    bw_db_kernel<<<a.N, 256, 0, st>>>(dz, a.T, a.N, dgate_bias);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

int backward_de_chunks(int T) { return (T + kBgDeRows - 1) / kBgDeRows; }

hipError_t launch_backward(int dtype, const BwdArgs& a, const float* gate, const float* scores,
                           const int32_t* idx, float* ds_pair, int32_t* slot_of, float* dz,
                           float* dgate_bias, void* du, int32_t* tab,
                           int32_t* tabs, hipStream_t stream) {
  if (dtype == 1 && tabs != nullptr)
    return backward_pipe_bf16(a, scores, idx, ds_pair, slot_of, dz, dgate_bias, du, tab,
                              tabs, stream);
  if (dtype == 1)
    return backward_t<ElemBF16>(a, gate, scores, idx, ds_pair, slot_of, dz, dgate_bias,
                                du, tab, stream);
  return backward_t<ElemF32>(a, gate, scores, idx, ds_pair, slot_of, dz, dgate_bias, du,
                             tab, stream);
}

}  // namespace moe
