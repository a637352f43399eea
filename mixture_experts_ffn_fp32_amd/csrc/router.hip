// Router kernel for gfx950: gate logits on MFMA, float32 softmax, top-K.
//
// Method (DeepSeekMoE paper summary, papercache.org, sec. A3 and 3.2 gate
// equations): s_{i,t} = Softmax_i(u_t . e_i) over the N routed experts; the K
// largest s of each token are kept as its gates, the rest are zero.  Ties
// are broken towards the lower expert index so that exactly K are kept.
//
// Layout of the work: one block = 64 tokens = 4 wavefronts x 16 tokens.
// Token rows and expert rows are staged through two LDS buffers, up to 512
// bytes of each row per stage.  A
// wavefront computes the logits of its 16 tokens against all N experts
// (padded to 16F) with 16x16 MFMA tiles, then each group of 16 lanes owns one
// token at a time (the MFMA output puts token rows on lane groups and
// experts on lanes), so softmax and top-K reductions are 4-step butterflies
// inside a 16-lane group.  Logits never leave registers.
#include <cstdlib>

#include "moe_internal.h"

namespace moe {
namespace {


// Lane exchange inside a row of 16 lanes through DPP (no LDS round trip), a
// butterfly: step 0 pairs lanes i and i ^ 1, step 1 i and i ^ 2 (quad
// permutations), step 2 i and i ^ 7 (half-row mirror: quad 0 with quad 1,
// quad 2 with quad 3), step 3 i and i ^ 15 (row mirror: half 0 with half 1).
// Every step combines two equal-sized partial results that the partner lane
// holds bit for bit, so after the four steps every lane of the row has the
// same combination of all 16 values, with the same bits (the combining
// operations being commutative).
template <int STEP>
__device__ __forceinline__ int row16_exchange(int v) {
  constexpr int ctrl = STEP == 0 ? 0xB1 : STEP == 1 ? 0x4E : STEP == 2 ? 0x141 : 0x140;
  return __builtin_amdgcn_mov_dpp(v, ctrl, 0xF, 0xF, false);
}
template <int STEP>
__device__ __forceinline__ float row16_exchange(float v) {
  return __int_as_float(row16_exchange<STEP>(__float_as_int(v)));
}

__device__ __forceinline__ f32x4 mfma16(ElemBF16, u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// float32: a 16-byte chunk holds 4 k values; step i takes element i from every lane.
__device__ __forceinline__ f32x4 mfma16(ElemF32, u32x4 a, u32x4 b, f32x4 c) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[i]), __uint_as_float(b[i]), c, 0,
                                             0, 0);
  return c;
}

// LDS slot of 16-byte chunk c of row r when a row holds CH chunks: rows of
// 128 bytes pair up in one 256-byte bank window (chunk c ^ ((r >> 1) & 7));
// longer rows rotate over 16 chunks (c ^ (r & 15)).  16 lanes reading one
// chunk of 16 consecutive rows then hit 16 distinct bank groups.
template <int CH>
__device__ __forceinline__ int router_lds_offset(int r, int c) {
  if (CH == 8) return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
  return r * (CH * 16) + ((c ^ (r & 15)) << 4);
}

// F: experts padded to 16F.  CH: 16-byte chunks of each row loaded per
// k-step (long k-steps keep many loads in flight per wavefront: the kernel
// is bound by the latency of reading u once).  TB: tokens per block; the
// 4 wavefronts form 4 / WG groups of 16 tokens, the WG = 64 / TB wavefronts
// of a group share its expert fragments (f % WG) and meet in LDS for the
// softmax, which the group's first wavefront computes.
template <class E, int F, int CH, int TB>
__global__ __launch_bounds__(256) void router_kernel(const typename E::T* __restrict__ u,
                                                     const typename E::T* __restrict__ Eg,
                                                     const float* __restrict__ bias, int T, int d,
                                                     int N, int K, int32_t* __restrict__ idx,
                                                     float* __restrict__ gate,
                                                     float* __restrict__ scores) {
  using Tp = typename E::T;
  constexpr int NP = 16 * F;            // experts, padded
  constexpr int ROWS = TB + NP;         // LDS rows per stage: tokens, then experts
  constexpr int WG = 64 / TB;           // wavefronts per group of 16 tokens
  constexpr int RPP = 256 / CH;         // rows covered by one pass of the block
  constexpr int PASSES = (ROWS + RPP - 1) / RPP;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][ROWS * CH * 16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * TB;
  const int tg = wave / WG, wr = wave % WG;  // token group, rank inside it
  constexpr int kStep = CH * E::kPerChunk;  // contraction elements per stage
  const int nsteps = d / kStep;

  // Each thread moves chunk c of rows tid / CH + RPP * i.  Rows past T or N
  // are clamped to a valid row; their results are never written.
  const int c = tid % CH;
  const Tp* rowp[PASSES];
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int r = tid / CH + RPP * i;
    if (r < TB) {
      rowp[i] = u + (size_t)min(t0 + r, T - 1) * d;
    } else {
      rowp[i] = Eg + (size_t)min(max(r - TB, 0), N - 1) * d;
    }
  }
  u32x4 stage[PASSES];
  auto gload = [&](int s) {
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int r = tid / CH + RPP * i;
      if (r < ROWS) stage[i] = *(const u32x4*)(rowp[i] + s * kStep + c * E::kPerChunk);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int r = tid / CH + RPP * i;
      if (r < ROWS) *(u32x4*)(lds[buf] + router_lds_offset<CH>(r, c)) = stage[i];
    }
  };

  f32x4 acc[F];
#pragma unroll
  for (int f = 0; f < F; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) gload(s + 1);
#pragma unroll
    for (int kg = 0; kg < CH / 4; ++kg) {  // k-groups of 4 chunks
      const int ch = kg * 4 + (lane >> 4);
      const u32x4 a = *(const u32x4*)(lds[buf] + router_lds_offset<CH>(tg * 16 + (lane & 15), ch));
#pragma unroll
      for (int f = 0; f < F; ++f) {
        if (WG > 1 && f % WG != wr) continue;
        const u32x4 b =
            *(const u32x4*)(lds[buf] + router_lds_offset<CH>(TB + f * 16 + (lane & 15), ch));
        acc[f] = mfma16(E{}, a, b, acc[f]);
      }
    }
    if (s + 1 < nsteps) lstore(buf ^ 1);
    __syncthreads();
  }

  // acc[f][r]: token row tg*16 + 4*(lane/16) + r, expert f*16 + lane%16.
  const int grp = lane >> 4, col = lane & 15;
  if constexpr (WG > 1) {
    // the group's fragments meet in LDS (the ring is free after the last barrier)
    float* lg = (float*)&lds[0][0] + tg * 16 * NP;
#pragma unroll
    for (int f = 0; f < F; ++f)
      if (f % WG == wr)
#pragma unroll
        for (int r = 0; r < 4; ++r) lg[(grp * 4 + r) * NP + f * 16 + col] = acc[f][r];
    __syncthreads();
    if (wr != 0) return;
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[f][r] = lg[(grp * 4 + r) * NP + f * 16 + col];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + tg * 16 + grp * 4 + r;
    float v[F];
    float m = -INFINITY;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int e = f * 16 + col;
      v[f] = (e < N) ? acc[f][r] + (bias ? bias[e] : 0.f) : -INFINITY;
      m = fmaxf(m, v[f]);
    }
    m = fmaxf(m, row16_exchange<0>(m));
    m = fmaxf(m, row16_exchange<1>(m));
    m = fmaxf(m, row16_exchange<2>(m));
    m = fmaxf(m, row16_exchange<3>(m));
    float sum = 0.f;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int e = f * 16 + col;
      v[f] = (e < N) ? expf(v[f] - m) : 0.f;
      sum += v[f];
    }
    // every lane of the group ends with the bit-identical sum
    sum += row16_exchange<0>(sum);
    sum += row16_exchange<1>(sum);
    sum += row16_exchange<2>(sum);
    sum += row16_exchange<3>(sum);
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int e = f * 16 + col;
      v[f] = (e < N) ? v[f] / sum : -2.f;  // scores are >= 0; -2 marks padding
      if (scores != nullptr && e < N && t < T) scores[(size_t)t * N + e] = v[f];
    }
    for (int k = 0; k < K; ++k) {
      float bv = -1.f;
      int bi = 0x7fffffff;
#pragma unroll
      for (int f = 0; f < F; ++f) {  // ascending expert id within the lane
        if (v[f] > bv) {
          bv = v[f];
          bi = f * 16 + col;
        }
      }
      auto take = [&](float ov, int oi) {
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      };
      take(row16_exchange<0>(bv), row16_exchange<0>(bi));
      take(row16_exchange<1>(bv), row16_exchange<1>(bi));
      take(row16_exchange<2>(bv), row16_exchange<2>(bi));
      take(row16_exchange<3>(bv), row16_exchange<3>(bi));
#pragma unroll
      for (int f = 0; f < F; ++f)
        if (f * 16 + col == bi) v[f] = -1.f;  // taken (-1 is below every score)
      if (col == 0 && t < T) {
        idx[(size_t)t * K + k] = bi;
        gate[(size_t)t * K + k] = bv;
      }
    }
  }
}

// Small batches (decode): one block per token.  Each of the 256 threads takes
// 16-byte chunks of the token's row and multiplies them with the same chunks
// of every expert row.  The token chunk is requested together with the first
// 32 expert chunks (E_gate through a buffer descriptor, one scalar offset per
// expert row; it stays in L2 across the blocks), so a 2048-wide bf16 row
// needs two round trips to memory, not three.  The 64 partial logits of an
// expert group are reduced across the wavefront by a halving exchange (each
// lane ends with one expert's sum), then across the four wavefronts in LDS in
// a fixed order.  Softmax and top-K work out of LDS with thread e owning
// expert e: every thread reads all logits (broadcast reads) and reduces them
// in the same order, so all hold the same maximum and sum; an expert's place
// in the top-K is its rank, the number of experts with a larger score or an
// equal score and a smaller index (the same choice as K rounds of argmax with
// the lowest index winning ties).
constexpr int kSmallRouterMaxT = 128;

// Element q of a 16-byte chunk as float32.
__device__ __forceinline__ float chunk_elem(ElemBF16, u32x4 w, int q) {
  return __uint_as_float((q & 1) ? (w[q >> 1] & 0xffff0000u) : (w[q >> 1] << 16));
}
__device__ __forceinline__ float chunk_elem(ElemF32, u32x4 w, int q) { return __uint_as_float(w[q]); }


template <class E>
__global__ __launch_bounds__(256) void router_small_kernel(const typename E::T* __restrict__ u,
                                                           const typename E::T* __restrict__ Eg,
                                                           const float* __restrict__ bias, int T,
                                                           int d, int N, int K,
                                                           int32_t* __restrict__ idx,
                                                           float* __restrict__ gate,
                                                           float* __restrict__ scores) {
  using Tp = typename E::T;
  constexpr int PC = E::kPerChunk;
  __shared__ float s_red[4][64];
  __shared__ float s_logit[256];  // logit + bias
  __shared__ float s_ex[256];     // exp(logit - max)
  __shared__ float s_p[256];      // scores
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = d / PC;  // 16-byte chunks per row
  const int row_bytes = d * (int)sizeof(Tp);
  const Tp* ur = u + (size_t)t * d;
  const __amdgpu_buffer_rsrc_t eg =
      __builtin_amdgcn_make_buffer_rsrc((void*)Eg, (short)0, N * row_bytes, 0x00020000);
  for (int eb = 0; eb < N; eb += 64) {
    float part[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) part[i] = 0.f;
    for (int c = tid; c < nch; c += 256) {
      float x[PC];
      u32x4 xw;  // the token chunk's raw words (bf16: four bf16 pairs)
      // 32 expert chunks in flight per batch
#pragma unroll
      for (int ib = 0; ib < 64; ib += 32) {
        u32x4 w[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int e = min(eb + ib + i, N - 1);  // experts past N: a valid row, never used
          w[i] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                         eg, c * 16, __builtin_amdgcn_readfirstlane(e * row_bytes), 0));
        }
        u32x4 xu;
        if (ib == 0) xu = *(const u32x4*)(ur + c * PC);  // the token chunk, with the first batch
        // every load of the batch is issued before the first wait
        __builtin_amdgcn_sched_barrier(0);
        if (ib == 0) {
          xw = xu;
#pragma unroll
          for (int q = 0; q < PC; ++q) x[q] = chunk_elem(E{}, xu, q);
        }
        if constexpr (PC == 8) {
          // bf16: a two-term dot product per instruction straight from the
          // packed pairs (products exact in float32, summed in float32).  The
          // words go through plain arrays: a bit cast of a subscripted vector
          // element compiles to element 0 for every subscript.
          const uint32_t xs[4] = {xw.x, xw.y, xw.z, xw.w};
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            const uint32_t ws[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
            float acc = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xs[q]),
                                                    __builtin_bit_cast(bf16x2, ws[q]), acc, false);
            part[ib + i] += acc;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int q = 0; q < PC; ++q) acc += x[q] * chunk_elem(E{}, w[i], q);
            part[ib + i] += acc;
          }
        }
      }
    }
    // halving exchange: after step s a lane holds 32 >> s partial sums of the
    // experts whose index agrees with the lane in the bits already folded
#pragma unroll
    for (int h = 32; h >= 1; h >>= 1) {
      const bool upper = (lane & h) != 0;
#pragma unroll
      for (int i = 0; i < h; ++i) {
        // keep expert (upper ? i + h : i) of each pair; send the other
        const float send = upper ? part[i] : part[i + h];
        const float recv = __shfl_xor(send, h);
        part[i] = (upper ? part[i + h] : part[i]) + recv;
      }
    }
    // lane l now holds the wavefront's sum for expert eb + l
    s_red[wave][lane] = part[0];
    __syncthreads();
    if (wave == 0 && eb + lane < N)
      s_logit[eb + lane] =
          (((s_red[0][lane] + s_red[1][lane]) + s_red[2][lane]) + s_red[3][lane]) +
          (bias ? bias[eb + lane] : 0.f);
    __syncthreads();
  }
  // softmax: the maximum and the sum in expert order, the same in every thread
  float m = -INFINITY;
  for (int e = 0; e < N; ++e) m = fmaxf(m, s_logit[e]);
  float ex = 0.f;
  if (tid < N) {
    ex = expf(s_logit[tid] - m);
    s_ex[tid] = ex;
  }
  __syncthreads();
  float sum = 0.f;
  for (int e = 0; e < N; ++e) sum += s_ex[e];
  float sc = 0.f;
  if (tid < N) {
    sc = ex / sum;
    s_p[tid] = sc;
    if (scores != nullptr) scores[(size_t)t * N + tid] = sc;
  }
  __syncthreads();
  if (tid < N) {
    int rank = 0;
    for (int e = 0; e < N; ++e) {
      const float o = s_p[e];
      rank += (o > sc || (o == sc && e < tid)) ? 1 : 0;
    }
    if (rank < K) {
      idx[(size_t)t * K + rank] = tid;
      gate[(size_t)t * K + rank] = sc;
    }
  }
}

template <class E, int F, int TB>
hipError_t launch_router_tb(const void* u, const void* Eg, const float* bias, int T, int d, int N,
                            int K, int32_t* idx, float* gate, float* scores, hipStream_t st) {
  using Tp = typename E::T;
  const dim3 grid((T + TB - 1) / TB), block(256);
  const Tp* up = (const Tp*)u;
  const Tp* ep = (const Tp*)Eg;
  // long k-steps (two stages of (TB + 16F) rows in LDS) where d allows
  constexpr int CH = F <= 4 ? 32 : F == 8 ? 16 : 8;
  if ((size_t)d * sizeof(Tp) % (CH * 16) == 0)
    router_kernel<E, F, CH, TB><<<grid, block, 0, st>>>(up, ep, bias, T, d, N, K, idx, gate, scores);
  else
    router_kernel<E, F, 8, TB><<<grid, block, 0, st>>>(up, ep, bias, T, d, N, K, idx, gate, scores);
  return hipGetLastError();
}

// Tokens per block: 64 (measured fastest at both the decode and the prefill
// sizes: each block is bound by the latency of its k-steps, not by the
// number of blocks).  MOE_ROUTER_TB=16 or 32 selects the expert-split
// layouts (tuning runs; results are identical).
int router_tb(int T) {
  (void)T;
  static const int v = [] {
    const char* e = getenv("MOE_ROUTER_TB");
    return e == nullptr ? 64 : atoi(e) == 16 ? 16 : atoi(e) == 32 ? 32 : 64;
  }();
  return v;
}

// Batches of at most kSmallRouterMaxT tokens take the one-block-per-token
// kernel unless MOE_ROUTER_SMALL=0.
bool router_small() {
  const char* e = getenv("MOE_ROUTER_SMALL");
  return !(e != nullptr && e[0] == '0');
}

template <class E, int F>
hipError_t launch_router_f(const void* u, const void* Eg, const float* bias, int T, int d, int N,
                           int K, int32_t* idx, float* gate, float* scores, hipStream_t st) {
  switch (router_tb(T)) {
    case 16: return launch_router_tb<E, F, 16>(u, Eg, bias, T, d, N, K, idx, gate, scores, st);
    case 32: return launch_router_tb<E, F, 32>(u, Eg, bias, T, d, N, K, idx, gate, scores, st);
    default: return launch_router_tb<E, F, 64>(u, Eg, bias, T, d, N, K, idx, gate, scores, st);
  }
}

template <class E>
hipError_t launch_router_t(const void* u, const void* Eg, const float* bias, int T, int d, int N,
                           int K, int32_t* idx, float* gate, float* scores, hipStream_t st) {
  using Tp = typename E::T;
  if (T <= kSmallRouterMaxT && router_small()) {
    router_small_kernel<E><<<T, 256, 0, st>>>((const Tp*)u, (const Tp*)Eg, bias, T, d, N, K, idx,
                                              gate, scores);
    return hipGetLastError();
  }
  if (N <= 16) return launch_router_f<E, 1>(u, Eg, bias, T, d, N, K, idx, gate, scores, st);
  if (N <= 32) return launch_router_f<E, 2>(u, Eg, bias, T, d, N, K, idx, gate, scores, st);
  if (N <= 64) return launch_router_f<E, 4>(u, Eg, bias, T, d, N, K, idx, gate, scores, st);
  if (N <= 128) return launch_router_f<E, 8>(u, Eg, bias, T, d, N, K, idx, gate, scores, st);
  return launch_router_f<E, 16>(u, Eg, bias, T, d, N, K, idx, gate, scores, st);
}

}  // namespace

hipError_t launch_router(int dtype, const void* u, const void* E_gate, const float* bias, int T,
                         int d, int N, int K, int32_t* idx, float* gate, float* scores,
                         hipStream_t stream) {
  if (dtype == 1)
    return launch_router_t<ElemBF16>(u, E_gate, bias, T, d, N, K, idx, gate, scores, stream);
  return launch_router_t<ElemF32>(u, E_gate, bias, T, d, N, K, idx, gate, scores, stream);
}

}  // namespace moe
