// Router kernel for gfx950: gate logits on MFMA, float32 softmax, top-K.
//
// Method (DeepSeekMoE paper summary, papercache.org, sec. A3 and 3.2 gate
// equations): s_{i,t} = Softmax_i(u_t . e_i) over the N routed experts; the K
// largest s of each token are kept as its gates, the rest are zero.  Ties
// are broken towards the lower expert index so that exactly K are kept.
//
// Layout of the work: one block = 64 tokens = 4 wavefronts x 16 tokens.  A
// wavefront computes the logits of its 16 tokens against all N experts
// (padded to 16F) with 16x16 MFMA tiles, then each group of 16 lanes owns one
// token at a time (the MFMA output puts token rows on lane groups and
// experts on lanes), so softmax and top-K reductions are 4-step butterflies
// inside a 16-lane group.  Logits never leave registers.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTokens = 64;

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

template <class E, int F>
__global__ __launch_bounds__(256) void router_kernel(const typename E::T* __restrict__ u,
                                                     const typename E::T* __restrict__ Eg,
                                                     const float* __restrict__ bias, int T, int d,
                                                     int N, int K, int32_t* __restrict__ idx,
                                                     float* __restrict__ gate,
                                                     float* __restrict__ scores) {
  using Tp = typename E::T;
  constexpr int NP = 16 * F;            // experts, padded
  constexpr int ROWS = kTokens + NP;    // LDS rows per stage: tokens, then experts
  constexpr int PASSES = (ROWS + 31) / 32;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][ROWS * 128];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kTokens;
  constexpr int kStep = 128 / (int)sizeof(Tp);  // contraction elements per stage
  const int nsteps = d / kStep;

  // Each thread moves chunk c of rows tid/8 + 32*i.  Rows past T or N are
  // clamped to a valid row; their results are never written.
  const int c = tid & 7;
  const Tp* rowp[PASSES];
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int r = (tid >> 3) + 32 * i;
    if (r < kTokens) {
      rowp[i] = u + (size_t)min(t0 + r, T - 1) * d;
    } else {
      rowp[i] = Eg + (size_t)min(r - kTokens, N - 1) * d;
    }
  }
  u32x4 stage[PASSES];
  auto gload = [&](int s) {
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int r = (tid >> 3) + 32 * i;
      if (r < ROWS) stage[i] = *(const u32x4*)(rowp[i] + s * kStep + c * E::kPerChunk);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int r = (tid >> 3) + 32 * i;
      if (r < ROWS) *(u32x4*)(lds[buf] + lds_chunk_offset(r, c)) = stage[i];
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
    for (int kg = 0; kg < 2; ++kg) {  // a 128-byte row = two k-groups of 4 chunks
      const int ch = kg * 4 + (lane >> 4);
      const u32x4 a = *(const u32x4*)(lds[buf] + lds_chunk_offset(wave * 16 + (lane & 15), ch));
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const u32x4 b =
            *(const u32x4*)(lds[buf] + lds_chunk_offset(kTokens + f * 16 + (lane & 15), ch));
        acc[f] = mfma16(E{}, a, b, acc[f]);
      }
    }
    if (s + 1 < nsteps) lstore(buf ^ 1);
    __syncthreads();
  }

  // acc[f][r]: token row wave*16 + 4*(lane/16) + r, expert f*16 + lane%16.
  const int grp = lane >> 4, col = lane & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + wave * 16 + grp * 4 + r;
    float v[F];
    float m = -INFINITY;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int e = f * 16 + col;
      v[f] = (e < N) ? acc[f][r] + (bias ? bias[e] : 0.f) : -INFINITY;
      m = fmaxf(m, v[f]);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    float sum = 0.f;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int e = f * 16 + col;
      v[f] = (e < N) ? expf(v[f] - m) : 0.f;
      sum += v[f];
    }
    // xor butterfly: every lane of the group ends with the bit-identical sum
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o);
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
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
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

template <class E>
hipError_t launch_router_t(const void* u, const void* Eg, const float* bias, int T, int d, int N,
                           int K, int32_t* idx, float* gate, float* scores, hipStream_t st) {
  using Tp = typename E::T;
  const dim3 grid((T + kTokens - 1) / kTokens), block(256);
  const Tp* up = (const Tp*)u;
  const Tp* ep = (const Tp*)Eg;
  if (N <= 16)
    router_kernel<E, 1><<<grid, block, 0, st>>>(up, ep, bias, T, d, N, K, idx, gate, scores);
  else if (N <= 32)
    router_kernel<E, 2><<<grid, block, 0, st>>>(up, ep, bias, T, d, N, K, idx, gate, scores);
  else if (N <= 64)
    router_kernel<E, 4><<<grid, block, 0, st>>>(up, ep, bias, T, d, N, K, idx, gate, scores);
  else if (N <= 128)
    router_kernel<E, 8><<<grid, block, 0, st>>>(up, ep, bias, T, d, N, K, idx, gate, scores);
  else
    router_kernel<E, 16><<<grid, block, 0, st>>>(up, ep, bias, T, d, N, K, idx, gate, scores);
  return hipGetLastError();
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
