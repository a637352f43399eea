// Router kernel for gfx950: gate logits on MFMA, float32 softmax, top-K.
//
// Method (DeepSeekMoE paper summary, papercache.org, sec. A3 and 3.2 gate
// equations): s_{i,t} = Softmax_i(u_t . e_i) over the N routed experts; the K
// largest s of each token are kept as its gates, the rest are zero.  Ties
// are broken towards the lower expert index so that exactly K are kept.
//
// Layout of the work: one block = 32 tokens x all experts, 4 computing
// wavefronts (two token groups x two expert halves) fed by 4 loading
// wavefronts through an LDS ring (see router_kernel); batches of at most 128
// tokens take a one-block-per-token kernel (router_small_kernel).
#include <cstdlib>

#include "lds_dma.h"
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

// One block = 32 tokens x all experts (padded to NP = 16F, F even), eight
// wavefronts.  Wavefronts 4-7 only load: a stage is CH 16-byte chunks of
// every token row and expert row, brought into an S-slot LDS ring by
// direct-to-LDS buffer loads (S - 1 stages in flight; the loaders wait for
// the oldest with an exact vmcnt and release it with a barrier).
// Wavefronts 0-3 only compute: wavefront w multiplies token group w & 1 (16
// tokens) against expert half w >> 1 (F / 2 fragments of 16), 16x16x32 bf16
// MFMAs (16x16x4 for float32) with float32 accumulation.  (With every
// wavefront both loading and reading, the compiler cannot tell a ring slot's
// reads from the other slots' loads and waits for all loads before reading.)
// After the last stage the computing wavefronts write their logits to LDS and
// each 16-lane row group of all eight wavefronts takes one token for the
// softmax and top-K: 4-step DPP butterflies inside the row group.
constexpr int kRouterTB = 32;

template <class E, int F, int CH>
struct RouterCfg {
  static constexpr int NP = 16 * F;                     // experts, padded
  static constexpr int ROWS = kRouterTB + NP;           // rows per stage: tokens, then experts
  static constexpr int RPI = 64 / CH;                   // rows per load instruction (1 KB)
  static constexpr int NI = ROWS / (4 * RPI);           // loads per loading wavefront per stage
  static constexpr int SLOT = ROWS * CH * 16;           // bytes per ring slot
  static constexpr int S = 4 * SLOT <= 144 * 1024 ? 4 : 3;  // ring slots
  static_assert(ROWS % (4 * RPI) == 0 && kRouterTB % RPI == 0, "stage shape");
  static_assert(S * SLOT <= 144 * 1024 && (S - 2) * NI < 64, "ring");
};

template <class E, int F, int CH>
__global__ __launch_bounds__(512) void router_kernel(const typename E::T* __restrict__ u,
                                                     const typename E::T* __restrict__ Eg,
                                                     const float* __restrict__ bias, int T, int d,
                                                     int N, int K, int32_t* __restrict__ idx,
                                                     float* __restrict__ gate,
                                                     float* __restrict__ scores,
                                                     int32_t* __restrict__ rank,
                                                     int32_t* __restrict__ tile_counts) {
  using Tp = typename E::T;
  using C = RouterCfg<E, F, CH>;
  constexpr int TB = kRouterTB, NP = C::NP, FW = F / 2, NI = C::NI, S = C::S;
  constexpr int SLOT = C::SLOT;
  constexpr int kStep = CH * E::kPerChunk;  // contraction elements per stage
  __shared__ __attribute__((aligned(1024))) uint8_t ring[S * SLOT];
  __shared__ uint32_t s_mask[NP];  // dispatch ranks: the block's tokens per expert, one bit each

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * TB;
  static_assert(TB == kRankTile && TB <= 32, "a rank tile is one block, one mask bit per token");
  if (rank != nullptr && tid < NP) s_mask[tid] = 0u;  // ordered before use by the barriers below
  const int nsteps = d / kStep;
  // the stages are taken in an order rotated per block (stage g reads
  // contraction slice (g + rot) mod nsteps): every block reads all of E_gate,
  // and all of them on the same lines at once would queue at one L2 channel
  const int rot = (int)(blockIdx.x % (unsigned)nsteps);
  const size_t row_bytes = (size_t)d * sizeof(Tp);

  if (wave >= 4) {
    // ---- loading wavefronts: wavefront 4 + w moves rows (w NI + i) RPI ..
    // + RPI - 1 of each stage with load i; lane L lands at LDS chunk
    // position L % CH of row L / CH of that group and fetches the chunk the
    // swizzle puts there.  Rows past T or N reread a valid row (never used).
    const int w = wave - 4;
    const uint8_t* base[NI];
    uint32_t off[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r0 = (w * NI + i) * C::RPI, r = r0 + lane / CH, pos = lane % CH;
      const int c = CH == 8 ? pos ^ ((r >> 1) & 7) : pos ^ (r & 15);
      if (r0 < TB) {
        base[i] = (const uint8_t*)(u + (size_t)t0 * d);
        off[i] = (uint32_t)((size_t)(min(t0 + r, T - 1) - t0) * row_bytes) + c * 16;
      } else {
        base[i] = (const uint8_t*)Eg;
        off[i] = (uint32_t)((size_t)min(r - TB, N - 1) * row_bytes) + c * 16;
      }
    }
    auto issue = [&](int g) __attribute__((always_inline)) {
      const int sr = g + rot < nsteps ? g + rot : g + rot - nsteps;
      uint8_t* wr = ring + (g % S) * SLOT;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        dma16(uni(base[i] + (size_t)sr * CH * 16), off[i],
              wr + ((w * NI + i) * C::RPI) * CH * 16);
    };
#pragma unroll
    for (int j = 0; j < S - 1; ++j)
      if (j < nsteps) issue(j);
    for (int g = 0; g < nsteps; ++g) {
      // stage g has landed: the stages after it in flight may stay
      if (g + S - 2 < nsteps) MOE_WAIT_VMCNT((S - 2) * NI);
      else MOE_WAIT_VMCNT(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // into the slot read at stage g - 1 (released by this barrier)
      if (g + S - 1 < nsteps) issue(g + S - 1);
    }
  }

  // ---- computing wavefronts
  const int tg = wave & 1, fh = (wave >> 1) & 1;
  f32x4 acc[FW];
#pragma unroll
  for (int f = 0; f < FW; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (wave < 4)
  for (int g = 0; g < nsteps; ++g) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const uint8_t* buf = ring + (g % S) * SLOT;
#pragma unroll
    for (int kg = 0; kg < CH / 4; ++kg) {  // k-groups of 4 chunks
      const int ch = kg * 4 + (lane >> 4);
      const u32x4 av = *(const u32x4*)(buf + router_lds_offset<CH>(tg * 16 + (lane & 15), ch));
#pragma unroll
      for (int f = 0; f < FW; ++f) {
        const u32x4 bv =
            *(const u32x4*)(buf + router_lds_offset<CH>(TB + (fh * FW + f) * 16 + (lane & 15), ch));
        acc[f] = mfma16(E{}, av, bv, acc[f]);
      }
    }
    MOE_WAIT_LGKMCNT0();  // this slot's reads are done before the next barrier
  }

  // acc[f][r]: token tg*16 + 4*(lane/16) + r, expert (fh*FW + f)*16 + lane%16.
  constexpr int LP = NP + 1;  // padded logit row (floats)
  static_assert(((TB * LP * 4 + 255) & ~255) + TB * NP * 4 <= S * SLOT,
                "logits and selections fit the ring");
  float* lg = (float*)ring;
  // each token's selected experts in order (dispatch ranks), after the logits
  int* sel = (int*)(ring + ((TB * LP * 4 + 255) & ~255));
  __syncthreads();  // every wavefront's last reads of the ring are done
  if (wave < 4) {
#pragma unroll
    for (int f = 0; f < FW; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        lg[(tg * 16 + 4 * (lane >> 4) + r) * LP + (fh * FW + f) * 16 + (lane & 15)] = acc[f][r];
  }
  __syncthreads();
  // softmax and top-K, all eight wavefronts: row group grp of wavefront w
  // takes token 4w + grp
  const int grp = lane >> 4, col = lane & 15;
  {
    const int tl = wave * 4 + grp;
    const int t = t0 + tl;
    float v[F];
    float m = -INFINITY;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int e = f * 16 + col;
      v[f] = (e < N) ? lg[tl * LP + e] + (bias ? bias[e] : 0.f) : -INFINITY;
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
        if (rank != nullptr) {
          sel[tl * K + k] = bi;
          // (no expert: scores that are all NaN; the dispatch ignores such ids)
          if ((unsigned)bi < (unsigned)N) atomicOr(&s_mask[bi], 1u << tl);
        }
      }
    }
  }
  if (rank == nullptr) return;
  // Dispatch step 1 for this tile of TB tokens (the block): the rank of each
  // pair among the tile's pairs of the same expert, in token order (the
  // number of the tile's lower tokens that selected it), and each expert's
  // count in the tile.
  __syncthreads();
  {
    const int tl = wave * 4 + grp;
    const int t = t0 + tl;
    if (t < T) {
      const uint32_t below = (1u << tl) - 1u;
      for (int k = col; k < K; k += 16) {
        const int e = sel[tl * K + k];
        rank[(size_t)t * K + k] = (unsigned)e < (unsigned)N ? __popc(s_mask[e] & below) : 0;
      }
    }
  }
  const int row = rank_row((int)gridDim.x);
  for (int e = tid; e < N; e += blockDim.x)
    tile_counts[(size_t)e * row + blockIdx.x] = __popc(s_mask[e]);
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
// the lowest index winning ties).  With at most 64 experts one wavefront
// does all of it, lane e holding expert e (maximum and sum by butterflies).
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
    for (int ci = tid; ci < nch; ci += 256) {
      // chunk order rotated per block: the blocks read E_gate at the same
      // time, and the same lines in the same order would queue at one L2
      // channel after another
      int c = ci + (int)((blockIdx.x * 8u) % (unsigned)nch);
      if (c >= nch) c -= nch;
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
  if (N <= 64) {
    // one wavefront, lane e holding expert e: the maximum and the sum by xor
    // butterflies (every lane ends with the same bits), the rank from the
    // scores in LDS (same wavefront: its LDS write is seen by its next read)
    if (wave != 0) return;
    const bool live = lane < N;
    const float z = live ? s_logit[lane] : -INFINITY;
    float m = z;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float ex = live ? expf(z - m) : 0.f;
    float sum = ex;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    const float sc = ex / sum;
    s_p[lane] = live ? sc : -1.f;  // -1: below every score
    if (live && scores != nullptr) scores[(size_t)t * N + lane] = sc;
    int rank = 0;
#pragma unroll 16
    for (int e = 0; e < 64; ++e) {
      const float o = s_p[e];
      rank += (o > sc || (o == sc && e < lane)) ? 1 : 0;
    }
    if (live && rank < K) {
      idx[(size_t)t * K + rank] = lane;
      gate[(size_t)t * K + rank] = sc;
    }
    return;
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

// The widest stage the row length allows (fewer, longer stages for few experts).
template <class E, int F>
hipError_t launch_router_f(const void* u, const void* Eg, const float* bias, int T, int d, int N,
                           int K, int32_t* idx, float* gate, float* scores, int32_t* rank,
                           int32_t* tile_counts, hipStream_t st) {
  using Tp = typename E::T;
  const dim3 grid((T + kRouterTB - 1) / kRouterTB), block(512);
  const Tp* up = (const Tp*)u;
  const Tp* ep = (const Tp*)Eg;
  const size_t row = (size_t)d * sizeof(Tp);
  constexpr int CHW = F <= 4 ? 32 : F == 8 ? 16 : 8;  // chunks per stage the LDS ring holds
  if (row % (CHW * 16) == 0)
    return launch_kernel(router_kernel<E, F, CHW>, grid, block, st, up, ep, bias, T, d, N, K, idx,
                         gate, scores, rank, tile_counts);
  return launch_kernel(router_kernel<E, F, 8>, grid, block, st, up, ep, bias, T, d, N, K, idx, gate,
                       scores, rank, tile_counts);
}

// Batches of at most kSmallRouterMaxT tokens take the one-block-per-token
// kernel unless MOE_ROUTER_SMALL=0 (read on every call).
bool router_small() {
  const char* e = getenv("MOE_ROUTER_SMALL");
  return !(e != nullptr && e[0] == '0');
}

template <class E>
hipError_t launch_router_t(const void* u, const void* Eg, const float* bias, int T, int d, int N,
                           int K, int32_t* idx, float* gate, float* scores, int32_t* rank,
                           int32_t* tile_counts, bool* ranked, hipStream_t st) {
  using Tp = typename E::T;
  if (ranked != nullptr) *ranked = false;
  if (T <= kSmallRouterMaxT && router_small()) {
    return launch_kernel(router_small_kernel<E>, dim3(T), dim3(256), st, (const Tp*)u,
                         (const Tp*)Eg, bias, T, d, N, K, idx, gate, scores);
  }
  if (rank == nullptr || tile_counts == nullptr) rank = tile_counts = nullptr;
  if (ranked != nullptr) *ranked = rank != nullptr;
  if (N <= 32)
    return launch_router_f<E, 2>(u, Eg, bias, T, d, N, K, idx, gate, scores, rank, tile_counts, st);
  if (N <= 64)
    return launch_router_f<E, 4>(u, Eg, bias, T, d, N, K, idx, gate, scores, rank, tile_counts, st);
  if (N <= 128)
    return launch_router_f<E, 8>(u, Eg, bias, T, d, N, K, idx, gate, scores, rank, tile_counts, st);
  return launch_router_f<E, 16>(u, Eg, bias, T, d, N, K, idx, gate, scores, rank, tile_counts, st);
}

}  // namespace

hipError_t launch_router(int dtype, const void* u, const void* E_gate, const float* bias, int T,
                         int d, int N, int K, int32_t* idx, float* gate, float* scores,
                         hipStream_t stream, int32_t* rank, int32_t* tile_counts, bool* ranked) {
  if (dtype == 1)
    return launch_router_t<ElemBF16>(u, E_gate, bias, T, d, N, K, idx, gate, scores, rank,
                                     tile_counts, ranked, stream);
  return launch_router_t<ElemF32>(u, E_gate, bias, T, d, N, K, idx, gate, scores, rank,
                                  tile_counts, ranked, stream);
}

}  // namespace moe
