// Weight-streaming expert GEMMs with long runs per weight row (gfx950, bf16).
//
// Decode-sized batches give each expert a few token rows (DeepSeekMoE paper
// summary, papercache.org, sec. 3.2 layer equation: each token goes through
// its K routed experts), so the expert GEMMs are bound by reading every
// selected expert's weights once.  HBM delivers more when each weight row is
// read in long runs: direct-to-LDS loads of 32 rows 4 KB apart reach
// 5.9-6.0 TB/s with 512-byte runs per row and step, 5.1-5.2 TB/s with
// 128-byte runs (measured on a 760 MB buffer, also with the rows in two
// runs of 16 like the gate and up rows below, and with consumers meeting the
// loaders at a barrier every step).  Long runs leave room for few weight rows
// per step, so the token rows of a tile stay in LDS for the whole tile
// instead of streaming beside the weights:
//
//  * a tile is (virtual expert, 16 token rows, 32 weight rows): GEMM1 the
//    gate and up rows of 16 columns of H, GEMM2 32 columns of Y; a k-step
//    takes 512 bytes of each weight row into one 16 KB ring slot;
//  * a segment is (virtual expert, 16-row group): its token rows (16 rows x
//    the whole contraction, at most 64 KB) are loaded into LDS once and stay
//    there while the segment's weight-row groups stream past;
//  * with at least as many segments as blocks, a block takes a contiguous
//    run of whole segments; with fewer, P blocks share a segment, each
//    taking a contiguous share of its weight-row groups;
//  * four wavefronts only load: they keep four k-steps in flight with
//    direct-to-LDS buffer loads, wait for the oldest with an exact vmcnt and
//    release it with a barrier; two wavefronts compute (16x16x32 bf16 MFMA,
//    weights as the 16-row operand so a lane holds four consecutive output
//    columns of one token), each on half of every k-step's k-groups; the
//    second hands its sums to the first through LDS, which finishes the tile
//    with 8-byte stores.
#include "dispatch_wave.h"
#include "lds_dma.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kSlBM = 16;                        // token rows per tile
constexpr int kSlBR = 32;                        // weight rows per tile
constexpr int kSlRB = 512;                       // bytes of each weight row per k-step
constexpr int kSlS = 5;                          // ring slots
constexpr int kSlLW = 4;                         // loading wavefronts
constexpr int kSlSlot = kSlBR * kSlRB;           // 16 KB
constexpr int kSlNI = kSlSlot / 1024 / kSlLW;    // loads per loading wavefront per k-step
constexpr int kSlThreads = 64 * (2 + kSlLW);  // two computing, four loading wavefronts
constexpr int kSlAMax = 64 * 1024;               // token-row region
constexpr int kSlMaxV = 256 + 16;
static_assert((kSlS - 2) * kSlNI < 64, "vmcnt range");
static_assert(kSlBR % (2 * kSlNI * kSlLW) == 0, "two weight rows per load");

// Position of 16-byte chunk c in an LDS row of >= 256 bytes whose row index
// is r: chunks rotate inside each 256-byte window, so 16 lanes reading one
// chunk index of 16 consecutive rows hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int sl_pos(int r, int c) { return (c & ~15) | ((c & 15) ^ (r & 15)); }

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float sl_silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}

// Tile coordinates: virtual expert v (routed experts, then the shared ones),
// 16-row group m, weight-row group n.
struct SlTile {
  int v, m, n;
};

// Contraction of virtual expert v (elements).
template <int MODE>
__device__ __forceinline__ int sl_k(const ExpertArgs& a, int v) {
  return MODE == 1 ? a.d : (v < a.N ? a.I : a.K_s * a.I);
}

// Weight row r (0..31) of tile t at contraction index 0.  GEMM1: rows 0..15
// are the gate rows of columns 16n .. 16n + 15, rows 16..31 their up rows.
template <int MODE>
__device__ __forceinline__ const uint8_t* sl_wrow(const ExpertArgs& a, const SlTile& t, int r) {
  const size_t Id = (size_t)a.I * a.d;
  const uint16_t* W = t.v < a.N ? (const uint16_t*)a.W_routed + (size_t)t.v * 3 * Id
                                : (const uint16_t*)a.W_shared +
                                      (size_t)(MODE == 1 ? t.v - a.N : 0) * 3 * Id;
  if (MODE == 1) return (const uint8_t*)(W + (r >= 16 ? Id : 0) + (size_t)(t.n * 16 + (r & 15)) * a.d);
  return (const uint8_t*)(W + 2 * Id + (size_t)(t.n * 32 + r) * a.I);
}

// Segment q of the tile table: virtual expert v and its 16-row group m (the
// table's prefix counts 16-row groups per virtual expert).
__device__ __forceinline__ void sl_segment(const int* s_tab, int V, int q, int& v, int& m) {
  int lo = 0, hi = V - 1;  // largest v with s_tab[v] <= q
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_tab[mid] <= q) lo = mid; else hi = mid - 1;
  }
  while (lo + 1 <= V && s_tab[lo + 1] <= q) ++lo;  // empty experts
  v = lo;
  m = q - s_tab[lo];
}

template <int MODE>
__global__ __launch_bounds__(kSlThreads, 1) void expert_stream_long_kernel(ExpertArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kSlS * kSlSlot];
  __shared__ __attribute__((aligned(1024))) uint8_t areg[kSlAMax];
  __shared__ __attribute__((aligned(16))) f32x4 xbuf[2][2][64];  // second wavefront's partial sums
  __shared__ int s_tab[kSlMaxV + 1];
  __shared__ int s_off[kSlMaxV + 1];
  __shared__ int s_sp[MODE == 1 ? kFusedDispatchPairs : 1];  // sorted pairs derived here
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int V = MODE == 1 ? a.N + a.K_s : a.N + (a.K_s > 0 ? 1 : 0);
  const int32_t* tab = MODE == 1 ? a.tiles1 : a.tiles2;
  // GEMM1 of a decode batch may derive the dispatch itself (the routing in
  // fd.idx): one wavefront of every block computes the offsets, the sorted
  // pairs and this launch's tile table into LDS (the lane masks in the token-
  // row region, free until the first segment); block 0 also writes them out,
  // with the tile tables, for the GEMM2 and combine launches.
  const bool derived = MODE == 1 && a.fd.idx != nullptr;
  if (derived) {
    if (wave == 0) {
      const bool b0 = blockIdx.x == 0;
      dispatch_wave(a.fd.idx, a.T, a.N, a.K, (unsigned long long*)areg, s_off, s_sp,
                    b0 ? a.fd.counts : nullptr, b0 ? a.fd.offsets : nullptr,
                    b0 ? a.fd.sorted_pair : nullptr);
      if (b0 && a.fd.tt.tiles1 != nullptr) tile_tables_wave(s_off, a.N, s_off[a.N], a.fd.tt);
      mtile_prefix_wave(s_off, a.N, V, a.T, a.T * a.K, kSlBM, s_tab);
    }
  } else {
    for (int i = tid; i <= V; i += blockDim.x) s_tab[i] = tab[i];
    for (int i = tid; i <= a.N; i += blockDim.x) s_off[i] = a.offsets[i];
  }
  __syncthreads();

  // The block's work: with at least as many segments as blocks, a
  // contiguous run of whole segments; with fewer, one segment and a share
  // of its weight-row groups (P blocks per segment).
  const int nt = MODE == 1 ? a.I / 16 : a.d / 32;
  const int S = s_tab[V];
  const int G = gridDim.x, b = blockIdx.x;
  int q0, q1, n0, n1;
  if (S >= G) {
    q0 = (int)((long long)S * b / G);
    q1 = (int)((long long)S * (b + 1) / G);
    n0 = 0;
    n1 = nt;
  } else {
    const int P = G / S;
    // A shared expert's M segments (its token rows in 16-row groups) stream
    // the same weights.  The blocks of one share of its weight-row groups
    // are placed 8 ids apart (workgroups are dealt round-robin over the 8
    // XCDs), so all M sit on one XCD, start together and read the same rows
    // in the same order: HBM serves the rows once and that XCD's L2 the
    // other M - 1 times.  Groups of 8 such block sets fill windows of 8 M
    // ids after the routed segments' blocks.
    const int Sr = s_tab[V - (MODE == 1 ? a.K_s : (a.K_s > 0 ? 1 : 0))];  // routed segments
    const int nsh = MODE == 1 ? a.K_s : (a.K_s > 0 ? 1 : 0);             // shared experts
    const int M = nsh > 0 ? (S - Sr) / nsh : 0;  // segments per shared expert
    const int base = Sr * P;
    const int need = M > 0 ? ((nsh * P + 7) / 8) * 8 * M : 0;
    int part = b % P;
    if (b < base || M == 0 || base + need > G) {
      q0 = b / P;
      q1 = b < S * P ? q0 + 1 : q0;
    } else {
      const int r = b - base, win = 8 * M;
      const int set = (r / win) * 8 + r % 8;  // block set: (shared expert, share)
      const int m = (r % win) / 8;
      const int e = set / P;
      part = set % P;
      q0 = Sr + e * M + m;
      q1 = e < nsh ? q0 + 1 : q0;
    }
    n0 = nt * part / P;
    n1 = nt * (part + 1) / P;
  }
  if (q0 >= q1 || n0 >= n1) return;  // whole block: no barrier is left behind

  const int lt = lane & 15, lg = lane >> 4;  // token / weight row in a fragment, k chunk
  const int TK = a.T * a.K;
  for (int q = q0; q < q1; ++q) {
    int v, m;
    sl_segment(s_tab, V, q, v, m);
    const int K = sl_k<MODE>(a, v), K2 = K * 2;
    const int ksteps = (K2 + kSlRB - 1) / kSlRB;
    const int nsteps = (n1 - n0) * ksteps;
    const int KP = (K2 + 1023) & ~1023;  // token row pitch in areg
    int row_base = 0, rows = a.T;
    if (v < a.N) {
      row_base = min(max(s_off[v], 0), TK);
      rows = min(max(s_off[v + 1], row_base), TK) - row_base;
    }
    const int live = min(kSlBM, rows - m * kSlBM);
    __syncthreads();  // the previous segment is done: ring and token rows are free

    if (wave >= 2) {
      // ---- loading wavefronts: wavefront w moves weight rows 8w .. 8w + 7 of
      // each slot, two rows per load (lane L: row L / 32, chunk position L % 32)
      const int w = wave - 2;
      const int pitch = (MODE == 1 ? a.d : a.I) * 2;  // (a shared GEMM2 segment: K_s == 1 here)
      // lane L of load i lands at LDS row 8w + 2i + L / 32, chunk position
      // L % 32, which holds the row's chunk sl_pos(row, L % 32)
      uint32_t coff[kSlNI];
#pragma unroll
      for (int i = 0; i < kSlNI; ++i)
        coff[i] = (uint32_t)((lane >> 5) * pitch + sl_pos(8 * w + 2 * i + (lane >> 5), lane & 31) * 16);
      int n = n0, s = 0;
      const uint8_t* rows_p[kSlNI];
      auto prepare = [&]() __attribute__((always_inline)) {
        const SlTile t{v, m, n};
#pragma unroll
        for (int i = 0; i < kSlNI; ++i) rows_p[i] = uni(sl_wrow<MODE>(a, t, 8 * w + 2 * i));
      };
      prepare();
      // issue the loads of the cursor's k-step, then advance it (past the
      // segment's last k-step it stays there: the spare loads reread valid
      // memory into slots nobody reads any more)
      auto issue = [&](int slot) __attribute__((always_inline)) {
        uint8_t* wr = ring + slot * kSlSlot + w * kSlNI * 1024;
        // bytes past a row's end: the next row, or past the pair's second
        // row zeros (the range bound); never multiplied
        const int nrec = pitch + K2 - s * kSlRB;
#pragma unroll
        for (int i = 0; i < kSlNI; ++i)
          dma16(uni(rows_p[i] + (size_t)s * kSlRB), coff[i], wr + i * 1024, nrec);
        if (s + 1 < ksteps) {
          ++s;
        } else if (n + 1 < n1) {
          ++n;
          s = 0;
          prepare();
        }
      };
#pragma unroll
      for (int j = 0; j < kSlS - 1; ++j) issue(j);
      __syncthreads();  // (the token rows have landed)
      int slot = kSlS - 1;
      for (int g = 0; g < nsteps; ++g) {
        MOE_WAIT_VMCNT((kSlS - 2) * kSlNI);  // k-step g has landed
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue(slot);  // k-step g + kSlS - 1 into the slot read at k-step g - 1
        slot = slot + 1 == kSlS ? 0 : slot + 1;
      }
      MOE_WAIT_VMCNT(0);
      __syncthreads();  // (the last tile's partial sums)
      continue;
    }

    // ---- computing wavefronts: wavefront c loads token rows 8c .. 8c + 7
    // and multiplies k-groups 4c .. 4c + 3 of every k-step; wavefront 1
    // hands its partial sums to wavefront 0, which finishes the tile
    const int c = wave;
    {
      int src_row = 0;  // lane i < 8: the source row of token row 8c + i
      if (lane < 8) {
        const int p = m * kSlBM + min(8 * c + lane, live - 1);
        if (MODE == 1) {
          src_row = p;
          if (v < a.N) {
            const int pair = derived ? s_sp[row_base + p] : a.sorted_pair[row_base + p];
            src_row = ((unsigned)pair < (unsigned)TK) ? pair / a.K : 0;
          }
        } else {
          src_row = v < a.N ? row_base + p : p;
        }
      }
      const size_t src_pitch =
          MODE == 1 ? (size_t)a.d : (v < a.N ? (size_t)a.I : (size_t)a.K_s * a.I);
      const uint16_t* src_base =
          MODE == 1 ? (const uint16_t*)a.u
                    : (v < a.N ? (const uint16_t*)a.H_routed : (const uint16_t*)a.H_shared);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * c + i;
        const int sr = __builtin_amdgcn_readlane(src_row, i);
        const uint8_t* src = uni((const uint8_t*)(src_base + (size_t)sr * src_pitch));
        for (int j = 0; j < KP / 1024; ++j) {
          const int nrec = r < live ? K2 - j * 1024 : 0;  // rows past the last slot: zeros
          const uint32_t o = (uint32_t)((sl_pos(r, j * 64 + lane) - j * 64) * 16);
          dma16(src + (size_t)j * 1024, o, areg + r * KP + j * 1024, nrec > 0 ? nrec : 0);
        }
      }
    }
    // GEMM2: destination pair and gate of this lane's token (wavefront 0 stores)
    int my_pair = 0;
    float my_gate = 1.f;
    if (MODE == 2 && c == 0 && v < a.N && lt < live) {
      int pair = a.sorted_pair[row_base + m * kSlBM + lt];
      pair = ((unsigned)pair < (unsigned)TK) ? pair : 0;
      my_pair = pair;
      my_gate = a.gate[pair];
    }
    MOE_WAIT_VMCNT(0);  // this wavefront's own loads only: its token rows are in
    __syncthreads();    // both halves of the token rows are in

    // two accumulators per fragment (k-groups kg % 2): four independent
    // MFMA chains per wavefront
    f32x4 acc[2][2];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[f][h] = f32x4{0.f, 0.f, 0.f, 0.f};
    // tile n's results: this lane's token, columns 4 lg + 0..3 of each fragment
    auto finish = [&](int n, int xb) __attribute__((always_inline)) {
      f32x4 y[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) y[f] = (acc[f][0] + acc[f][1]) + xbuf[xb][f][lane];
      const int p = m * kSlBM + lt;
      if (p >= rows) return;
      if (MODE == 1) {
        uint16_t* dst = v < a.N ? (uint16_t*)a.H_routed + (size_t)(row_base + p) * a.I
                                : (uint16_t*)a.H_shared + (size_t)p * a.K_s * a.I +
                                      (size_t)(v - a.N) * a.I;
        uint2 wv;
        wv.x = pack_bf16x2(sl_silu_mul(y[0][0], y[1][0]), sl_silu_mul(y[0][1], y[1][1]));
        wv.y = pack_bf16x2(sl_silu_mul(y[0][2], y[1][2]), sl_silu_mul(y[0][3], y[1][3]));
        *(uint2*)(dst + n * 16 + 4 * lg) = wv;
      } else {
        uint16_t* dst = v < a.N ? (uint16_t*)a.Y + (size_t)my_pair * a.d
                                : (uint16_t*)a.Y_shared + (size_t)p * a.d;
        const float gt = v < a.N ? my_gate : 1.f;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          uint2 wv;
          wv.x = pack_bf16x2(y[f][0] * gt, y[f][1] * gt);
          wv.y = pack_bf16x2(y[f][2] * gt, y[f][3] * gt);
          *(uint2*)(dst + n * 32 + f * 16 + 4 * lg) = wv;
        }
      }
    };

    int n = n0, s = 0, slot = 0, pending = -1;  // pending: tile whose sums wait for wavefront 1
    for (int g = 0; g < nsteps; ++g) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (c == 0 && pending >= 0) {  // wavefront 1's sums of the last tile are in
        finish(pending, (pending - n0) & 1);
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int h = 0; h < 2; ++h) acc[f][h] = f32x4{0.f, 0.f, 0.f, 0.f};
        pending = -1;
      }
      const uint8_t* rd = ring + slot * kSlSlot;
      // k-groups of this step that lie inside the contraction
      const int kg_n = min(kSlRB / 64, (K - s * (kSlRB / 2)) / 32);
      // the step's fragments are requested first (k-groups past the
      // contraction read in-range bytes that are never used), then multiplied
      u32x4 xt[4], wv[2][4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int ch = (4 * c + k) * 4 + lg;  // chunk of this step's 512 bytes
        xt[k] = *(const u32x4*)(areg + lt * KP + sl_pos(lt, s * (kSlRB / 16) + ch) * 16);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int r = f * 16 + lt;
          wv[f][k] = *(const u32x4*)(rd + r * kSlRB + sl_pos(r, ch) * 16);
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (4 * c + k < kg_n)
#pragma unroll
          for (int f = 0; f < 2; ++f)  // lane: token lt, weight rows 4 lg + 0..3
            acc[f][k & 1] = mfma16(wv[f][k], xt[k], acc[f][k & 1]);
      MOE_WAIT_LGKMCNT0();  // this slot's reads are done before the next barrier
      slot = slot + 1 == kSlS ? 0 : slot + 1;
      if (++s < ksteps) continue;
      // end of tile n: wavefront 1 hands over its sums (read by wavefront 0
      // after the next barrier; two buffers, so the next tile's hand-over
      // cannot overwrite them first)
      if (c == 1) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          xbuf[(n - n0) & 1][f][lane] = acc[f][0] + acc[f][1];
#pragma unroll
          for (int h = 0; h < 2; ++h) acc[f][h] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        MOE_WAIT_LGKMCNT0();  // written before the barrier that lets wavefront 0 read them
      } else {
        pending = n;
      }
      s = 0;
      ++n;
    }
    __syncthreads();  // the last tile's sums
    if (c == 0 && pending >= 0) finish(pending, (pending - n0) & 1);
  }
}

}  // namespace

bool stream_long_ok(int mode, const ExpertArgs& a) {
  // the token rows of a tile fit the LDS region; a shared GEMM2 tile of more
  // than one shared expert would span two weight blocks per row
  const int K = mode == 1 ? a.d : (a.K_s > 1 ? a.K_s * a.I : a.I);
  if (mode == 2 && a.K_s > 1) return false;
  return ((K * 2 + 1023) & ~1023) * kSlBM <= kSlAMax && a.I % 16 == 0 && a.d % 32 == 0;
}

int stream_long_rows() { return kSlBM; }

hipError_t launch_stream_long(int mode, const ExpertArgs& a, int cus, hipStream_t st) {
  const int nt = mode == 1 ? a.I / 16 : a.d / 32;
  // upper bound of the tile count (the kernel reads the exact one)
  const long long routed = ((long long)a.T * a.K + (long long)a.N * (kSlBM - 1)) / kSlBM;
  const long long mt = (a.T + kSlBM - 1) / kSlBM;
  const long long shared = mode == 1 ? (long long)a.K_s * mt : (a.K_s > 0 ? mt : 0);
  long long g = (routed + shared) * nt;
  if (g <= 0) return hipSuccess;
  g = g < cus ? g : cus;  // persistent: one block per CU
  if (mode == 1)
    return launch_kernel(expert_stream_long_kernel<1>, dim3((unsigned)g), dim3(kSlThreads), st, a);
  return launch_kernel(expert_stream_long_kernel<2>, dim3((unsigned)g), dim3(kSlThreads), st, a);
}

}  // namespace moe
