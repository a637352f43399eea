// Combine kernel for gfx950: h_t = u_t + Y_shared_t + sum_k Y_{t*K+k}.
//
// The layer output adds the shared experts' outputs, the gate-weighted
// routed outputs and the residual (DeepSeekMoE paper summary, papercache.org,
// sec. 3.2 layer equation).  The gates were applied when Y was written, so
// this is a deterministic gather: each thread owns one 16-byte chunk of a
// row of h, reads the matching chunks of u, Y_shared and the token's K rows
// of Y (contiguous, token-major), all in flight at once, sums in float32 in
// that fixed order and rounds once.  HBM-bound: (K + 2) reads and one write
// per output element.
#include "moe_internal.h"

namespace moe {
namespace {

template <class E>
__global__ __launch_bounds__(256) void combine_kernel(const typename E::T* __restrict__ u,
                                                      const typename E::T* __restrict__ Y,
                                                      const typename E::T* __restrict__ Ys,
                                                      int T, int d, int K,
                                                      typename E::T* __restrict__ h) {
  using Tp = typename E::T;
  constexpr int V = E::kPerChunk;
  const long long chunk = (long long)blockIdx.x * 256 + threadIdx.x;
  const int cpr = d / V;  // chunks per row
  if (chunk >= (long long)T * cpr) return;
  const int t = (int)(chunk / cpr);
  const int col = (int)(chunk % cpr) * V;

  // every row of the token is requested before any is added (in groups of
  // eight Y rows; the sum keeps the fixed order u, Y_shared, Y_0 .. Y_{K-1}).
  // The inputs are read once here: non-temporal loads, so they do not push
  // other data out of the caches.
  constexpr int G = 8;
  const Tp* yr = Y + (size_t)t * K * d + col;
  u32x4 xu = __builtin_nontemporal_load((const u32x4*)(u + (size_t)t * d + col));
  u32x4 xs = Ys != nullptr ? __builtin_nontemporal_load((const u32x4*)(Ys + (size_t)t * d + col))
                           : u32x4{0u, 0u, 0u, 0u};
  u32x4 xy[G];
#pragma unroll
  for (int j = 0; j < G; ++j)
    if (j < K) xy[j] = __builtin_nontemporal_load((const u32x4*)(yr + (size_t)j * d));
  float acc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) acc[j] = load_as_f32<E>((const Tp*)&xu + j);
  if (Ys != nullptr) {
#pragma unroll
    for (int j = 0; j < V; ++j) acc[j] += load_as_f32<E>((const Tp*)&xs + j);
  }
  for (int k0 = 0; k0 < K; k0 += G) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (k0 + i >= K) break;
#pragma unroll
      for (int j = 0; j < V; ++j) acc[j] += load_as_f32<E>((const Tp*)&xy[i] + j);
    }
    if (k0 + G < K) {  // the next group
#pragma unroll
      for (int i = 0; i < G; ++i)
        if (k0 + G + i < K) xy[i] = __builtin_nontemporal_load((const u32x4*)(yr + (size_t)(k0 + G + i) * d));
    }
  }
  u32x4 out;
  Tp* os = (Tp*)&out;
#pragma unroll
  for (int j = 0; j < V; ++j) store_from_f32<E>(os + j, acc[j]);
  *(u32x4*)(h + (size_t)t * d + col) = out;
}

template <class E>
hipError_t launch_t(const void* u, const void* Y, const void* Ys, int T, int d, int K, void* h,
                    hipStream_t st) {
  using Tp = typename E::T;
  const long long chunks = (long long)T * (d / E::kPerChunk);
  const long long blocks = (chunks + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  return launch_kernel(combine_kernel<E>, dim3((unsigned)blocks), dim3(256), st, (const Tp*)u,
                       (const Tp*)Y, (const Tp*)Ys, T, d, K, (Tp*)h);
}

}  // namespace

hipError_t launch_combine(int dtype, const void* u, const void* Y, const void* Y_shared, int T,
                          int d, int K, int K_s, void* h, hipStream_t stream) {
  const void* ys = K_s > 0 ? Y_shared : nullptr;
  return dtype == 1 ? launch_t<ElemBF16>(u, Y, ys, T, d, K, h, stream)
                    : launch_t<ElemF32>(u, Y, ys, T, d, K, h, stream);
}

}  // namespace moe
