// Balance statistics of one routed batch (DeepSeekMoE paper summary,
// papercache.org, sec. 3.3, expert-level and device-level balance losses):
//   f_i = N / (K T) * #{t : token t selects expert i},  P_i = (1/T) sum_t s_{i,t}
//   L_ExpBal = alpha1 * sum_i f_i P_i
//   f'_g = mean_{i in group g} f_i,  P'_g = sum_{i in group g} P_i
//   L_DevBal = alpha2 * sum_g f'_g P'_g
// (N, K: routed experts and experts kept per token, the paper's N' and K'.)
//
// Two launches, both deterministic: per-chunk column sums of the scores (in
// float64) and selection counts (integers), then one block that adds the
// chunks in order and forms f, P and the two sums.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBalThreads = 256;

__global__ __launch_bounds__(kBalThreads) void balance_partial_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ idx, int T, int N, int K,
    double* __restrict__ psum, int32_t* __restrict__ pcnt) {
  __shared__ int cnt[256];
  const int tid = threadIdx.x, b = blockIdx.x;
  const int t0 = b * kBalRows, t1 = min(t0 + kBalRows, T);
  for (int c = tid; c < N; c += kBalThreads) cnt[c] = 0;
  __syncthreads();
  for (int j = t0 * K + tid; j < t1 * K; j += kBalThreads) {
    const int e = idx[j];
    if ((unsigned)e < (unsigned)N) atomicAdd(&cnt[e], 1);
  }
  for (int c = tid; c < N; c += kBalThreads) {
    double s = 0.0;
    for (int t = t0; t < t1; ++t) s += (double)scores[(size_t)t * N + c];
    psum[(size_t)b * N + c] = s;
  }
  __syncthreads();
  for (int c = tid; c < N; c += kBalThreads) pcnt[(size_t)b * N + c] = cnt[c];
}

__global__ __launch_bounds__(kBalThreads) void balance_final_kernel(
    const double* __restrict__ psum, const int32_t* __restrict__ pcnt, int nb, int T, int N,
    int K, BalanceGroups groups, float alpha1, float alpha2, float* __restrict__ f,
    float* __restrict__ P, float* __restrict__ f_dev, float* __restrict__ P_dev,
    float* __restrict__ losses) {
  __shared__ double sf[256], sP[256], gf[256], gP[256];
  const int tid = threadIdx.x;
  for (int c = tid; c < N; c += kBalThreads) {
    double s = 0.0;
    long long n = 0;
    for (int b = 0; b < nb; ++b) {
      s += psum[(size_t)b * N + c];
      n += pcnt[(size_t)b * N + c];
    }
    const double fc = (double)N * (double)n / ((double)K * (double)T);
    const double Pc = s / (double)T;
    sf[c] = fc;
    sP[c] = Pc;
    f[c] = (float)fc;
    P[c] = (float)Pc;
  }
  __syncthreads();
  const int D = groups.D;
  for (int g = tid; g < D; g += kBalThreads) {
    double fs = 0.0, ps = 0.0;
    int size = 0;
    for (int c = 0; c < N; ++c)
      if (groups.of[c] == g) {
        fs += sf[c];
        ps += sP[c];
        ++size;
      }
    gf[g] = size > 0 ? fs / size : 0.0;
    gP[g] = ps;
    f_dev[g] = (float)gf[g];
    P_dev[g] = (float)ps;
  }
  __syncthreads();
  if (tid == 0) {
    double l1 = 0.0, l2 = 0.0;
    for (int c = 0; c < N; ++c) l1 += sf[c] * sP[c];
    for (int g = 0; g < D; ++g) l2 += gf[g] * gP[g];
    losses[0] = (float)(alpha1 * l1);
    losses[1] = (float)(alpha2 * l2);
  }
}

}  // namespace

size_t balance_workspace_bytes(int T, int N) {
  const size_t nb = (size_t)(T + kBalRows - 1) / kBalRows;
  const size_t a = (nb * N * 8 + 255) & ~size_t(255);
  return a + nb * N * 4;
}

hipError_t launch_balance(const float* scores, const int32_t* idx, int T, int N, int K,
                          const BalanceGroups& groups, float alpha1, float alpha2, float* f,
                          float* P, float* f_dev, float* P_dev, float* losses, void* workspace,
                          hipStream_t stream) {
  const int nb = (T + kBalRows - 1) / kBalRows;
  double* psum = (double*)workspace;
  int32_t* pcnt = (int32_t*)((char*)workspace + (((size_t)nb * N * 8 + 255) & ~size_t(255)));
  hipLaunchKernelGGL(balance_partial_kernel, dim3(nb), dim3(kBalThreads), 0, stream, scores, idx,
                     T, N, K, psum, pcnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(balance_final_kernel, dim3(1), dim3(kBalThreads), 0, stream, psum, pcnt, nb,
                     T, N, K, groups, alpha1, alpha2, f, P, f_dev, P_dev, losses);
  return hipGetLastError();
}

}  // namespace moe
