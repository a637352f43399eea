// Host-side checks of the C ABI's validation and workspace arithmetic, built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code (the
// library's argument checks, workspace layouts and host-array reads).  Every
// call here fails validation (or is an empty batch) before any HIP call, so
// no GPU is needed.  Prints one line per failed expectation and "ALL OK".
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "moe.h"

static int g_bad = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    printf("FAIL %s: status %d, want %d (%s)\n", what, got, want, moe_last_error());
    ++g_bad;
  } else if (want != MOE_OK && moe_last_error()[0] == '\0') {
    printf("FAIL %s: empty error message\n", what);
    ++g_bad;
  }
}

static void* fake(uintptr_t x) { return reinterpret_cast<void*>(x); }

int main() {
  size_t b = 0;
  // workspace sizes: the five workload shapes, the limits, overflow-prone shapes
  const int shapes[][7] = {
      {256, 256, 128, 16, 4, 1, 0},       {4096, 1280, 896, 63, 7, 1, 1},
      {8192, 2048, 1408, 64, 6, 2, 1},    {64, 2048, 1408, 64, 6, 2, 1},
      {16384, 4096, 1536, 128, 12, 4, 1}, {1, 64, 64, 256, 256, 16, 0},
      {0, 64, 64, 1, 1, 0, 1},
  };
  for (auto& s : shapes) {
    expect(moe_workspace_size(s[0], s[1], s[2], s[3], s[4], s[5], s[6], &b), MOE_OK, "ws size");
    expect(moe_backward_workspace_size(s[0], s[1], s[2], s[3], s[4], s[5], s[6], &b), MOE_OK,
           "bwd ws size");
    expect(moe_dispatch_workspace_size(s[0], s[3], s[4], &b), MOE_OK, "dispatch ws size");
    expect(moe_expert_ffn_workspace_size(s[0], s[3], s[4], s[5], &b), MOE_OK, "ffn ws size");
  }
  expect(moe_workspace_size(0x7fffffff, 64, 64, 256, 256, 0, 1, &b), MOE_ERR_UNSUPPORTED,
         "T*K overflow");
  expect(moe_workspace_size(32768, 2048, 1536, 64, 12, 2, 0, &b), MOE_ERR_UNSUPPORTED,
         "H_routed past 2 GiB");
  expect(moe_workspace_size(8, 64, 64, 8, 2, 0, 1, nullptr), MOE_ERR_INVALID_ARG, "bytes NULL");
  expect(moe_workspace_size(8, 65, 64, 8, 2, 0, 1, &b), MOE_ERR_UNSUPPORTED, "d % 64");
  expect(moe_workspace_size(8, 64, 64, 8, 9, 0, 1, &b), MOE_ERR_INVALID_ARG, "K > N");
  expect(moe_workspace_size(8, 64, 64, 8, 2, 0, 3, &b), MOE_ERR_UNSUPPORTED, "dtype");

  // forward: every argument check before the first HIP call
  const int T = 64, d = 2048, I = 1408, N = 64, K = 6, Ks = 2;
  size_t ws = 0;
  expect(moe_workspace_size(T, d, I, N, K, Ks, 1, &ws), MOE_OK, "ws");
  void* u = fake(0x100000);
  void* E = fake(0x200000);
  void* Wr = fake(0x300000);
  void* Ws = fake(0x400000);
  void* h = fake(0x10000000);
  void* w = fake(0x20000000);
  expect(moe_layer_forward(u, E, Wr, Ws, N, K, Ks, 0, d, I, 1, nullptr, nullptr, nullptr, 0,
                           nullptr),
         MOE_OK, "empty batch");
  expect(moe_layer_forward(nullptr, E, Wr, Ws, N, K, Ks, T, d, I, 1, nullptr, h, w, ws, nullptr),
         MOE_ERR_INVALID_ARG, "u NULL");
  expect(moe_layer_forward(fake(0x100008), E, Wr, Ws, N, K, Ks, T, d, I, 1, nullptr, h, w, ws,
                           nullptr),
         MOE_ERR_ALIGNMENT, "u misaligned");
  expect(moe_layer_forward(u, E, Wr, nullptr, N, K, Ks, T, d, I, 1, nullptr, h, w, ws, nullptr),
         MOE_ERR_INVALID_ARG, "W_shared NULL with K_s > 0");
  expect(moe_layer_forward(u, E, Wr, Ws, N, K, Ks, T, d, I, 1, nullptr, h, w, ws - 1, nullptr),
         MOE_ERR_WORKSPACE, "workspace too small");
  expect(moe_layer_forward(u, E, Wr, Ws, N, K, Ks, T, d, I, 1, nullptr, fake(0x100000 + 4096), w,
                           ws, nullptr),
         MOE_ERR_INVALID_ARG, "h overlaps u");
  expect(moe_layer_forward(u, E, Wr, Ws, N, K, Ks, T, d, I, 1, nullptr, fake(0x20000000 + 256), w,
                           ws, nullptr),
         MOE_ERR_INVALID_ARG, "h overlaps workspace");
  expect(moe_layer_forward(u, E, Wr, Ws, N, K, Ks, T, d, I, 1, (const float*)fake(0x500004), h, w,
                           ws, nullptr),
         MOE_ERR_ALIGNMENT, "bias misaligned");

  // stage entry points
  expect(moe_route(u, E, nullptr, T, d, N, K, 1, nullptr, (float*)w, nullptr, nullptr),
         MOE_ERR_INVALID_ARG, "route idx NULL");
  expect(moe_route(u, E, nullptr, T, d, N, N + 1, 1, (int32_t*)w, (float*)w, nullptr, nullptr),
         MOE_ERR_INVALID_ARG, "route K > N");
  expect(moe_dispatch((const int32_t*)u, T, N, K, (int32_t*)w, (int32_t*)w, (int32_t*)w, w, 0,
                      nullptr),
         MOE_ERR_WORKSPACE, "dispatch workspace");
  expect(moe_expert_ffn(u, Wr, Ws, T, d, I, N, K, Ks, 1, (const int32_t*)w, (const int32_t*)w,
                        (const float*)w, w, nullptr, w, w, w, 1 << 20, nullptr),
         MOE_ERR_INVALID_ARG, "expert_ffn H_shared NULL");
  expect(moe_combine(u, w, nullptr, T, d, K, Ks, 1, h, nullptr), MOE_ERR_INVALID_ARG,
         "combine Y_shared NULL");
  expect(moe_combine(u, w, w, T, 100, K, Ks, 1, h, nullptr), MOE_ERR_UNSUPPORTED, "combine d");

  // balance statistics: the host group array is read in full before any device call
  std::vector<int32_t> groups(N);
  for (int i = 0; i < N; ++i) groups[i] = i * 8 / N;
  expect(moe_balance_workspace_size(T, N, &b), MOE_OK, "balance ws");
  expect(moe_balance_stats(nullptr, (const int32_t*)w, T, N, K, groups.data(), 8, 1.f, 1.f,
                           (float*)w, (float*)w, (float*)w, (float*)w, (float*)w, w, b, nullptr),
         MOE_ERR_INVALID_ARG, "balance scores NULL");
  groups[N - 1] = 8;
  expect(moe_balance_stats((const float*)w, (const int32_t*)w, T, N, K, groups.data(), 8, 1.f,
                           1.f, (float*)w, (float*)w, (float*)w, (float*)w, (float*)w, w, b,
                           nullptr),
         MOE_ERR_INVALID_ARG, "balance group out of range");
  groups[N - 1] = 6;
  for (int i = 0; i < N; ++i) groups[i] = i < N - 1 ? 0 : 2;
  expect(moe_balance_stats((const float*)w, (const int32_t*)w, T, N, K, groups.data(), 3, 1.f,
                           1.f, (float*)w, (float*)w, (float*)w, (float*)w, (float*)w, w, b,
                           nullptr),
         MOE_ERR_INVALID_ARG, "balance empty group");

  // backward
  size_t bws = 0;
  expect(moe_backward_workspace_size(T, d, I, N, K, Ks, 1, &bws), MOE_OK, "bwd ws");
  expect(moe_layer_backward(u, E, Wr, Ws, N, K, Ks, T, d, I, 1, nullptr, fake(0x600000), u,
                            (float*)w, nullptr, (float*)w, (float*)w, w, bws, nullptr),
         MOE_ERR_INVALID_ARG, "du overlaps u");
  expect(moe_layer_backward(u, E, Wr, Ws, N, K, Ks, T, d, I, 1, nullptr, fake(0x600000), h,
                            (float*)w, nullptr, (float*)w, (float*)w, w, bws - 1, nullptr),
         MOE_ERR_WORKSPACE, "bwd workspace");

  // timing with nothing recorded
  double ms[MOE_NUM_STAGES];
  int n[MOE_NUM_STAGES];
  expect(moe_timing_stages(0x10), MOE_OK, "timing stages");
  expect(moe_timing_read(ms, n), MOE_OK, "timing read");
  expect(moe_timing_read(nullptr, n), MOE_ERR_INVALID_ARG, "timing read NULL");
  for (int i = 0; i < MOE_NUM_STAGES; ++i)
    if (n[i] != 0) ++g_bad;

  if (g_bad == 0) printf("ALL OK\n");
  return g_bad == 0 ? 0 : 1;
}
