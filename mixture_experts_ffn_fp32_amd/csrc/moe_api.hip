// C ABI of the DeepSeekMoE layer forward: argument validation, workspace
// layout and the stream-ordered launch sequence.  No device memory is
// allocated here and nothing waits on the device (except moe_timing_read).
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "moe.h"
#include "moe_internal.h"

namespace {

thread_local std::string g_err;

moe_status_t fail(moe_status_t s, const std::string& msg) {
  g_err = msg;
  return s;
}
moe_status_t ok() {
  g_err.clear();
  return MOE_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
size_t elem_size(int dtype) { return dtype == MOE_DTYPE_BF16 ? 2 : 4; }

// ---------------------------------------------------------------- validation
moe_status_t check_dtype(int dtype) {
  if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "dtype must be MOE_DTYPE_F32 (0) or MOE_DTYPE_BF16 (1)");
  return MOE_OK;
}

moe_status_t check_routing(int T, int N, int K) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0");
  if (N < 1) return fail(MOE_ERR_INVALID_ARG, "N must be >= 1");
  if (N > 256) return fail(MOE_ERR_UNSUPPORTED, "N > 256 routed experts is not supported");
  if (K < 1 || K > N) return fail(MOE_ERR_INVALID_ARG, "K must satisfy 1 <= K <= N");
  if ((long long)T * K > 0x7fffffffLL - 1024)
    return fail(MOE_ERR_UNSUPPORTED, "T*K must stay below 2^31");
  return MOE_OK;
}

moe_status_t check_dim(const char* name, int x) {
  if (x <= 0) return fail(MOE_ERR_INVALID_ARG, std::string(name) + " must be positive");
  if (x % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, std::string(name) + " must be a multiple of 64");
  return MOE_OK;
}

// The MFMA GEMMs address the rows of an operand as 32-bit byte offsets from
// one base inside a buffer resource whose range ends at 2^31 bytes: the
// gathered token rows (u, and dh in the backward), the expert-sorted H
// rows, the shared experts' H rows, one expert's weight block, and in the
// backward the 256-row tiles of the transposed token copies.  Larger
// operands are refused rather than read wrong.
constexpr long long kMaxOperandBytes = 0x7fffffffLL - 4096;

moe_status_t check_extent(const char* what, long long bytes) {
  if (bytes > kMaxOperandBytes)
    return fail(MOE_ERR_UNSUPPORTED, std::string(what) + " would span " +
                                         std::to_string(bytes) + " bytes; the limit is 2^31");
  return MOE_OK;
}

moe_status_t check_shapes(int T, int d, int I, int N, int K, int K_s, int dtype) {
  moe_status_t s;
  if ((s = check_dtype(dtype)) != MOE_OK) return s;
  if ((s = check_routing(T, N, K)) != MOE_OK) return s;
  if (K_s < 0) return fail(MOE_ERR_INVALID_ARG, "K_s must be >= 0");
  if (K_s > 16) return fail(MOE_ERR_UNSUPPORTED, "K_s > 16 shared experts is not supported");
  if ((s = check_dim("d", d)) != MOE_OK) return s;
  if ((s = check_dim("I", I)) != MOE_OK) return s;
  const long long es = dtype == MOE_DTYPE_BF16 ? 2 : 4;
  if ((s = check_extent("u [T][d]", (long long)T * d * es)) != MOE_OK) return s;
  if ((s = check_extent("H_routed [T*K][I]", (long long)T * K * I * es)) != MOE_OK) return s;
  if ((s = check_extent("H_shared [T][K_s*I]", (long long)T * K_s * I * es)) != MOE_OK) return s;
  if ((s = check_extent("one expert's weights [3][I][d]", 3LL * I * d * es)) != MOE_OK) return s;
  return MOE_OK;
}

moe_status_t check_ptr(const char* name, const void* p, bool required) {
  if (p == nullptr) {
    if (required) return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is NULL");
    return MOE_OK;
  }
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(MOE_ERR_ALIGNMENT, std::string(name) + " is not 16-byte aligned");
  return MOE_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

moe_status_t hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// ---------------------------------------------------------------- workspace
struct Layout {
  size_t idx, gate, rank, tile_counts, tile_base, counts, offsets, sorted_pair, tiles, tiles_side;
  size_t H_routed, H_shared, Y, Y_shared, total;
};

int rank_tiles(int T) { return (T + moe::kRankTile - 1) / moe::kRankTile; }

Layout make_layout(int T, int d, int I, int N, int K, int K_s, int dtype) {
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  const size_t TK = (size_t)T * K, es = elem_size(dtype);
  const size_t nt = (size_t)moe::rank_row(rank_tiles(T));
  L.idx = take(TK * 4);
  L.gate = take(TK * 4);
  L.rank = take(TK * 4);
  L.tile_counts = take(nt * N * 4);
  L.tile_base = take(nt * N * 4);
  L.counts = take((size_t)N * 4);
  L.offsets = take((size_t)(N + 1) * 4);
  L.sorted_pair = take(TK * 4);
  L.tiles = take((size_t)moe::expert_tile_table_ints(N, K_s) * 4);
  L.tiles_side = take((size_t)moe::expert_tile_table_ints(0, K_s) * 4);
  L.H_routed = take(TK * I * es);
  L.H_shared = take((size_t)T * K_s * I * es);
  L.Y = take(TK * d * es);
  L.Y_shared = take(K_s > 0 ? (size_t)T * d * es : 0);
  L.total = o;
  return L;
}

size_t dispatch_ws_bytes(int T, int N, int K) {
  const size_t nt = (size_t)moe::rank_row(rank_tiles(T));
  return align256((size_t)T * K * 4) + 2 * align256(nt * N * 4);
}
size_t expert_ws_bytes(int N, int K_s) {
  return align256((size_t)moe::expert_tile_table_ints(N, K_s) * 4);
}

// ---------------------------------------------------------------- timing
struct Timing {
  std::mutex mu;
  bool on = false;
  unsigned mask = ~0u;  // stages that get an event pair
  std::vector<hipEvent_t> pool;
  struct Rec {
    int stage;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Timing g_timing;

// The stage being enqueued on this thread and its event pair (see
// moe::stage_launch_events): the first launch of the stage carries the start
// event, every launch the stop event.
struct ScopeTiming {
  bool active = false, launched = false;
  hipEvent_t a = nullptr, b = nullptr;
};
thread_local ScopeTiming g_scope;

// Times one stage when timing is on: the pair of events rides on the stage's
// kernel launches.  Calls that must not allocate pass record = false (event
// creation allocates).
struct StageScope {
  int stage;
  bool mine = false;
  StageScope(int s, hipStream_t, bool record = true) : stage(s) {
    if (!record) return;
    std::lock_guard<std::mutex> g(g_timing.mu);
    if (!g_timing.on || !((g_timing.mask >> s) & 1u)) return;
    hipEvent_t a = g_timing.get(), b = g_timing.get();
    if (!(a && b)) {
      if (a) g_timing.pool.push_back(a);
      if (b) g_timing.pool.push_back(b);
      return;
    }
    g_scope = ScopeTiming{true, false, a, b};
    mine = true;
  }
  ~StageScope() {
    if (!mine) return;
    std::lock_guard<std::mutex> g(g_timing.mu);
    if (g_scope.launched) {
      g_timing.recs.push_back({stage, g_scope.a, g_scope.b});
    } else {  // nothing was launched (an empty batch)
      g_timing.pool.push_back(g_scope.a);
      g_timing.pool.push_back(g_scope.b);
    }
    g_scope = ScopeTiming{};
  }
};

// ---------------------------------------------------------------- shared experts beside the routing
// In decode-sized batches the router and the dispatch are latency-bound
// launches during which HBM is idle, and the shared experts need no routing:
// their two GEMMs run on a second stream of the library's own (default
// priority) meanwhile, forked from and joined into the caller's stream with
// events.  One set per device; the enqueue sequence holds a lock, so calls
// from several host threads keep each fork and join paired.
constexpr int kSideMaxT = 128;
struct Side {
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
Side g_side[64];

// MOE_SHARED_SIDE=1 runs a decode-sized batch's shared experts on the side
// stream (read on every call).  Off by default: with the long-run streaming
// GEMMs, keeping the shared experts' segments in the routed launches is
// faster (16B decode batch 0.246 -> 0.238 ms): the side kernels hold CUs that
// the dispatch and the routed GEMM1 then wait for.
bool side_enabled() {
  const char* e = getenv("MOE_SHARED_SIDE");
  return e != nullptr && e[0] == '1';
}

// Caller holds g_side_mu.
hipError_t side_of_device(Side** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  Side& sd = g_side[dev];
  if (sd.st == nullptr) {
    if ((e = hipStreamCreateWithFlags(&sd.st, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&sd.join, hipEventDisableTiming)) != hipSuccess) return e;
  }
  *out = &sd;
  return hipSuccess;
}

// ---------------------------------------------------------------- launches
// tables: the grouped GEMMs' tile tables to write as well (NULL: none).
moe_status_t run_dispatch(const int32_t* idx, int T, int N, int K, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pair, int32_t* rank,
                          int32_t* tile_counts, int32_t* tile_base, hipStream_t st,
                          const moe::TileTableOut* tables = nullptr, bool rec = true,
                          bool ranked = false) {
  hipError_t e;
  const moe::TileTableOut tt = tables != nullptr ? *tables : moe::TileTableOut{};
  if (T <= moe::kSmallDispatchT) {  // ranks, scan and scatter in one launch
    StageScope sc(1, st, rec);
    if ((e = moe::launch_dispatch_small(idx, T, N, K, counts, offsets, sorted_pair, tt, st)) !=
        hipSuccess)
      return hip_fail(e, "dispatch launch");
    return MOE_OK;
  }
  if (!ranked) {  // (ranked: the router wrote them)
    StageScope sc(1, st, rec);
    if ((e = moe::launch_tile_rank(idx, T, N, K, tile_counts, rank, st)) != hipSuccess)
      return hip_fail(e, "tile rank launch");
  }
  if (moe::scan_scatter_fits(T, N)) {  // scan and scatter in one launch
    StageScope sc(3, st, rec);
    if ((e = moe::launch_scan_scatter(idx, rank, tile_counts, T, N, K, counts, offsets,
                                      sorted_pair, tt, st)) != hipSuccess)
      return hip_fail(e, "scan and scatter launch");
    return MOE_OK;
  }
  {
    StageScope sc(2, st, rec);
    if ((e = moe::launch_dispatch_scan(tile_counts, rank_tiles(T), N, counts, offsets, tile_base,
                                       tt, st)) != hipSuccess)
      return hip_fail(e, "dispatch scan launch");
  }
  {
    StageScope sc(3, st, rec);
    if ((e = moe::launch_scatter(idx, rank, tile_base, T, N, K, sorted_pair, st)) != hipSuccess)
      return hip_fail(e, "scatter launch");
  }
  return MOE_OK;
}

// tables_ready: the dispatch launch has already written the tile tables.
moe_status_t run_experts(int dtype, const moe::ExpertArgs& a, hipStream_t st,
                         bool tables_ready = false, bool rec = true) {
  hipError_t e;
  {
    StageScope sc(4, st, rec);
    if (!tables_ready && (e = moe::launch_tile_table(dtype, a, st)) != hipSuccess)
      return hip_fail(e, "tile table launch");
    if ((e = moe::launch_gemm1(dtype, a, st)) != hipSuccess)
      return hip_fail(e, "expert GEMM1 launch");
  }
  {
    StageScope sc(5, st, rec);
    if ((e = moe::launch_gemm2(dtype, a, st)) != hipSuccess)
      return hip_fail(e, "expert GEMM2 launch");
  }
  return MOE_OK;
}

// ---------------------------------------------------------------- the forward
// Argument checks of the layer forward that do not involve the workspace.
moe_status_t check_forward(const void* u, const void* E_gate, const void* W_routed,
                           const void* W_shared, int N, int K, int K_s, int T, int d, int I,
                           int dtype, const float* gate_bias, void* h) {
  moe_status_t s = check_shapes(T, d, I, N, K, K_s, dtype);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  if ((s = check_ptr("u", u, true)) != MOE_OK) return s;
  if ((s = check_ptr("E_gate", E_gate, true)) != MOE_OK) return s;
  if ((s = check_ptr("W_routed", W_routed, true)) != MOE_OK) return s;
  if ((s = check_ptr("W_shared", W_shared, K_s > 0)) != MOE_OK) return s;
  if ((s = check_ptr("gate_bias", gate_bias, false)) != MOE_OK) return s;
  if ((s = check_ptr("h", h, true)) != MOE_OK) return s;
  const size_t act = (size_t)T * d * elem_size(dtype);
  if (overlap(h, act, u, act)) return fail(MOE_ERR_INVALID_ARG, "h overlaps u");
  return MOE_OK;
}

// The launch sequence of the layer forward on workspace `ws` (layout L).
// rec: record timing events when timing is on and allow the side stream
// (both create HIP objects on first use; the allocation-free entry point
// passes false).
moe_status_t forward_enqueue(const void* u, const void* E_gate, const void* W_routed,
                             const void* W_shared, int N, int K, int K_s, int T, int d, int I,
                             int dtype, const float* gate_bias, void* h, char* ws,
                             const Layout& L, hipStream_t st, bool rec) {
  moe_status_t s;
  int32_t* idx = (int32_t*)(ws + L.idx);
  float* gate = (float*)(ws + L.gate);
  hipError_t e;
  int32_t* offsets = (int32_t*)(ws + L.offsets);
  int32_t* sorted_pair = (int32_t*)(ws + L.sorted_pair);
  moe::ExpertArgs a{};
  a.u = u;
  a.W_routed = W_routed;
  a.W_shared = W_shared;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.gate = gate;
  a.H_routed = ws + L.H_routed;
  a.H_shared = ws + L.H_shared;
  a.Y = ws + L.Y;
  a.Y_shared = ws + L.Y_shared;
  a.tiles1 = (int32_t*)(ws + L.tiles);
  a.tiles2 = a.tiles1 + (N + K_s + 1);
  a.counters = a.tiles2 + (N + 2);
  a.T = T;
  a.d = d;
  a.I = I;
  a.N = N;
  a.K = K;
  a.K_s = K_s;
  // decode-sized batches with MOE_SHARED_SIDE=1: the shared experts on the
  // side stream, the routed ones (a K_s = 0 view of the same buffers) after
  // the dispatch
  const bool side = rec && K_s > 0 && T <= kSideMaxT && side_enabled();
  std::unique_lock<std::mutex> side_lock(g_side_mu, std::defer_lock);
  Side* sd = nullptr;
  moe::ExpertArgs ar = a;
  if (side) {
    side_lock.lock();
    if ((e = side_of_device(&sd)) != hipSuccess) return hip_fail(e, "side stream");
    moe::ExpertArgs as = a;
    as.N = 0;
    as.sel_N = N;
    as.tiles1 = (int32_t*)(ws + L.tiles_side);
    as.tiles2 = as.tiles1 + (K_s + 1);
    as.counters = as.tiles2 + 2;
    if ((e = hipEventRecord(sd->fork, st)) != hipSuccess ||
        (e = hipStreamWaitEvent(sd->st, sd->fork, 0)) != hipSuccess ||
        (e = moe::launch_tile_table(dtype, as, sd->st)) != hipSuccess ||
        (e = moe::launch_gemm1(dtype, as, sd->st)) != hipSuccess ||
        (e = moe::launch_gemm2(dtype, as, sd->st)) != hipSuccess ||
        (e = hipEventRecord(sd->join, sd->st)) != hipSuccess)
      return hip_fail(e, "shared-expert launches");
    ar.K_s = 0;
  }
  // the tiled router also writes the dispatch ranks of large batches
  bool ranked = false;
  const bool want_ranks = T > moe::kSmallDispatchT;
  {
    StageScope sc(0, st, rec);
    if ((e = moe::launch_router(dtype, u, E_gate, gate_bias, T, d, N, K, idx, gate, nullptr, st,
                                want_ranks ? (int32_t*)(ws + L.rank) : nullptr,
                                want_ranks ? (int32_t*)(ws + L.tile_counts) : nullptr,
                                &ranked)) != hipSuccess)
      return hip_fail(e, "router launch");
  }
  const moe::TileTableOut tables = moe::expert_tile_tables(dtype, ar);
  if (moe::gemm1_derives_dispatch(dtype, ar)) {
    // a decode batch: GEMM1 derives the dispatch itself, in every block
    ar.fd.idx = idx;
    ar.fd.counts = (int32_t*)(ws + L.counts);
    ar.fd.offsets = offsets;
    ar.fd.sorted_pair = sorted_pair;
    ar.fd.tt = tables;
  } else if ((s = run_dispatch(idx, T, N, K, (int32_t*)(ws + L.counts), offsets, sorted_pair,
                               (int32_t*)(ws + L.rank), (int32_t*)(ws + L.tile_counts),
                               (int32_t*)(ws + L.tile_base), st, &tables, rec, ranked)) != MOE_OK) {
    return s;
  }
  if ((s = run_experts(dtype, ar, st, true, rec)) != MOE_OK) return s;
  if (side && (e = hipStreamWaitEvent(st, sd->join, 0)) != hipSuccess)
    return hip_fail(e, "shared-expert join");
  if (side) side_lock.unlock();
  {
    StageScope sc(6, st, rec);
    if ((e = moe::launch_combine(dtype, u, a.Y, a.Y_shared, T, d, K, K_s, h, st)) != hipSuccess)
      return hip_fail(e, "combine launch");
  }
  return ok();
}

// ---------------------------------------------------------------- static scratch
// The workspace of moe_layer_forward_static: a device array of the library's
// own (each device holds its copy until the process ends).  Host code never
// uses its name as an address: its device address is looked up once per
// device and kept.
constexpr size_t kScratchBytes = MOE_STATIC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
char* g_scratch_ptr[64] = {nullptr};

// The scratch array's address on the current device (looked up on the first
// call made with that device current).
hipError_t scratch_of_device(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = (char*)ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

namespace moe {
LaunchEvents stage_launch_events() {
  if (!g_scope.active) return LaunchEvents{nullptr, nullptr};
  const LaunchEvents ev{g_scope.launched ? nullptr : g_scope.a, g_scope.b};
  g_scope.launched = true;
  return ev;
}
}  // namespace moe

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

moe_status_t moe_workspace_size(int T, int d, int I, int N, int K, int K_s, int dtype,
                                size_t* bytes) {
  moe_status_t s = check_shapes(T, d, I, N, K, K_s, dtype);
  if (s != MOE_OK) return s;
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = T == 0 ? 0 : make_layout(T, d, I, N, K, K_s, dtype).total;
  return ok();
}

moe_status_t moe_layer_forward(const void* u, const void* E_gate, const void* W_routed,
                               const void* W_shared, int N, int K, int K_s, int T, int d, int I,
                               int dtype, const float* gate_bias, void* h, void* workspace,
                               size_t workspace_bytes, void* stream) {
  moe_status_t s = check_forward(u, E_gate, W_routed, W_shared, N, K, K_s, T, d, I, dtype,
                                 gate_bias, h);
  if (s != MOE_OK || T == 0) return s;
  if ((s = check_ptr("workspace", workspace, true)) != MOE_OK) return s;
  const Layout L = make_layout(T, d, I, N, K, K_s, dtype);
  if (workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_workspace_size()");
  const size_t act = (size_t)T * d * elem_size(dtype);
  if (overlap(h, act, workspace, L.total)) return fail(MOE_ERR_INVALID_ARG, "h overlaps workspace");
  return forward_enqueue(u, E_gate, W_routed, W_shared, N, K, K_s, T, d, I, dtype, gate_bias, h,
                         (char*)workspace, L, (hipStream_t)stream, true);
}

moe_status_t moe_layer_forward_static(const void* u, const void* E_gate, const void* W_routed,
                                      const void* W_shared, int N, int K, int K_s, int T, int d,
                                      int I, int dtype, const float* gate_bias, void* h,
                                      void* stream) {
  moe_status_t s = check_forward(u, E_gate, W_routed, W_shared, N, K, K_s, T, d, I, dtype,
                                 gate_bias, h);
  if (s != MOE_OK || T == 0) return s;
  const Layout L = make_layout(T, d, I, N, K, K_s, dtype);
  if (L.total > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE, "these shapes need " + std::to_string(L.total) +
                                       " bytes of workspace; the static scratch holds " +
                                       std::to_string(kScratchBytes) +
                                       " (use moe_layer_forward with a workspace)");
  char* ws = nullptr;
  hipError_t e = scratch_of_device(&ws);
  if (e != hipSuccess) return hip_fail(e, "static scratch address");
  return forward_enqueue(u, E_gate, W_routed, W_shared, N, K, K_s, T, d, I, dtype, gate_bias, h,
                         ws, L, (hipStream_t)stream, false);
}

moe_status_t moe_route(const void* u, const void* E_gate, const float* gate_bias, int T, int d,
                       int N, int K, int dtype, int32_t* idx, float* gate, float* scores,
                       void* stream) {
  moe_status_t s;
  if ((s = check_dtype(dtype)) != MOE_OK) return s;
  if ((s = check_routing(T, N, K)) != MOE_OK) return s;
  if ((s = check_dim("d", d)) != MOE_OK) return s;
  if (T == 0) return ok();
  if ((s = check_ptr("u", u, true)) != MOE_OK) return s;
  if ((s = check_ptr("E_gate", E_gate, true)) != MOE_OK) return s;
  if ((s = check_ptr("gate_bias", gate_bias, false)) != MOE_OK) return s;
  if ((s = check_ptr("idx", idx, true)) != MOE_OK) return s;
  if ((s = check_ptr("gate", gate, true)) != MOE_OK) return s;
  if ((s = check_ptr("scores", scores, false)) != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  StageScope sc(0, st);
  hipError_t e = moe::launch_router(dtype, u, E_gate, gate_bias, T, d, N, K, idx, gate, scores, st);
  if (e != hipSuccess) return hip_fail(e, "router launch");
  return ok();
}

moe_status_t moe_dispatch_workspace_size(int T, int N, int K, size_t* bytes) {
  moe_status_t s = check_routing(T, N, K);
  if (s != MOE_OK) return s;
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = T == 0 ? 0 : dispatch_ws_bytes(T, N, K);
  return ok();
}

moe_status_t moe_dispatch(const int32_t* idx, int T, int N, int K, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pair, void* workspace,
                          size_t workspace_bytes, void* stream) {
  moe_status_t s = check_routing(T, N, K);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  if ((s = check_ptr("idx", idx, true)) != MOE_OK) return s;
  if ((s = check_ptr("counts", counts, true)) != MOE_OK) return s;
  if ((s = check_ptr("offsets", offsets, true)) != MOE_OK) return s;
  if ((s = check_ptr("sorted_pair", sorted_pair, true)) != MOE_OK) return s;
  if ((s = check_ptr("workspace", workspace, true)) != MOE_OK) return s;
  if (workspace_bytes < dispatch_ws_bytes(T, N, K))
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_dispatch_workspace_size()");
  char* ws = (char*)workspace;
  const size_t nt = (size_t)moe::rank_row(rank_tiles(T));
  int32_t* rank = (int32_t*)ws;
  int32_t* tile_counts = (int32_t*)(ws + align256((size_t)T * K * 4));
  int32_t* tile_base = (int32_t*)((char*)tile_counts + align256(nt * N * 4));
  if ((s = run_dispatch(idx, T, N, K, counts, offsets, sorted_pair, rank, tile_counts, tile_base,
                        (hipStream_t)stream)) != MOE_OK)
    return s;
  return ok();
}

moe_status_t moe_expert_ffn_workspace_size(int T, int N, int K, int K_s, size_t* bytes) {
  moe_status_t s = check_routing(T, N, K);
  if (s != MOE_OK) return s;
  if (K_s < 0 || K_s > 16) return fail(MOE_ERR_INVALID_ARG, "K_s must satisfy 0 <= K_s <= 16");
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = T == 0 ? 0 : expert_ws_bytes(N, K_s);
  return ok();
}

moe_status_t moe_expert_ffn(const void* u, const void* W_routed, const void* W_shared, int T,
                            int d, int I, int N, int K, int K_s, int dtype,
                            const int32_t* offsets, const int32_t* sorted_pair,
                            const float* gate, void* H_routed, void* H_shared, void* Y,
                            void* Y_shared, void* workspace, size_t workspace_bytes,
                            void* stream) {
  moe_status_t s = check_shapes(T, d, I, N, K, K_s, dtype);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  if ((s = check_ptr("u", u, true)) != MOE_OK) return s;
  if ((s = check_ptr("W_routed", W_routed, true)) != MOE_OK) return s;
  if ((s = check_ptr("W_shared", W_shared, K_s > 0)) != MOE_OK) return s;
  if ((s = check_ptr("offsets", offsets, true)) != MOE_OK) return s;
  if ((s = check_ptr("sorted_pair", sorted_pair, true)) != MOE_OK) return s;
  if ((s = check_ptr("gate", gate, true)) != MOE_OK) return s;
  if ((s = check_ptr("H_routed", H_routed, true)) != MOE_OK) return s;
  if ((s = check_ptr("H_shared", H_shared, K_s > 0)) != MOE_OK) return s;
  if ((s = check_ptr("Y", Y, true)) != MOE_OK) return s;
  if ((s = check_ptr("Y_shared", Y_shared, K_s > 0)) != MOE_OK) return s;
  if ((s = check_ptr("workspace", workspace, true)) != MOE_OK) return s;
  if (workspace_bytes < expert_ws_bytes(N, K_s))
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_expert_ffn_workspace_size()");
  moe::ExpertArgs a{};
  a.u = u;
  a.W_routed = W_routed;
  a.W_shared = W_shared;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.gate = gate;
  a.H_routed = H_routed;
  a.H_shared = H_shared;
  a.Y = Y;
  a.Y_shared = Y_shared;
  a.tiles1 = (int32_t*)workspace;
  a.tiles2 = a.tiles1 + (N + K_s + 1);
  a.counters = a.tiles2 + (N + 2);
  a.T = T;
  a.d = d;
  a.I = I;
  a.N = N;
  a.K = K;
  a.K_s = K_s;
  if ((s = run_experts(dtype, a, (hipStream_t)stream)) != MOE_OK) return s;
  return ok();
}

moe_status_t moe_combine(const void* u, const void* Y, const void* Y_shared, int T, int d, int K,
                         int K_s, int dtype, void* h, void* stream) {
  moe_status_t s;
  if ((s = check_dtype(dtype)) != MOE_OK) return s;
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0");
  if (K < 1) return fail(MOE_ERR_INVALID_ARG, "K must be >= 1");
  if (K_s < 0) return fail(MOE_ERR_INVALID_ARG, "K_s must be >= 0");
  if ((s = check_dim("d", d)) != MOE_OK) return s;
  if (T == 0) return ok();
  if ((s = check_ptr("u", u, true)) != MOE_OK) return s;
  if ((s = check_ptr("Y", Y, true)) != MOE_OK) return s;
  if ((s = check_ptr("Y_shared", Y_shared, K_s > 0)) != MOE_OK) return s;
  if ((s = check_ptr("h", h, true)) != MOE_OK) return s;
  StageScope sc(6, (hipStream_t)stream);
  hipError_t e = moe::launch_combine(dtype, u, Y, Y_shared, T, d, K, K_s, h, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return ok();
}

// ---------------------------------------------------------------- backward
namespace {

struct BwdLayout {
  size_t idx, gate, scores, rank, tile_counts, tile_base, counts, offsets, sorted_pair;
  size_t AC, ACs, dP, dPs, dAC, dACs, P, Ps, dY, dX, dXs, dzE, dz, dE_part, ds_pair, slot_of,
      tab, total;
  // pipelined bfloat16 path
  bool pipe;
  size_t XT, dhT, dsp, tabs;
  long long ldx;
};

int pad8(int n) { return (n + 7) & ~7; }

// bfloat16 backward on the pipelined GEMMs unless MOE_BWD_GENERIC=1 asks for
// the generic kernels (the float32 path).
bool bwd_pipe(int dtype) {
  if (dtype != MOE_DTYPE_BF16) return false;
  const char* s = getenv("MOE_BWD_GENERIC");
  return !(s != nullptr && s[0] == '1');
}

BwdLayout make_bwd_layout(int T, int d, int I, int N, int K, int K_s, int dtype) {
  BwdLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  const size_t TK = (size_t)T * K, es = elem_size(dtype), nt = (size_t)moe::rank_row(rank_tiles(T));
  L.pipe = bwd_pipe(dtype);
  const size_t gen = L.pipe ? 0 : 1;  // buffers only the generic path uses
  L.idx = take(TK * 4);
  L.gate = take(TK * 4);
  L.scores = take((size_t)T * N * 4);
  L.rank = take(TK * 4);
  L.tile_counts = take(nt * N * 4);
  L.tile_base = take(nt * N * 4);
  L.counts = take((size_t)N * 4);
  L.offsets = take((size_t)(N + 1) * 4);
  L.sorted_pair = take(TK * 4);
  L.AC = take(gen * TK * 2 * I * 4);
  L.ACs = take(gen * (size_t)T * K_s * 2 * I * 4);
  L.dP = take(TK * I * 4);
  L.dPs = take((size_t)T * K_s * I * 4);
  L.dAC = take(TK * 2 * I * es);
  L.dACs = take((size_t)T * K_s * 2 * I * es);
  L.P = take(TK * I * es);
  L.Ps = take((size_t)T * K_s * I * es);
  L.dY = take(gen * TK * d * es);
  L.dX = take(TK * d * 4);
  L.dXs = take((size_t)K_s * T * d * 4);
  L.dzE = take((size_t)T * pad8(N) * es);
  L.dz = take((size_t)T * N * 4);
  L.dE_part = take((size_t)moe::backward_de_chunks(T) * N * d * 4);
  L.ds_pair = take(TK * 4);
  L.slot_of = take(TK * 4);
  L.tab = take((size_t)(std::max(N + K_s, moe::backward_de_chunks(T)) + 1) * 4);
  if (L.pipe) {
    const long long R = moe::bt_routed_cols(T, K, N), Tp = moe::bt_pad64(T);
    L.ldx = R + Tp;
    L.XT = take((size_t)d * L.ldx * 2);
    L.dhT = take((size_t)d * L.ldx * 2);
    L.dsp = take(TK * ((I + 127) / 128) * 4);
    L.tabs = take((size_t)(moe::bt_tables_ints(N, K_s) + N + 1) * 4);
  }
  L.total = o;
  return L;
}

// The backward's operands beyond the forward's: [da dc] rows (2I wide) and
// 256-row tiles of the transposed token copies (pitch: every padded slot
// column plus the shared experts' tokens).
moe_status_t check_bwd_shapes(int T, int d, int I, int N, int K, int K_s, int dtype) {
  moe_status_t s = check_shapes(T, d, I, N, K, K_s, dtype);
  if (s != MOE_OK) return s;
  const long long es = dtype == MOE_DTYPE_BF16 ? 2 : 4;
  if ((s = check_extent("[da dc] [T*K][2I]", (long long)T * K * 2 * I * es)) != MOE_OK) return s;
  const long long ldx = moe::bt_routed_cols(T, K, N) + moe::bt_pad64(T);
  if ((s = check_extent("a 256-row tile of the transposed tokens", 256LL * ldx * 2)) != MOE_OK)
    return s;
  return MOE_OK;
}

}  // namespace

moe_status_t moe_backward_workspace_size(int T, int d, int I, int N, int K, int K_s, int dtype,
                                         size_t* bytes) {
  moe_status_t s = check_bwd_shapes(T, d, I, N, K, K_s, dtype);
  if (s != MOE_OK) return s;
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = T == 0 ? 0 : make_bwd_layout(T, d, I, N, K, K_s, dtype).total;
  return ok();
}

moe_status_t moe_layer_backward(const void* u, const void* E_gate, const void* W_routed,
                                const void* W_shared, int N, int K, int K_s, int T, int d, int I,
                                int dtype, const float* gate_bias, const void* dh, void* du,
                                float* dE_gate, float* dgate_bias, float* dW_routed,
                                float* dW_shared, void* workspace, size_t workspace_bytes,
                                void* stream) {
  moe_status_t s = check_bwd_shapes(T, d, I, N, K, K_s, dtype);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  if ((s = check_ptr("u", u, true)) != MOE_OK) return s;
  if ((s = check_ptr("E_gate", E_gate, true)) != MOE_OK) return s;
  if ((s = check_ptr("W_routed", W_routed, true)) != MOE_OK) return s;
  if ((s = check_ptr("W_shared", W_shared, K_s > 0)) != MOE_OK) return s;
  if ((s = check_ptr("gate_bias", gate_bias, false)) != MOE_OK) return s;
  if ((s = check_ptr("dh", dh, true)) != MOE_OK) return s;
  if ((s = check_ptr("du", du, true)) != MOE_OK) return s;
  if ((s = check_ptr("dE_gate", dE_gate, true)) != MOE_OK) return s;
  if ((s = check_ptr("dgate_bias", dgate_bias, false)) != MOE_OK) return s;
  if ((s = check_ptr("dW_routed", dW_routed, true)) != MOE_OK) return s;
  if ((s = check_ptr("dW_shared", dW_shared, K_s > 0)) != MOE_OK) return s;
  if ((s = check_ptr("workspace", workspace, true)) != MOE_OK) return s;
  const size_t act = (size_t)T * d * elem_size(dtype);
  if (overlap(du, act, u, act)) return fail(MOE_ERR_INVALID_ARG, "du overlaps u");
  if (overlap(du, act, dh, act)) return fail(MOE_ERR_INVALID_ARG, "du overlaps dh");
  const BwdLayout L = make_bwd_layout(T, d, I, N, K, K_s, dtype);
  if (workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_backward_workspace_size()");
  if (overlap(du, act, workspace, L.total))
    return fail(MOE_ERR_INVALID_ARG, "du overlaps workspace");
  const size_t wr = (size_t)N * 3 * I * d * 4;
  if (overlap(dW_routed, wr, workspace, L.total))
    return fail(MOE_ERR_INVALID_ARG, "dW_routed overlaps workspace");

  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  int32_t* idx = (int32_t*)(ws + L.idx);
  float* gate = (float*)(ws + L.gate);
  float* scores = (float*)(ws + L.scores);
  hipError_t e;
  if ((e = moe::launch_router(dtype, u, E_gate, gate_bias, T, d, N, K, idx, gate, scores, st)) !=
      hipSuccess)
    return hip_fail(e, "router launch");
  int32_t* offsets = (int32_t*)(ws + L.offsets);
  int32_t* sorted_pair = (int32_t*)(ws + L.sorted_pair);
  if ((s = run_dispatch(idx, T, N, K, (int32_t*)(ws + L.counts), offsets, sorted_pair,
                        (int32_t*)(ws + L.rank), (int32_t*)(ws + L.tile_counts),
                        (int32_t*)(ws + L.tile_base), st)) != MOE_OK)
    return s;
  moe::BwdArgs a{};
  a.u = u;
  a.dh = dh;
  a.E_gate = E_gate;
  a.W_routed = W_routed;
  a.W_shared = W_shared;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.AC = (float*)(ws + L.AC);
  a.ACs = (float*)(ws + L.ACs);
  a.dP = (float*)(ws + L.dP);
  a.dPs = (float*)(ws + L.dPs);
  a.dAC = ws + L.dAC;
  a.dACs = ws + L.dACs;
  a.P = ws + L.P;
  a.Ps = ws + L.Ps;
  a.dY = ws + L.dY;
  a.dX = (float*)(ws + L.dX);
  a.dXs = (float*)(ws + L.dXs);
  a.dzE = ws + L.dzE;
  a.dE_part = (float*)(ws + L.dE_part);
  a.dE_gate = dE_gate;
  a.dW_routed = dW_routed;
  a.dW_shared = dW_shared;
  a.T = T;
  a.d = d;
  a.I = I;
  a.N = N;
  a.K = K;
  a.K_s = K_s;
  a.NP = pad8(N);
  a.gate = gate;
  int32_t* tabs = nullptr;
  if (L.pipe) {
    tabs = (int32_t*)(ws + L.tabs);
    a.XT = ws + L.XT;
    a.dhT = ws + L.dhT;
    a.dsp = (float*)(ws + L.dsp);
    a.pcol = tabs + moe::bt_tables_ints(N, K_s);
    a.ldx = L.ldx;
    a.Tp = moe::bt_pad64(T);
  }
  if ((e = moe::launch_backward(dtype, a, gate, scores, idx, (float*)(ws + L.ds_pair),
                                (int32_t*)(ws + L.slot_of), (float*)(ws + L.dz),
                                dgate_bias, du,
                                (int32_t*)(ws + L.tab), tabs, st)) != hipSuccess)
    return hip_fail(e, "backward launch");
  return ok();
}

moe_status_t moe_balance_workspace_size(int T, int N, size_t* bytes) {
  if (T < 1) return fail(MOE_ERR_INVALID_ARG, "balance statistics need T >= 1");
  if (N < 1) return fail(MOE_ERR_INVALID_ARG, "N must be >= 1");
  if (N > 256) return fail(MOE_ERR_UNSUPPORTED, "N > 256 routed experts is not supported");
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = moe::balance_workspace_bytes(T, N);
  return ok();
}

moe_status_t moe_balance_stats(const float* scores, const int32_t* idx, int T, int N, int K,
                               const int32_t* group_of, int D, float alpha1, float alpha2,
                               float* f, float* P, float* f_dev, float* P_dev, float* losses,
                               void* workspace, size_t workspace_bytes, void* stream) {
  moe_status_t s = check_routing(T, N, K);
  if (s != MOE_OK) return s;
  if (T < 1) return fail(MOE_ERR_INVALID_ARG, "balance statistics need T >= 1");
  moe::BalanceGroups groups{};
  if (group_of != nullptr) {
    if (D < 1 || D > N) return fail(MOE_ERR_INVALID_ARG, "D must satisfy 1 <= D <= N");
    std::vector<int> size(D, 0);
    for (int i = 0; i < N; ++i) {
      if (group_of[i] < 0 || group_of[i] >= D)
        return fail(MOE_ERR_INVALID_ARG, "group_of[" + std::to_string(i) + "] is outside [0, D)");
      ++size[group_of[i]];
      groups.of[i] = group_of[i];
    }
    for (int g = 0; g < D; ++g)
      if (size[g] == 0)
        return fail(MOE_ERR_INVALID_ARG, "device group " + std::to_string(g) + " has no expert");
    groups.D = D;
  }
  if ((s = check_ptr("scores", scores, true)) != MOE_OK) return s;
  if ((s = check_ptr("idx", idx, true)) != MOE_OK) return s;
  if ((s = check_ptr("f", f, true)) != MOE_OK) return s;
  if ((s = check_ptr("P", P, true)) != MOE_OK) return s;
  if ((s = check_ptr("f_dev", f_dev, group_of != nullptr)) != MOE_OK) return s;
  if ((s = check_ptr("P_dev", P_dev, group_of != nullptr)) != MOE_OK) return s;
  if ((s = check_ptr("losses", losses, true)) != MOE_OK) return s;
  if ((s = check_ptr("workspace", workspace, true)) != MOE_OK) return s;
  if (workspace_bytes < moe::balance_workspace_bytes(T, N))
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_balance_workspace_size()");
  hipError_t e = moe::launch_balance(scores, idx, T, N, K, groups, alpha1, alpha2, f, P, f_dev,
                                     P_dev, losses, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "balance statistics launch");
  return ok();
}

moe_status_t moe_timing_enable(int on) {
  std::lock_guard<std::mutex> g(g_timing.mu);
  g_timing.on = on != 0;
  return ok();
}

moe_status_t moe_timing_stages(unsigned mask) {
  std::lock_guard<std::mutex> g(g_timing.mu);
  g_timing.mask = mask;
  return ok();
}

moe_status_t moe_timing_read(double* ms_per_stage, int* launches_per_stage) {
  if (ms_per_stage == nullptr || launches_per_stage == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "output arrays are NULL");
  std::lock_guard<std::mutex> g(g_timing.mu);
  for (int i = 0; i < MOE_NUM_STAGES; ++i) {
    ms_per_stage[i] = 0.0;
    launches_per_stage[i] = 0;
  }
  moe_status_t st = MOE_OK;
  for (auto& r : g_timing.recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) {
      st = hip_fail(e, "timing event");
    } else if (r.stage >= 0 && r.stage < MOE_NUM_STAGES) {
      ms_per_stage[r.stage] += ms;
      launches_per_stage[r.stage] += 1;
    }
    g_timing.pool.push_back(r.a);
    g_timing.pool.push_back(r.b);
  }
  g_timing.recs.clear();
  return st == MOE_OK ? ok() : st;
}

}  // extern "C"
