/*
 * moe.h -- C ABI of the MI355X (gfx950) DeepSeekMoE layer (forward and backward).
 *
 * The operation (DeepSeekMoE paper summary, papercache.org, sec. 3.2 "Shared
 * Expert Isolation", full layer equation; the conventional top-K layer of
 * sec. A3 is the case K_s = 0):
 *
 *   s_{i,t} = Softmax_i(u_t . e_i + b_i)       over the N routed experts
 *   g_{i,t} = s_{i,t} for the K largest s_{.,t} of token t (ties: lower i), else 0
 *   h_t     = u_t + sum_{j<K_s} FFN_shared_j(u_t) + sum_{i<N} g_{i,t} FFN_routed_i(u_t)
 *   FFN(x)  = W_down (SiLU(W_gate x) * (W_up x)),   SiLU(a) = a / (1 + e^-a)
 *
 * In the paper's notation N = mN - K_s routed experts, K = mK - K_s kept per
 * token, and each expert's intermediate size I is the 1/m slice of sec. 3.1.
 * The gates are not renormalised.  b is an optional per-expert logit bias.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers unless stated; the caller owns
 *    every buffer.  The library keeps no pointer after a call returns and
 *    never allocates or frees device memory on these paths.
 *  - Row-major layouts.  dtype selects the storage type of u, E_gate, the
 *    weights, h and the intermediate H / Y buffers: MOE_DTYPE_F32 (float) or
 *    MOE_DTYPE_BF16 (bfloat16).  Router logits, softmax, gates and every
 *    accumulation are float32 in both cases.
 *  - One expert's weight block (W_routed holds N of them back to back,
 *    W_shared K_s of them): W_gate [I][d], then W_up [I][d], then
 *    W_down [d][I], contiguous, 3*I*d elements.
 *  - stream is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued asynchronously; MOE_OK means "enqueued".  A fault inside a
 *    kernel surfaces at the caller's next synchronisation.  No entry point
 *    synchronises with the host.
 *  - Validation runs before any HIP call.  On error nothing is enqueued, the
 *    status says why and moe_last_error() gives a message.
 *  - Limits: T >= 0; 1 <= K <= N <= 256; 0 <= K_s <= 16; d and I positive
 *    multiples of 64; device pointers 16-byte aligned; inputs finite.
 *    T = 0 is a valid empty call that enqueues nothing.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype_t;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* a size, a count or a pointer is wrong          */
  MOE_ERR_UNSUPPORTED = 2,  /* valid input outside the implemented limits     */
  MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required     */
  MOE_ERR_ALIGNMENT = 4,    /* a pointer is not 16-byte aligned               */
  MOE_ERR_HIP = 5           /* a HIP launch call failed                       */
} moe_status_t;

/* Message of the last failed call on this thread ("" if none).  Valid until
 * the next call into the library from the same thread. */
const char* moe_last_error(void);

/* Bytes of device workspace moe_layer_forward needs for these shapes.
 * Writes the size to *bytes (host pointer). */
moe_status_t moe_workspace_size(int T, int d, int I, int N, int K, int K_s, int dtype,
                                size_t* bytes);

/* The whole layer forward, h = MoE(u) as above (sec. 3.2 layer equation).
 *   u         [T][d]            dtype
 *   E_gate    [N][d]            dtype   gate vector (centroid) e_i per routed expert
 *   W_routed  N weight blocks   dtype
 *   W_shared  K_s weight blocks dtype   may be NULL iff K_s == 0
 *   gate_bias [N] float or NULL         added to the logits before the softmax
 *   h         [T][d]            dtype   output; must not overlap any input
 *   workspace device buffer of at least moe_workspace_size() bytes
 * Routing ties are broken towards the lower expert index; each token's K
 * routed contributions are summed in descending-score order, after the
 * shared experts' sum, in float32, and h is rounded once.
 * With MOE_SHARED_SIDE=1 in the environment, K_s > 0 and T <= 128, the
 * shared experts' GEMMs run on a stream the library owns (one per device,
 * default priority), forked from `stream` by an event before the router and
 * joined back into it before the combine: everything the call does is still
 * ordered on `stream` for the caller, and the result is the same bits as
 * without it, which keeps them on `stream`. */
moe_status_t moe_layer_forward(const void* u, const void* E_gate, const void* W_routed,
                               const void* W_shared, int N, int K, int K_s, int T, int d,
                               int I, int dtype, const float* gate_bias, void* h,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ---- allocation-free forward ----
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same kernels and results as moe_layer_forward (the same
 * bits for the same inputs), with the workspace taken from a static device
 * array of MOE_STATIC_SCRATCH_BYTES that the library holds on every device it
 * runs on until the process ends (its address is looked up on the first call
 * made with that device current).  No hipMalloc, hipFree, stream, event or
 * other allocating call is made; timing events and the MOE_SHARED_SIDE side
 * stream are not used.
 * Limits: shapes whose moe_workspace_size() exceeds MOE_STATIC_SCRATCH_BYTES
 * are refused with MOE_ERR_WORKSPACE (at d = 2048, I = 1408, 64 routed
 * experts, top-6 and 2 shared experts: up to about 1300 tokens).
 * Every call on a device shares that device's one array: calls that overlap
 * on one device (two streams, or two host threads) race and give undefined
 * results; calls ordered on one stream are safe.  Nothing in the array needs
 * to start at zero (each call writes every region before reading it). */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status_t moe_layer_forward_static(const void* u, const void* E_gate, const void* W_routed,
                                      const void* W_shared, int N, int K, int K_s, int T, int d,
                                      int I, int dtype, const float* gate_bias, void* h,
                                      void* stream);

/* ---- stage entry points: the kernels moe_layer_forward launches, one stage
 * at a time, for callers that want the intermediate results. ---- */

/* Router (sec. A3 / 3.2 affinity and gate equations): logits z = u E_gate^T
 * (+ gate_bias) in float32, softmax over the N routed experts, top-K.
 *   idx    [T][K] int32   expert ids, descending score, ties lower id first
 *   gate   [T][K] float   the kept softmax values (not renormalised)
 *   scores [T][N] float   all softmax values, or NULL */
moe_status_t moe_route(const void* u, const void* E_gate, const float* gate_bias, int T, int d,
                       int N, int K, int dtype, int32_t* idx, float* gate, float* scores,
                       void* stream);

/* Workspace bytes moe_dispatch needs (per-tile counters). */
moe_status_t moe_dispatch_workspace_size(int T, int N, int K, size_t* bytes);

/* Group the (token, k) pairs by expert (the tokens each expert computes,
 * sec. A3: token t is computed only by its K experts).  Pair p = t*K + k.
 *   idx         [T][K] int32 input, each row holding K distinct ids in [0, N)
 *   counts      [N]    int32 pairs per expert
 *   offsets     [N+1]  int32 exclusive prefix sum of counts
 *   sorted_pair [T*K]  int32 pair ids grouped by expert, ascending pair id
 *                            (hence ascending token) within each expert */
moe_status_t moe_dispatch(const int32_t* idx, int T, int N, int K, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pair, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Workspace bytes moe_expert_ffn needs (tile tables). */
moe_status_t moe_expert_ffn_workspace_size(int T, int N, int K, int K_s, size_t* bytes);

/* The expert FFNs on grouped tokens (SwiGLU; gate applied in the output).
 * Inputs: offsets, sorted_pair from moe_dispatch; gate [T][K] from moe_route.
 *   H_routed [T*K][I]     dtype  SiLU(W_gate x)*(W_up x), row = slot in sorted order
 *   H_shared [T][K_s*I]   dtype  the same for the shared experts (expert j at
 *                                columns j*I ..), NULL iff K_s == 0
 *   Y        [T*K][d]     dtype  row p = t*K+k: g_{t,k} * FFN_{idx[t][k]}(u_t)
 *   Y_shared [T][d]       dtype  sum over shared experts of FFN_j(u_t), NULL iff K_s == 0 */
moe_status_t moe_expert_ffn(const void* u, const void* W_routed, const void* W_shared, int T,
                            int d, int I, int N, int K, int K_s, int dtype,
                            const int32_t* offsets, const int32_t* sorted_pair,
                            const float* gate, void* H_routed, void* H_shared, void* Y,
                            void* Y_shared, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Combine with the residual (sec. 3.2 layer equation):
 *   h_t = u_t + Y_shared_t + sum_{k<K} Y_{t*K+k}, float32 sum in that order,
 *   rounded once to dtype.  Y_shared may be NULL iff K_s == 0. */
moe_status_t moe_combine(const void* u, const void* Y, const void* Y_shared, int T, int d,
                         int K, int K_s, int dtype, void* h, void* stream);

/* ---- balance statistics (beside the forward path) ----
 * DeepSeekMoE paper summary, papercache.org, sec. 3.3 (expert-level and
 * device-level balance losses), over one batch of T >= 1 tokens:
 *   f_i = N / (K T) * #{t : token t selects routed expert i}
 *   P_i = (1/T) * sum_t s_{i,t}
 *   L_ExpBal = alpha1 * sum_i f_i P_i
 *   f'_g = mean of f_i over the experts of device group g
 *   P'_g = sum of P_i over the experts of device group g
 *   L_DevBal = alpha2 * sum_g f'_g P'_g
 * (N, K are the paper's N' = mN - K_s and K' = mK - K_s.)
 * Inputs: scores [T][N] float32 (the softmax s from moe_route), idx [T][K]
 * int32 (entries outside [0, N) are not counted).
 * group_of is a HOST array of N ints giving each routed expert's group in
 * [0, D), every group non-empty; or NULL (then D is ignored, f_dev / P_dev may
 * be NULL and L_DevBal is written as 0).
 * Outputs (device, float32): f [N], P [N], f_dev [D], P_dev [D],
 * losses [2] = {L_ExpBal, L_DevBal}.  Sums are formed in float64 in a fixed
 * order, so repeated calls give identical bits.
 * Workspace: moe_balance_workspace_size() bytes (partial sums). */
moe_status_t moe_balance_workspace_size(int T, int N, size_t* bytes);
moe_status_t moe_balance_stats(const float* scores, const int32_t* idx, int T, int N, int K,
                               const int32_t* group_of, int D, float alpha1, float alpha2,
                               float* f, float* P, float* f_dev, float* P_dev, float* losses,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ---- layer backward ----
 * Gradients of the scalar sum_t dh_t . h_t for h = moe_layer_forward(u, ...),
 * by the chain rule through the sec. 3.2 layer equation (DeepSeekMoE paper
 * summary, papercache.org; the pages train the layer but print no backward
 * formulas), with the top-K set of each token held fixed -- the selection is
 * piecewise constant in the scores, so it contributes no derivative:
 *   per expert slot (x = u_t, a = W_gate x, c = W_up x, p = SiLU(a) c,
 *   dy = g dh for a routed slot, dh for a shared one):
 *     dW_down += dy p^T, dp = W_down^T dy, da = dp c SiLU'(a), dc = dp SiLU(a),
 *     dW_gate += da x^T, dW_up += dc x^T, du_t += W_gate^T da + W_up^T dc;
 *   routed gate: ds_{i,t} = dh_t . FFN_i(u_t) for i in the top-K, else 0;
 *   softmax:     dz_{i,t} = s_{i,t} (ds_{i,t} - sum_j s_{j,t} ds_{j,t});
 *   router:      du_t += E_gate^T dz_t, dE_gate += dz_t u_t^T, db += dz_t;
 *   residual:    du_t += dh_t.
 * The forward's routing is recomputed from u (same kernels, same bits).
 * Inputs: u, E_gate, W_routed, W_shared, gate_bias as for moe_layer_forward;
 *   dh [T][d] dtype (upstream gradient).
 * Outputs (device):
 *   du         [T][d]             dtype    must not overlap u or dh
 *   dE_gate    [N][d]             float32
 *   dgate_bias [N]                float32  may be NULL (then not written;
 *                                          gate_bias may still be given)
 *   dW_routed  [N][3*I*d]         float32  in the weights' block layout
 *   dW_shared  [K_s][3*I*d]       float32  NULL iff K_s == 0
 * Intermediates: dP and the softmax gradient in float32; [da dc], g p, the
 * per-slot dx rows and the operands of the router-gradient product in dtype
 * (bfloat16: rounded once each); products accumulate in float32.  Experts
 * that no token selects get zero weight gradients.  Every sum has a fixed
 * order: repeated calls give identical bits.
 * T = 0 writes nothing (the gradients of an empty batch are zero).
 * Workspace: moe_backward_workspace_size() bytes, 256-byte aligned (for
 * T = 8192, d = 2048, I = 1408, N = 64, K = 6, K_s = 2: about 2.0 GB in
 * bfloat16, 3.2 GB in float32). */
moe_status_t moe_backward_workspace_size(int T, int d, int I, int N, int K, int K_s, int dtype,
                                         size_t* bytes);
moe_status_t moe_layer_backward(const void* u, const void* E_gate, const void* W_routed,
                                const void* W_shared, int N, int K, int K_s, int T, int d, int I,
                                int dtype, const float* gate_bias, const void* dh, void* du,
                                float* dE_gate, float* dgate_bias, float* dW_routed,
                                float* dW_shared, void* workspace, size_t workspace_bytes,
                                void* stream);

/* ---- per-stage timing (for profiling; off by default) ----
 * When enabled, moe_layer_forward records a HIP event pair around each of its
 * kernel stages on the stream it was given.  moe_timing_read() waits for
 * those events, writes the summed milliseconds and launch counts per stage
 * (host arrays of MOE_NUM_STAGES entries), and clears them. */
#define MOE_NUM_STAGES 7
/* stage order: 0 router, 1 tile ranks, 2 dispatch scan, 3 scatter,
 *              4 expert GEMM1 (gate/up + SwiGLU), 5 expert GEMM2 (down x gate),
 *              6 combine.  The tile-table kernel is counted in stage 4; a batch
 *              of at most 64 tokens runs the whole dispatch as stage 1. */
moe_status_t moe_timing_enable(int on);
moe_status_t moe_timing_read(double* ms_per_stage, int* launches_per_stage);
/* Stages that get an event pair while timing is on: bit s selects stage s
 * (default all).  Fewer events disturb the timed launches less (each pair
 * separates back-to-back kernels on the stream). */
moe_status_t moe_timing_stages(unsigned mask);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
