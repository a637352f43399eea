"""Shared helpers of the GPU parity tests: upload seeded inputs, compare with the oracle.

Every expected value comes from the oracle fed with the seeded inputs (or
with the oracle's own intermediate results); nothing the GPU computes is fed
back into the oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import moe_inputs
import oracle

BF16_TOL = 2e-2     # max|dh| <= 2e-2 * max|h_ref| for bfloat16 storage
F32_TOL = 1e-4      # max|dh| <= 1e-4 * max|h_ref| for float32 storage
TIE_EPS = 1e-6      # routing must be exact where the K-th vs (K+1)-th score margin exceeds this
GATE_RTOL = 1e-5    # kept gates within this relative error of the oracle's scores


def say(msg: str):
    """Name the case before a GPU step (a fault ends the process without a traceback)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def tol_for(w) -> float:
    return BF16_TOL if w.dtype == "bf16" else F32_TOL


def to_device(raw: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Storage-form array (float32 or uint16 bf16 bits) -> device tensor of the storage type."""
    t = torch.from_numpy(np.ascontiguousarray(raw))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(device)


def device_f32(x: torch.Tensor) -> np.ndarray:
    return x.float().cpu().numpy()


class Uploaded:
    """Inputs of one workload on the GPU, plus host views for the oracle."""

    def __init__(self, inp: moe_inputs.MoEInputs, device="cuda"):
        w = inp.w
        self.inp, self.w = inp, w
        self.u = to_device(inp.u_raw(), w.dtype, device)
        self.E = to_device(inp.E_gate_raw(), w.dtype, device)
        self.W_routed_raw = inp.routed_all_raw()
        self.W_shared_raw = inp.shared_all_raw()
        self.W_routed = to_device(self.W_routed_raw, w.dtype, device)
        self.W_shared = to_device(self.W_shared_raw, w.dtype, device) if w.K_s > 0 else None
        b = inp.gate_bias()
        self.bias = None if b is None else torch.from_numpy(b).to(device)

    def _f32(self, raw):
        return moe_inputs.bf16_bits_to_f32(raw) if self.w.dtype == "bf16" else raw

    def routed(self, e):
        """(W_gate, W_up, W_down) of routed expert e as float32 (same values the GPU holds)."""
        return self.inp.split_block(self._f32(self.W_routed_raw[e]))

    def shared(self, j):
        return self.inp.split_block(self._f32(self.W_shared_raw[j]))


def admissible_set(s_row: np.ndarray, K: int, chosen, eps: float = TIE_EPS) -> bool:
    """Whether `chosen` (K distinct expert ids) is a correct top-K of the float64 scores s_row
    in finite precision.  With s_K the K-th largest score: every expert scoring above
    s_K + eps is chosen, no chosen expert scores below s_K - eps (so any near-tie group at
    the boundary, of any size, may be split either way), and exact ties go to the lower
    index (exactly K gates are non-zero, [DSMoE] A3): an expert is chosen only if every
    lower-indexed expert with the same score is chosen too."""
    chosen = [int(i) for i in chosen]
    if len(set(chosen)) != K:
        return False
    sK = np.sort(s_row)[::-1][K - 1]
    cs = set(chosen)
    if any(i not in cs for i in np.nonzero(s_row > sK + eps)[0]):
        return False
    if any(s_row[i] < sK - eps for i in chosen):
        return False
    for i in chosen:
        if any(j not in cs for j in np.nonzero(s_row[:i] == s_row[i])[0]):
            return False
    return True


def check_routing(idx_gpu: np.ndarray, gate_gpu: np.ndarray, s_ref: np.ndarray, K: int,
                  gate_rtol: float = GATE_RTOL):
    """Routing parity.  Returns (tokens whose GPU set differs from the oracle's,
    {t: (GPU set, oracle scores of it)} for those tokens).

    * tokens with margin > TIE_EPS: the GPU index set equals the oracle's, and the
      order equals it wherever adjacent kept scores differ by more than TIE_EPS;
    * exact ties (margin 0): the oracle's set (lower index), never the other one;
    * adjacent kept experts with exactly equal scores are in ascending index order;
    * every kept gate is within GATE_RTOL of the oracle's score of that expert;
    * other near-tie tokens: the GPU set is admissible (admissible_set).
    """
    idx_ref, g_ref, margin = oracle.top_k_gates(s_ref, K)
    T = s_ref.shape[0]
    assert idx_gpu.shape == (T, K)
    assert np.all((idx_gpu >= 0) & (idx_gpu < s_ref.shape[1]))
    for t in range(T):
        assert len(set(idx_gpu[t].tolist())) == K, f"token {t}: repeated expert"
    same_set = np.all(np.sort(idx_gpu, axis=1) == np.sort(idx_ref, axis=1), axis=1)
    clear = margin > TIE_EPS
    bad = np.nonzero(clear & ~same_set)[0]
    assert bad.size == 0, f"routing differs on clear-margin tokens {bad[:10]}"
    bad = np.nonzero((margin == 0) & ~same_set)[0]
    assert bad.size == 0, f"exact tie not broken towards the lower index on tokens {bad[:10]}"
    # order where adjacent kept scores are separated
    gaps = -np.diff(g_ref, axis=1) > TIE_EPS
    for t in np.nonzero(clear)[0]:
        for k in range(K):
            left_ok = k == 0 or gaps[t, k - 1]
            right_ok = k == K - 1 or gaps[t, k]
            if left_ok and right_ok:
                assert idx_gpu[t, k] == idx_ref[t, k], f"token {t} slot {k}: order differs"
    s_at = np.take_along_axis(s_ref, idx_gpu.astype(np.int64), axis=1)
    eq = s_at[:, 1:] == s_at[:, :-1]
    bad = np.nonzero(np.any(eq & (idx_gpu[:, 1:] < idx_gpu[:, :-1]), axis=1))[0]
    assert bad.size == 0, f"equal kept scores not in ascending index order on tokens {bad[:10]}"
    rel = np.abs(gate_gpu - s_at) / np.maximum(s_at, 1e-30)
    assert rel.max() <= gate_rtol, f"gate error {rel.max():.3e}"
    differing = np.nonzero(~same_set)[0]
    alts = {}
    for t in differing:
        assert admissible_set(s_ref[t], K, idx_gpu[t]), f"token {t}: GPU set is not admissible"
        order = np.argsort(-s_at[t], kind="stable")
        sel = idx_gpu[t][order].astype(np.int64)
        alts[int(t)] = (sel, s_ref[t, sel])
    return differing, alts


def reference_h(up: Uploaded, tokens=None):
    """Oracle h (float64) for `tokens` (all if None) and its routing info."""
    w = up.w
    inp = up.inp
    return oracle.moe_forward_tokens(inp.u_f32(), inp.E_gate_f32(), up.routed, up.shared,
                                     w.N, w.K, w.K_s, inp.gate_bias(), tokens)


def check_h(h_gpu: np.ndarray, h_ref: np.ndarray, u: np.ndarray, tol: float, dtype: str,
            K: int, label: str = ""):
    """End-to-end bar: max|dh| <= tol * max|h_ref|.  Also the MoE delta h - u, to tol of its
    own scale plus what the output's float32 sum and final rounding may add (K + 2 terms of
    size up to |u| and max|h_ref - u|; one ulp of bf16 when stored in bf16)."""
    err = np.abs(h_gpu.astype(np.float64) - h_ref)
    scale = np.abs(h_ref).max()
    assert err.max() <= tol * scale, f"{label} max|dh| {err.max():.3e} > {tol} * {scale:.3e}"
    delta_scale = np.abs(h_ref - u).max()
    rounding = (K + 1) * 2.0 ** -24 * (np.abs(u) + (K + 1) * delta_scale)
    if dtype == "bf16":
        rounding = rounding + np.exp2(np.floor(np.log2(np.maximum(np.abs(h_ref), 1e-30))) - 7)
    assert np.all(err <= tol * delta_scale + rounding), \
        f"{label} MoE delta error {(err - rounding).max():.3e} > {tol} * {delta_scale:.3e}"
    return err.max() / scale


# Small workloads (several tiles, ragged tails, degenerate cases) shared by the
# forward and backward parity tests.
SMALL = {
    "ragged_f32": dict(T=300, d=256, N=20, K=5, K_s=2, I=192, dtype="f32"),
    "ragged_bf16": dict(T=300, d=256, N=20, K=5, K_s=2, I=192, dtype="bf16"),
    "no_shared_bf16": dict(T=200, d=128, N=8, K=2, K_s=0, I=128, dtype="bf16"),
    "k_equals_n_f32": dict(T=70, d=64, N=6, K=6, K_s=1, I=64, dtype="f32"),
    "one_token_bf16": dict(T=1, d=128, N=16, K=4, K_s=1, I=128, dtype="bf16"),
    "n63_bf16": dict(T=513, d=320, N=63, K=7, K_s=1, I=128, dtype="bf16"),
    "n256_bf16": dict(T=130, d=128, N=256, K=8, K_s=3, I=64, dtype="bf16"),
    "n1_f32": dict(T=33, d=64, N=1, K=1, K_s=0, I=64, dtype="f32"),
    "wide_tokens_bf16": dict(T=2050, d=512, N=16, K=4, K_s=1, I=256, dtype="bf16"),
    # ends of the granularity sweep (conventional top-2 and 8x finer experts with a
    # shared one) at a reduced size: I0 = 4096, d = 128
    "gran_m1_ks0_bf16": dict(T=300, d=128, N=16, K=2, K_s=0, I=4096, dtype="bf16", seed=1101),
    "gran_m8_ks1_bf16": dict(T=300, d=128, N=127, K=15, K_s=1, I=512, dtype="bf16", seed=1181),
    # the ping-pong GEMMs (d, I >= 192): ragged expert tails, partial last n-tiles of
    # both GEMMs (I = 320: 3 GEMM1 tiles of 128 columns, the last half full; d = 448:
    # 2 GEMM2 tiles of 256, the last 192 wide), an odd k-step count (I / 64 = 5), two
    # shared experts whose down projections cross W_down blocks inside one contraction
    "pp_ragged_bf16": dict(T=700, d=448, N=12, K=3, K_s=2, I=320, dtype="bf16", seed=1301),
    # decode-sized batches (the one-block-per-token router): many experts, a ragged
    # expert count, float32
    "decode_n256_bf16": dict(T=96, d=256, N=256, K=8, K_s=1, I=128, dtype="bf16", seed=1201),
    "decode_n200_f32": dict(T=100, d=192, N=200, K=5, K_s=0, I=64, dtype="f32", seed=1202),
    # batches of at most 64 tokens: GEMM1 derives the dispatch itself (at most 1024
    # pairs; 256 experts are four rounds of the wavefront's expert loop, two shared
    # experts), and past 1024 pairs the one-launch dispatch (K = 20: ids past the 16
    # held in registers)
    "decode64_n256_bf16": dict(T=64, d=256, N=256, K=8, K_s=2, I=128, dtype="bf16", seed=1203),
    "decode64_k20_bf16": dict(T=64, d=128, N=64, K=20, K_s=1, I=128, dtype="bf16", seed=1204),
    # decode batches with a model width that is not a multiple of 128 (six 32-column
    # GEMM2 groups, the one-shared-expert GEMM2 on the long-run kernel) and with three
    # shared experts (three shared virtual experts in GEMM1, GEMM2 on the short-run
    # kernel)
    "decode_d192_bf16": dict(T=40, d=192, N=24, K=3, K_s=1, I=192, dtype="bf16", seed=1205),
    "decode_ks3_bf16": dict(T=48, d=128, N=32, K=4, K_s=3, I=64, dtype="bf16", seed=1206),
    # a decode GEMM2 neither streaming kernel takes (d = 320, two shared experts): the
    # register-staged kernel in bf16
    "decode_reg_bf16": dict(T=24, d=320, N=16, K=2, K_s=2, I=128, dtype="bf16", seed=1207),
    # the two routers' boundary: 128 tokens (the last batch routed one block per token)
    # and 129 (the tiled router, its last 32-token block holding one token)
    "t128_bf16": dict(T=128, d=128, N=32, K=4, K_s=1, I=64, dtype="bf16", seed=1208),
    "t129_f32": dict(T=129, d=64, N=8, K=2, K_s=1, I=64, dtype="f32", seed=1209),
    # a wide model (d = 7168): token rows too long for the long-run streaming kernel
    # (decode batch: the short-run kernels), 112 k-steps per pipelined GEMM1 tile; weights
    # at sigma = 0.015 as the pages' widest layer (0.08 would give logits of std ~7, far
    # from any trained router)
    "wide_d_decode_bf16": dict(T=16, d=7168, N=8, K=2, K_s=1, I=256, dtype="bf16", seed=1210,
                               sigma=0.015),
    "wide_d_bf16": dict(T=300, d=7168, N=8, K=2, K_s=1, I=256, dtype="bf16", seed=1211,
                        sigma=0.015),
    # the most shared experts the ABI takes (16), each I = 64: the pipelined GEMM2's
    # shared tiles change W_down block at every k-step; the decode GEMM1 has 32 virtual
    # experts
    "ks16_bf16": dict(T=300, d=128, N=16, K=2, K_s=16, I=64, dtype="bf16", seed=1212),
    "ks16_decode_bf16": dict(T=40, d=128, N=16, K=2, K_s=16, I=64, dtype="bf16", seed=1213),
    # every token to every routed expert (K = N = 32): in a decode batch exactly the 1024
    # pairs GEMM1 derives the dispatch of itself; at 96 tokens the pipelined GEMMs
    "k_equals_n_decode_bf16": dict(T=32, d=128, N=32, K=32, K_s=1, I=64, dtype="bf16",
                                   seed=1214),
    "k_equals_n_bf16": dict(T=96, d=128, N=32, K=32, K_s=0, I=64, dtype="bf16", seed=1215),
    # the narrowest model (d = 64) in bf16: one real k-step per GEMM1 tile (padded with a
    # zero one), a GEMM2 n-tile a quarter full; and its decode batch on the long-run kernels
    "d64_bf16": dict(T=600, d=64, N=4, K=2, K_s=1, I=64, dtype="bf16", seed=1216),
    "d64_decode_bf16": dict(T=100, d=64, N=8, K=2, K_s=1, I=64, dtype="bf16", seed=1217),
}


def small_inputs(name):
    kw = dict(SMALL[name])
    seed = kw.pop("seed", None)
    sigma = kw.pop("sigma", 0.08)
    if seed is None:
        seed = 1000 + sorted(k for k in SMALL if "seed" not in SMALL[k]).index(name)
    return moe_inputs.custom(**kw, sigma=sigma, seed=seed, name=name)
