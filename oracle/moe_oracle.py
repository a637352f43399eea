"""CPU oracle of the DeepSeekMoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The GPU path never calls it, and it shares no code with
the GPU path: it is plain NumPy in float64, written from the method's
defining equations, slow and literal on purpose.

Source of every equation: the papercache.org summary of "DeepSeekMoE: Towards
Ultimate Expert Specialization in Mixture-of-Experts Language Models"
(cited below as [DSMoE]):

* A3 (background), conventional MoE layer: h_t = sum_i g_{i,t} FFN_i(u_t) + u_t,
  g_{i,t} = s_{i,t} if s_{i,t} is among the top-K affinities of token t, else 0,
  s_{i,t} = Softmax_i(u_t^T e_i); exactly K of the N gates are non-zero.
* sec. 3.1, fine-grained segmentation: the same formula over mN experts with
  mK kept; each small expert is one 1/m slice of an FFN's intermediate width.
* sec. 3.2, shared-expert isolation (the full layer):
  h_t = sum_{shared} FFN_i(u_t) + sum_{routed} g_{i,t} FFN_i(u_t) + u_t,
  top-(mK - K_s) among the routed experts; shared experts take coefficient 1
  regardless of the router.
* sec. 3.3, expert- and device-level balance losses (forward statistics).

The expert FFN is a SwiGLU FFN (Swish-gated linear unit, as the dtcms.com
notes "DeepSeek LLM和DeepSeek Moe解读", section on the DeepSeek LLM model
structure, state for DeepSeek's blocks):
FFN(x) = W_down (SiLU(W_gate x) * (W_up x)), SiLU(a) = a / (1 + e^-a), no biases.

Readings taken where the pages are silent or ambiguous:
* the softmax runs over the routed experts only (shared experts have no
  centroid and no gate);
* the kept gates are the softmax values themselves, not renormalised;
* exactly K experts are kept; equal scores are ordered lower index first;
* an optional per-expert bias is added to the logits before the softmax.

Every function here is pinned by tests/test_oracle_pins.py against closed
forms, hand-computed values, brute force and the invariants the pages state.
"""
from __future__ import annotations

import itertools

import numpy as np

__all__ = [
    "affinity_logits", "affinity_scores", "top_k_gates", "swiglu_ffn",
    "moe_layer_forward", "moe_forward_tokens", "dense_gate_weighted_forward",
    "permute_by_expert", "expert_slot_activations", "balance_statistics",
    "brute_force_top_k", "moe_forward_given_routing", "near_tie_alternatives",
    "combine_outputs",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# Router: [DSMoE] A3 / sec. 3.2, affinity s_{i,t} = Softmax_i(u_t^T e_i)
# --------------------------------------------------------------------------
def affinity_logits(u, E_gate, gate_bias=None) -> np.ndarray:
    """z[t, i] = u_t . e_i (+ b_i), float64.  u: [T][d], E_gate: [N][d]."""
    z = _f64(u) @ _f64(E_gate).T
    if gate_bias is not None:
        z = z + _f64(gate_bias)[None, :]
    return z


def affinity_scores(u, E_gate, gate_bias=None) -> np.ndarray:
    """s[t, i] = Softmax over the N routed experts of the logits, float64, [T][N]."""
    z = affinity_logits(u, E_gate, gate_bias)
    z = z - z.max(axis=1, keepdims=True)   # exact shift: softmax is shift invariant
    ez = np.exp(z)
    return ez / ez.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# Top-K gate: [DSMoE] A3 gate equation, sec. 3.2 gate equation
# --------------------------------------------------------------------------
def top_k_gates(s, K: int):
    """Keep exactly K experts per token.

    Experts are ordered by score descending, equal scores lower index first
    (a stable sort of -s); the first K are kept and their gate is the score
    itself.  Returns idx [T][K] int64 in that order, g [T][K] float64, and the
    margin s_(K) - s_(K+1) per token (+inf when K == N).
    """
    s = _f64(s)
    T, N = s.shape
    if not 1 <= K <= N:
        raise ValueError("need 1 <= K <= N")
    order = np.argsort(-s, axis=1, kind="stable")
    idx = order[:, :K]
    g = np.take_along_axis(s, idx, axis=1)
    if K < N:
        nxt = np.take_along_axis(s, order[:, K:K + 1], axis=1)[:, 0]
        margin = g[:, K - 1] - nxt
    else:
        margin = np.full(T, np.inf)
    return idx, g, margin


def brute_force_top_k(s_row, K: int):
    """The unique K-subset S with: for i in S, j not in S, s_i > s_j or (s_i == s_j and i < j).

    Enumerates every K-subset of range(N) (tiny N only).  Returns the subset as
    a sorted tuple and the number of subsets enumerated.
    """
    s_row = [float(v) for v in s_row]
    N = len(s_row)
    winners, count = [], 0
    for S in itertools.combinations(range(N), K):
        count += 1
        inside = set(S)
        ok = all(s_row[i] > s_row[j] or (s_row[i] == s_row[j] and i < j)
                 for i in S for j in range(N) if j not in inside)
        if ok:
            winners.append(S)
    if len(winners) != 1:
        raise AssertionError(f"dominance rule admits {len(winners)} subsets")
    return winners[0], count


# --------------------------------------------------------------------------
# Expert FFN (SwiGLU)
# --------------------------------------------------------------------------
def swiglu_ffn(x, W_gate, W_up, W_down) -> np.ndarray:
    """FFN(x) = W_down (SiLU(W_gate x) * W_up x) for each row x of X [R][d].

    W_gate, W_up: [I][d]; W_down: [d][I].  Returns [R][d] float64.
    """
    X = _f64(x)
    a = X @ _f64(W_gate).T                       # [R][I]
    b = X @ _f64(W_up).T                         # [R][I]
    with np.errstate(over="ignore"):
        silu = a / (1.0 + np.exp(-a))            # SiLU(a) = a * sigmoid(a)
    return (silu * b) @ _f64(W_down).T           # [R][d]


def _expert(weights, i):
    """weights is a sequence of (W_gate, W_up, W_down) or a callable i -> tuple."""
    return weights(i) if callable(weights) else weights[i]


# --------------------------------------------------------------------------
# The layer: [DSMoE] sec. 3.2, full DeepSeekMoE layer output
# --------------------------------------------------------------------------
def moe_forward_tokens(u, E_gate, routed, shared, N: int, K: int, K_s: int,
                       gate_bias=None, tokens=None):
    """h for the rows `tokens` of u (all rows if None).

    h_t = u_t + sum_{j < K_s} FFN_shared_j(u_t) + sum_{i < N} g_{i,t} FFN_routed_i(u_t),
    evaluated as the formula's sums: shared experts with coefficient 1, then
    routed experts in index order, each over the tokens whose gate is
    non-zero.  Returns (h [R][d] float64, info dict with s, idx, g, margin).
    """
    u = _f64(u)
    if tokens is not None:
        u = u[np.asarray(tokens)]
    if E_gate.shape[0] != N:
        raise ValueError("E_gate must have N rows")
    s = affinity_scores(u, E_gate, gate_bias)
    idx, g, margin = top_k_gates(s, K)
    R = u.shape[0]
    gate = np.zeros((R, N))                      # the sparse gate matrix g_{i,t}
    np.put_along_axis(gate, idx, g, axis=1)

    h = u.copy()                                 # residual term u_t
    for j in range(K_s):
        h += swiglu_ffn(u, *_expert(shared, j))  # shared: coefficient 1
    for i in range(N):
        rows = np.nonzero(gate[:, i])[0]
        if rows.size:
            h[rows] += gate[rows, i, None] * swiglu_ffn(u[rows], *_expert(routed, i))
    return h, {"s": s, "idx": idx, "g": g, "margin": margin}


def moe_layer_forward(u, E_gate, routed, shared, N: int, K: int, K_s: int, gate_bias=None):
    """Whole-batch layer forward; see moe_forward_tokens."""
    return moe_forward_tokens(u, E_gate, routed, shared, N, K, K_s, gate_bias, None)


def moe_forward_given_routing(u, idx, g, routed, shared, K_s: int):
    """h_t = u_t + sum_j FFN_shared_j(u_t) + sum_k g[t,k] FFN_{idx[t,k]}(u_t) for given gates.

    The same layer equation with the routing supplied (used where a token's
    top-K set is not unique, to evaluate each admissible set).
    """
    u = _f64(u)
    idx = np.asarray(idx)
    g = _f64(g)
    h = u.copy()
    for j in range(K_s):
        h += swiglu_ffn(u, *_expert(shared, j))
    for e in np.unique(idx):
        rows, ks = np.nonzero(idx == e)
        h[rows] += g[rows, ks][:, None] * swiglu_ffn(u[rows], *_expert(routed, int(e)))
    return h


def near_tie_alternatives(s, K: int, eps: float = 1e-6):
    """For tokens whose K-th and (K+1)-th scores are within eps, the other admissible set.

    Returns {t: (idx_alt [K], g_alt [K])}: the top-K set with its K-th expert
    replaced by the (K+1)-th.  Either set satisfies "keep the K largest" up to
    eps, so either is a correct routing in finite precision.  An exact tie
    (margin 0) has one correct answer, the lower index (exactly K gates are
    non-zero, [DSMoE] A3), so it has no alternative.
    """
    s = _f64(s)
    idx, g, margin = top_k_gates(s, K)
    out = {}
    if K >= s.shape[1]:
        return out
    order = np.argsort(-s, axis=1, kind="stable")
    for t in np.nonzero((margin > 0) & (margin <= eps))[0]:
        alt = idx[t].copy()
        alt[K - 1] = order[t, K]
        out[int(t)] = (alt, s[t, alt])
    return out


def dense_gate_weighted_forward(u, E_gate, routed, gate_bias=None):
    """h_t = u_t + sum_i s_{i,t} FFN_i(u_t) over all N experts, no selection at all.

    This is the conventional MoE formula ([DSMoE] A3) with K = N and no shared
    experts, written as its own loop so that it shares no selection code with
    moe_forward_tokens.
    """
    u = _f64(u)
    s = affinity_scores(u, E_gate, gate_bias)
    h = u.copy()
    for i in range(s.shape[1]):
        h += s[:, i:i + 1] * swiglu_ffn(u, *_expert(routed, i))
    return h


# --------------------------------------------------------------------------
# Dispatch reference: tokens grouped by expert
# --------------------------------------------------------------------------
def permute_by_expert(idx, N: int):
    """Stable grouping of the (token, k) pairs by expert.

    idx: [T][K] expert ids.  Pair p = t*K + k.  Returns counts [N],
    offsets [N+1] (exclusive prefix of counts) and sorted_pair [T*K]: the pair
    ids ordered by expert, then by pair id (so by token, since one token never
    selects an expert twice).
    """
    flat = np.asarray(idx, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=N).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    sorted_pair = np.argsort(flat, kind="stable")
    return counts, offsets, sorted_pair


def expert_slot_activations(u, routed, shared, idx, g, sorted_pair, offsets, K: int, K_s: int,
                            experts=None):
    """Per-slot intermediate values, for stage checks of the expert GEMMs.

    For routed expert e and each slot p in [offsets[e], offsets[e+1]), with
    pair = sorted_pair[p], t = pair // K, k = pair % K:
      H[p] = SiLU(W_gate x) * (W_up x) with x = u_t     ([I] float64)
      Y[p] = g[t, k] * W_down H[p]                       ([d] float64)
    Returns dicts {e: (H_e, Y_e)} for the experts asked for (all if None),
    and for the shared experts {j: (H_j, Y_j)} over all tokens (coefficient 1).
    """
    u = _f64(u)
    N = len(offsets) - 1
    experts = range(N) if experts is None else experts
    out = {}
    for e in experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        pairs = np.asarray(sorted_pair[lo:hi])
        t, k = pairs // K, pairs % K
        Wg, Wu, Wd = (_f64(w) for w in _expert(routed, e))
        X = u[t]
        a, b = X @ Wg.T, X @ Wu.T
        with np.errstate(over="ignore"):
            H = a / (1.0 + np.exp(-a)) * b
        out[e] = (H, _f64(g)[t, k][:, None] * (H @ Wd.T))
    sh = {}
    for j in range(K_s):
        Wg, Wu, Wd = (_f64(w) for w in _expert(shared, j))
        a, b = u @ Wg.T, u @ Wu.T
        with np.errstate(over="ignore"):
            H = a / (1.0 + np.exp(-a)) * b
        sh[j] = (H, H @ Wd.T)
    return out, sh


def combine_outputs(u, Y, Y_shared, K: int):
    """h_t = u_t + Y_shared_t + sum_k Y[t*K + k]: the layer equation's final sum, float64.

    Y [T*K][d] holds gate-weighted routed outputs in token-major pair order,
    Y_shared [T][d] (or None) the summed shared-expert outputs.
    """
    u = _f64(u)
    T, d = u.shape
    h = u + (0.0 if Y_shared is None else _f64(Y_shared))
    return h + _f64(Y).reshape(T, K, d).sum(axis=1)


# --------------------------------------------------------------------------
# Balance statistics: [DSMoE] sec. 3.3 (forward values only)
# --------------------------------------------------------------------------
def balance_statistics(s, idx, K: int, groups=None, alpha1: float = 1.0, alpha2: float = 1.0):
    """Expert-level and device-level balance statistics of one batch.

    f_i = N'/(K' T) * #{t : token t selects expert i},  P_i = (1/T) sum_t s_{i,t},
    L_ExpBal = alpha1 * sum_i f_i P_i   (N' = routed experts, K' = kept per token).
    With groups = list of expert-index lists (one per device):
    f'_g = mean_{j in group} f_j,  P'_g = sum_{j in group} P_j,
    L_DevBal = alpha2 * sum_g f'_g P'_g.
    """
    s = _f64(s)
    T, N = s.shape
    sel = np.zeros((T, N))
    np.put_along_axis(sel, np.asarray(idx), 1.0, axis=1)
    f = N / (K * T) * sel.sum(axis=0)
    P = s.sum(axis=0) / T
    out = {"f": f, "P": P, "L_ExpBal": alpha1 * float(np.sum(f * P))}
    if groups is not None:
        fg = np.array([f[list(gr)].mean() for gr in groups])
        Pg = np.array([P[list(gr)].sum() for gr in groups])
        out.update({"f_dev": fg, "P_dev": Pg, "L_DevBal": alpha2 * float(np.sum(fg * Pg))})
    return out
