"""CPU oracle of the DeepSeekMoE layer BACKWARD pass -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module; the GPU path never calls it and shares no code with it.
Plain NumPy in float64.

The pages train the layer but state no backward equations, so this is the
exact derivative of the forward layer of the DeepSeekMoE paper summary
(papercache.org, sec. 3.2 layer equation, with the router of sec. A3):

    z_t = E_gate u_t (+ b),  s_t = Softmax(z_t),  S_t = top-K of s_t,
    h_t = u_t + sum_j FFN_shared_j(u_t) + sum_{i in S_t} s_{i,t} FFN_routed_i(u_t),
    FFN(x) = W_down (SiLU(W_gate x) * (W_up x)),  SiLU(a) = a sigma(a),

differentiated by the chain rule with the top-K set S_t held fixed (it is
piecewise constant in the scores: its derivative is zero wherever the
selection does not change).  For an upstream gradient dh:

    FFN backward (a = W_gate x, c = W_up x, p = SiLU(a) c, y = W_down p, dy):
      dW_down += dy p^T,  dp = W_down^T dy,
      da = dp * c * SiLU'(a),  SiLU'(a) = sigma(a) (1 + a (1 - sigma(a))),
      dc = dp * SiLU(a),
      dW_gate += da x^T,  dW_up += dc x^T,  dx = W_gate^T da + W_up^T dc;
    shared expert j:  dy = dh;
    routed expert i in S_t:  dy = s_{i,t} dh  and  ds_{i,t} = dh . FFN_i(u_t);
    ds_{i,t} = 0 for i outside S_t;
    softmax:  dz_{i,t} = s_{i,t} (ds_{i,t} - sum_j s_{j,t} ds_{j,t});
    router:   du_t += E_gate^T dz_t,  dE_gate += dz_t u_t^T,  db += dz_t;
    residual: du_t += dh_t.

Pinned by tests/test_oracle_backward.py against central finite differences of
sum(dh * h) and against closed forms.
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import affinity_scores, top_k_gates

__all__ = ["silu", "silu_grad", "swiglu_ffn_backward", "moe_layer_backward"]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def silu(a):
    a = _f64(a)
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def silu_grad(a):
    """d SiLU / da = sigma(a) (1 + a (1 - sigma(a)))."""
    a = _f64(a)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-a))
    return sig * (1.0 + a * (1.0 - sig))


def swiglu_ffn_backward(x, W_gate, W_up, W_down, dy):
    """Gradients of y = W_down (SiLU(W_gate x) * W_up x) for rows x of X [R][d].

    dy: [R][d].  Returns (y, dx [R][d], dW_gate [I][d], dW_up [I][d], dW_down [d][I]).
    """
    X, dY = _f64(x), _f64(dy)
    Wg, Wu, Wd = _f64(W_gate), _f64(W_up), _f64(W_down)
    a = X @ Wg.T                       # [R][I]
    c = X @ Wu.T                       # [R][I]
    p = silu(a) * c                    # [R][I]
    y = p @ Wd.T                       # [R][d]
    dWd = dY.T @ p                     # [d][I]
    dp = dY @ Wd                       # [R][I]
    da = dp * c * silu_grad(a)
    dc = dp * silu(a)
    dWg = da.T @ X                     # [I][d]
    dWu = dc.T @ X                     # [I][d]
    dx = da @ Wg + dc @ Wu             # [R][d]
    return y, dx, dWg, dWu, dWd


def _expert(weights, i):
    return weights(i) if callable(weights) else weights[i]


def moe_layer_backward(u, E_gate, routed, shared, N: int, K: int, K_s: int, dh, gate_bias=None,
                       replace_sets=None):
    """All gradients of sum(dh * h) for the layer; the chain rule in the order of the
    formula (residual, shared experts, routed experts, softmax, router).

    replace_sets: optional {t: (idx [K], g [K])} of tokens whose held-fixed set is
    another admissible one (near_tie_alternatives) instead of the top-K of s.

    Returns a dict: du [T][d], dE_gate [N][d], dgate_bias [N], d_routed (list of
    (dW_gate, dW_up, dW_down) per routed expert), d_shared (same per shared expert),
    and the forward's s, idx, g, ds, dz.
    """
    u, dh = _f64(u), _f64(dh)
    T, d = u.shape
    s = affinity_scores(u, E_gate, gate_bias)
    idx, g, margin = top_k_gates(s, K)
    for t, (ia, ga) in (replace_sets or {}).items():
        idx[t], g[t] = ia, ga
    gate = np.zeros((T, N))
    np.put_along_axis(gate, idx, g, axis=1)

    du = dh.copy()                                     # residual
    d_shared = []
    for j in range(K_s):                               # shared experts: coefficient 1
        _, dx, dWg, dWu, dWd = swiglu_ffn_backward(u, *_expert(shared, j), dh)
        du += dx
        d_shared.append((dWg, dWu, dWd))
    ds = np.zeros((T, N))
    d_routed = []
    for i in range(N):                                 # routed experts, gate s_{i,t}
        Wi = _expert(routed, i)
        I = np.asarray(Wi[0]).shape[0]
        rows = np.nonzero(gate[:, i])[0]
        if rows.size == 0:
            d_routed.append((np.zeros((I, d)), np.zeros((I, d)), np.zeros((d, I))))
            continue
        gi = gate[rows, i, None]
        y, dx, dWg, dWu, dWd = swiglu_ffn_backward(u[rows], *Wi, gi * dh[rows])
        du[rows] += dx
        ds[rows, i] = np.sum(dh[rows] * y, axis=1)     # d(g_i y_i)/d g_i
        d_routed.append((dWg, dWu, dWd))
    dz = s * (ds - np.sum(s * ds, axis=1, keepdims=True))   # softmax backward
    du += dz @ _f64(E_gate)
    dE = dz.T @ u
    db = dz.sum(axis=0)
    return {"du": du, "dE_gate": dE, "dgate_bias": db, "d_routed": d_routed,
            "d_shared": d_shared, "s": s, "idx": idx, "g": g, "ds": ds, "dz": dz,
            "margin": margin}
