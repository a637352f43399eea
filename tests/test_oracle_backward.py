"""Pins of the backward oracle (oracle/moe_backward.py).

The pages give no backward equations; the oracle is the exact derivative of
the forward layer ([DSMoE] sec. 3.2 with the router of sec. A3) with the top-K
set held fixed.  It is pinned here by what fixes a derivative independently of
the oracle's formulas: central finite differences of L = sum(dh * h) through
the (already pinned) forward oracle, on tiny float64 layers whose top-K margins
are far larger than the perturbation, plus closed forms.
"""
import numpy as np
import pytest

import oracle

EPS = 1e-6


def _layer(seed, T=3, d=6, N=5, K=2, K_s=1, I=4, scale=0.6):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((T, d))
    E = rng.standard_normal((N, d)) * 0.8
    b = rng.standard_normal(N) * 0.3
    routed = [(rng.standard_normal((I, d)) * scale, rng.standard_normal((I, d)) * scale,
               rng.standard_normal((d, I)) * scale) for _ in range(N)]
    shared = [(rng.standard_normal((I, d)) * scale, rng.standard_normal((I, d)) * scale,
               rng.standard_normal((d, I)) * scale) for _ in range(K_s)]
    dh = rng.standard_normal((T, d))
    return u, E, b, routed, shared, dh


def _loss(u, E, b, routed, shared, N, K, K_s, dh):
    h, info = oracle.moe_forward_tokens(u, E, routed, shared, N, K, K_s, gate_bias=b)
    return float(np.sum(dh * h)), info


def _fd(f, x, eps=EPS):
    """Central differences of scalar f with respect to every entry of array x (in place)."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        fp = f()
        x[i] = old - eps
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_backward_matches_finite_differences(seed):
    N, K, K_s = 5, 2, 1
    u, E, b, routed, shared, dh = _layer(seed)
    _, info = _loss(u, E, b, routed, shared, N, K, K_s, dh)
    # the selection must not change under the perturbation
    assert np.min(info["margin"]) > 1e-3
    res = oracle.moe_layer_backward(u, E, routed, shared, N, K, K_s, dh, gate_bias=b)
    f = lambda: _loss(u, E, b, routed, shared, N, K, K_s, dh)[0]   # noqa: E731
    checks = [("du", u, res["du"]), ("dE_gate", E, res["dE_gate"]), ("dgate_bias", b, res["dgate_bias"])]
    for i in range(N):
        for w, name in enumerate(("dW_gate", "dW_up", "dW_down")):
            checks.append((f"routed {i} {name}", routed[i][w], res["d_routed"][i][w]))
    for j in range(K_s):
        for w, name in enumerate(("dW_gate", "dW_up", "dW_down")):
            checks.append((f"shared {j} {name}", shared[j][w], res["d_shared"][j][w]))
    for name, x, got in checks:
        want = _fd(f, x)
        np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-7, err_msg=name)


def test_unselected_experts_get_zero_weight_gradient():
    N, K, K_s = 5, 1, 0
    u, E, b, routed, shared, dh = _layer(4, T=2, K_s=0)
    res = oracle.moe_layer_backward(u, E, routed, [], N, K, 0, dh, gate_bias=b)
    chosen = set(res["idx"].ravel().tolist())
    for i in range(N):
        if i not in chosen:
            assert all(np.all(w == 0) for w in res["d_routed"][i])


def test_zero_weights_pass_the_gradient_through_the_residual():
    # W = 0: every FFN is 0, so h = u and dL/du = dh exactly; every gradient but du is 0
    rng = np.random.default_rng(5)
    T, d, N, K, I = 4, 6, 4, 2, 3
    u = rng.standard_normal((T, d))
    E = rng.standard_normal((N, d))
    z = [(np.zeros((I, d)), np.zeros((I, d)), np.zeros((d, I))) for _ in range(N)]
    dh = rng.standard_normal((T, d))
    res = oracle.moe_layer_backward(u, E, z, z[:1], N, K, 1, dh)
    np.testing.assert_array_equal(res["du"], dh)
    assert np.all(res["dE_gate"] == 0) and np.all(res["dgate_bias"] == 0)
    for ws in res["d_routed"] + res["d_shared"]:
        assert all(np.all(w == 0) for w in ws)


def test_softmax_gradient_sums_to_zero_per_token():
    # sum_i dz_{i,t} = sum_i s_i ds_i - (sum_i s_i) (sum_j s_j ds_j) = 0, so the bias
    # gradient (the token sum of dz) sums to zero over the experts
    u, E, b, routed, shared, dh = _layer(6, T=5, N=6, K=3)
    res = oracle.moe_layer_backward(u, E, routed, shared, 6, 3, 1, dh, gate_bias=b)
    assert abs(res["dgate_bias"].sum()) < 1e-12 * (1 + np.abs(res["dgate_bias"]).sum())


def test_silu_grad_closed_forms():
    # SiLU'(0) = 1/2; SiLU'(a) -> 1 as a -> +inf and -> 0 as a -> -inf
    assert oracle.silu_grad(np.array([0.0]))[0] == 0.5
    np.testing.assert_allclose(oracle.silu_grad(np.array([40.0, -40.0])), [1.0, 0.0], atol=1e-15)
    # against a central difference of SiLU itself at a few points
    a = np.array([-3.0, -0.7, 0.2, 1.9])
    fd = (oracle.silu(a + 1e-6) - oracle.silu(a - 1e-6)) / 2e-6
    np.testing.assert_allclose(oracle.silu_grad(a), fd, rtol=1e-8)
