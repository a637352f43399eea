"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the passage of the DeepSeekMoE paper summary (papercache.org,
cited as [DSMoE]) or the mathematical fact it pins.  None of them recomputes
the oracle's own formula: they use closed forms, hand-derived values,
brute-force enumeration and invariants stated on the pages, chosen so that a
plausible mistake in the oracle (wrong softmax axis, min instead of max,
tie-break the wrong way, renormalised gates, gate/up swapped, W_down
transposed, missing residual, shared experts routed, bias after the softmax,
tokens mixed up) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import moe_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LN2, LN3 = math.log(2.0), math.log(3.0)


def _rand_experts(rng, n, d, I, scale=0.3):
    return [(rng.standard_normal((I, d)) * scale, rng.standard_normal((I, d)) * scale,
             rng.standard_normal((d, I)) * scale) for _ in range(n)]


# --------------------------------------------------------------------------
# softmax  ([DSMoE] A3, affinity s_{i,t} = Softmax_i(u_t^T e_i))
# --------------------------------------------------------------------------
def test_softmax_closed_form():
    # d = 1, u = 1, centroids 0, ln2, ln3  ->  logits 0, ln2, ln3  ->  s = 1/6, 2/6, 3/6
    u = np.array([[1.0]])
    E = np.array([[0.0], [LN2], [LN3]])
    s = oracle.affinity_scores(u, E)
    np.testing.assert_allclose(s[0], [1 / 6, 2 / 6, 3 / 6], rtol=0, atol=1e-15)


def test_softmax_over_experts_not_tokens():
    # two tokens with different logits: each row is its own distribution
    u = np.array([[1.0], [2.0]])
    E = np.array([[0.0], [LN2]])          # token 0: logits 0, ln2; token 1: 0, 2 ln2
    s = oracle.affinity_scores(u, E)
    np.testing.assert_allclose(s, [[1 / 3, 2 / 3], [1 / 5, 4 / 5]], atol=1e-15)


def test_bias_enters_before_softmax():
    # zero logits plus bias (ln2, 0): s = 2/3, 1/3
    u = np.zeros((1, 4))
    E = np.ones((2, 4))
    s = oracle.affinity_scores(u, E, gate_bias=np.array([LN2, 0.0]))
    np.testing.assert_allclose(s[0], [2 / 3, 1 / 3], atol=1e-15)


@pytest.mark.parametrize("name", ["tiny_fp32", "moe2b_bf16"])
def test_softmax_sums_to_one(name):
    inp = moe_inputs.make(name, T=64)
    s = oracle.affinity_scores(inp.u_f32(), inp.E_gate_f32(), inp.gate_bias())
    assert s.shape == (64, inp.w.N)
    assert np.all(s > 0)
    np.testing.assert_allclose(s.sum(axis=1), 1.0, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# top-K  ([DSMoE] A3 gate equation: exactly K of N gates non-zero)
# --------------------------------------------------------------------------
def test_combinatorics_printed_on_the_page():
    gold = json.load(open(os.path.join(GOLDEN, "combinatorics.json")))
    for case in gold["cases"]:
        assert math.comb(case["N"], case["K"]) == case["combinations"]
    # the brute-force enumerator used below really visits C(16,2) = 120 subsets
    s = np.linspace(0.0, 1.0, 16)
    _, count = oracle.brute_force_top_k(s, 2)
    assert count == gold["cases"][0]["combinations"]


@pytest.mark.parametrize("seed", range(6))
def test_top_k_matches_brute_force_random(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(2, 11))
    s = rng.random((5, N))
    for K in range(1, N + 1):
        idx, g, margin = oracle.top_k_gates(s, K)
        for t in range(5):
            S, _ = oracle.brute_force_top_k(s[t], K)
            assert tuple(sorted(idx[t])) == S
            np.testing.assert_array_equal(g[t], s[t][idx[t]])
            # order: score descending
            assert np.all(np.diff(g[t]) <= 0)
            if K < N:
                rest = np.setdiff1d(np.arange(N), idx[t])
                assert margin[t] == pytest.approx(g[t, -1] - s[t][rest].max(), abs=0)
            else:
                assert margin[t] == np.inf


def test_top_k_planted_ties_lower_index_wins():
    # integer logits give exact ties in the softmax values
    u = np.array([[1.0]])
    E = np.array([[1.0], [3.0], [3.0], [2.0], [3.0], [0.0]])
    s = oracle.affinity_scores(u, E)
    for K in range(1, 7):
        idx, g, _ = oracle.top_k_gates(s, K)
        S, _ = oracle.brute_force_top_k(s[0], K)
        assert tuple(sorted(idx[0])) == S
    idx, _, margin = oracle.top_k_gates(s, 2)
    assert list(idx[0]) == [1, 2]          # experts 1, 2, 4 tie: the two lowest win
    assert margin[0] == 0.0
    idx, _, _ = oracle.top_k_gates(s, 4)
    assert list(idx[0]) == [1, 2, 4, 3]


def test_top_k_keeps_largest_not_smallest():
    s = np.array([[0.1, 0.5, 0.05, 0.35]])
    idx, g, margin = oracle.top_k_gates(s, 2)
    assert list(idx[0]) == [1, 3]
    np.testing.assert_array_equal(g[0], [0.5, 0.35])
    assert margin[0] == pytest.approx(0.25)


# --------------------------------------------------------------------------
# SwiGLU expert, residual  (single-expert layer = textbook FFN block)
# --------------------------------------------------------------------------
def test_single_expert_hand_computed():
    # N = 1, K = 1, K_s = 0: s = 1, so h = u + W_down(SiLU(W_gate u) * W_up u).
    # u = (2, -1); W_gate = [[ln3/2, 0]] -> a = ln3, SiLU(ln3) = ln3 * sigmoid(ln3) = (3/4) ln3
    # W_up = [[1, 1]] -> b = 1;  W_down = [[2], [-4]]  (d = 2, I = 1)
    # h = (2 + 2*(3/4)ln3, -1 - 4*(3/4)ln3) = (2 + 1.5 ln3, -1 - 3 ln3)
    u = np.array([[2.0, -1.0]])
    E = np.array([[0.7, -0.2]])
    W = (np.array([[LN3 / 2, 0.0]]), np.array([[1.0, 1.0]]), np.array([[2.0], [-4.0]]))
    h, info = oracle.moe_layer_forward(u, E, [W], [], N=1, K=1, K_s=0)
    assert info["g"][0, 0] == 1.0
    np.testing.assert_allclose(h[0], [2 + 1.5 * LN3, -1 - 3 * LN3], rtol=0, atol=1e-14)


def test_single_expert_gate_and_up_roles():
    # swap the roles: SiLU now sees a = 1 and the linear branch b = ln3:
    # p = SiLU(1) * ln3 = ln3 / (1 + e^-1)   (differs from the case above)
    u = np.array([[2.0, -1.0]])
    W = (np.array([[1.0, 1.0]]), np.array([[LN3 / 2, 0.0]]), np.array([[2.0], [-4.0]]))
    h, _ = oracle.moe_layer_forward(u, np.zeros((1, 2)), [W], [], N=1, K=1, K_s=0)
    p = LN3 / (1 + math.exp(-1.0))
    np.testing.assert_allclose(h[0], [2 + 2 * p, -1 - 4 * p], rtol=0, atol=1e-14)


def test_silu_zero_gives_residual_only():
    u = np.array([[3.0, 5.0]])
    W = (np.array([[5.0, -3.0]]), np.array([[1.0, 2.0]]), np.array([[7.0], [9.0]]))   # a = 0
    h, _ = oracle.moe_layer_forward(u, np.zeros((1, 2)), [W], [], N=1, K=1, K_s=0)
    np.testing.assert_array_equal(h, u)


def test_w_down_orientation_non_square():
    # d = 3, I = 2: W_down is [d][I]; column k of W_down carries intermediate unit k.
    u = np.array([[1.0, 0.0, 0.0]])
    Wg = np.array([[LN3, 0.0, 0.0], [0.0, 0.0, 0.0]])      # a = (ln3, 0)
    Wu = np.array([[1.0, 0.0, 0.0], [1.0, 0.0, 0.0]])      # b = (1, 1)
    Wd = np.array([[1.0, 10.0], [2.0, 20.0], [3.0, 30.0]])
    # p = (SiLU(ln3), SiLU(0)) = (0.75 ln3, 0)  ->  y = 0.75 ln3 * (1, 2, 3)
    h, _ = oracle.moe_layer_forward(u, np.zeros((1, 3)), [(Wg, Wu, Wd)], [], N=1, K=1, K_s=0)
    np.testing.assert_allclose(h[0], [1 + 0.75 * LN3, 1.5 * LN3, 2.25 * LN3], atol=1e-14)


# --------------------------------------------------------------------------
# gates are the softmax values, not renormalised; shared experts outside the softmax
# ([DSMoE] sec. 3.2 layer and gate equations)
# --------------------------------------------------------------------------
def _one_unit_expert():
    # d = 2, I = 1, FFN(u) = W_down * SiLU(ln3) * 1 for u = (1, 0)
    return (np.array([[LN3, 0.0]]), np.array([[1.0, 0.0]]), np.array([[1.0], [2.0]]))


@pytest.mark.parametrize("K,gsum", [(1, 1 / 2), (2, 5 / 6), (3, 1.0)])
def test_identical_experts_closed_form(K, gsum):
    # routed logits 0, ln2, ln3 -> s = 1/6, 1/3, 1/2; all routed experts identical,
    # so h = u + (sum of kept s) FFN(u).  Renormalised gates would give sum 1 for every K.
    u = np.array([[1.0, 0.0]])
    E = np.array([[0.0, 0.0], [LN2, 0.0], [LN3, 0.0]])
    W = _one_unit_expert()
    ffn = 0.75 * LN3 * np.array([1.0, 2.0])
    h, info = oracle.moe_layer_forward(u, E, [W, W, W], [], N=3, K=K, K_s=0)
    np.testing.assert_allclose(h[0], u[0] + gsum * ffn, atol=1e-14)
    np.testing.assert_allclose(info["g"].sum(), gsum, atol=1e-15)


def test_shared_expert_coefficient_one_and_outside_softmax():
    # the same three routed experts plus one shared expert whose FFN is 2x the routed one:
    # h = u + 2 FFN(u) + (1/2) FFN(u) for K = 1.  A softmax over all four experts, or a
    # gated shared expert, would give something else.
    u = np.array([[1.0, 0.0]])
    E = np.array([[0.0, 0.0], [LN2, 0.0], [LN3, 0.0]])
    W = _one_unit_expert()
    Ws = (W[0], W[1], 2 * W[2])
    ffn = 0.75 * LN3 * np.array([1.0, 2.0])
    h, info = oracle.moe_layer_forward(u, E, [W, W, W], [Ws], N=3, K=1, K_s=1)
    np.testing.assert_allclose(h[0], u[0] + 2 * ffn + 0.5 * ffn, atol=1e-14)
    assert list(info["idx"][0]) == [2]


def test_zero_weights_give_residual_exactly():
    inp = moe_inputs.custom(T=16, d=64, N=8, K=3, K_s=2, I=32)
    z = lambda i: (np.zeros((32, 64)), np.zeros((32, 64)), np.zeros((64, 32)))  # noqa: E731
    h, _ = oracle.moe_layer_forward(inp.u_f32(), inp.E_gate_f32(), z, z, N=8, K=3, K_s=2)
    np.testing.assert_array_equal(h, inp.u_f32().astype(np.float64))


def test_zero_centroids_give_uniform_gates():
    # e_i = 0 -> s = 1/N for every expert; with K = N identical routed experts
    # h = u + FFN(u) (sum of gates is exactly 1)
    rng = np.random.default_rng(3)
    d, I, N = 6, 4, 5
    W = _rand_experts(rng, 1, d, I)[0]
    u = rng.standard_normal((4, d))
    h, info = oracle.moe_layer_forward(u, np.zeros((N, d)), [W] * N, [], N=N, K=N, K_s=0)
    np.testing.assert_allclose(info["g"], 1 / N, atol=1e-16)
    np.testing.assert_allclose(h, u + oracle.swiglu_ffn(u, *W), atol=1e-13)


# --------------------------------------------------------------------------
# K = N, no shared experts: the dense gate-weighted sum, by a loop with no selection
# --------------------------------------------------------------------------
def test_k_equals_n_is_dense_weighted_sum():
    rng = np.random.default_rng(11)
    d, I, N, T = 12, 8, 6, 20
    routed = _rand_experts(rng, N, d, I)
    u = rng.standard_normal((T, d))
    E = rng.standard_normal((N, d))
    h, _ = oracle.moe_layer_forward(u, E, routed, [], N=N, K=N, K_s=0)
    h_dense = oracle.dense_gate_weighted_forward(u, E, routed)
    np.testing.assert_allclose(h, h_dense, rtol=0, atol=1e-12 * np.abs(h_dense).max())


# --------------------------------------------------------------------------
# fine-grained segmentation keeps the function ([DSMoE] sec. 3.1: an FFN cut into m
# experts of intermediate width 1/m); shared concatenation is the same identity read back
# --------------------------------------------------------------------------
def _segments(Wg, Wu, Wd, m):
    I = Wg.shape[0] // m
    return [(Wg[j * I:(j + 1) * I], Wu[j * I:(j + 1) * I], Wd[:, j * I:(j + 1) * I]) for j in range(m)]


@pytest.mark.parametrize("m", [2, 4, 8])
def test_segmentation_reproduces_unsplit_ffn(m):
    rng = np.random.default_rng(m)
    d, I_big, T = 16, 64, 10
    big = _rand_experts(rng, 1, d, I_big)[0]
    u = rng.standard_normal((T, d))
    zero = (np.zeros((8, d)), np.zeros((8, d)), np.zeros((d, 8)))
    # all m segments as shared experts (gate 1), one dummy routed expert with zero weights
    h, _ = oracle.moe_layer_forward(u, np.zeros((1, d)), [zero], _segments(*big, m), N=1, K=1, K_s=m)
    ref = u + oracle.swiglu_ffn(u, *big)
    np.testing.assert_allclose(h, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    # and through the router: zero centroids give s = 1/m on every segment
    h2, _ = oracle.moe_layer_forward(u, np.zeros((m, d)), _segments(*big, m), [], N=m, K=m, K_s=0)
    np.testing.assert_allclose(h2, u + oracle.swiglu_ffn(u, *big) / m, rtol=0,
                               atol=1e-12 * np.abs(ref).max())


def test_shared_experts_equal_one_concatenated_ffn():
    rng = np.random.default_rng(5)
    d, I, Ks, T = 16, 8, 3, 7
    shared = _rand_experts(rng, Ks, d, I)
    cat = (np.concatenate([w[0] for w in shared]), np.concatenate([w[1] for w in shared]),
           np.concatenate([w[2] for w in shared], axis=1))
    u = rng.standard_normal((T, d))
    zero = (np.zeros((I, d)), np.zeros((I, d)), np.zeros((d, I)))
    h, _ = oracle.moe_layer_forward(u, np.zeros((1, d)), [zero], shared, N=1, K=1, K_s=Ks)
    np.testing.assert_allclose(h, u + oracle.swiglu_ffn(u, *cat), atol=1e-12)


# --------------------------------------------------------------------------
# invariances of the formula
# --------------------------------------------------------------------------
def test_shift_invariance_of_bias():
    inp = moe_inputs.custom(T=32, d=64, N=10, K=3, K_s=1, I=16, seed=9)
    u, E = inp.u_f32(), inp.E_gate_f32()
    h0, i0 = oracle.moe_layer_forward(u, E, inp.routed_expert_f32, inp.shared_expert_f32, 10, 3, 1)
    h1, i1 = oracle.moe_layer_forward(u, E, inp.routed_expert_f32, inp.shared_expert_f32, 10, 3, 1,
                                      gate_bias=np.full(10, 3.25))
    np.testing.assert_array_equal(i0["idx"], i1["idx"])
    np.testing.assert_allclose(i0["g"], i1["g"], rtol=1e-13)
    np.testing.assert_allclose(h0, h1, rtol=0, atol=1e-13)


def test_token_chunk_invariance():
    inp = moe_inputs.custom(T=40, d=32, N=8, K=2, K_s=1, I=16, seed=4)
    args = (inp.E_gate_f32(), inp.routed_expert_f32, inp.shared_expert_f32, 8, 2, 1)
    u = inp.u_f32()
    h, _ = oracle.moe_layer_forward(u, *args)
    ha, _ = oracle.moe_layer_forward(u[:13], *args)
    hb, _ = oracle.moe_layer_forward(u[13:], *args)
    np.testing.assert_allclose(np.concatenate([ha, hb]), h, rtol=0, atol=1e-14)
    hs, _ = oracle.moe_forward_tokens(u, *args, tokens=[39, 0, 17])
    np.testing.assert_allclose(hs, h[[39, 0, 17]], rtol=0, atol=1e-14)


def test_identical_experts_random_batch():
    # all routed experts identical: h = u + shared + (sum of the brute-force top-K scores) FFN(u)
    rng = np.random.default_rng(21)
    d, I, N, K, T = 10, 6, 7, 3, 9
    W = _rand_experts(rng, 1, d, I)[0]
    Ws = _rand_experts(rng, 1, d, I)[0]
    u = rng.standard_normal((T, d))
    E = rng.standard_normal((N, d))
    h, info = oracle.moe_layer_forward(u, E, [W] * N, [Ws], N=N, K=K, K_s=1)
    z = u @ E.T
    for t in range(T):
        p = np.exp(z[t] - z[t].max())
        p /= p.sum()
        S, _ = oracle.brute_force_top_k(p, K)
        ref = u[t] + oracle.swiglu_ffn(u[t:t + 1], *Ws)[0] + p[list(S)].sum() * oracle.swiglu_ffn(u[t:t + 1], *W)[0]
        np.testing.assert_allclose(h[t], ref, atol=1e-12)


# --------------------------------------------------------------------------
# dispatch reference
# --------------------------------------------------------------------------
def test_permute_brute_force():
    rng = np.random.default_rng(8)
    T, N, K = 37, 9, 4
    idx = np.stack([rng.permutation(N)[:K] for _ in range(T)])
    counts, offsets, sp = oracle.permute_by_expert(idx, N)
    assert offsets[0] == 0 and offsets[-1] == T * K == counts.sum()
    assert sorted(sp.tolist()) == list(range(T * K))
    for e in range(N):
        want = [t * K + k for t in range(T) for k in range(K) if idx[t, k] == e]
        assert sp[offsets[e]:offsets[e + 1]].tolist() == want
        assert counts[e] == len(want)


def test_slot_activations_reassemble_the_layer():
    inp = moe_inputs.custom(T=24, d=32, N=6, K=2, K_s=2, I=16, seed=12)
    u, E = inp.u_f32(), inp.E_gate_f32()
    h, info = oracle.moe_layer_forward(u, E, inp.routed_expert_f32, inp.shared_expert_f32, 6, 2, 2)
    counts, offsets, sp = oracle.permute_by_expert(info["idx"], 6)
    per_e, per_s = oracle.expert_slot_activations(u, inp.routed_expert_f32, inp.shared_expert_f32,
                                                  info["idx"], info["g"], sp, offsets, 2, 2)
    acc = u.astype(np.float64).copy()
    for e, (H, Y) in per_e.items():
        np.add.at(acc, sp[offsets[e]:offsets[e + 1]] // 2, Y)
    for j, (H, Y) in per_s.items():
        acc += Y
    np.testing.assert_allclose(acc, h, atol=1e-13)


# --------------------------------------------------------------------------
# balance statistics ([DSMoE] sec. 3.3)
# --------------------------------------------------------------------------
def test_balance_statistics_closed_forms():
    rng = np.random.default_rng(2)
    T, N, K = 50, 8, 3
    s = rng.random((T, N))
    s /= s.sum(axis=1, keepdims=True)
    idx, _, _ = oracle.top_k_gates(s, K)
    st = oracle.balance_statistics(s, idx, K, groups=[[0, 1], [2, 3, 4], [5, 6, 7]], alpha1=0.5, alpha2=2.0)
    assert st["f"].sum() == pytest.approx(N)          # sum_i f_i = N'
    assert st["P"].sum() == pytest.approx(1.0)        # sum_i P_i = 1
    assert st["P_dev"].sum() == pytest.approx(1.0)
    # perfectly uniform routing: f_i = 1, P_i = 1/N -> L_ExpBal = alpha1
    T2 = N
    s2 = np.full((T2, N), 1 / N)
    idx2 = np.array([[(t + k) % N for k in range(K)] for t in range(T2)])
    st2 = oracle.balance_statistics(s2, idx2, K, groups=[[i] for i in range(N)], alpha1=0.5, alpha2=2.0)
    np.testing.assert_allclose(st2["f"], 1.0)
    assert st2["L_ExpBal"] == pytest.approx(0.5)
    assert st2["L_DevBal"] == pytest.approx(2.0)
    # collapse: every token picks experts 0..K-1 -> f = N/K on those, 0 elsewhere
    idx3 = np.tile(np.arange(K), (T2, 1))
    st3 = oracle.balance_statistics(s2, idx3, K)
    np.testing.assert_allclose(st3["f"], [N / K] * K + [0] * (N - K))


def test_device_balance_with_multi_expert_groups():
    """Device groups of several experts ([DSMoE] sec. 3.3 device-level loss): f'_g is the
    MEAN of f over the group and P'_g the SUM of P over it.  Collapsed routing (every token
    keeps experts 0, 1, 2 of N = 8) with groups {0, 1} and {2, ..., 7}, worked by hand:
    f = (8/3, 8/3, 8/3, 0, 0, 0, 0, 0), so f'_0 = 8/3 and f'_1 = (8/3) / 6 = 4/9;
    every token has the scores below, so P = s and P' = (0.5, 0.5);
    L_DevBal = alpha2 * (8/3 * 0.5 + 4/9 * 0.5) = alpha2 * 14/9."""
    T, N, K = 10, 8, 3
    row = np.array([0.3, 0.2, 0.1, 0.1, 0.1, 0.1, 0.05, 0.05])
    s = np.tile(row, (T, 1))
    idx = np.tile(np.arange(K), (T, 1))
    groups = [[0, 1], [2, 3, 4, 5, 6, 7]]
    st = oracle.balance_statistics(s, idx, K, groups=groups, alpha1=1.0, alpha2=3.0)
    np.testing.assert_allclose(st["f"], [8 / 3] * 3 + [0] * 5, rtol=1e-15)
    np.testing.assert_allclose(st["f_dev"], [8 / 3, 4 / 9], rtol=1e-15)
    np.testing.assert_allclose(st["P_dev"], [0.5, 0.5], rtol=1e-15)
    assert st["L_DevBal"] == pytest.approx(3.0 * 14 / 9, rel=1e-15)
    # L_ExpBal over the same batch: sum_i f_i P_i = 8/3 * (0.3 + 0.2 + 0.1) = 1.6
    assert st["L_ExpBal"] == pytest.approx(1.6, rel=1e-15)
    # uneven groups {0..5}, {6}, {7}: f' = (8/3 * 3 / 6, 0, 0), P' = (0.9, 0.05, 0.05)
    st2 = oracle.balance_statistics(s, idx, K, groups=[[0, 1, 2, 3, 4, 5], [6], [7]], alpha2=1.0)
    np.testing.assert_allclose(st2["f_dev"], [4 / 3, 0.0, 0.0], rtol=1e-15)
    np.testing.assert_allclose(st2["P_dev"], [0.9, 0.05, 0.05], rtol=1e-15)
    assert st2["L_DevBal"] == pytest.approx(4 / 3 * 0.9, rel=1e-15)


def test_given_routing_equals_layer_and_identical_experts():
    # with the oracle's own routing it reproduces the layer; with identical experts it
    # gives u + shared + (sum of the supplied gates) FFN(u) for any supplied set
    inp = moe_inputs.custom(T=12, d=32, N=6, K=2, K_s=1, I=16, seed=13)
    u, E = inp.u_f32(), inp.E_gate_f32()
    h, info = oracle.moe_layer_forward(u, E, inp.routed_expert_f32, inp.shared_expert_f32, 6, 2, 1)
    h2 = oracle.moe_forward_given_routing(u, info["idx"], info["g"], inp.routed_expert_f32,
                                          inp.shared_expert_f32, 1)
    np.testing.assert_allclose(h2, h, atol=1e-14)
    W = _one_unit_expert()
    u1 = np.array([[1.0, 0.0], [1.0, 0.0]])
    h3 = oracle.moe_forward_given_routing(u1, np.array([[0, 2], [1, 0]]), np.array([[0.25, 0.5], [0.125, 0.0]]),
                                          [W, W, W], [], 0)
    ffn = 0.75 * LN3 * np.array([1.0, 2.0])
    np.testing.assert_allclose(h3, [u1[0] + 0.75 * ffn, u1[1] + 0.125 * ffn], atol=1e-14)


def test_near_tie_alternative_swaps_boundary_expert():
    s = np.array([[0.3, 0.2, 0.2 + 5e-7, 0.1, 0.2 - 1e-3 + 0.0]])
    s = s / s.sum()
    alts = oracle.near_tie_alternatives(s, 2)
    assert list(alts) == [0]
    assert sorted(alts[0][0].tolist()) == [0, 1]      # expert 2 (K-th) swapped for expert 1
    assert oracle.near_tie_alternatives(s, 1) == {}
    # an exact tie at the boundary is decided by the lower index: no alternative
    s_tie = np.array([[0.4, 0.2, 0.1, 0.2, 0.1]])
    assert oracle.near_tie_alternatives(s_tie, 2) == {}
    idx, _, margin = oracle.top_k_gates(s_tie, 2)
    assert idx.tolist() == [[0, 1]] and margin[0] == 0.0


def test_combine_outputs_closed_form():
    u = np.array([[1.0, 2.0], [3.0, 4.0]])
    Y = np.array([[0.5, 0.0], [0.0, 0.25], [1.0, 1.0], [2.0, -2.0]])   # T = 2, K = 2
    Ys = np.array([[10.0, 20.0], [30.0, 40.0]])
    np.testing.assert_array_equal(oracle.combine_outputs(u, Y, Ys, 2), [[11.5, 22.25], [36.0, 43.0]])
    np.testing.assert_array_equal(oracle.combine_outputs(u, Y, None, 2), [[1.5, 2.25], [6.0, 3.0]])
