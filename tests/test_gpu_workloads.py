"""GPU parity at the five workload shapes (tiny fp32, 2B-, 16B-prefill-, 16B-decode- and
145B-skewed-shaped bf16 layers), in the launch configuration the benchmark times.

Routing is checked on every token; dispatch on every pair (integer exact); the
expert stage on every slot of every expert (H and Y, so every m-tile including
each expert's ragged tail tile) and on every token row of the shared experts,
except at the 145B shape, where it covers every slot of the hottest, the
coldest and two random experts (plus every shared row); h on every token,
except at the 145B shape: 2048 tokens holding the first and last tokens, every
near-tie token, tokens of the hottest and coldest experts and random tokens.
"""
import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from parity_helpers import (Uploaded, check_h, check_routing, device_f32, say, tol_for)

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mixture_experts_ffn_fp32_amd")

# tokens whose h is recomputed by the oracle (None = all)
SAMPLE = {"tiny_fp32": None, "moe16b_decode_bf16": None, "moe2b_bf16": None,
          "moe16b_prefill_bf16": None, "moe145b_skewed_bf16": 2048}
# experts whose every slot the expert-stage test checks (None = all)
STAGE_EXPERTS = {"moe145b_skewed_bf16": 4}


@pytest.fixture(scope="module", params=list(moe_inputs.WORKLOADS))
def wl(request):
    name = request.param
    say(f"upload workload {name}")
    up = Uploaded(moe_inputs.make(name))
    inp = up.inp
    s = oracle.affinity_scores(inp.u_f32(), inp.E_gate_f32(), inp.gate_bias())
    yield up, s
    del up
    torch.cuda.empty_cache()


def _sample(up, s, n):
    w = up.w
    if n is None or n >= w.T:
        return np.arange(w.T)
    idx, _, margin = oracle.top_k_gates(s, w.K)
    counts = np.bincount(idx.ravel(), minlength=w.N)
    hot = int(np.argmax(counts))
    nz = np.nonzero(counts)[0]
    cold = int(nz[np.argmin(counts[nz])])
    rng = np.random.default_rng(w.seed)
    pick = {0, w.T - 1}
    pick |= set(np.nonzero(margin <= 1e-6)[0].tolist())
    pick |= set(np.nonzero((idx == cold).any(axis=1))[0].tolist())     # all of the coldest
    pick |= set(np.nonzero((idx == hot).any(axis=1))[0][:64].tolist())
    while len(pick) < n:
        pick.add(int(rng.integers(w.T)))
    return np.array(sorted(pick))


def test_routing_all_tokens(wl):
    up, s = wl
    w = up.w
    say(f"route {w.name}")
    idx, gate, _ = mx.route(up.u, up.E, w.K, up.bias)
    torch.cuda.synchronize()
    differing, _ = check_routing(idx.cpu().numpy(), gate.cpu().numpy(), s, w.K)
    assert len(differing) <= max(1, w.T // 1000)


def test_dispatch_all_pairs(wl):
    up, s = wl
    w = up.w
    idx_ref, _, _ = oracle.top_k_gates(s, w.K)
    say(f"dispatch {w.name}")
    counts, offsets, sp = mx.dispatch(torch.from_numpy(idx_ref.astype(np.int32)).cuda(), w.N)
    torch.cuda.synchronize()
    c_ref, o_ref, sp_ref = oracle.permute_by_expert(idx_ref, w.N)
    np.testing.assert_array_equal(counts.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(offsets.cpu().numpy(), o_ref)
    np.testing.assert_array_equal(sp.cpu().numpy(), sp_ref)
    if w.zipf_s is not None:   # the skew really is there
        assert c_ref.max() > 5 * c_ref.mean()


def test_expert_stage_selected_experts(wl):
    up, s = wl
    w = up.w
    idx_ref, g_ref, _ = oracle.top_k_gates(s, w.K)
    c_ref, o_ref, sp_ref = oracle.permute_by_expert(idx_ref, w.N)
    say(f"expert_ffn {w.name}")
    H, Hs, Y, Ys = mx.expert_ffn(up.u, up.W_routed, up.W_shared, w.N, w.K, w.K_s,
                                 torch.from_numpy(o_ref.astype(np.int32)).cuda(),
                                 torch.from_numpy(sp_ref.astype(np.int32)).cuda(),
                                 torch.from_numpy(g_ref.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    nz = np.nonzero(c_ref)[0]
    n_pick = STAGE_EXPERTS.get(w.name)
    if n_pick is None:
        experts = nz.tolist()
    else:
        rng = np.random.default_rng(3)
        experts = sorted({int(np.argmax(c_ref)), int(nz[np.argmin(c_ref[nz])]),
                          *rng.choice(nz, size=min(n_pick - 2, nz.size), replace=False).tolist()})
    tol = tol_for(w)
    u32 = up.inp.u_f32()
    for e in experts:    # every slot of the expert: all its m-tiles, the ragged last one too
        acts, _ = oracle.expert_slot_activations(u32, up.routed, up.shared, idx_ref, g_ref,
                                                 sp_ref, o_ref, w.K, 0, experts=[e])
        H_ref, Y_ref = acts[e]
        lo, hi = int(o_ref[e]), int(o_ref[e + 1])
        Hg = device_f32(H[lo:hi])
        Yg = device_f32(Y[torch.from_numpy(sp_ref[lo:hi]).cuda()])
        assert np.abs(Hg - H_ref).max() <= tol * np.abs(H_ref).max(), f"H of expert {e}"
        assert np.abs(Yg - Y_ref).max() <= tol * np.abs(Y_ref).max(), f"Y of expert {e}"
    say(f"{w.name}: H and Y of {len(experts)} experts, {int(c_ref[experts].sum())} slots")
    if w.K_s:
        Hs_g = device_f32(Hs)
        Ys_g = device_f32(Ys)
        for r0 in range(0, w.T, 4096):     # every token row, in row blocks
            rows = np.arange(r0, min(w.T, r0 + 4096))
            _, sh = oracle.expert_slot_activations(u32[rows], up.routed, up.shared,
                                                   idx_ref[rows], g_ref[rows], sp_ref[:0],
                                                   np.zeros(1, dtype=np.int64), w.K, w.K_s,
                                                   experts=[])
            for j in range(w.K_s):
                H_ref = sh[j][0]
                Hg = Hs_g[rows][:, j * w.I:(j + 1) * w.I]
                assert np.abs(Hg - H_ref).max() <= tol * np.abs(H_ref).max(), f"H_shared {j}"
            Ys_ref = sum(sh[j][1] for j in range(w.K_s))
            assert np.abs(Ys_g[rows] - Ys_ref).max() <= tol * np.abs(Ys_ref).max(), "Y_shared"


def test_layer_forward_sampled(wl):
    up, s = wl
    w = up.w
    say(f"layer_forward {w.name}")
    h = mx.layer_forward(up.u, up.E, up.W_routed, up.W_shared, w.N, w.K, w.K_s, up.bias)
    idx, gate, _ = mx.route(up.u, up.E, w.K, up.bias)
    torch.cuda.synchronize()
    tokens = _sample(up, s, SAMPLE[w.name])
    inp = up.inp
    h_ref, info = oracle.moe_forward_tokens(inp.u_f32(), inp.E_gate_f32(), up.routed, up.shared,
                                            w.N, w.K, w.K_s, inp.gate_bias(), tokens)
    idx_s = idx.cpu().numpy()[tokens]
    differing, alts = check_routing(idx_s, gate.cpu().numpy()[tokens], info["s"], w.K)
    for i in differing:
        a_idx, a_g = alts[int(i)]
        t = tokens[i]
        h_ref[i] = oracle.moe_forward_given_routing(inp.u_f32()[t:t + 1], a_idx[None], a_g[None],
                                                    up.routed, up.shared, w.K_s)[0]
    hs = device_f32(h[torch.from_numpy(tokens).cuda()])
    rel = check_h(hs, h_ref, inp.u_f32()[tokens].astype(np.float64), tol_for(w), w.dtype, w.K,
                  w.name)
    say(f"{w.name}: max|dh|/max|h| = {rel:.2e} over {len(tokens)} tokens")


def test_balance_statistics(wl):
    """GPU statistics from the GPU's routing against the oracle's statistics from the
    oracle's routing: P to float32 softmax accuracy, f to the tokens whose routing may
    legitimately differ (near ties), and the definitions' exact sums."""
    up, s = wl
    w = up.w
    D = 8 if w.N % 8 == 0 else 7 if w.N % 7 == 0 else 4
    group_of = [i * D // w.N for i in range(w.N)]
    groups = [[i for i in range(w.N) if group_of[i] == g] for g in range(D)]
    say(f"balance {w.name}")
    idx, _, scores = mx.route(up.u, up.E, w.K, up.bias, want_scores=True)
    res = mx.balance_stats(scores, idx, w.K, group_of, alpha1=0.001, alpha2=0.05)
    torch.cuda.synchronize()
    idx_ref, _, margin = oracle.top_k_gates(s, w.K)
    ref = oracle.balance_statistics(s, idx_ref, w.K, groups, alpha1=0.001, alpha2=0.05)
    n_near = int(np.count_nonzero(margin <= 1e-6))
    f_step = w.N / (w.K * w.T)
    assert np.abs(res["f"].cpu().numpy() - ref["f"]).max() <= f_step * n_near + 2.0 ** -23 * w.N
    np.testing.assert_allclose(res["P"].cpu().numpy(), ref["P"], rtol=1e-5, atol=1e-7)
    assert abs(float(res["L_ExpBal"]) - ref["L_ExpBal"]) <= 1e-4 * ref["L_ExpBal"] + 1e-3 * n_near
    np.testing.assert_allclose(res["P_dev"].cpu().numpy(), ref["P_dev"], rtol=1e-5, atol=1e-7)
    # f'_g: the mean of f over the group's N / D experts (a near tie moves one f by f_step)
    assert np.abs(res["f_dev"].cpu().numpy() - ref["f_dev"]).max() <= \
        f_step * n_near + 2.0 ** -22 * ref["f_dev"].max()
    assert abs(float(res["L_DevBal"]) - ref["L_DevBal"]) <= \
        1e-4 * ref["L_DevBal"] + 2 * 0.05 * f_step * n_near
    assert abs(float(res["f"].double().sum()) - w.N) <= 1e-5 * w.N
    assert abs(float(res["P"].double().sum()) - 1.0) <= 1e-5
    if w.zipf_s is not None:   # the skew shows: the hottest expert far above f = 1
        assert ref["f"].max() > 5.0
    say(f"{w.name}: max f = {ref['f'].max():.3f}, L_ExpBal/alpha1 = {ref['L_ExpBal'] / 0.001:.4f}")
