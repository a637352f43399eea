"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Stage tests feed the GPU and the oracle the same inputs (seeded inputs, or
the oracle's own routing / dispatch / expert outputs) and compare each stage;
end-to-end tests compare h.  Shapes span several tiles with ragged tails,
and include the degenerate cases (one token, K = N, no shared expert,
N = 1, N = 256, a non-power-of-two N).
"""
import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from parity_helpers import (SMALL, Uploaded, check_h, check_routing, device_f32, say,
                            small_inputs, to_device, tol_for)

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mixture_experts_ffn_fp32_amd")

@pytest.fixture(scope="module", params=sorted(SMALL))
def small(request):
    say(f"upload {request.param}")
    return Uploaded(small_inputs(request.param))


def test_route(small):
    w = small.w
    say(f"route {w.name}")
    idx, gate, scores = mx.route(small.u, small.E, w.K, small.bias, want_scores=True)
    torch.cuda.synchronize()
    s_ref = oracle.affinity_scores(small.inp.u_f32(), small.inp.E_gate_f32(), small.inp.gate_bias())
    sc = scores.cpu().numpy()
    assert np.all(np.abs(sc - s_ref) <= 1e-5 * s_ref + 1e-9)
    check_routing(idx.cpu().numpy(), gate.cpu().numpy(), s_ref, w.K)


@pytest.mark.parametrize("name", ["decode_n256_bf16", "one_token_bf16", "k_equals_n_f32"])
def test_route_small_batch_kernels_agree(name, monkeypatch):
    """Batches of at most 128 tokens use the one-block-per-token router; the tiled
    router (MOE_ROUTER_SMALL=0) must give the same routing wherever the margin is
    clear, and both must meet the oracle's bar."""
    up = Uploaded(small_inputs(name))
    w = up.w
    say(f"route small-batch kernels {w.name}")
    idx_s, gate_s, sc_s = mx.route(up.u, up.E, w.K, up.bias, want_scores=True)
    monkeypatch.setenv("MOE_ROUTER_SMALL", "0")
    idx_t, gate_t, sc_t = mx.route(up.u, up.E, w.K, up.bias, want_scores=True)
    torch.cuda.synchronize()
    s_ref = oracle.affinity_scores(up.inp.u_f32(), up.inp.E_gate_f32(), up.inp.gate_bias())
    for idx, gate, sc in ((idx_s, gate_s, sc_s), (idx_t, gate_t, sc_t)):
        assert np.all(np.abs(sc.cpu().numpy() - s_ref) <= 1e-5 * s_ref + 1e-9)
        check_routing(idx.cpu().numpy(), gate.cpu().numpy(), s_ref, w.K)


def _tie_inputs(T, d, N, K, pattern, dtype, with_bias, seed):
    """Router inputs whose scores have planted EXACT ties: every token ranks the experts in
    the same order (expert perm[r] at rank r, logits about one unit apart, the top one near
    0), and the experts of one tie group have bit-identical centroid rows (and biases), so
    their logits are equal on both sides whatever the token.  `pattern` lists the rank
    groups that tie."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(N)
    level = np.zeros(N, dtype=np.float32)
    noise = rng.standard_normal((N, d - 1)).astype(np.float32) * 0.01
    bias = rng.standard_normal(N).astype(np.float32) * 0.05
    lead = {}
    for grp in pattern:
        for r in grp[1:]:
            lead[r] = grp[0]
    for r in range(N):
        level[perm[r]] = -0.5 * lead.get(r, r)
        noise[perm[r]] = noise[perm[lead.get(r, r)]]
        bias[perm[r]] = bias[perm[lead.get(r, r)]]
    E = np.concatenate([level[:, None], noise], axis=1)
    u = rng.standard_normal((T, d)).astype(np.float32) * 0.5
    u[:, 0] = 2.0 + 0.25 * rng.random(T).astype(np.float32)
    if dtype == "bf16":
        E = moe_inputs.bf16_bits_to_f32(moe_inputs.f32_to_bf16_bits(E))
        u = moe_inputs.bf16_bits_to_f32(moe_inputs.f32_to_bf16_bits(u))
    tie_sets = [sorted(int(perm[r]) for r in grp) for grp in pattern]
    return u, E, (bias if with_bias else None), tie_sets


TIE_CASES = {
    # (T, d, N, K, tie groups of ranks)
    "boundary_pair": (100, 128, 16, 4, [(3, 4), (0, 1)]),
    "boundary_triple": (300, 256, 64, 6, [(4, 5, 6)]),
    "boundary_pair_tiled": (300, 128, 16, 4, [(3, 4)]),
    "top1_pair": (70, 64, 8, 1, [(0, 1)]),
    "decode_n256_pair": (64, 256, 256, 8, [(7, 8), (2, 3, 4)]),
}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", sorted(TIE_CASES))
@pytest.mark.parametrize("router", ["auto", "tiled"])
def test_route_exact_ties_go_to_lower_index(case, dtype, router, monkeypatch):
    """Exact ties at the K-th / (K+1)-th rank (and inside the top-K) are broken towards
    the lower expert index, bit-exact, by both router kernels (one block per token for
    T <= 128, the tiled kernel otherwise or with MOE_ROUTER_SMALL=0)."""
    T, d, N, K, pattern = TIE_CASES[case]
    for with_bias in (False, True):
        u, E, bias, tie_sets = _tie_inputs(T, d, N, K, pattern, dtype, with_bias,
                                           seed=4000 + sorted(TIE_CASES).index(case))
        s_ref = oracle.affinity_scores(u, E, bias)
        idx_ref, g_ref, margin = oracle.top_k_gates(s_ref, K)
        boundary = any(K - 1 in grp and K in grp for grp in pattern)
        if boundary:
            assert np.all(margin == 0.0)     # the planted tie really is exact
        if router == "tiled":
            monkeypatch.setenv("MOE_ROUTER_SMALL", "0")
        say(f"route ties {case} {dtype} bias={with_bias} router={router} T={T} N={N} K={K}")
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        ud = torch.from_numpy(u).to("cuda", tdt)
        Ed = torch.from_numpy(E).to("cuda", tdt)
        bd = None if bias is None else torch.from_numpy(bias).cuda()
        idx, gate, scores = mx.route(ud, Ed, K, bd, want_scores=True)
        torch.cuda.synchronize()
        monkeypatch.delenv("MOE_ROUTER_SMALL", raising=False)
        ig = idx.cpu().numpy()
        sc = scores.cpu().numpy()
        for grp in tie_sets:                 # equal on the GPU too
            assert np.all(sc[:, grp] == sc[:, grp[:1]])
        np.testing.assert_array_equal(ig, idx_ref)   # set and order, bit-exact
        # logits of a few units here (float32 products and sums of inputs this large move
        # a score by ~|z| 2^-24 sqrt(d) relative), so the gates get a wider band
        np.testing.assert_allclose(gate.cpu().numpy(), g_ref, rtol=1e-4)
        check_routing(ig, gate.cpu().numpy(), s_ref, K, gate_rtol=1e-4)


def test_dispatch(small):
    w = small.w
    s_ref = oracle.affinity_scores(small.inp.u_f32(), small.inp.E_gate_f32(), small.inp.gate_bias())
    idx_ref, _, _ = oracle.top_k_gates(s_ref, w.K)
    say(f"dispatch {w.name}")
    counts, offsets, sp = mx.dispatch(torch.from_numpy(idx_ref.astype(np.int32)).cuda(), w.N)
    torch.cuda.synchronize()
    c_ref, o_ref, sp_ref = oracle.permute_by_expert(idx_ref, w.N)
    np.testing.assert_array_equal(counts.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(offsets.cpu().numpy(), o_ref)
    np.testing.assert_array_equal(sp.cpu().numpy(), sp_ref)


@pytest.mark.parametrize("T,N,K", [(65, 7, 3), (700, 12, 3), (4096, 63, 7), (20000, 256, 8)])
def test_dispatch_sizes(T, N, K):
    """The tiled dispatch at sizes on both sides of its one-launch form (every block
    re-deriving the scan it needs, while the tile counts are small enough to read whole:
    N x tiles up to 16384 counts) and the separate scan and scatter launches beyond it
    (T = 20000, N = 256): integer exact against the oracle, with random expert ids (each
    token's K distinct)."""
    rng = np.random.default_rng(7000 + T)
    idx = np.stack([rng.choice(N, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    say(f"dispatch T={T} N={N} K={K}")
    counts, offsets, sp = mx.dispatch(torch.from_numpy(idx).cuda(), N)
    torch.cuda.synchronize()
    c_ref, o_ref, sp_ref = oracle.permute_by_expert(idx, N)
    np.testing.assert_array_equal(counts.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(offsets.cpu().numpy(), o_ref)
    np.testing.assert_array_equal(sp.cpu().numpy(), sp_ref)


def test_expert_ffn(small):
    w = small.w
    inp = small.inp
    u = inp.u_f32()
    s_ref = oracle.affinity_scores(u, inp.E_gate_f32(), inp.gate_bias())
    idx_ref, g_ref, _ = oracle.top_k_gates(s_ref, w.K)
    _, o_ref, sp_ref = oracle.permute_by_expert(idx_ref, w.N)
    say(f"expert_ffn {w.name}")
    H, Hs, Y, Ys = mx.expert_ffn(small.u, small.W_routed, small.W_shared, w.N, w.K, w.K_s,
                                 torch.from_numpy(o_ref.astype(np.int32)).cuda(),
                                 torch.from_numpy(sp_ref.astype(np.int32)).cuda(),
                                 torch.from_numpy(g_ref.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    per_e, per_s = oracle.expert_slot_activations(u, small.routed, small.shared, idx_ref, g_ref,
                                                  sp_ref, o_ref, w.K, w.K_s)
    tol = tol_for(w)
    Hg, Yg = device_f32(H), device_f32(Y)
    for e, (H_ref, Y_ref) in per_e.items():
        lo, hi = o_ref[e], o_ref[e + 1]
        if hi == lo:
            continue
        assert np.abs(Hg[lo:hi] - H_ref).max() <= tol * np.abs(H_ref).max(), f"H of expert {e}"
        rows = sp_ref[lo:hi]
        assert np.abs(Yg[rows] - Y_ref).max() <= tol * np.abs(Y_ref).max(), f"Y of expert {e}"
    if w.K_s:
        Hsg, Ysg = device_f32(Hs), device_f32(Ys)
        Ys_ref = sum(per_s[j][1] for j in range(w.K_s))
        for j in range(w.K_s):
            H_ref = per_s[j][0]
            got = Hsg[:, j * w.I:(j + 1) * w.I]
            assert np.abs(got - H_ref).max() <= tol * np.abs(H_ref).max(), f"H of shared {j}"
        assert np.abs(Ysg - Ys_ref).max() <= tol * np.abs(Ys_ref).max(), "Y_shared"


def test_combine(small):
    w = small.w
    rng = np.random.default_rng(5)
    T, d, K = w.T, w.d, w.K
    # any values do for this stage; round them to the storage type first
    Yr = (rng.standard_normal((T * K, d)) * 0.1).astype(np.float32)
    Ysr = (rng.standard_normal((T, d)) * 0.1).astype(np.float32)
    if w.dtype == "bf16":
        Yr, Ysr = moe_inputs.f32_to_bf16_bits(Yr), moe_inputs.f32_to_bf16_bits(Ysr)
        Yf, Ysf = moe_inputs.bf16_bits_to_f32(Yr), moe_inputs.bf16_bits_to_f32(Ysr)
    else:
        Yf, Ysf = Yr, Ysr
    say(f"combine {w.name}")
    h = mx.combine(small.u, to_device(Yr, w.dtype), to_device(Ysr, w.dtype) if w.K_s else None,
                   K, w.K_s)
    torch.cuda.synchronize()
    u = small.inp.u_f32()
    ref = oracle.combine_outputs(u, Yf, Ysf if w.K_s else None, K)
    # float32 summation of K + 2 terms: |err| <= (K + 1) * 2^-24 * sum|terms|, then one
    # rounding to the storage type (one bf16 ulp of the result)
    mag = np.abs(u) + (np.abs(Ysf) if w.K_s else 0) + np.abs(Yf).reshape(T, K, d).sum(axis=1)
    bound = (K + 1) * 2.0 ** -24 * mag
    if w.dtype == "bf16":
        bound = bound + np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(device_f32(h) - ref) <= bound)


def test_layer_forward(small):
    w = small.w
    say(f"layer_forward {w.name}")
    h = mx.layer_forward(small.u, small.E, small.W_routed, small.W_shared, w.N, w.K, w.K_s,
                         small.bias)
    idx, gate, _ = mx.route(small.u, small.E, w.K, small.bias)
    torch.cuda.synchronize()
    inp = small.inp
    h_ref, info = oracle.moe_forward_tokens(inp.u_f32(), inp.E_gate_f32(), small.routed,
                                            small.shared, w.N, w.K, w.K_s, inp.gate_bias())
    differing, alts = check_routing(idx.cpu().numpy(), gate.cpu().numpy(), info["s"], w.K)
    for t in differing:   # an admissible near-tie set: compare with the oracle's h for that set
        a_idx, a_g = alts[int(t)]
        h_ref[t] = oracle.moe_forward_given_routing(inp.u_f32()[t:t + 1], a_idx[None], a_g[None],
                                                    small.routed, small.shared, w.K_s)[0]
    check_h(device_f32(h), h_ref, inp.u_f32().astype(np.float64), tol_for(w), w.dtype, w.K,
            w.name)


@pytest.mark.parametrize("name", ["one_token_bf16", "n256_bf16", "decode_n256_bf16",
                                  "gran_m8_ks1_bf16"])
def test_layer_forward_short_run_streaming(name, monkeypatch):
    """Decode-sized bf16 batches take the long-run streaming GEMMs by default;
    MOE_STREAM=short keeps them on the short-run streaming kernel, which must
    match the oracle as well."""
    up = Uploaded(small_inputs(name))
    w = up.w
    say(f"layer_forward MOE_STREAM=short {w.name}")
    monkeypatch.setenv("MOE_STREAM", "short")
    h = mx.layer_forward(up.u, up.E, up.W_routed, up.W_shared, w.N, w.K, w.K_s, up.bias)
    idx, gate, _ = mx.route(up.u, up.E, w.K, up.bias)
    torch.cuda.synchronize()
    inp = up.inp
    h_ref, info = oracle.moe_forward_tokens(inp.u_f32(), inp.E_gate_f32(), up.routed, up.shared,
                                            w.N, w.K, w.K_s, inp.gate_bias())
    differing, alts = check_routing(idx.cpu().numpy(), gate.cpu().numpy(), info["s"], w.K)
    for t in differing:
        a_idx, a_g = alts[int(t)]
        h_ref[t] = oracle.moe_forward_given_routing(inp.u_f32()[t:t + 1], a_idx[None], a_g[None],
                                                    up.routed, up.shared, w.K_s)[0]
    check_h(device_f32(h), h_ref, inp.u_f32().astype(np.float64), tol_for(w), w.dtype, w.K,
            w.name)


@pytest.mark.parametrize("name", ["decode_n256_bf16", "k_equals_n_f32", "one_token_bf16"])
def test_layer_forward_tiled_router_small_batch(name, monkeypatch):
    """MOE_ROUTER_SMALL=0 sends batches of at most 128 tokens to the tiled router, which
    then also writes the dispatch ranks of its 32-token blocks when the batch has more
    than 64 tokens (T = 96 and 70 here; T = 1 keeps the one-launch dispatch): the layer
    must match the oracle on that path as well."""
    up = Uploaded(small_inputs(name))
    w = up.w
    say(f"layer_forward MOE_ROUTER_SMALL=0 {w.name}")
    monkeypatch.setenv("MOE_ROUTER_SMALL", "0")
    h = mx.layer_forward(up.u, up.E, up.W_routed, up.W_shared, w.N, w.K, w.K_s, up.bias)
    idx, gate, _ = mx.route(up.u, up.E, w.K, up.bias)
    torch.cuda.synchronize()
    inp = up.inp
    h_ref, info = oracle.moe_forward_tokens(inp.u_f32(), inp.E_gate_f32(), up.routed, up.shared,
                                            w.N, w.K, w.K_s, inp.gate_bias())
    differing, alts = check_routing(idx.cpu().numpy(), gate.cpu().numpy(), info["s"], w.K)
    for t in differing:
        a_idx, a_g = alts[int(t)]
        h_ref[t] = oracle.moe_forward_given_routing(inp.u_f32()[t:t + 1], a_idx[None], a_g[None],
                                                    up.routed, up.shared, w.K_s)[0]
    check_h(device_f32(h), h_ref, inp.u_f32().astype(np.float64), tol_for(w), w.dtype, w.K,
            w.name)


@pytest.mark.parametrize("name", ["pp_ragged_bf16", "decode_n256_bf16", "one_token_bf16"])
def test_stage_timing_covers_every_launched_stage(name):
    """Timing on: every stage the forward launches reports one launch per call with a
    positive time (the events ride on the stage's kernel dispatches), stages limited by the
    mask report nothing, and the output is the same bits as without timing."""
    up = Uploaded(small_inputs(name))
    w = up.w
    say(f"stage timing {w.name}")
    args = (up.u, up.E, up.W_routed, up.W_shared, w.N, w.K, w.K_s, up.bias)
    h0 = mx.layer_forward(*args)
    torch.cuda.synchronize()
    mx.timing_read()
    mx.timing_enable(True)
    h1 = mx.layer_forward(*args)
    h2 = mx.layer_forward(*args)
    torch.cuda.synchronize()
    mx.timing_enable(False)
    st = mx.timing_read()
    small_batch = w.T <= 64      # one dispatch launch (timed as tile_rank) ...
    # ... unless GEMM1 derives the dispatch itself (a bf16 decode batch on the
    # long-run streaming kernel, as these small shapes are)
    derived = small_batch and w.dtype == "bf16" and w.T * w.K <= 1024
    tiled_router = w.T > 128     # the router also writes the dispatch ranks
    expect = {"router", "expert_gemm1_swiglu", "expert_gemm2_down", "combine"}
    if (small_batch and not derived) or (not small_batch and not tiled_router):
        expect.add("tile_rank")
    if not small_batch:
        expect.add("scatter")    # (with the scan, in one launch at these sizes)
    for name_, (ms, n) in st.items():
        if name_ in expect:
            assert n == 2 and ms > 0, (name_, ms, n)
        else:
            assert n == 0, (name_, ms, n)
    mx.timing_enable(True, ["expert_gemm1_swiglu"])
    h3 = mx.layer_forward(*args)
    torch.cuda.synchronize()
    mx.timing_enable(False)
    st = mx.timing_read()
    assert st["expert_gemm1_swiglu"][1] == 1 and st["expert_gemm1_swiglu"][0] > 0
    assert sum(n for k, (_, n) in st.items() if k != "expert_gemm1_swiglu") == 0
    for hx in (h1, h2, h3):
        assert torch.equal(hx, h0)


def test_deterministic_and_chunk_invariant(small):
    w = small.w
    if w.T < 4:
        pytest.skip("needs a few tokens")
    say(f"determinism {w.name}")
    args = (small.E, small.W_routed, small.W_shared, w.N, w.K, w.K_s, small.bias)
    h1 = mx.layer_forward(small.u, *args)
    h2 = mx.layer_forward(small.u, *args)
    a = w.T // 3
    ha = mx.layer_forward(small.u[:a].contiguous(), *args)
    hb = mx.layer_forward(small.u[a:].contiguous(), *args)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)
    hc = torch.cat([ha, hb])
    tol = tol_for(w) * h1.float().abs().max().item()
    assert (hc.float() - h1.float()).abs().max().item() <= tol


@pytest.mark.parametrize("name", ["one_token_bf16", "k_equals_n_f32", "decode_n256_bf16"])
def test_shared_experts_beside_routing_same_bits(name, monkeypatch):
    """With MOE_SHARED_SIDE=1, batches of at most 128 tokens run the shared
    experts' GEMMs on a second stream while the router and the dispatch run;
    the result must be the same bits as with every expert in the same
    launches (the default): each tile is the same arithmetic either way."""
    up = Uploaded(small_inputs(name))
    w = up.w
    assert w.K_s > 0 and w.T <= 128
    say(f"shared experts beside routing {w.name}")
    args = (up.E, up.W_routed, up.W_shared, w.N, w.K, w.K_s, up.bias)
    monkeypatch.setenv("MOE_SHARED_SIDE", "1")
    h_side = mx.layer_forward(up.u, *args)
    torch.cuda.synchronize()
    monkeypatch.setenv("MOE_SHARED_SIDE", "0")
    h_one = mx.layer_forward(up.u, *args)
    torch.cuda.synchronize()
    assert torch.equal(h_side, h_one)


def test_empty_batch():
    inp = small_inputs("ragged_bf16")
    up = Uploaded(inp)
    w = inp.w
    say("empty batch")
    h = mx.layer_forward(up.u[:0], up.E, up.W_routed, up.W_shared, w.N, w.K, w.K_s)
    torch.cuda.synchronize()
    assert h.shape == (0, w.d)


def _check_balance(res, ref, groups):
    f, P = res["f"].cpu().numpy(), res["P"].cpu().numpy()
    # f_i = N count_i / (K T): an exact rational rounded once to float32
    np.testing.assert_allclose(f, ref["f"], rtol=2.0 ** -23, atol=0)
    np.testing.assert_allclose(P, ref["P"], rtol=2.0 ** -22, atol=1e-30)
    assert abs(float(res["L_ExpBal"]) - ref["L_ExpBal"]) <= 2.0 ** -22 * abs(ref["L_ExpBal"])
    if groups is not None:
        np.testing.assert_allclose(res["f_dev"].cpu().numpy(), ref["f_dev"], rtol=2.0 ** -22)
        np.testing.assert_allclose(res["P_dev"].cpu().numpy(), ref["P_dev"], rtol=2.0 ** -22)
        assert abs(float(res["L_DevBal"]) - ref["L_DevBal"]) <= 2.0 ** -22 * abs(ref["L_DevBal"])


@pytest.mark.parametrize("grouping", ["none", "contiguous", "scattered"])
def test_balance_statistics(small, grouping):
    """Balance statistics of the GPU's own routing against the oracle's formulas on the
    same scores and indices (float32 scores read exactly as float64)."""
    w = small.w
    idx, _, scores = mx.route(small.u, small.E, w.K, small.bias, want_scores=True)
    D = min(4, w.N)
    if grouping == "none":
        group_of = None
    elif grouping == "contiguous":
        group_of = [i * D // w.N for i in range(w.N)]
    else:
        perm = np.random.default_rng(w.seed).permutation(w.N)
        group_of = [int(perm[i]) % D for i in range(w.N)]
    say(f"balance {w.name} {grouping}")
    res = mx.balance_stats(scores, idx, w.K, group_of, alpha1=0.003, alpha2=0.05)
    res2 = mx.balance_stats(scores, idx, w.K, group_of, alpha1=0.003, alpha2=0.05)
    torch.cuda.synchronize()
    groups = None if group_of is None else [[i for i in range(w.N) if group_of[i] == g]
                                            for g in range(D)]
    ref = oracle.balance_statistics(scores.cpu().numpy().astype(np.float64), idx.cpu().numpy(),
                                    w.K, groups, alpha1=0.003, alpha2=0.05)
    _check_balance(res, ref, groups)
    for k in res:   # fixed summation order: identical bits on a second call
        assert torch.equal(res[k], res2[k]), k
    # the sums the definitions fix: sum_i f_i = N, sum_i P_i = 1
    assert abs(float(res["f"].double().sum()) - w.N) <= 1e-5 * w.N
    assert abs(float(res["P"].double().sum()) - 1.0) <= 1e-5


def test_balance_statistics_ignores_out_of_range_indices():
    T, N, K = 257, 12, 3
    rng = np.random.default_rng(7)
    s = rng.random((T, N))
    s /= s.sum(axis=1, keepdims=True)
    idx = np.stack([rng.permutation(N)[:K] for _ in range(T)]).astype(np.int32)
    bad = idx.copy()
    bad[::5, 0] = -1
    bad[1::7, 1] = N
    say("balance out-of-range indices")
    res = mx.balance_stats(torch.from_numpy(s.astype(np.float32)).cuda(),
                           torch.from_numpy(bad).cuda(), K)
    torch.cuda.synchronize()
    keep = (bad >= 0) & (bad < N)
    counts = np.bincount(bad[keep], minlength=N)
    np.testing.assert_allclose(res["f"].cpu().numpy(), N / (K * T) * counts, rtol=2.0 ** -23)
    np.testing.assert_allclose(res["P"].cpu().numpy(),
                               s.astype(np.float32).astype(np.float64).sum(0) / T, rtol=2.0 ** -22)
