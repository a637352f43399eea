"""GPU parity of the layer backward: the HIP path through the C ABI against the
float64 backward oracle (chain rule with each token's top-K set held fixed).

Bars: every gradient tensor within tol * max|reference| of the oracle, where tol
is the forward's (2e-2 for bfloat16 storage, 1e-4 for float32); per expert and
per matrix for the weight gradients, so a mistake confined to one expert or one
of W_gate / W_up / W_down shows.  Experts no token selects must get exact zeros.
Tokens whose GPU top-K set is an admissible near-tie alternative are compared
with the oracle holding that alternative set fixed.
"""
import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from parity_helpers import (SMALL, Uploaded, check_routing, device_f32, say, small_inputs,
                            to_device, tol_for)

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mixture_experts_ffn_fp32_amd")


def _close(got, ref, tol, label):
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max() if ref.size else 0.0
    err = np.abs(np.asarray(got, dtype=np.float64) - ref).max() if ref.size else 0.0
    assert err <= tol * scale, f"{label}: max|err| {err:.3e} > {tol} * {scale:.3e}"


def run_backward(up, bias=None):
    w = up.w
    dh = to_device(up.inp.dh_raw(), w.dtype)
    say(f"layer_backward {w.name} T={w.T} d={w.d} I={w.I} N={w.N} K={w.K} K_s={w.K_s} {w.dtype}")
    out = mx.layer_backward(up.u, up.E, up.W_routed, up.W_shared, w.N, w.K, w.K_s, dh,
                            up.bias if bias is None else bias)
    idx, gate, _ = mx.route(up.u, up.E, w.K, up.bias if bias is None else bias)
    torch.cuda.synchronize()
    return out, idx.cpu().numpy(), gate.cpu().numpy()


def reference(up, idx_gpu, gate_gpu, bias=None):
    w, inp = up.w, up.inp
    b = inp.gate_bias() if bias is None else bias.cpu().numpy()
    s_ref = oracle.affinity_scores(inp.u_f32(), inp.E_gate_f32(), b)
    differing, alts = check_routing(idx_gpu, gate_gpu, s_ref, w.K)
    return oracle.moe_layer_backward(inp.u_f32(), inp.E_gate_f32(), up.routed, up.shared, w.N,
                                     w.K, w.K_s, inp.dh_f32(), b,
                                     replace_sets={int(t): alts[int(t)] for t in differing})


def check_gradients(w, out, ref):
    du, dE, db, dWr, dWs = out
    tol = tol_for(w)
    _close(device_f32(du), ref["du"], tol, "du")
    _close(dE.cpu().numpy(), ref["dE_gate"], tol, "dE_gate")
    _close(db.cpu().numpy(), ref["dgate_bias"], tol, "dgate_bias")
    Id = w.I * w.d
    dWr = dWr.cpu().numpy().reshape(w.N, 3 * Id)
    names = ("dW_gate", "dW_up", "dW_down")
    for e in range(w.N):
        for m, r in enumerate(ref["d_routed"][e]):
            _close(dWr[e, m * Id:(m + 1) * Id].reshape(r.shape), r, tol, f"routed {e} {names[m]}")
    if w.K_s:
        dWs = dWs.cpu().numpy().reshape(w.K_s, 3 * Id)
        for j in range(w.K_s):
            for m, r in enumerate(ref["d_shared"][j]):
                _close(dWs[j, m * Id:(m + 1) * Id].reshape(r.shape), r, tol,
                       f"shared {j} {names[m]}")


@pytest.mark.parametrize("name", sorted(SMALL))
def test_layer_backward(name):
    up = Uploaded(small_inputs(name))
    out, idx, gate = run_backward(up)
    check_gradients(up.w, out, reference(up, idx, gate))


def test_layer_backward_with_bias_and_unused_experts():
    """A strong logit bias leaves some experts unselected: their weight gradients are
    exact zeros, and the bias gradient matches the oracle."""
    up = Uploaded(small_inputs("ragged_bf16"))
    w = up.w
    b = np.zeros(w.N, dtype=np.float32)
    b[: w.N // 2] = -30.0          # softmax weight ~e^-30: never in any top-5 of 20
    bias = torch.from_numpy(b).cuda()
    out, idx, gate = run_backward(up, bias)
    assert idx.max() >= w.N // 2 and idx.min() >= w.N // 2
    ref = reference(up, idx, gate, bias)
    check_gradients(w, out, ref)
    dWr = out[3].view(w.N, -1)
    assert torch.count_nonzero(dWr[: w.N // 2]).item() == 0


def test_backward_is_deterministic():
    up = Uploaded(small_inputs("n63_bf16"))
    a, _, _ = run_backward(up)
    b, _, _ = run_backward(up)
    for x, y in zip(a, b):
        if x is not None:
            assert torch.equal(x, y)


def test_backward_empty_batch():
    up = Uploaded(small_inputs("ragged_bf16"))
    w = up.w
    say("layer_backward empty batch")
    du, dE, db, dWr, dWs = mx.layer_backward(up.u[:0], up.E, up.W_routed, up.W_shared, w.N, w.K,
                                             w.K_s, up.u[:0])
    torch.cuda.synchronize()
    assert du.shape == (0, w.d)
    assert torch.count_nonzero(dWr).item() == 0 and torch.count_nonzero(dE).item() == 0


@pytest.mark.timeout(600)
def test_layer_backward_16b_prefill_full():
    """The 16B-shaped prefill layer (T=8192, d=2048, 64 routed + 2 shared experts,
    top-6, I=1408, bf16) in the launch configuration the benchmark times: every
    gradient element against the float64 oracle (about 15 s of CPU)."""
    up = Uploaded(moe_inputs.make("moe16b_prefill_bf16"))
    out, idx, gate = run_backward(up)
    check_gradients(up.w, out, reference(up, idx, gate))


@pytest.mark.parametrize("name", ["ragged_bf16", "n63_bf16", "gran_m8_ks1_bf16"])
def test_layer_backward_generic_kernels_bf16(name, monkeypatch):
    """bfloat16 through the generic grouped kernels (the float32 path's) instead of
    the pipelined ones: the same bar against the oracle."""
    monkeypatch.setenv("MOE_BWD_GENERIC", "1")
    up = Uploaded(small_inputs(name))
    out, idx, gate = run_backward(up)
    check_gradients(up.w, out, reference(up, idx, gate))


@pytest.mark.timeout(600)
def test_layer_backward_2b_full():
    """The 2B-shaped layer (T=4096, d=1280, 63 routed + 1 shared experts, top-7,
    I=896, bf16): a routed-expert count that is not a power of two and an n-tile
    count of 7; every gradient element against the float64 oracle."""
    up = Uploaded(moe_inputs.make("moe2b_bf16"))
    out, idx, gate = run_backward(up)
    check_gradients(up.w, out, reference(up, idx, gate))
