"""The allocation-free layer forward (moe_layer_forward_static) through the C ABI.

It runs the same kernels as moe_layer_forward on the library's static device
scratch instead of a caller workspace, so for the same inputs it must give the
same bits; two calls in a row (the second on a smaller batch, over the first
call's leftovers in the scratch) are checked against moe_layer_forward and
against the float64 oracle's bar.
"""
import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from parity_helpers import Uploaded, check_h, check_routing, device_f32, say, small_inputs, tol_for

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mixture_experts_ffn_fp32_amd")


def _oracle_check(up, h, T):
    w = up.w
    inp = up.inp
    tokens = np.arange(T)
    h_ref, info = oracle.moe_forward_tokens(inp.u_f32(), inp.E_gate_f32(), up.routed, up.shared,
                                            w.N, w.K, w.K_s, inp.gate_bias(), tokens)
    idx, gate, _ = mx.route(up.u[:T], up.E, w.K, up.bias)
    torch.cuda.synchronize()
    differing, alts = check_routing(idx.cpu().numpy(), gate.cpu().numpy(), info["s"], w.K)
    for t in differing:
        a_idx, a_g = alts[int(t)]
        h_ref[t] = oracle.moe_forward_given_routing(inp.u_f32()[t:t + 1], a_idx[None], a_g[None],
                                                    up.routed, up.shared, w.K_s)[0]
    check_h(device_f32(h), h_ref, inp.u_f32()[:T].astype(np.float64), tol_for(w), w.dtype, w.K,
            f"{w.name} T={T} static")


@pytest.mark.parametrize("case", ["moe16b_decode_bf16", "ragged_f32", "n63_bf16"])
def test_static_forward_matches_workspace_forward(case):
    up = Uploaded(moe_inputs.make(case) if case in moe_inputs.WORKLOADS else small_inputs(case))
    w = up.w
    for T in (w.T, max(1, w.T // 3)):       # the second call on a smaller batch
        u = up.u[:T].contiguous()
        say(f"static forward {w.name} T={T}")
        h_static = mx.layer_forward_static(u, up.E, up.W_routed, up.W_shared, w.N, w.K, w.K_s,
                                           up.bias)
        say(f"workspace forward {w.name} T={T}")
        h_ws = mx.layer_forward(u, up.E, up.W_routed, up.W_shared, w.N, w.K, w.K_s, up.bias)
        torch.cuda.synchronize()
        assert torch.equal(h_static.view(torch.int16 if w.dtype == "bf16" else torch.int32),
                           h_ws.view(torch.int16 if w.dtype == "bf16" else torch.int32)), \
            f"{w.name} T={T}: static-scratch forward differs from the workspace forward"
        _oracle_check(up, h_static, T)


def test_static_forward_refuses_shapes_beyond_the_scratch():
    up = Uploaded(small_inputs("wide_tokens_bf16"))
    w = up.w
    big = torch.zeros((16384, w.d), dtype=torch.bfloat16, device="cuda")
    say("static forward refusal")
    with pytest.raises(mx.MoEError) as ei:
        mx.layer_forward_static(big, up.E, up.W_routed, up.W_shared, w.N, w.K, w.K_s, up.bias)
    assert ei.value.status == 3 and "static scratch" in ei.value.message
