"""The seeded input generator: determinism, bf16 rounding, per-expert streams."""
import numpy as np
import pytest

import moe_inputs


def test_bf16_rounding_matches_torch_rne():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 3,
                        # exact halfway cases: low 16 bits = 0x8000, both parities of bit 16
                        (np.arange(1000, dtype=np.uint32) * 0x10000 + 0x3F808000).view(np.float32),
                        np.array([0.0, -0.0, 1e-30, -7.5e20], dtype=np.float32)])
    ours = moe_inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = moe_inputs.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_deterministic_and_independent_streams():
    a = moe_inputs.make("moe2b_bf16", T=8)
    b = moe_inputs.make("moe2b_bf16", T=8)
    np.testing.assert_array_equal(a.u_raw(), b.u_raw())
    np.testing.assert_array_equal(a.routed_block_raw(5), b.routed_block_raw(5))
    assert not np.array_equal(a.routed_block_raw(5), a.routed_block_raw(6))
    # the T override changes u's length, not its leading values
    c = moe_inputs.make("moe2b_bf16", T=16)
    np.testing.assert_array_equal(c.u_raw()[:8], a.u_raw())


def test_distribution_scale():
    inp = moe_inputs.make("tiny_fp32")
    u = inp.u_f32()
    assert abs(u.std() - 1) < 0.02 and abs(u.mean()) < 0.02
    Wg, Wu, Wd = inp.routed_expert_f32(0)
    assert Wg.shape == (128, 256) and Wd.shape == (256, 128)
    assert abs(np.concatenate([Wg.ravel(), Wu.ravel(), Wd.ravel()]).std() - 0.02) < 0.001


def test_parallel_block_draw_equals_single():
    inp = moe_inputs.make("tiny_fp32")
    allb = inp.routed_all_raw(threads=4)
    for e in (0, 7, 15):
        np.testing.assert_array_equal(allb[e], inp.routed_block_raw(e))


def test_zipf_bias_profile():
    inp = moe_inputs.make("moe145b_skewed_bf16", T=1)
    b = inp.gate_bias().astype(np.float64)
    r = np.exp(-b / 1.1)                       # recovers the ranks 1..N
    np.testing.assert_allclose(np.sort(r), np.arange(1, 129), rtol=1e-5)
    p = np.exp(b) / np.exp(b).sum()
    ranks = np.rint(r).astype(int)
    np.testing.assert_allclose(p, ranks ** -1.1 / (np.arange(1, 129) ** -1.1).sum(), rtol=1e-5)
    assert moe_inputs.make("moe16b_prefill_bf16", T=1).gate_bias() is None


def test_granularity_sweep_keeps_parameters_and_compute():
    """Every point of the sweep has the conventional layer's expert parameters and
    per-token expert FLOPs ([DSMoE] sec. 3.1/3.2, Fig. 2: both stay unchanged)."""
    base = moe_inputs.granularity(1, 0)
    assert (base.N, base.K, base.K_s, base.I) == (16, 2, 0, 5632)
    params = lambda w: (w.N + w.K_s) * 3 * w.I * w.d           # noqa: E731
    expert_flops = lambda w: 6 * w.d * w.I * (w.K + w.K_s)     # noqa: E731
    for m, ks in moe_inputs.GRANULARITY_SWEEP:
        w = moe_inputs.granularity(m, ks)
        assert params(w) == params(base), (m, ks)
        assert expert_flops(w) == expert_flops(base), (m, ks)
        assert w.N + w.K_s == 16 * m and w.K + w.K_s == 2 * m
        assert w.I % 64 == 0
