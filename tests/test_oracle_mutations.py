"""The oracle's pins catch planted mistakes.

Each case copies the oracle into a temporary directory, plants one plausible
mistake in the copy (CPU only), and runs the pin tests against that copy: the
run must fail.  The real oracle is never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    "renormalised_gates": ('g = np.take_along_axis(s, idx, axis=1)',
                           'g = np.take_along_axis(s, idx, axis=1); g = g / g.sum(axis=1, keepdims=True)'),
    "ties_to_higher_index": ('order = np.argsort(-s, axis=1, kind="stable")',
                             'order = s.shape[1] - 1 - np.argsort(-s[:, ::-1], axis=1, kind="stable")'),
    "smallest_k": ('order = np.argsort(-s, axis=1, kind="stable")',
                   'order = np.argsort(s, axis=1, kind="stable")'),
    "softmax_over_tokens": ('ez / ez.sum(axis=1, keepdims=True)', 'ez / ez.sum(axis=0, keepdims=True)'),
    "silu_on_up_branch": ('return (silu * b) @ _f64(W_down).T',
                          'return (b / (1.0 + np.exp(-b)) * a) @ _f64(W_down).T'),
    "sigmoid_not_silu": ('silu = a / (1.0 + np.exp(-a))            # SiLU(a) = a * sigmoid(a)',
                         'silu = 1 / (1.0 + np.exp(-a))'),
    "no_residual": ('h = u.copy()                                 # residual term u_t',
                    'h = np.zeros_like(u)'),
    "gated_shared_expert": ('h += swiglu_ffn(u, *_expert(shared, j))  # shared: coefficient 1',
                            'h += 0.5 * swiglu_ffn(u, *_expert(shared, j))'),
    "bias_dropped": ('        z = z + _f64(gate_bias)[None, :]\n', '        pass\n'),
    "unstable_permutation": ('sorted_pair = np.argsort(flat, kind="stable")',
                             'sorted_pair = np.argsort(flat, kind="stable")[::-1]'),
    "margin_wrong_neighbour": ('margin = g[:, K - 1] - nxt', 'margin = g[:, 0] - nxt'),
    "device_f_sum_not_mean": ('fg = np.array([f[list(gr)].mean() for gr in groups])',
                              'fg = np.array([f[list(gr)].sum() for gr in groups])'),
    "device_P_mean_not_sum": ('Pg = np.array([P[list(gr)].sum() for gr in groups])',
                              'Pg = np.array([P[list(gr)].mean() for gr in groups])'),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "moe_oracle.py")).read()
    assert before in src, "mutation anchor no longer present in the oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle")
    shutil.copytree(os.path.join(ROOT, "moe_inputs"), tmp_path / "moe_inputs")
    (tmp_path / "tests").mkdir()
    for f in ("test_oracle_pins.py", "conftest.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    (tmp_path / "oracle" / "moe_oracle.py").write_text(src.replace(before, after))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        str(tmp_path / "tests" / "test_oracle_pins.py")],
                       cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"planted mistake {name!r} passed every pin:\n{r.stdout[-2000:]}"


# Planted mistakes in the backward oracle; tests/test_oracle_backward.py must catch each.
BACKWARD_MUTATIONS = {
    "silu_grad_is_sigmoid": ('return sig * (1.0 + a * (1.0 - sig))', 'return sig'),
    "routed_dy_without_gate": ('y, dx, dWg, dWu, dWd = swiglu_ffn_backward(u[rows], *Wi, gi * dh[rows])',
                               'y, dx, dWg, dWu, dWd = swiglu_ffn_backward(u[rows], *Wi, dh[rows])'),
    "softmax_backward_no_centering": ('dz = s * (ds - np.sum(s * ds, axis=1, keepdims=True))',
                                      'dz = s * ds'),
    "no_residual_gradient": ('du = dh.copy()                                     # residual',
                             'du = np.zeros_like(dh)'),
    "dc_uses_silu_grad": ('dc = dp * silu(a)', 'dc = dp * silu_grad(a)'),
    "gate_scales_ds": ('ds[rows, i] = np.sum(dh[rows] * y, axis=1)',
                       'ds[rows, i] = np.sum(gi * dh[rows] * y, axis=1)'),
    "router_gradient_dropped": ('du += dz @ _f64(E_gate)', 'pass'),
    "gate_and_up_swapped": ('dx = da @ Wg + dc @ Wu', 'dx = da @ Wu + dc @ Wg'),
}


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTATIONS))
def test_backward_pins_catch_planted_mistake(name, tmp_path):
    before, after = BACKWARD_MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "moe_backward.py")).read()
    assert before in src, "mutation anchor no longer present in the backward oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle")
    shutil.copytree(os.path.join(ROOT, "moe_inputs"), tmp_path / "moe_inputs")
    (tmp_path / "tests").mkdir()
    for f in ("test_oracle_backward.py", "conftest.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    (tmp_path / "oracle" / "moe_backward.py").write_text(src.replace(before, after))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        str(tmp_path / "tests" / "test_oracle_backward.py")],
                       cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"planted mistake {name!r} passed every pin:\n{r.stdout[-2000:]}"
