"""CPU checks of the routing-parity rule the GPU tests apply (tests/parity_helpers.py).

The rule must accept exactly the routings that are correct in finite precision:
the oracle's set where the K-th vs (K+1)-th margin is clear, either side of a
near-tie group at the boundary (of any size), and only the lower index on an
exact tie ([DSMoE] A3: exactly K gates are non-zero; ties go to the lower index).
"""
import numpy as np
import pytest

import oracle
from parity_helpers import admissible_set, check_routing


def test_exact_tie_only_lower_index():
    s = np.array([0.4, 0.2, 0.1, 0.2, 0.1])          # experts 1 and 3 tie at rank 2 / 3
    assert admissible_set(s, 2, [0, 1])
    assert not admissible_set(s, 2, [0, 3])           # the higher index of the tie
    idx, g, _ = oracle.top_k_gates(s[None], 2)
    with pytest.raises(AssertionError, match="exact tie"):
        check_routing(np.array([[0, 3]]), s[[0, 3]][None].astype(np.float32), s[None], 2)
    check_routing(idx.astype(np.int32), g.astype(np.float32), s[None], 2)


def test_three_way_near_tie_any_split():
    eps = 1e-7
    s = np.array([0.5, 0.2, 0.2 + eps, 0.2 - eps, 0.1 - eps])
    s = s / s.sum()
    for chosen in ([0, 1], [0, 2], [0, 3]):
        assert admissible_set(s, 2, chosen)
    assert not admissible_set(s, 2, [0, 4])           # clearly below the boundary
    assert not admissible_set(s, 2, [1, 2])           # drops the clear winner
    # check_routing accepts the farthest admissible split of the three-way group
    idx = np.array([[0, 3]], dtype=np.int32)
    differing, alts = check_routing(idx, s[[0, 3]][None].astype(np.float32), s[None], 2)
    assert differing.tolist() == [0] and sorted(alts[0][0].tolist()) == [0, 3]


def test_clear_margin_must_match_and_order():
    s = np.array([[0.1, 0.6, 0.05, 0.25]])
    with pytest.raises(AssertionError):
        check_routing(np.array([[1, 0]], dtype=np.int32), np.float32([[0.6, 0.1]]), s, 2)
    with pytest.raises(AssertionError, match="order"):
        check_routing(np.array([[3, 1]], dtype=np.int32), np.float32([[0.25, 0.6]]), s, 2)
    check_routing(np.array([[1, 3]], dtype=np.int32), np.float32([[0.6, 0.25]]), s, 2)


def test_equal_kept_scores_ascending_index():
    s = np.array([[0.3, 0.1, 0.3, 0.3]])              # a three-way exact tie inside the top-3
    with pytest.raises(AssertionError, match="ascending"):
        check_routing(np.array([[2, 0, 3]], dtype=np.int32), np.float32([[0.3, 0.3, 0.3]]), s, 3)
    check_routing(np.array([[0, 2, 3]], dtype=np.int32), np.float32([[0.3, 0.3, 0.3]]), s, 3)
