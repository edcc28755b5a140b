"""Host-side logic of bench.py (no GPU): the accepted-token count of a verification block, the
Belady bound simulator against the oracle's, the static-pin selection."""
import numpy as np
import pytest

import bench
import oracle


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_expected_accepted_closed_form(T):
    assert bench.expected_accepted(T, 1.0) == T  # every draft accepted
    assert bench.expected_accepted(T, 0.0) == 1  # only the target's own token
    a = 0.7
    assert abs(bench.expected_accepted(T, a) - (1 - a ** T) / (1 - a)) < 1e-12


def test_belady_simulator_matches_the_oracle():
    rng = np.random.default_rng(4)
    p = 1.0 / np.arange(1, 65) ** 1.1
    p /= p.sum()
    groups = [set(rng.choice(64, size=6, p=p).tolist()) for _ in range(300)]
    hb, _ = oracle.belady(20, [sorted(g) for g in groups])
    assert bench.belady_hits(20, groups) == hb.sum()


def test_static_pins_take_the_most_used():
    class M:
        E = 6

    calib = {0: [np.array([1, 1, 2]), np.array([2, 3]), np.array([2, 1])], 1: [np.array([5]), np.array([4, 5])]}
    pins = bench.static_pins(M, calib, 2)
    assert pins[0].tolist() == [1, 2] and pins[1].tolist() == [4, 5]
