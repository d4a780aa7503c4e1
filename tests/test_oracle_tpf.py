"""Pins of oracle.tpf and of the block reading behind the A/B state machine (CPU only).

The pages print TPF = (2 + p + ... + p^(N-2)) / (2 - p^(N-1)) and the figures in
tests/golden/pages_tpf.json; the state machine of oracle.isd must reproduce the
formula exactly, and the printed figures must follow from it.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import tpf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_tpf.json")


@pytest.mark.parametrize("N", range(1, 9))
@pytest.mark.parametrize("p", [Fraction(0), Fraction(1, 2), Fraction(9, 10), Fraction(1)])
def test_state_machine_equals_closed_form_exactly(N, p):
    if N == 1:
        assert tpf.tpf_state_machine(p, N) == 1
        return
    assert tpf.tpf_state_machine(p, N) == tpf.tpf_closed_form(p, N)


def test_monte_carlo_converges():
    for N, p in [(4, 0.9), (2, 0.5), (3, 0.7)]:
        mc = tpf.tpf_monte_carlo(p, N, 300_000, seed=N)
        assert abs(mc - tpf.tpf_closed_form(p, N)) < 0.01


def test_pages_printed_figures():
    g = json.load(open(GOLDEN))["entries"]
    t = tpf.tpf_closed_form(0.9, 4)
    # 2.9 (printed to 1 decimal) at p = 0.9
    assert round(t, 1) == g[1]["printed"]
    # efficiency TPF^2 / (2N-1) = 1.22 at p = 0.9: the 2N-1 = 7 query rows of the block
    assert round(tpf.efficiency(t, 2 * 4 - 1), 2) == g[2]["printed"]
    # 2.96 is a measured-acceptance figure: some p that rounds to 0.9 gives it
    ps = np.linspace(0.895, 0.905, 1001)
    assert any(round(tpf.tpf_closed_form(p, 4), 2) == g[0]["printed"] for p in ps)


def test_extreme_acceptance():
    N = 5
    assert tpf.tpf_state_machine(Fraction(1), N) == N      # every pending accepted: N tokens per pass
    assert tpf.tpf_state_machine(Fraction(0), N) == 1      # none: A pass + B pass commit 2 tokens
    assert tpf.tpf_closed_form(Fraction(1), N) == N and tpf.tpf_closed_form(Fraction(0), N) == 1
