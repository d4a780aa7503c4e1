"""Tokens per forward (TPF) of the ISD state machine (oracle; test infrastructure only).

The pages print the memory-bound TPF closed form (2 + p + ... + p^(N-2)) / (2 - p^(N-1))
(wiki note, *Method*; GeekNews, *Speedup Factor Explorer*) and its value at N = 4 with
acceptance p ~ 0.9 (about 2.9 to 2.96), plus the compute efficiency
TPF^2 / queries-per-forward (1.22 for ISD with 2N-1 = 7 queries).

``tpf_closed_form`` is that formula; ``tpf_state_machine`` derives the same quantity
from the A/B block machine of ``oracle.isd`` (expected tokens per A-cycle over
expected passes per A-cycle, exact in rationals), and ``tpf_monte_carlo`` simulates
the machine with i.i.d. Bernoulli(p) acceptances.
"""
from fractions import Fraction

import numpy as np


def tpf_closed_form(p, N):
    num = 2 + sum(p ** k for k in range(1, N - 1))
    return num / (2 - p ** (N - 1))


def tpf_state_machine(p, N):
    """Exact renewal-reward TPF of the A/B machine (p may be a Fraction)."""
    if N == 1:
        return Fraction(1) if isinstance(p, Fraction) else 1.0
    one = Fraction(1) if isinstance(p, Fraction) else 1.0
    tokens = 0 * one
    passes = 0 * one
    for i in range(1, N):                      # first rejection at pending i
        pr = p ** (i - 1) * (one - p)
        tokens += pr * (i + 1)                 # (i-1) accepted + resample, then z_1 of the B pass
        passes += pr * 2
    pr_all = p ** (N - 1)
    tokens += pr_all * N                       # N-1 accepted + z_1
    passes += pr_all * 1
    return tokens / passes


def tpf_monte_carlo(p, N, n_passes, seed=0):
    rng = np.random.default_rng(seed)
    state_a = False
    tokens = 0
    for _ in range(n_passes):
        if not state_a:
            tokens += 1
            state_a = True
            continue
        acc = 0
        while acc < N - 1 and rng.random() < p:
            acc += 1
        if acc == N - 1:
            tokens += N
        else:
            tokens += acc + 1
            state_a = False
    return tokens / n_passes


def efficiency(tpf, queries_per_forward):
    return tpf * tpf / queries_per_forward
