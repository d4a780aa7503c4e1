"""Pins of oracle.sampler (CPU only).

* Exact enumeration: drawing x ~ q, accepting with u < p(x)/q(x) and otherwise
  resampling from normalize(max(0, p - q)) yields exactly p (the speculative-sampling
  guarantee the pages state for the rule: Agentic Commons post, *How Introspective
  Strided Decoding Works*; GeekNews, *Inference & ISD*).  Integrated over a grid of
  K = 2^12 uniforms, so exact up to the grid's resolution.
* p = q accepts every pending token.
* Cat returns the token whose CDF interval holds u*S (brute-force interval check).
* argmax ties go to the lowest index.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import sampler as S

K = 1 << 12
GRID = (np.arange(K) + 0.5) / K


def _rational_dist(rng, V):
    w = rng.integers(1, 20, size=V)
    w[rng.integers(0, V)] = 0 if V > 2 else w[0]
    return np.array([Fraction(int(x), int(w.sum())) for x in w])


def _enumerate_output(p, q, argmax_q=False):
    """P(output = y) of one pending decision, integrating the oracle functions over u grids."""
    V = len(p)
    pf = p.astype(float)
    qf = q.astype(float)
    out = np.zeros(V)
    resid_hist = np.zeros(V)
    if argmax_q:
        xs = [(int(np.argmax(qf)), 1.0)]
    else:
        xs = [(x, float(q[x])) for x in range(V) if q[x] > 0]
    for x, wx in xs:
        qx = 1.0 if argmax_q else qf[x]
        acc = np.array([S.accept(pf[x], qx, u)[0] for u in GRID])
        pa = acc.mean()
        out[x] += wx * pa
        qq = np.zeros(V) if argmax_q else qf
        if argmax_q:
            qq[x] = 1.0
        hist = np.bincount([S.resid_draw(pf, qq, u)[0] for u in GRID], minlength=V) / K
        out += wx * (1 - pa) * hist
    return out


@pytest.mark.parametrize("seed", range(6))
def test_accept_resample_preserves_p_exactly(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 7))
    p, q = _rational_dist(rng, V), _rational_dist(rng, V)
    if all(q[i] == 0 for i in range(V)):
        return
    got = _enumerate_output(p, q)
    np.testing.assert_allclose(got, p.astype(float), atol=3.0 / K)


@pytest.mark.parametrize("seed", range(4))
def test_argmax_proposal_with_delta_q_preserves_p(seed):
    rng = np.random.default_rng(100 + seed)
    V = 5
    p, q = _rational_dist(rng, V), _rational_dist(rng, V)
    got = _enumerate_output(p, q, argmax_q=True)
    np.testing.assert_allclose(got, p.astype(float), atol=3.0 / K)


def test_closed_form_of_the_rule():
    # P(y) = min(p,q)(y) + (1 - sum min(p,q)) r(y)/sum r = p(y): the algebra behind the rule
    rng = np.random.default_rng(9)
    for _ in range(20):
        V = int(rng.integers(2, 9))
        p, q = _rational_dist(rng, V), _rational_dist(rng, V)
        mn = np.array([min(a, b) for a, b in zip(p, q)])
        r = np.array([max(Fraction(0), a - b) for a, b in zip(p, q)])
        if sum(r) == 0:
            assert all(p == q)
            continue
        tot = mn + (1 - sum(mn)) * r / sum(r)
        assert all(tot == p)


def test_p_equal_q_accepts_everything():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal(1000).astype(np.float32) * 3
    p = S.probs_T(logits, 1.0)
    us = np.concatenate([rng.random(2000), [1 - 2.0 ** -25, 0.5 * 2.0 ** -24]])
    for x in rng.integers(0, 1000, size=50):
        for u in us:
            assert S.accept(p[x], p[x], u)[0]


def test_resid_fallback_when_p_equals_q():
    p = np.array([0.25, 0.5, 0.25])
    tok, _ = S.resid_draw(p, p, 0.6)
    assert tok == S.cat(p, 0.6)[0] == 1


def test_cat_interval_brute_force():
    rng = np.random.default_rng(2)
    w = rng.random(50).astype(np.float32)
    w[[3, 17, 18]] = 0
    C = np.cumsum(w.astype(np.float64))
    for j in range(50):
        lo = C[j - 1] if j else 0.0
        if w[j] == 0:
            continue
        u = (lo + C[j]) / 2 / C[-1]
        assert S.cat(w, u)[0] == j
    # zero-weight tokens are never drawn
    draws = [S.cat(w, u)[0] for u in GRID]
    assert not set(draws) & {3, 17, 18}


def test_cat_matches_frequencies():
    rng = np.random.default_rng(3)
    w = rng.random(16)
    draws = np.bincount([S.cat(w, u)[0] for u in GRID], minlength=16) / K
    np.testing.assert_allclose(draws, w / w.sum(), atol=1.5 / K)


def test_argmax_lowest_index_on_ties():
    l = np.array([0.0, 3.0, 1.0, 3.0, 3.0], np.float32)
    assert S.argmax(l) == 1


def test_temperature_scaling():
    l = np.array([0.0, 1.0, 2.0], np.float32)
    p = S.probs_T(l, 0.5)
    e = np.exp(np.array([0.0, 2.0, 4.0]))
    np.testing.assert_allclose(p, e / e.sum(), rtol=1e-6)


def test_top2_gap_hand_values():
    """top2_gap: the largest logit minus the second largest; a repeated maximum gives 0."""
    assert S.top2_gap([1.0, 5.0, 3.0]) == 2.0
    assert S.top2_gap([5.0, 1.0, 5.0]) == 0.0
    assert S.top2_gap([0.5, -1.0, 0.25, 0.5]) == 0.0
    assert S.top2_gap([-np.inf, 2.0, -3.0]) == 5.0
    assert S.top2_gap([7.0]) == np.inf


def test_top2_gap_brute_force_and_margin_meaning():
    """Against the definition written out (max over the others removed one at a time), and as
    the greedy near-tie margin: no perturbation of every logit by less than half the gap moves
    the argmax, and one of half the gap plus a little can."""
    rng = np.random.default_rng(5)
    for trial in range(200):
        V = int(rng.integers(2, 40))
        l = rng.standard_normal(V).astype(np.float32) * 3
        if trial % 5 == 0:
            l[rng.integers(V)] = l.max()           # a repeated maximum
        j = int(np.argmax(l))
        brute = float(l[j]) - max(float(l[i]) for i in range(V) if i != j)
        gap = S.top2_gap(l)
        assert gap == brute
        if gap > 0:
            e = rng.uniform(-1, 1, V) * (0.499 * gap)
            assert S.argmax(l.astype(np.float64) + e) == j
            k = max((i for i in range(V) if i != j), key=lambda i: l[i])
            flip = l.astype(np.float64).copy()
            flip[j] -= 0.5 * gap + 1e-6
            flip[k] += 0.5 * gap + 1e-6
            assert S.argmax(flip) == k
