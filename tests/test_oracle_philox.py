"""Pins of oracle.philox: published known-answer vectors and uniformity."""
import os

import numpy as np
import pytest

from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            w = [int(x, 16) for x in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,out", _kat())
def test_known_answer_vectors(ctr, key, out):
    got = philox.philox4x32(np.array(ctr), np.array(key))
    assert [int(x) for x in got] == out


def test_fewer_rounds_differ():
    # a dropped round must not pass the known-answer check
    ctr, key, out = _kat()[2]
    assert [int(x) for x in philox.philox4x32(np.array(ctr), np.array(key), rounds=9)] != out


def test_uniform_open_interval_and_moments():
    n = 200_000
    u = philox.uniform(1, np.arange(n) % 64, np.arange(n) // 64, 1234, 0)
    assert u.min() > 0.0 and u.max() < 1.0
    # KS distance against U(0,1)
    s = np.sort(u)
    d = np.max(np.maximum(np.arange(1, n + 1) / n - s, s - np.arange(n) / n))
    assert d < 1.63 / np.sqrt(n) * 1.5
    assert abs(u.mean() - 0.5) < 5 / np.sqrt(12 * n)


def test_uniform_is_24bit_grid():
    u = philox.uniform(7, 3, 5, np.arange(1000), 1)
    k = u * 2 ** 24 - 0.5
    assert np.all(k == np.round(k)) and np.all((k >= 0) & (k < 2 ** 24))
    # (2k+1) * 2^-25: exact in float64, so both sides compare u in float64
    assert np.all(((2 * (u * 2 ** 24 - 0.5) + 1) * 2.0 ** -25) == u)


def test_streams_depend_on_every_field():
    base = philox.uniform(1, 2, 3, 4, 0)
    assert base != philox.uniform(1, 2, 3, 4, 1)
    assert base != philox.uniform(1, 2, 3, 5, 0)
    assert base != philox.uniform(1, 2, 4, 4, 0)
    assert base != philox.uniform(1, 3, 3, 4, 0)
    assert base != philox.uniform(2, 2, 3, 4, 0)
    assert base != philox.uniform(1 + (1 << 32), 2, 3, 4, 0)   # high key word
