"""Sampling primitives of the ISD step (oracle; test infrastructure only).

From the pages: a pending token x drawn from q (the MASK-row distribution of the
previous pass) is accepted when u < p(x)/q(x), u ~ U(0,1), p being the anchor
distribution of the current pass (wiki note, *Key claims* and *Method*).  The rule
is the speculative-sampling rule and keeps the AR output distribution (Agentic
Commons post, *How Introspective Strided Decoding Works*; GeekNews, *Inference &
ISD*).  The pages do not write out what happens on rejection; the plainest reading
that keeps that guarantee is the speculative-sampling residual draw from
normalize(max(0, p - q)).

Precision (the same on both sides of the parity tests): logits are float32;
w_j = exp((l_j - max l)/T) is evaluated in float32; sums, prefix sums, ratios and
the residual are float64.

Definitions used here and in the HIP sampler:
  softmax_T(l)    w / S with w as above and S = sum w.  T = 0 means greedy.
  Cat(w, u)       smallest j with C_j > u*S, C_j the inclusive prefix sums of w in
                  index order (S = C_{V-1}); if rounding leaves no such j, the last j
                  with w_j > 0.
  Accept(x,p,q,u) u < p(x)/q(x) (strict), u in the open interval (0, 1).
  Resid(p,q,u)    r = max(0, p - q); Cat(r, u) if sum r > 0 else Cat(p, u).
  argmax          lowest index among the maxima.
"""
import numpy as np


def weights_T(logits, T):
    """(w float32 [V], S float64, m float32): w_j = exp((l_j - m)/T)."""
    l = np.asarray(logits, dtype=np.float32)
    m = l.max()
    w = np.exp((l - m) / np.float32(T)).astype(np.float32)
    S = float(np.cumsum(w.astype(np.float64))[-1])
    return w, S, m


def probs_T(logits, T):
    w, S, _ = weights_T(logits, T)
    return w.astype(np.float64) / S


def argmax(logits):
    return int(np.argmax(np.asarray(logits)))     # numpy returns the first maximum


def top2_gap(logits):
    l = np.sort(np.asarray(logits, dtype=np.float64))
    return float(l[-1] - l[-2]) if l.size > 1 else np.inf


def cat(w, u):
    """Cat(w, u) and its near-tie margin.

    Returns (j, margin) where margin = distance of u*S to the nearest edge of the
    chosen interval [C_{j-1}, C_j), divided by S.
    """
    w = np.asarray(w, dtype=np.float64)
    C = np.cumsum(w)
    S = C[-1]
    target = u * S
    j = int(np.searchsorted(C, target, side="right"))
    if j >= len(w):
        nz = np.nonzero(w > 0)[0]
        j = int(nz[-1])
    lo = C[j - 1] if j > 0 else 0.0
    margin = min(target - lo, C[j] - target) / S if S > 0 else 0.0
    return j, float(margin)


def accept(px, qx, u):
    """(accepted, margin): accepted iff u < p(x)/q(x); margin = |u - min(1, p/q)|."""
    ratio = px / qx
    return bool(u < ratio), float(abs(u - min(1.0, ratio)))


def residual(p, q):
    """max(0, p - q) in float64."""
    return np.maximum(0.0, np.asarray(p, np.float64) - np.asarray(q, np.float64))


def resid_draw(p, q, u):
    """Resid(p, q, u) -> (token, margin)."""
    r = residual(p, q)
    if r.sum() > 0:
        return cat(r, u)
    return cat(p, u)
