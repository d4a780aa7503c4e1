"""Decision-by-decision comparison of a GPU pass with the oracle's (test helper).

The oracle's decisions of one pass are, in order: the acceptance tests of the pending
tokens, then either the residual draw (first rejection) or z_1 and the proposals.  The
GPU's outputs (committed tokens, accepted count, next pending tokens) determine the
outcome of each of those decisions.  A GPU pass agrees with the oracle if every outcome
matches; otherwise the FIRST differing decision must be a near-tie on the oracle side
(its margin below the threshold of its kind), since every later decision depends on it.
"""

ACC_TAU = 1e-3      # |u - min(1, p/q)| of an acceptance test
CAT_TAU = 1e-5      # distance of u*S to the chosen interval's edge, relative to S


def gpu_outcomes(state, N, g_tokens, g_nacc, g_pending):
    """Outcome of each oracle decision slot as the GPU took it (kind -> list)."""
    out = []
    if state == "A":
        for i in range(N - 1):
            if i < g_nacc:
                out.append(("accept", True, g_tokens[i] if i < len(g_tokens) else None))
            else:
                out.append(("accept", False, None))
                out.append(("resid", None, g_tokens[i] if i < len(g_tokens) else None))
                return out
        out.append(("z1", None, g_tokens[N - 1] if N - 1 < len(g_tokens) else None))
    else:
        out.append(("z1", None, g_tokens[0] if g_tokens else None))
    for j in range(N - 1):
        out.append(("propose", None, g_pending[j] if g_pending is not None and j < len(g_pending) else None))
    return out


def first_divergence(decisions, state, N, g_tokens, g_nacc, g_pending, greedy_tau=None):
    """None if the GPU took every decision as the oracle did, else (decision, is_near_tie).

    g_tokens may be truncated by max_new; missing GPU outcomes are not compared.
    greedy_tau: for greedy decoding, the top-2 logit gap below which an argmax is a
    near-tie (0 when both sides decide on identical logits).
    """
    g = gpu_outcomes(state, N, list(g_tokens), g_nacc, g_pending)
    for d, (kind, acc, tok) in zip(decisions, g):
        if d.kind != kind:
            return d, _near(d, greedy_tau)
        if kind == "accept":
            same = d.accepted == acc
        else:
            same = tok is None or d.token == tok
        if not same:
            return d, _near(d, greedy_tau)
    return None


def _near(d, greedy_tau):
    if greedy_tau is not None:
        return d.margin < greedy_tau
    return d.margin < (ACC_TAU if d.kind == "accept" else CAT_TAU)
