"""Pins of the oracle's ISD / R-ISD / AR decoders (CPU only).

* greedy ISD (any N, with or without the MASK-gated LoRA) commits exactly the tokens
  of plain AR greedy decoding by full recomputation (the lossless claim: wiki note,
  *Key claims* and *Method*; GeekNews, *Lossless R-ISD*);
* N = 1 sampling equals AR sampling draw for draw under the shared uniforms;
* the output distribution of sampled ISD equals the exact AR distribution, enumerated
  over a 4-token vocabulary (Agentic Commons post, *How Introspective Strided Decoding
  Works*: the rule aligns the output distribution with the AR model);
* after any pass the cache equals a fresh prefill of the committed tokens (logit shift
  and first-rejection rollback, wiki note *Method*);
* anchor rows of an A pass equal the AR next-token logits of the prefix they verify;
* the page allocator reproduces a hand-worked example and its invariants.
"""
import os

import numpy as np
import pytest

import isd_inputs as I
from _golden import prefill_golden
from oracle import isd, philox, sampler
from oracle import model as M
from oracle.paged_kv import PagePool

SHAPE = I.ModelShape("tiny-gqa", 2, 64, 4, 2, 16, 96, 50, "f32")


def spec_of(shape):
    return M.Spec(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                  shape.d_ffn, shape.vocab, shape.rope_base, shape.rms_eps)


def _peaky(shape, seed, scale):
    """Random weights with a larger scale so that distributions are far from uniform."""
    return I.weights_numpy(shape, seed=seed, scale=scale)


# sticky variants (alpha, beta, gamma): None rejects every greedy proposal of the random
# model; (0, 10, 2) makes MASK rows propose the token the AR model falls into, so most
# proposals are accepted and a few rejected.  Together they cover both branches.
STICKY = [None, (0.0, 10.0, 2.0)]


def _model(lora_rank=0, scale=40.0, sticky=None):
    w = I.weights_numpy(SHAPE, seed=21, scale=scale, sticky=None if sticky is None else sticky + (7,))
    lora = I.lora_numpy(SHAPE, lora_rank, seed=22) if lora_rank else None
    if lora is not None:
        for layer in lora:
            for t in layer:
                a, b = layer[t]
                layer[t] = (a * np.float32(10), b * np.float32(10))
    return M.Model(spec_of(SHAPE), w, lora)


@pytest.mark.parametrize("sticky", STICKY)
@pytest.mark.parametrize("N", [2, 3, 4])
@pytest.mark.parametrize("lora_rank", [0, 8])
def test_greedy_isd_equals_ar_greedy(N, lora_rank, sticky):
    m = _model(lora_rank, sticky=sticky)
    base = M.Model(m.spec, m.w, None)
    lens = [9, 14]
    ps = I.ragged_prompts(lens, m.spec.vocab, seed=N)
    n_new = 24
    dec = isd.Decoder(m, N, 0.0, seed=1, page_size=4)
    dec.prefill([0, 1], ps, [n_new, n_new])
    dec.run()
    for s, p in enumerate(ps):
        assert dec.slots[s].generated == isd.ar_greedy_reference(base, p, n_new)


def test_sticky_model_exercises_accept_and_reject():
    acc = tot = 0
    for N in (2, 3, 4):
        m = _model(sticky=STICKY[1])
        dec = isd.Decoder(m, N, 0.0, seed=1, page_size=4)
        dec.prefill([0, 1], I.ragged_prompts([9, 14], m.spec.vocab, seed=N), [30, 30])
        while any(st.state != isd.STATE_DONE for st in dec.slots.values()):
            for rec in dec.step().values():
                for d in rec.decisions:
                    if d.kind == "accept":
                        tot += 1
                        acc += d.accepted
    assert 0 < acc < tot


def test_n1_sampling_equals_ar_sampling_draw_for_draw():
    m = _model()
    prompt = I.ragged_prompts([7], m.spec.vocab, seed=5)[0]
    n_new, slot, seed = 15, 3, 1
    dec = isd.Decoder(m, 1, 1.0, seed=seed, page_size=4)
    dec.prefill([slot], [prompt], [n_new])
    dec.run()
    seq = list(prompt)
    for k in range(n_new):     # token k sits at position len(prompt)+k and is drawn in pass t = k
        logits, _ = m.forward(seq, np.arange(len(seq)), M.empty_cache(m.spec))
        w, _, _ = sampler.weights_T(logits[-1], 1.0)
        seq.append(sampler.cat(w, philox.uniform(seed, slot, k, len(seq), 1))[0])
    assert dec.slots[slot].generated == seq[len(prompt):]


def _exact_ar_distribution(m, prompt, n):
    """P(first n generated tokens) by enumeration over the vocabulary."""
    V = m.spec.vocab
    probs = {}

    def rec(seq, pr):
        if len(seq) - len(prompt) == n:
            probs[tuple(seq[len(prompt):])] = pr
            return
        logits, _ = m.forward(seq, np.arange(len(seq)), M.empty_cache(m.spec))
        p = sampler.probs_T(logits[-1], 1.0)
        for x in range(V):
            rec(seq + [x], pr * p[x])

    rec(list(prompt), 1.0)
    return probs


@pytest.mark.slow
@pytest.mark.parametrize("N,propose", [(2, "sample"), (3, "sample"), (2, "argmax")])
def test_isd_sampling_distribution_equals_ar(N, propose):
    shape = I.ModelShape("v4", 1, 16, 2, 1, 8, 32, 4, "f32")
    w = _peaky(shape, 31, 60.0)
    m = M.Model(spec_of(shape), w)
    prompt = [1, 3, 0]
    n = 3
    exact = _exact_ar_distribution(m, prompt, n)
    runs = 3000
    counts = {k: 0 for k in exact}
    for r in range(runs):
        dec = isd.Decoder(m, N, 1.0, propose=propose, seed=1000 + r, page_size=4)
        dec.prefill([0], [prompt], [n])
        dec.run()
        counts[tuple(dec.slots[0].generated)] += 1
    keys = sorted(exact)
    e = np.array([exact[k] for k in keys]) * runs
    o = np.array([counts[k] for k in keys])
    # pool cells with small expectation, then chi-square
    big = e >= 5
    e2 = np.append(e[big], e[~big].sum())
    o2 = np.append(o[big], o[~big].sum())
    chi2 = ((o2 - e2) ** 2 / np.maximum(e2, 1e-12)).sum()
    from scipy.stats import chi2 as C
    assert C.sf(chi2, len(e2) - 1) > 1e-4, (chi2, len(e2))


@pytest.mark.parametrize("N,T,propose", [(2, 1.0, "sample"), (4, 1.0, "argmax"), (3, 0.7, "sample")])
def test_cache_equals_fresh_prefill_of_committed(N, T, propose):
    m = _model()
    ps = I.ragged_prompts([6, 11], m.spec.vocab, seed=9)
    dec = isd.Decoder(m, N, T, propose=propose, seed=4, page_size=4)
    dec.prefill([0, 1], ps, [25, 25])
    for _ in range(6):
        dec.step()
        for st in dec.slots.values():
            if st.state == isd.STATE_DONE:
                continue
            committed = st.committed
            assert st.L == len(committed) - 1 and committed[-1] == st.c
            _, kv = m.forward(committed[:st.L], np.arange(st.L), M.empty_cache(m.spec))
            for (ck, cv), (fk, fv) in zip(st.cache, kv):
                np.testing.assert_allclose(ck, fk, atol=2e-5)
                np.testing.assert_allclose(cv, fv, atol=2e-5)


def test_anchor_rows_are_ar_next_token_logits():
    m = _model()
    p = I.ragged_prompts([8], m.spec.vocab, seed=10)[0]
    dec = isd.Decoder(m, 4, 1.0, seed=2, page_size=4, keep_logits=True)
    dec.prefill([0], [p], [40])
    rec = None
    for _ in range(10):
        st = dec.slots[0]
        before = list(st.committed) + list(st.pending)
        state = st.state
        r = dec.step()[0]
        if state == isd.STATE_A:
            rec = r
            break
    assert rec is not None
    for i in range(1, 4):      # row i-1 predicts the token at position L+i
        prefix = before[:len(before) - 3 + i - 1]      # committed tokens + v_1 .. v_{i-1}
        logits, _ = m.forward(prefix, np.arange(len(prefix)), M.empty_cache(m.spec))
        np.testing.assert_allclose(rec.logits[i - 1], logits[-1], atol=5e-4, rtol=1e-4)


def test_max_new_truncates_and_finishes():
    m = _model(scale=200.0)
    p = I.ragged_prompts([5], m.spec.vocab, seed=11)[0]
    for n_new in (1, 2, 5):
        dec = isd.Decoder(m, 4, 0.0, seed=2, page_size=4)
        dec.prefill([0], [p], [n_new])
        dec.run()
        st = dec.slots[0]
        assert len(st.generated) == n_new and st.state == isd.STATE_DONE
        assert dec.pool.table(0) == [] and dec.pool.n_free == dec.pool.n_pages


def _golden_ops():
    path = os.path.join(os.path.dirname(__file__), "golden", "page_allocator_example.txt")
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        lhs, rhs = line.split("->")
        op, slot, length = lhs.split()
        table, stack = [x.strip() for x in rhs.split("|")]
        table = [] if table == "-" else [int(x) for x in table.split(",")]
        stack = [int(x) for x in stack.split(",")]
        yield op, int(slot), int(length), table, stack


def test_page_allocator_golden_example():
    pool = PagePool(8, 4)
    for op, slot, length, table, stack in _golden_ops():
        getattr(pool, op)(slot, length)
        assert pool.table(slot) == table, (op, slot, length)
        assert pool.stack == stack, (op, slot, length)


def test_page_invariants_during_decoding():
    m = _model()
    ps = I.ragged_prompts([3, 17, 9], m.spec.vocab, seed=12)
    dec = isd.Decoder(m, 3, 1.0, seed=5, page_size=4, n_pages=64)
    dec.prefill([0, 2, 5], ps, [12, 30, 7])
    while any(st.state != isd.STATE_DONE for st in dec.slots.values()):
        dec.step()
        lens = {s: (st.L if st.state != isd.STATE_DONE else 0) for s, st in dec.slots.items()}
        dec.pool.check(lens)
    assert dec.pool.n_free == 64


def _meter_run(m, N, T, propose, n_new=30):
    """Meter-mode decode of two prompts; returns (decoder, {slot: [(position, token)] of the
    re-scored pending tokens})."""
    ps = I.ragged_prompts([7, 12], m.spec.vocab, seed=13)
    dec = isd.Decoder(m, N, T, propose=propose, seed=6, page_size=4, meter=True)
    dec.prefill([0, 1], ps, [n_new, n_new])
    scored = {0: [], 1: []}
    for _ in range(40):
        if all(st.state == isd.STATE_DONE for st in dec.slots.values()):
            break
        for s, r in dec.step().items():
            scored[s] += [(d.position, d.token) for d in r.decisions if d.kind == "accept"]
    return dec, scored


def _extended(committed, scored):
    """The committed sequence followed by the re-scored tokens that max_new dropped (the last
    pass re-scores its pending tokens before the output is truncated)."""
    seq = list(committed)
    for pos, tok in sorted(scored):
        if pos == len(seq):
            seq.append(tok)
    return seq


@pytest.mark.parametrize("sticky", STICKY)
@pytest.mark.parametrize("N", [2, 4])
def test_meter_greedy_counts_ar_agreement(N, sticky):
    """At T = 0 the meter counts the re-scored tokens equal to the AR greedy token of their
    prefix, recomputed here by one full forward of the committed sequence."""
    m = _model(sticky=sticky)
    dec, scored = _meter_run(m, N, 0.0, "argmax")
    total = 0
    for s, st in dec.slots.items():
        seq = _extended(st.committed, scored[s])
        logits, _ = m.forward(seq, np.arange(len(seq)), M.empty_cache(m.spec))
        agree = sum(1 for pos, tok in scored[s] if seq[pos] == tok and tok == int(np.argmax(logits[pos - 1])))
        assert st.meter_n == len(scored[s]) and st.meter_n > 0
        assert st.meter_sum == agree
        total += agree
    if sticky is not None:
        assert total > 0                # the sticky model's own proposals are often AR tokens


@pytest.mark.parametrize("sticky", STICKY)
def test_meter_argmax_proposals_sum_ar_probabilities(sticky):
    """At T = 1 with argmax proposals (q = delta) the meter sums p(x), the AR probability of
    each re-scored token given its prefix (one full forward of the committed sequence)."""
    m = _model(sticky=sticky)
    dec, scored = _meter_run(m, 3, 1.0, "argmax")
    for s, st in dec.slots.items():
        seq = _extended(st.committed, scored[s])
        logits, _ = m.forward(seq, np.arange(len(seq)), M.empty_cache(m.spec))
        want = 0.0
        for pos, tok in scored[s]:
            assert seq[pos] == tok
            z = logits[pos - 1].astype(np.float64)
            p = np.exp(z - z.max())
            want += p[tok] / p.sum()
        assert st.meter_n == len(scored[s]) and st.meter_n > 0
        np.testing.assert_allclose(st.meter_sum, want, rtol=1e-5)


def test_meter_commits_the_models_own_proposals():
    """Meter mode never rejects: after the first pass every pass commits N tokens, the
    pending tokens of the previous pass followed by the new z_1."""
    m = _model()
    N = 4
    ps = I.ragged_prompts([9], m.spec.vocab, seed=14)
    dec = isd.Decoder(m, N, 1.0, propose="sample", seed=8, page_size=4, meter=True)
    dec.prefill([0], ps, [60])
    first = True
    while dec.slots[0].state != isd.STATE_DONE:
        st = dec.slots[0]
        pend = list(st.pending)
        r = dec.step()[0]
        if first:
            assert len(r.tokens) == 1
            first = False
            continue
        if dec.slots[0].state == isd.STATE_DONE:
            break
        assert r.tokens[:N - 1] == pend and len(r.tokens) == N
    assert dec.slots[0].meter_n > 0 and 0.0 <= dec.slots[0].meter_sum <= dec.slots[0].meter_n


def test_prefill_page_order_golden_example():
    """Several slots per prefill call, recycled slots and slots finished at admission: the
    decoder's page tables and free stack follow the hand-worked example."""
    m = _model()
    dec = isd.Decoder(m, 2, 1.0, seed=1, page_size=4, n_pages=8)
    for slots, lens, mx, tables, stack in prefill_golden():
        prompts = I.ragged_prompts(lens, m.spec.vocab, seed=sum(lens))
        dec.prefill(slots, prompts, mx)
        for s, t in tables.items():
            assert dec.pool.table(s) == t, (slots, s)
        assert dec.pool.stack == stack, slots
