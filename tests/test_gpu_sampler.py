"""GPU parity: the fused acceptance / resample / propose kernel (isd_sample_step) vs
oracle.isd.decide on identical logits and identical Philox counters.

Integer outputs (committed tokens, accept counts, next state, pending proposals) must be
bit-identical.  The only allowed difference: a slot whose FIRST differing decision is a
near-tie on the oracle side (acceptance |u - min(1, p/q)| < 1e-3, categorical draw within
1e-5 * S of an interval edge); such slots are counted, and their number is held to what
those widths make likely (u is uniform, so a decision is a near-tie with probability about
twice its width).  The kernel's own record of every decision (kind and margin) equals the
oracle's decisions up to the first divergence.  Inputs follow the acceptance microbench
recipe (p-logits ~ N(0, 3^2), q = p + N(0, 0.3^2)).
"""
import numpy as np
import pytest
import torch

import isd_inputs as I
from oracle import isd as OI
from oracle import philox, sampler

from _decisions import ACC_TAU, CAT_TAU, first_divergence

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ST = {"A": 1, "B": 2, "DONE": 3}


def _slots(B, N, states, L, t, pending, q_row, n_gen, max_new, c):
    a = np.zeros((B, 32), np.int32)
    a[:, 0] = [ST[s] for s in states]
    a[:, 1] = L
    a[:, 2] = c
    a[:, 3] = t
    a[:, 4] = n_gen
    a[:, 5] = max_new
    a[:, 8:15] = -1
    a[:, 15:22] = -1
    a[:, 8:8 + N - 1] = pending
    a[:, 15:15 + N - 1] = q_row
    return a


def _case(B, N, V, T, propose, seed, states, max_new=None):
    cfg = I.AttnSamplerMicro(batch=B, stride=N, vocab=V)
    lg = I.sampler_micro(cfg, seed=seed)
    p, q = lg["p_logits"], lg["q_logits"]           # [B, R, V], [B, N-1, V]
    rng = np.random.default_rng(seed)
    L = rng.integers(20, 3000, size=B).astype(np.int32)
    t = rng.integers(1, 50, size=B).astype(np.int32)
    pending = np.zeros((B, N - 1), np.int32)
    for b in range(B):
        for i in range(N - 1):
            if T == 0.0 or propose == "argmax":
                pending[b, i] = sampler.argmax(q[b, i])
            else:
                pending[b, i] = OI.draw(q[b, i], philox.uniform(99, b, i, 7, 1), T)[0]
    q_row = np.arange(B * (N - 1), dtype=np.int32).reshape(B, N - 1)
    n_gen = np.ones(B, np.int32)
    mx = np.full(B, 1 << 20, np.int32) if max_new is None else max_new
    slots = _slots(B, N, states, L, t, pending, q_row, n_gen, mx, c=5)
    return dict(p=p, q=q.reshape(B * (N - 1), V), L=L, t=t, pending=pending, slots=slots, states=states, mx=mx)


def _run_gpu(cs, N, T, propose, seed, meter=False):
    from strided_decoding_amd import sample
    B = cs["p"].shape[0]
    slots = torch.from_numpy(cs["slots"]).to(DEV)
    p = torch.from_numpy(cs["p"]).to(DEV)
    q = torch.from_numpy(cs["q"]).to(DEV)
    tok = torch.full((B, N), -7, dtype=torch.int32, device=DEV)
    nc = torch.zeros(B, dtype=torch.int32, device=DEV)
    na = torch.zeros(B, dtype=torch.int32, device=DEV)
    mg = torch.full((B, 2 * N), -7.0, dtype=torch.float64, device=DEV)
    kd = torch.full((B, 2 * N), -7, dtype=torch.int32, device=DEV)
    print(f"sampler case B={B} N={N} V={p.shape[2]} T={T} {propose}", flush=True)
    sample(slots, p, q, N, T, propose, seed, tok, nc, na, meter=meter, margins=mg, kinds=kd)
    torch.cuda.synchronize()
    return (slots.cpu().numpy(), tok.cpu().numpy(), nc.cpu().numpy(), na.cpu().numpy(), mg.cpu().numpy(),
            kd.cpu().numpy())


KIND = {"accept": 0, "resid": 1, "z1": 2, "propose": 3}


def _check_record(decisions, g_margins, g_kinds, upto):
    """The kernel's decision record equals the oracle's decisions [0, upto)."""
    for j, d in enumerate(decisions[:upto]):
        assert g_kinds[j] == KIND[d.kind], (j, d.kind, g_kinds[j])
        if np.isinf(d.margin):
            assert np.isinf(g_margins[j])
        else:
            # acceptance: |u - min(1, p/q)|; draws: an interval-edge distance of a prefix sum, over
            # the total.  Both sides take float32 exps, which may differ in the last bit (2^-23
            # relative per weight), so these agree to ~2^-22 of the total; argmax gaps exactly
            np.testing.assert_allclose(g_margins[j], d.margin, rtol=1e-5, atol=3e-7, err_msg=f"decision {j}")
    if upto == len(decisions):
        assert np.all(g_kinds[upto:] == -1) and np.all(g_margins[upto:] == -1.0)


def _compare(cs, N, T, propose, seed, gpu, meter=False):
    g_slots, g_tok, g_nc, g_na, g_mg, g_kd = gpu
    B = cs["p"].shape[0]
    near = 0
    checked = 0
    expected = 0.0          # expected near-ties: about 2 tau per decision of width tau
    for b in range(B):
        st = cs["states"][b]
        if st == "DONE":
            assert g_nc[b] == 0 and np.all(g_tok[b] == -1)
            assert np.all(g_kd[b] == -1)
            continue
        pq = None
        if T > 0 and propose == "sample":
            pq = [sampler.weights_T(cs["q"][b * (N - 1) + i], T)[:2] for i in range(N - 1)]
        out = OI.decide(st, int(cs["L"][b]), int(cs["t"][b]), b, list(cs["pending"][b]), pq, cs["p"][b], N, T,
                        propose, seed, meter=meter)
        gs = g_slots[b]
        g_pend = list(gs[8:8 + N - 1]) if gs[0] == 1 else None
        if T > 0:
            expected += sum(2 * (ACC_TAU if d.kind == "accept" else CAT_TAU) for d in out.decisions
                            if not np.isinf(d.margin) and not (d.kind == "propose" and propose == "argmax"))
        div = first_divergence(out.decisions, st, N, g_tok[b, :g_nc[b]], int(g_na[b]), g_pend)
        if div is not None:
            d, is_near = div
            assert is_near, (b, d)
            _check_record(out.decisions, g_mg[b], g_kd[b], out.decisions.index(d))
            near += 1
            continue
        _check_record(out.decisions, g_mg[b], g_kd[b], len(out.decisions))
        checked += 1
        room = int(cs["mx"][b]) - 1
        toks = out.tokens[:room]
        assert g_nc[b] == len(toks), (b, g_nc[b], toks)
        assert list(g_tok[b, :len(toks)]) == toks, (b, g_tok[b], toks)
        assert np.all(g_tok[b, len(toks):] == -1)
        assert g_na[b] == out.n_accept
        if meter:
            g_msum = gs[26:28].copy().view(np.float64)[0]
            assert gs[28] == out.meter_n and out.meter_n == (N - 1 if st == "A" else 0)
            np.testing.assert_allclose(g_msum, out.meter_sum, rtol=1e-6, atol=1e-12)
        assert gs[1] == out.new_L and gs[2] == out.new_c and gs[3] == cs["t"][b] + 1
        done = 1 + len(toks) >= cs["mx"][b]
        exp_state = 3 if done else ST[out.new_state]
        assert gs[0] == exp_state, (b, gs[0], exp_state)
        if exp_state == 1:
            assert list(gs[8:8 + N - 1]) == out.new_pending
            for j, qr in enumerate(out.new_q):
                # a sampled proposal records its MASK row (b*R + row), an argmax one -1
                assert (gs[15 + j] >= 0) == (qr is not None)
    print(f"checked {checked} slots exactly, {near} diverged at a near-tie decision "
          f"({expected:.2f} expected)", flush=True)
    # a Poisson count with mean `expected`: far above mean + 4 sd would be a systematic difference
    assert near <= expected + 4.0 * np.sqrt(expected) + 1.0, (near, expected)
    return near


@pytest.mark.parametrize("T,propose", [(1.0, "sample"), (1.0, "argmax"), (0.0, "argmax"), (0.7, "sample")])
def test_sampler_small_vocab(T, propose):
    B, N, V = 32, 4, 5000
    rng = np.random.default_rng(1)
    states = list(rng.choice(["A", "A", "B", "DONE"], size=B))
    cs = _case(B, N, V, T, propose, 3, states)
    _compare(cs, N, T, propose, 1, _run_gpu(cs, N, T, propose, 1))


@pytest.mark.parametrize("N", [2, 3, 8])
def test_sampler_strides(N):
    B, V = 16, 3000
    states = ["A"] * 12 + ["B"] * 4
    cs = _case(B, N, V, 1.0, "sample", 4 + N, states)
    _compare(cs, N, 1.0, "sample", 2, _run_gpu(cs, N, 1.0, "sample", 2))


def test_sampler_max_new_truncation():
    B, N, V = 16, 4, 2000
    states = ["A"] * 8 + ["B"] * 8
    mx = np.array([2, 3, 4, 5] * 4, np.int32)
    cs = _case(B, N, V, 1.0, "sample", 8, states, max_new=mx)
    _compare(cs, N, 1.0, "sample", 3, _run_gpu(cs, N, 1.0, "sample", 3))


@pytest.mark.parametrize("propose", ["sample", "argmax"])
def test_sampler_full_vocab_microbench(propose):
    B, N, V = 64, 4, 151936
    cs = _case(B, N, V, 1.0, propose, 5, ["A"] * B)
    _compare(cs, N, 1.0, propose, 1, _run_gpu(cs, N, 1.0, propose, 1))


@pytest.mark.parametrize("T,propose", [(1.0, "sample"), (1.0, "argmax"), (0.0, "argmax")])
def test_sampler_meter_mode(T, propose):
    """Introspective acceptance meter: pending tokens are committed untested and their
    acceptance probabilities (min(1, p/q), p(x) for argmax proposals, argmax agreement at
    T = 0) accumulate in the slot record, as in the oracle."""
    B, N, V = 32, 4, 5000
    rng = np.random.default_rng(2)
    states = list(rng.choice(["A", "A", "B", "DONE"], size=B))
    cs = _case(B, N, V, T, propose, 6, states)
    _compare(cs, N, T, propose, 1, _run_gpu(cs, N, T, propose, 1, meter=True), meter=True)
