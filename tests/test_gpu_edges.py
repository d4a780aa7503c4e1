"""Edge cases of the decode path through the C ABI: a pass before any prefill, passes over
slots that are empty or finished, a batch with holes, generation that fills a slot's
capacity exactly, and admission errors that must leave the context usable.

Greedy decoding (T = 0, argmax proposals) makes a slot's tokens independent of its slot id
and of the other slots (every kernel computes a row from that row alone), so a slot decoded
in a batch with holes must produce exactly the tokens of the same prompt decoded alone.
"""
import numpy as np
import pytest
import torch

import isd_inputs as I
from strided_decoding_amd import Engine
from strided_decoding_amd._abi import IsdError

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SHAPE = I.SMALL_BF16
N = 4


def _engine(w, B, max_seq=96):
    return Engine(SHAPE, w, stride=N, temperature=0.0, propose="argmax", seed=1, max_batch=B, max_seq_len=max_seq)


def _run(eng, slots, max_steps=200):
    """Step until every listed slot is DONE; returns each slot's committed tokens and the
    per-pass commit counts of every slot."""
    out = {b: [] for b in slots}
    counts = []
    for _ in range(max_steps):
        tok, nc, _ = eng.step()
        torch.cuda.synchronize()
        tok, nc = tok.cpu().numpy(), nc.cpu().numpy()
        counts.append(nc.copy())
        for b in slots:
            out[b] += [int(x) for x in tok[b, :nc[b]]]
        st = eng.slots_host()
        if all(st[b]["state"] == 3 for b in slots):
            break
    return out, counts


def test_steps_before_prefill_and_after_every_slot_finished():
    """A pass before any prefill is refused on the host (ISD_E_STATE, nothing enqueued); once
    every slot has finished, passes commit nothing and the pool stays whole."""
    w = I.weights_numpy(SHAPE, seed=0, scale=20.0)
    eng = _engine(w, 3)
    n_pages = eng.cfg.n_pages
    with pytest.raises(IsdError, match="ISD_E_STATE"):
        eng.step()
    p = I.ragged_prompts([11], SHAPE.vocab, seed=20)
    eng.prefill([1], p, [5])
    out, _ = _run(eng, [1])
    assert len(out[1]) == 4
    for _ in range(3):
        tok, nc, na = eng.step()
        torch.cuda.synchronize()
        assert nc.cpu().numpy().tolist() == [0, 0, 0]
        assert na.cpu().numpy().tolist() == [0, 0, 0]
    assert eng.status() == 0
    assert int(eng.free_stack().numel()) == n_pages
    assert [s["state"] for s in eng.slots_host()] == [0, 3, 0]


def test_batch_with_holes_and_finished_slots_equals_alone():
    """Slots 1 and 3 stay empty, slot 0 finishes early and keeps being stepped while slot 2
    continues: empty and finished slots commit nothing and hold no pages, and slot 2's greedy
    tokens equal the same prompt decoded in a context of its own."""
    w = I.weights_numpy(SHAPE, seed=0, scale=20.0, sticky=(0.0, 20.0, 4.0, 7))
    p0, p2 = I.ragged_prompts([13, 29], SHAPE.vocab, seed=21)
    eng = _engine(w, 4)
    eng.prefill([0, 2], [p0, p2], [3, 40])
    out, counts = _run(eng, [0, 2])
    for nc in counts:
        assert nc[1] == 0 and nc[3] == 0
    done0 = next(i for i, nc in enumerate(counts) if sum(c[0] for c in counts[:i + 1]) >= 2)
    assert all(nc[0] == 0 for nc in counts[done0 + 1:])            # finished: nothing more
    assert len(out[0]) == 2 and len(out[2]) == 39                    # max_new minus the first token
    st = eng.slots_host()
    assert st[0]["state"] == 3 and st[2]["state"] == 3
    assert int(eng.free_stack().numel()) == eng.cfg.n_pages         # every page returned
    alone = _engine(w, 1)
    alone.prefill([0], [p2], [40])
    ref, _ = _run(alone, [0])
    assert out[2] == ref[0]


def test_generation_fills_capacity_exactly():
    """prompt + max_new + 2N == max_seq_len: the slot generates exactly max_new tokens and
    returns all of its pages."""
    w = I.weights_numpy(SHAPE, seed=0, scale=20.0)
    max_seq = 80
    p = I.ragged_prompts([20], SHAPE.vocab, seed=22)[0]
    max_new = max_seq - len(p) - 2 * N
    eng = _engine(w, 1, max_seq=max_seq)
    eng.prefill([0], [p], [max_new])
    out, _ = _run(eng, [0])
    assert len(out[0]) == max_new - 1
    assert eng.slots_host()[0]["n_gen"] == max_new
    assert int(eng.free_stack().numel()) == eng.cfg.n_pages


def test_admission_errors_leave_the_context_usable():
    """A prompt beyond the capacity and a repeated slot are refused on the host (nothing is
    enqueued); a valid prefill and decode then proceed normally."""
    w = I.weights_numpy(SHAPE, seed=0, scale=20.0)
    eng = _engine(w, 2, max_seq=64)
    long_p = I.ragged_prompts([60], SHAPE.vocab, seed=23)[0]
    with pytest.raises(IsdError):
        eng.prefill([0], [long_p], [8])
    p = I.ragged_prompts([10, 12], SHAPE.vocab, seed=24)
    with pytest.raises(IsdError):
        eng.prefill([1, 1], p, [5, 5])
    assert int(eng.free_stack().numel()) == eng.cfg.n_pages
    eng.prefill([0, 1], p, [6, 6])
    out, _ = _run(eng, [0, 1])
    assert len(out[0]) == 5 and len(out[1]) == 5
    assert eng.status() == 0


def _lockstep(ref, eng, slots, n_active, log, max_steps=200):
    """Step `ref` over every slot and `eng` over the first n_active slots until the listed
    slots are DONE; each pass's tokens, commit and accept counts of the listed slots agree."""
    for i in range(max_steps):
        rt, rn, ra = [t.cpu().numpy().copy() for t in ref.step()]
        gt, gn, ga = [t.cpu().numpy().copy() for t in eng.step(n_active)]
        torch.cuda.synchronize()
        for b in slots:
            assert rn[b] == gn[b] and ra[b] == ga[b], (i, b, rn[b], gn[b])
            assert list(rt[b, :rn[b]]) == list(gt[b, :gn[b]]), (i, b)
        log.append(i)
        if all(s["state"] == 3 for k, s in enumerate(eng.slots_host()) if k in slots):
            return
    raise AssertionError("slots did not finish")


@pytest.mark.parametrize("graphs", [False, True])
def test_active_prefix_equals_full_batch(graphs):
    """isd_step_active over the live prefix of a partly filled context gives every live slot
    exactly the tokens that isd_step over all slots gives it (sampled proposals, T = 1, so the
    stored proposal rows of the previous pass are used), also when a slot is admitted in the
    middle of the run and the prefix grows; the page pool ends the same."""
    w = I.weights_numpy(SHAPE, seed=0, scale=20.0)
    mk = lambda: Engine(SHAPE, w, stride=N, temperature=1.0, propose="sample", seed=5, max_batch=6, max_seq_len=96)
    ref, eng = mk(), mk()
    if graphs:
        ref.set_graphs(True)
        eng.set_graphs(True)
    p = I.ragged_prompts([9, 17, 30, 12], SHAPE.vocab, seed=30)
    for e in (ref, eng):
        e.prefill([0, 1, 2], p[:3], [12, 20, 9])
    done = []
    for _ in range(3):
        rt = ref.step()
        gt = eng.step(3)
        torch.cuda.synchronize()
        r, g = [t.cpu().numpy() for t in rt], [t.cpu().numpy() for t in gt]
        for b in range(3):
            assert r[1][b] == g[1][b] and list(r[0][b, :r[1][b]]) == list(g[0][b, :g[1][b]])
    for e in (ref, eng):
        e.prefill([3], [p[3]], [15])
    _lockstep(ref, eng, [0, 1, 2, 3], 4, done)
    assert eng.status() == 0 and ref.status() == 0
    assert int(eng.free_stack().numel()) == eng.cfg.n_pages == int(ref.free_stack().numel())
    assert eng.slots_host()[:4] == ref.slots_host()[:4]


def test_live_slot_past_active_prefix_is_flagged():
    """A live slot at or past n_active is not advanced and reports ISD_E_STATE; the slots in
    the prefix advance normally."""
    w = I.weights_numpy(SHAPE, seed=0, scale=20.0)
    eng = _engine(w, 6)
    p = I.ragged_prompts([10, 14], SHAPE.vocab, seed=31)
    eng.prefill([0, 4], p, [8, 8])
    before = eng.slots_host()[4]
    tok, nc, _ = eng.step(2)
    torch.cuda.synchronize()
    assert int(nc.cpu().numpy()[0]) >= 1
    after = eng.slots_host()
    assert after[0]["passes"] == 1
    assert {k: v for k, v in after[4].items() if k != "status"} == {k: v for k, v in before.items() if k != "status"}
    assert after[4]["status"] == -4
    assert eng.status() == -4
    with pytest.raises(IsdError, match="ISD_E_ARG"):
        eng.step(7)
    with pytest.raises(IsdError, match="ISD_E_ARG"):
        eng.step(0)


def test_nonfinite_logits_end_only_that_slot():
    """isd_sample_step with a NaN in one slot's logits: that slot ends DONE with
    ISD_E_NONFINITE and commits nothing; every other slot's outputs and record equal those of
    the same call without the NaN."""
    from strided_decoding_amd import sample
    B, N, V = 8, 4, 3000
    R = 2 * N - 1
    g = torch.Generator(device=DEV).manual_seed(77)
    logits = torch.randn((B, R, V), generator=g, device=DEV) * 3.0
    q = torch.randn((B * R, V), generator=g, device=DEV) * 3.0
    base = torch.zeros((B, 32), dtype=torch.int32, device=DEV)
    base[:, 0] = torch.tensor([1, 2] * (B // 2), dtype=torch.int32)   # A and B slots
    base[:, 1] = 50
    base[:, 3] = 3
    base[:, 4] = 1
    base[:, 5] = 100
    base[:, 8:22] = -1
    base[:, 8:8 + N - 1] = torch.randint(0, V, (B, N - 1), generator=g, device=DEV).int()
    base[:, 15:15 + N - 1] = (torch.arange(B, device=DEV)[:, None] * R + N +
                              torch.arange(N - 1, device=DEV)[None, :]).int()
    outs = []
    for poison in (None, 3, 6):
        slots = base.clone()
        lg = logits.clone()
        if poison is not None:
            lg[poison, 0, 17] = float("nan")
        tok = torch.full((B, N), -7, dtype=torch.int32, device=DEV)
        nc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        na = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        print(f"nonfinite logits: poisoned slot {poison}", flush=True)
        sample(slots, lg, q, N, 1.0, "sample", 1, tok, nc, na)
        torch.cuda.synchronize()
        outs.append((slots.cpu().numpy(), tok.cpu().numpy(), nc.cpu().numpy(), na.cpu().numpy()))
    ref = outs[0]
    assert np.all(ref[0][:, 7] == 0)
    for poison, out in zip((3, 6), outs[1:]):
        for b in range(B):
            if b == poison:
                assert out[0][b, 0] == 3 and out[0][b, 7] == -6      # DONE, ISD_E_NONFINITE
                assert out[2][b] == 0 and np.all(out[1][b] == -1)
            else:
                assert np.array_equal(out[0][b], ref[0][b]) and np.array_equal(out[1][b], ref[1][b])
                assert out[2][b] == ref[2][b] and out[3][b] == ref[3][b]


def test_nonfinite_weight_row_is_confined_to_its_slot():
    """A NaN in the embedding row of one token: the slot whose prompt holds that token sees
    non-finite logits at its prefill and ends DONE with ISD_E_NONFINITE; the context's sticky
    status reports it (isd_get_status, and the return of the next pass once the prefill has
    run); the other slots decode exactly as they do without that slot (greedy)."""
    w = I.weights_numpy(SHAPE, seed=0, scale=20.0)
    p = I.ragged_prompts([12, 15, 9], SHAPE.vocab, seed=41)
    bad = int(p[1][4])
    assert bad not in set(p[0].tolist()) | set(p[2].tolist())
    w_bad = dict(w)
    emb = w["embed"].copy()
    emb[bad] = np.uint16(0x7FC0)                  # bf16 NaN
    w_bad["embed"] = emb
    eng = _engine(w_bad, 3)
    ref = _engine(w, 3)
    eng.prefill([0, 1, 2], p, [12, 12, 12])
    ref.prefill([0, 2], [p[0], p[2]], [12, 12])
    assert eng.status() == -6                       # synchronizes: the prefill has run
    st = eng.slots_host()
    assert st[1]["state"] == 3 and st[1]["status"] == -6 and st[0]["status"] == 0 and st[2]["status"] == 0
    tok, nc, _ = eng.step()
    assert eng.device_status == -6                  # returned by isd_step itself
    torch.cuda.synchronize()
    first = {b: [int(x) for x in tok[b, :int(nc[b])].cpu()] for b in (0, 2)}
    assert int(nc[1]) == 0
    out, _ = _run(eng, [0, 2])
    out_ref, _ = _run(ref, [0, 2])
    assert first[0] + out[0] == out_ref[0] and first[2] + out[2] == out_ref[2]
    assert int(eng.free_stack().numel()) == eng.cfg.n_pages


def test_prefill_page_order_matches_golden():
    """The hand-worked multi-slot prefill example (tests/golden/prefill_pages_example.txt, page
    size 4) at page size 16 with every prompt 4 times as long (the same page counts): the
    GPU's page tables and free stack after each isd_prefill call equal the example's."""
    from _golden import prefill_golden
    shape = I.TINY
    w = I.weights_numpy(shape)
    eng = Engine(shape, w, stride=2, temperature=1.0, propose="sample", seed=1, max_batch=3, max_seq_len=64,
                 n_pages=8, graphs=False)
    for slots, lens, mx, tables, stack in prefill_golden():
        prompts = I.ragged_prompts([4 * n for n in lens], shape.vocab, seed=sum(lens))
        eng.prefill(slots, prompts, mx)
        torch.cuda.synchronize()
        pt = eng.page_table().cpu().numpy()
        for s, t in tables.items():
            assert pt[s, :len(t)].tolist() == t and np.all(pt[s, len(t):] == -1), (slots, s, pt[s])
        assert eng.free_stack().cpu().numpy().tolist() == stack, slots
