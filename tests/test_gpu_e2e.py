"""GPU parity of whole decode passes through the C ABI (isd_prefill / isd_step).

Teacher-forced: before every pass the oracle holds the GPU's slot state (committed
tokens, pending tokens, L, state), runs its own forward and decisions, the two are
compared, and the oracle then adopts the GPU's resulting state.
  * fp32 path (tiny model): logits max-abs <= 1e-4; the decisions the oracle takes on its
    own logits must equal the GPU's, except near-ties (acceptance |u - min(1,p/q)| < 1e-3,
    categorical draw within 1e-5 of an interval edge relative to the mass), counted.
  * bf16 path: logits ||gpu - oracle||_inf <= 2e-2 ||oracle||_inf per row; the decisions
    are checked on the GPU's own logits (both sides decide in the same precision), the
    prefill's first token included (on the GPU's prefill logits, exposed by isd_buffers).
Each test runs with the passes replayed from captured HIP graphs (the path the benchmark
times) and, where parametrized, also launched kernel by kernel.
Page tables and the free stack are compared bit-exactly with the oracle's allocator while
every slot is in lock-step.
"""
import numpy as np
import pytest
import torch

import isd_inputs as I
from oracle import isd as OI
from oracle import model as M
from oracle import philox, sampler

from _decisions import CAT_TAU, first_divergence

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
STATE_NAME = {1: "A", 2: "B", 3: "DONE", 0: "EMPTY"}


def spec_of(s):
    return M.Spec(s.n_layers, s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim, s.d_ffn, s.vocab, s.rope_base,
                  s.rms_eps)


def make_engine(shape, w, N, T, propose, B, max_seq, lora=None, seed=1, n_pages=None, graphs=True):
    from strided_decoding_amd import Engine
    return Engine(shape, w, stride=N, temperature=T, propose=propose, seed=seed, max_batch=B,
                  max_seq_len=max_seq, lora=lora, n_pages=n_pages, graphs=graphs)


def _rel(a, r):
    return float((np.abs(a - r).max(axis=-1) / np.maximum(np.abs(r).max(axis=-1), 1e-6)).max())


def _adopt(dec, model, b, g, committed, rec_logits, row0, N, T, propose):
    """Make the oracle slot equal the GPU's state (cache rebuilt when L differs).  rec_logits:
    the slot's block rows of the pass that proposed its pending tokens, whose first row is the
    pass's packed row row0 (the GPU's q_row entries are packed rows)."""
    st = dec.slots[b]
    st.committed = list(committed)
    st.n_gen = len(committed) - st.prompt_len
    st.c = g["c"]
    st.t = g["t"]
    st.state = STATE_NAME[g["state"]]
    st.pending, st.pending_q = [], []
    if st.state == "A":
        for j in range(N - 1):
            st.pending.append(g[f"pending{j}"])
            qr = g[f"q_row{j}"]
            if qr >= 0 and T > 0 and propose == "sample":
                st.pending_q.append(sampler.weights_T(rec_logits[qr - row0], T)[:2])
            else:
                st.pending_q.append(None)
    if g["L"] != st.L:
        st.L = g["L"]
        _, kv = model.forward(st.committed[:st.L], np.arange(st.L), M.empty_cache(model.spec))
        st.cache = M.extend_cache(M.empty_cache(model.spec), kv, st.L)
    if st.state == "DONE":
        dec.pool.truncate(b, 0)


def teacher_forced(shape, w, N, T, propose, prompts, max_new, steps, lora=None, on_gpu_logits=False,
                   logits_tol=1e-4, rel=False, graphs=True):
    B = len(prompts)
    max_seq = max(len(p) for p in prompts) + max(max_new) + 2 * N + 2
    eng = make_engine(shape, w, N, T, propose, B, max_seq, lora=lora, graphs=graphs)
    model = M.Model(spec_of(shape), w, lora)
    dec = OI.Decoder(model, N, T, propose=propose, seed=1, page_size=16, n_pages=eng.cfg.n_pages,
                     keep_logits=True)
    slots = list(range(B))
    print(f"e2e {shape.name} N={N} T={T} {propose} B={B} graphs={graphs}", flush=True)
    first = eng.prefill(slots, prompts, max_new).cpu().numpy()
    ofirst = dec.prefill(slots, prompts, max_new)
    gpl = eng.prefill_logits(B).cpu().numpy() if on_gpu_logits else None
    near, lockstep = 0, True
    committed = [[int(x) for x in p] + [int(first[b])] for b, p in enumerate(prompts)]
    for b in range(B):
        L0 = len(prompts[b])
        u = philox.uniform(1, b, 0, L0, 1)
        if on_gpu_logits:
            # the first token is decided on the GPU's own prefill logits, which follow the oracle's
            ol, _ = model.forward(prompts[b], np.arange(L0), M.empty_cache(model.spec))
            err = _rel(gpl[b], ol[-1])
            assert err <= logits_tol, ("prefill logits", b, err)
            z, m = OI.draw(gpl[b], u, T)
            if z != first[b]:
                assert T > 0 and m < CAT_TAU, ("first token differs on the GPU's logits", b, m)
                near += 1
        elif first[b] != ofirst[b]:
            logits, _ = model.forward(prompts[b], np.arange(L0), M.empty_cache(model.spec))
            _, m = OI.draw(logits[-1], u, T)
            assert T > 0 and m < CAT_TAU, ("first token differs", b, m)
            near += 1
        if first[b] != ofirst[b]:
            lockstep = False
            dec.slots[b].committed[-1] = int(first[b])
            dec.slots[b].c = int(first[b])
    R = 2 * N - 1
    n_steps, max_err = 0, 0.0
    for _ in range(steps):
        if all(st.state == "DONE" for st in dec.slots.values()):
            break
        snap = {b: (dec.slots[b].state, dec.slots[b].L, dec.slots[b].t, list(dec.slots[b].pending),
                    list(dec.slots[b].pending_q)) for b in slots}
        tok, nc, na = eng.step()
        recs = dec.step()
        n_steps += 1
        torch.cuda.synchronize()
        g_tok, g_nc, g_na = tok.cpu().numpy(), nc.cpu().numpy(), na.cpu().numpy()
        g_logits = eng.logits().cpu().numpy()
        g_off = eng.row_offsets()
        gs = eng.slots_host()
        for b in slots:
            if b not in recs:
                assert g_nc[b] == 0
                continue
            rec = recs[b]
            nrows = len(rec.ids)
            ol, gl = rec.logits, g_logits[b, :nrows]
            if rel:
                err = _rel(gl, ol)
            else:
                err = float(np.abs(gl - ol).max())
            assert err <= logits_tol, (b, err)
            max_err = max(max_err, err)
            if on_gpu_logits:
                state, L, t, pend, pq = snap[b]
                out = OI.decide(state, L, t, b, pend, pq, gl, N, T, propose, 1)
                room = max_new[b] - (len(committed[b]) - len(prompts[b]))
                decisions, otoks, onacc = out.decisions, out.tokens[:room], out.n_accept
            else:
                decisions, otoks, onacc = rec.decisions, rec.tokens, rec.n_accept
            gt = [int(x) for x in g_tok[b, :g_nc[b]]]
            g_pend = [gs[b][f"pending{j}"] for j in range(N - 1)] if gs[b]["state"] == 1 else None
            greedy_tau = None if T > 0 else (0.0 if on_gpu_logits else 2 * logits_tol)
            div = first_divergence(decisions, rec.state, N, gt, int(g_na[b]), g_pend, greedy_tau)
            if div is not None:
                d, is_near = div
                assert is_near, (b, gt, otoks, (d.kind, d.token, d.margin))
                near += 1
                lockstep = False
            else:
                assert gt == list(otoks) and g_na[b] == onacc, (b, gt, otoks)
            committed[b] += gt
        if lockstep:
            pt = eng.page_table().cpu().numpy()
            for b in slots:
                np.testing.assert_array_equal(pt[b], dec.pool.table_array(b, pt.shape[1]))
            np.testing.assert_array_equal(eng.free_stack().cpu().numpy(), np.array(dec.pool.stack, np.int32))
        for b in slots:
            if b in recs:
                q_src = g_logits[b] if on_gpu_logits else recs[b].logits
                _adopt(dec, model, b, gs[b], committed[b], q_src, int(g_off[b]), N, T, propose)
    print(f"steps={n_steps} near_ties={near} max_logit_err={max_err:.3g}", flush=True)
    return eng, dec, committed, near


@pytest.mark.parametrize("graphs", [True, False])
def test_tiny_fp32_end_to_end(graphs):
    wl = I.TINY_E2E
    w = I.weights_numpy(wl.model)
    prompts = list(I.prompts(wl.batch, wl.prompt_len, wl.model.vocab))
    eng, dec, committed, near = teacher_forced(wl.model, w, wl.stride, wl.temperature, wl.propose, prompts,
                                               [wl.max_new] * wl.batch, steps=64, graphs=graphs)
    for b in range(wl.batch):
        assert len(committed[b]) - wl.prompt_len == wl.max_new
    assert near <= 6
    st = eng.slots_host()
    assert all(s["state"] == 3 for s in st[:wl.batch])
    assert int(eng.free_stack().numel()) == eng.cfg.n_pages


@pytest.mark.parametrize("N,T,propose", [(3, 1.0, "argmax"), (4, 0.0, "argmax"), (1, 1.0, "sample"),
                                         (8, 1.0, "sample"), (8, 0.0, "argmax")])
def test_tiny_fp32_variants(N, T, propose):
    shape = I.ModelShape("tiny-gqa", 2, 128, 4, 2, 32, 256, 512, "f32")
    w = I.weights_numpy(shape, seed=4, scale=8.0)
    prompts = I.ragged_prompts([5, 17, 33], shape.vocab, seed=6)
    teacher_forced(shape, w, N, T, propose, prompts, [20, 9, 15], steps=40)


@pytest.mark.parametrize("graphs", [True, False])
def test_small_bf16_end_to_end(graphs):
    shape = I.SMALL_BF16
    w = I.weights_numpy(shape, seed=0, scale=20.0)
    prompts = I.ragged_prompts([40, 7, 130, 19], shape.vocab, seed=3)
    teacher_forced(shape, w, 4, 1.0, "sample", prompts, [12, 20, 8, 16], steps=14, logits_tol=2e-2, rel=True,
                   on_gpu_logits=True, graphs=graphs)


@pytest.mark.parametrize("propose,T", [("sample", 1.0), ("argmax", 1.0)])
def test_small_bf16_stride8_end_to_end(propose, T):
    """N = 8: blocks of 15 rows (7 pending, 7 MASK)."""
    shape = I.SMALL_BF16
    w = I.weights_numpy(shape, seed=0, scale=20.0, sticky=(0.0, 20.0, 4.0, 7))
    prompts = I.ragged_prompts([23, 61, 9], shape.vocab, seed=21)
    teacher_forced(shape, w, 8, T, propose, prompts, [30, 24, 17], steps=12, logits_tol=2e-2, rel=True,
                   on_gpu_logits=True)


def test_small_bf16_long_prompt():
    """A prompt longer than 2048 tokens: prefill attention spans more than one 128-page window of
    page ids, and decode passes merge many context splits."""
    shape = I.SMALL_BF16
    w = I.weights_numpy(shape, seed=0, scale=20.0)
    prompts = I.ragged_prompts([2300, 90], shape.vocab, seed=8)
    teacher_forced(shape, w, 4, 1.0, "sample", prompts, [6, 6], steps=4, logits_tol=2e-2, rel=True,
                   on_gpu_logits=True)


def test_bf16_eight_heads_per_group_end_to_end():
    """The 32B shape's grouping (8 query heads per KV head: a block's 7 rows x 8 heads take the
    four-wave attention workgroup in decode, and prefill tiles of 8 positions) on a small model."""
    shape = I.ModelShape("small-g8-bf16", 2, 512, 16, 2, 128, 1024, 4096, "bf16")
    w = I.weights_numpy(shape, seed=1, scale=20.0)
    prompts = I.ragged_prompts([33, 9, 150], shape.vocab, seed=9)
    teacher_forced(shape, w, 4, 1.0, "sample", prompts, [10, 14, 8], steps=10, logits_tol=2e-2, rel=True,
                   on_gpu_logits=True)


@pytest.mark.parametrize("graphs", [True, False])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lora_mask_rows_end_to_end(dtype, graphs):
    """Gated LoRA (R-ISD adapter) on q, k, v, o, gate, up, down at the MASK rows: the GPU
    logits of every row, MASK rows included, follow the oracle's; the adapter is scaled up so
    that its contribution is of the order of the base projections' (bf16: scale 4 at rank 64
    and d 512 makes the delta about 2.6 times the base projection; at scale 15 it is ~36
    times, the MASK rows' attention becomes one-hot, and a near-tie of two keys turns bf16
    storage of q and k into an attention change of up to ~18 % in the oracle's own bf16
    precision model - an ill-conditioned input, not a measure of the path)."""
    shape = I.TINY if dtype == "f32" else I.SMALL_BF16
    rank = 8 if dtype == "f32" else 64
    w = I.weights_numpy(shape, seed=0, scale=1.0 if dtype == "f32" else 20.0)
    lora = I.lora_numpy(shape, rank, scale=15.0 if dtype == "f32" else 4.0)
    prompts = I.ragged_prompts([21, 9, 40], shape.vocab, seed=14)
    if dtype == "f32":
        teacher_forced(shape, w, 3, 1.0, "sample", prompts, [10, 12, 8], steps=10, lora=lora, graphs=graphs)
    else:
        teacher_forced(shape, w, 3, 1.0, "sample", prompts, [10, 12, 8], steps=8, lora=lora, logits_tol=2e-2,
                       rel=True, on_gpu_logits=True, graphs=graphs)


@pytest.mark.parametrize("scale", [3.0, 6.0])
def test_lora_split_shrink_end_to_end(scale):
    """The MASK-row shrink as several k-splits: at d_model 2048 and d_ffn 4096 the q/k/v and
    gate/up shrinks run as 2 splits and the down shrink as 4, summed by the last workgroup of
    each tile to arrive; the GPU logits of every row follow the oracle's.  At adapter scale 6
    the MASK rows' q is several times the base projection and their attention scores are
    large, so bf16 storage of q and k shows up in the logits (the oracle's bf16 precision model
    sits 1.7 % from the fp32 forward here): the path rounds q, k, v once, after RoPE (rounding
    the projection before RoPE as well doubles that error to about 3 %)."""
    shape = I.ModelShape("mid-bf16", 1, 2048, 16, 4, 128, 4096, 4096, "bf16")
    w = I.weights_numpy(shape, seed=2, scale=20.0)
    lora = I.lora_numpy(shape, 64, scale=scale)
    prompts = I.ragged_prompts([19, 33], shape.vocab, seed=15)
    teacher_forced(shape, w, 4, 1.0, "sample", prompts, [10, 8], steps=6, lora=lora, logits_tol=2e-2, rel=True,
                   on_gpu_logits=True)


def test_lora_8b_widths_end_to_end():
    """One layer at the 8B shape's widths (d_model 4096, 32 x 128 query heads, 8 KV heads,
    d_ffn 12288) with the rank-128 adapter: the shrinks run as 4 (q/k/v, o, gate/up) and 12
    (down) k-splits, the expands are fused into the projections at their real widths, and
    the GPU logits of every row follow the oracle's."""
    shape = I.ModelShape("8b-widths-1-layer", 1, 4096, 32, 8, 128, 12288, 4096, "bf16")
    w = I.weights_numpy(shape, seed=3, scale=20.0)
    lora = I.lora_numpy(shape, 128, scale=2.0)   # delta of the order of the base projection at d 4096
    prompts = I.ragged_prompts([17, 29], shape.vocab, seed=16)
    teacher_forced(shape, w, 4, 1.0, "sample", prompts, [8, 8], steps=4, lora=lora, logits_tol=2e-2, rel=True,
                   on_gpu_logits=True)


@pytest.mark.parametrize("B", [20, 33])
def test_lora_tiled_rows_end_to_end(B):
    """The adapter on the tiled GEMM kernel: 20 and 33 slots of 7 rows (140 and 231 rows, past
    the skinny kernel's 128) at the 8B shape's widths, so that the fused LoRA expands run in
    the tiled kernel with 2 waves per workgroup (140 rows), and with 3 (gate/up) and 4 (q/k/v,
    o, down) at 231 rows; the GPU logits of every row follow the oracle's.  Every decision,
    the prefill's first token included, is checked on the GPU's own logits."""
    shape = I.ModelShape("8b-widths-1-layer", 1, 4096, 32, 8, 128, 12288, 4096, "bf16")
    w = I.weights_numpy(shape, seed=3, scale=20.0)
    lora = I.lora_numpy(shape, 128, scale=2.0)
    lens = [int(x) for x in np.random.default_rng(17).integers(5, 30, B)]
    prompts = I.ragged_prompts(lens, shape.vocab, seed=17)
    teacher_forced(shape, w, 4, 1.0, "sample", prompts, [8] * B, steps=2, lora=lora, logits_tol=2e-2, rel=True,
                   on_gpu_logits=True)


@pytest.mark.parametrize("N,T,propose", [(3, 0.0, "argmax"), (4, 1.0, "argmax")])
def test_meter_mode_end_to_end(N, T, propose):
    """Introspective acceptance meter through isd_step: the model's own proposals are
    committed untested and re-scored; the committed sequences and the per-slot meter sums
    equal the oracle decoder's in meter mode (tiny fp32 model, peaky weights so that no
    decision is near a tie)."""
    shape = I.ModelShape("tiny-gqa", 2, 128, 4, 2, 32, 256, 512, "f32")
    w = I.weights_numpy(shape, seed=4, scale=40.0, sticky=(0.0, 10.0, 2.0, 7))
    prompts = I.ragged_prompts([5, 17, 33], shape.vocab, seed=6)
    max_new = [20, 9, 15]
    B = len(prompts)
    eng = make_engine(shape, w, N, T, propose, B, max(len(p) for p in prompts) + max(max_new) + 2 * N + 2)
    eng.set_meter(True)
    model = M.Model(spec_of(shape), w, None)
    dec = OI.Decoder(model, N, T, propose=propose, seed=1, page_size=16, n_pages=eng.cfg.n_pages, meter=True)
    print(f"meter e2e N={N} T={T} {propose}", flush=True)
    first = eng.prefill(list(range(B)), prompts, max_new).cpu().numpy()
    assert list(first) == dec.prefill(list(range(B)), prompts, max_new)
    gen = [[int(first[b])] for b in range(B)]
    for _ in range(40):
        if all(st.state == OI.STATE_DONE for st in dec.slots.values()):
            break
        tok, nc, _ = eng.step()
        dec.step()
        torch.cuda.synchronize()
        t, n = tok.cpu().numpy(), nc.cpu().numpy()
        for b in range(B):
            gen[b] += [int(x) for x in t[b, :n[b]]]
    gs = eng.slots_host()
    for b in range(B):
        st = dec.slots[b]
        assert gen[b] == st.generated, b
        assert gs[b]["meter_n"] == st.meter_n and st.meter_n > 0
        np.testing.assert_allclose(gs[b]["meter_sum"], st.meter_sum, rtol=1e-5, atol=1e-9)
