"""Full-size parity at the Qwen3-8B shape in the benchmark's launch configuration (64 slots x
7 rows = 448 rows, N = 4, argmax proposals, T = 1: the same GEMM tiles, split-K factors and
attention split length as the timed pass).

test_fullsize_8b_layer_by_layer (the benchmark's own workload: 1024-token prompts, contexts
sized for 1024 + 1024 tokens) follows three sampled slots through two passes (a B pass of 4
live rows, then an A pass of 7) with the isd_debug record, and checks every one of the 36
layers on its own: the oracle's fp32 layer, fed the GPU's residual input of that layer and
the GPU's KV cache of the context, must give the GPU's attention output, the GPU's output
residual and the GPU's residual update within the bf16 bar, ||gpu - ref||_inf <= 2e-2
||ref||_inf per tensor.  The final RMSNorm and the LM head are checked the same way from the
GPU's final residual, and the decisions taken on the GPU's logits equal the committed tokens
(with the kernel's decision record equal to the oracle's).  Teacher-forcing every layer keeps
errors from compounding, so a wrong head, position, weight or a systematic percent-level
error in any one layer fails here.

test_fullsize_8b_decode_pass_end_to_end (short prompts, so that the oracle can run whole
prefills) records the other reading: the whole 36-layer pass against the fp32 forward and the
oracle's bf16 precision model.  Through 36 random-init layers any bf16-level perturbation
grows to a few percent of the logit range (the precision model and the fp32 forward differ
by ~4-5 %; the GPU and the precision model are two different rounding sequences, as far
apart), so that test holds the GPU to the size of that storage error.  The oracle needs the
weights in fp32 on the host (one layer at a time for the layer-by-layer test).
"""
import numpy as np
import pytest
import torch

import isd_inputs as I
from oracle import isd as OI
from oracle import model as M

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16_REL = 2e-2
KIND = {"accept": 0, "resid": 1, "z1": 2, "propose": 3}


def _host_f32(t):
    return t.float().cpu().numpy()


def _rel(a, r):
    """||a - r||_inf / ||r||_inf over the whole tensor."""
    return float(np.abs(a - r).max() / max(float(np.abs(r).max()), 1e-30))


def _spec(shape):
    return M.Spec(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.d_ffn,
                  shape.vocab, shape.rope_base, shape.rms_eps)


@pytest.mark.timeout(900)
def test_fullsize_8b_layer_by_layer():
    from strided_decoding_amd import Engine
    shape, wl = I.QWEN3_8B, I.QWEN3_8B_DECODE
    B, N, T, plen, gen = wl.batch, wl.stride, wl.temperature, wl.prompt_len, wl.max_new
    R = 2 * N - 1
    print("layer-by-layer: generating weights on the device", flush=True)
    weights, _ = I.weights_torch(shape, DEV)
    eng = Engine(shape, weights, stride=N, temperature=T, propose=wl.propose, seed=I.SEED_PHILOX, max_batch=B,
                 max_seq_len=plen + gen + 2 * N + 8, max_prefill_tokens=16 * plen, device=DEV)
    prompts = I.prompts(B, plen, shape.vocab)
    for s0 in range(0, B, 16):
        sl = list(range(s0, s0 + 16))
        eng.prefill(sl, [prompts[b] for b in sl], [gen] * 16)
    sampled = [0, 37, 63]
    rows = [b * R + i for b in sampled for i in range(R)]
    passes = []
    for p in range(2):
        before = eng.slots_host()
        dbg = eng.make_debug(rows)
        tok, nc, _ = eng.step(debug=dbg)
        torch.cuda.synchronize()
        lg = eng.logits()
        passes.append(dict(
            slots={b: before[b] for b in sampled},
            layer_in=dbg.layer_in.cpu().numpy(), attn=_host_f32(dbg.layer_attn), final=_host_f32(dbg.final_normed),
            logits={b: lg[b].cpu().numpy() for b in sampled}, tok=tok.cpu().numpy(), nc=nc.cpu().numpy(),
            margins=dbg.margins.cpu().numpy(), kinds=dbg.kinds.cpu().numpy()))
        print(f"layer-by-layer: pass {p} done (slot states {[before[b]['state'] for b in sampled]})", flush=True)
    assert eng.status() == 0
    pt = eng.page_table().cpu().numpy()
    kp, vp = eng.kv_pools()
    spec = _spec(shape)
    P = eng.cfg.page_size

    def context_kv(layer, b, L):
        ids = pt[b, :-(-L // P)].astype(np.int64)
        assert np.all(ids >= 0) and np.all(ids < eng.cfg.n_pages), (b, L)    # checked before indexing
        pages = torch.from_numpy(ids).to(DEV)
        k = kp[layer].index_select(0, pages).permute(0, 2, 1, 3).reshape(-1, shape.n_kv_heads, shape.head_dim)
        v = vp[layer].index_select(0, pages).permute(0, 3, 1, 2).reshape(-1, shape.n_kv_heads, shape.head_dim)
        return _host_f32(k[:L]), _host_f32(v[:L])

    worst = {"attn": 0.0, "out": 0.0, "delta": 0.0}
    for layer in range(shape.n_layers):
        Wl = {k: _host_f32(v) for k, v in weights["layers"][layer].items()}
        e = {"attn": 0.0, "out": 0.0, "delta": 0.0}
        for rec in passes:
            for si, b in enumerate(sampled):
                st = rec["slots"][b]
                L = st["L"]
                n_live = R if st["state"] == 1 else N
                ri = slice(si * R, si * R + n_live)
                x_in = rec["layer_in"][layer, ri]
                ck, cv = context_kv(layer, b, L)
                x_out, _, o = M.layer_forward(spec, Wl, x_in, L + np.arange(n_live), ck, cv)
                g_out = rec["layer_in"][layer + 1, ri]
                e["attn"] = max(e["attn"], _rel(rec["attn"][layer, ri], o.reshape(n_live, -1)))
                e["out"] = max(e["out"], _rel(g_out, x_out))
                e["delta"] = max(e["delta"], _rel(g_out - x_in, x_out - x_in))
        print(f"layer {layer:2d}: attention {e['attn']:.2e}  output residual {e['out']:.2e}  "
              f"residual update {e['delta']:.2e}", flush=True)
        for k in worst:
            worst[k] = max(worst[k], e[k])
        del Wl
    print(f"layer-by-layer worst: {worst}", flush=True)
    for k, v in worst.items():
        assert v <= BF16_REL, (k, v)

    # final RMSNorm and LM head from the GPU's final residual; decisions on the GPU's logits
    fn = _host_f32(weights["final_norm"])
    W_lm = _host_f32(weights["lm_head"])
    for rec in passes:
        for si, b in enumerate(sampled):
            st = rec["slots"][b]
            n_live = R if st["state"] == 1 else N
            ri = slice(si * R, si * R + n_live)
            ref_norm = M.rmsnorm(rec["layer_in"][shape.n_layers, ri], fn, shape.rms_eps)
            e_norm = _rel(rec["final"][ri], ref_norm)
            ref_logits = rec["final"][ri] @ W_lm.T
            e_lm = _rel(rec["logits"][b][:n_live], ref_logits)
            print(f"slot {b} state {st['state']}: final norm {e_norm:.2e}  LM head {e_lm:.2e}", flush=True)
            assert e_norm <= BF16_REL and e_lm <= BF16_REL, (b, e_norm, e_lm)
            state = "A" if st["state"] == 1 else "B"
            pend = [st[f"pending{j}"] for j in range(N - 1)] if state == "A" else []
            out = OI.decide(state, st["L"], st["t"], b, pend, [None] * len(pend), rec["logits"][b][:n_live],
                            N, T, wl.propose, I.SEED_PHILOX)
            assert [int(x) for x in rec["tok"][b, :rec["nc"][b]]] == out.tokens, (b, rec["tok"][b], out.tokens)
            for j, d in enumerate(out.decisions):
                assert rec["kinds"][b, j] == KIND[d.kind]
                np.testing.assert_allclose(rec["margins"][b, j], d.margin, rtol=1e-5, atol=3e-7)
            assert np.all(rec["kinds"][b, len(out.decisions):] == -1)


@pytest.mark.timeout(900)
def test_fullsize_8b_decode_pass_end_to_end():
    from strided_decoding_amd import Engine
    shape = I.QWEN3_8B
    B, N, T, prompt_len, gen = 64, 4, 1.0, 24, 1024
    print("full-size: generating weights on the device", flush=True)
    weights, _ = I.weights_torch(shape, DEV)
    eng = Engine(shape, weights, stride=N, temperature=T, propose="argmax", seed=I.SEED_PHILOX, max_batch=B,
                 max_seq_len=prompt_len + gen + 2 * N + 8, max_prefill_tokens=16 * 1024, device=DEV)
    prompts = I.prompts(B, prompt_len, shape.vocab)
    first = []
    for s0 in range(0, B, 16):
        sl = list(range(s0, s0 + 16))
        first += eng.prefill(sl, [prompts[b] for b in sl], [gen] * 16).cpu().tolist()
    tok, nc, _ = eng.step()
    torch.cuda.synchronize()
    logits = eng.logits()
    sampled = [0, 37, 63]
    got = {b: logits[b, :N].cpu().numpy() for b in sampled}
    tok, nc = tok.cpu().numpy(), nc.cpu().numpy()
    print("full-size: GPU pass done; weights to the host in fp32", flush=True)

    w = {k: _host_f32(weights[k]) for k in ("embed", "final_norm", "lm_head")}
    w["layers"] = [{k: _host_f32(v) for k, v in layer.items()} for layer in weights["layers"]]
    del weights, eng
    torch.cuda.empty_cache()
    spec = _spec(shape)
    model = M.Model(spec, w)
    model16 = M.Model(spec, w, act_bf16=True)
    for b in sampled:
        print(f"full-size: oracle forwards of slot {b}", flush=True)
        p = [int(x) for x in prompts[b]]
        L = len(p)
        ids = [int(first[b])] + [shape.vocab] * (N - 1)
        refs = []
        for m in (model, model16):
            _, kv = m.forward(p, np.arange(L), M.empty_cache(spec))
            cache = M.extend_cache(M.empty_cache(spec), kv, L)
            refs.append(m.forward(ids, L + np.arange(N), cache)[0])
        ref32, ref16 = refs

        def rel(a, r):
            return float((np.abs(a - r).max(axis=1) / np.abs(r).max(axis=1)).max())
        e_gpu16, e_gpu32, e_16_32 = rel(got[b], ref16), rel(got[b], ref32), rel(ref16, ref32)
        print(f"full-size: slot {b}: GPU vs bf16 model {e_gpu16:.2e}, GPU vs fp32 {e_gpu32:.2e}, "
              f"bf16 model vs fp32 {e_16_32:.2e}", flush=True)
        assert e_gpu32 <= 2 * e_16_32 + 1e-2, (b, e_gpu32, e_16_32)
        assert e_gpu16 <= 3 * e_16_32 + 1e-2, (b, e_gpu16, e_16_32)
        out = OI.decide("B", L, 1, b, [], [], got[b], N, T, "argmax", I.SEED_PHILOX)
        assert [int(x) for x in tok[b, :nc[b]]] == out.tokens, (b, tok[b, :nc[b]], out.tokens)
