"""Pins of oracle.model against library routines and invariants (CPU only).

Independent references: torch's scaled_dot_product_attention (GQA and boolean mask),
torch.nn.functional.rms_norm, RoPE written as complex multiplication, and closed forms
(a single visible key returns its value; zero queries average the visible values).
Invariants: causality, KV-cache incremental == one-shot forward, RoPE relative-position
invariance, LoRA gating (clean rows bit-identical to the base model, MASK rows equal to
the merged weight W + B A).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import isd_inputs as I
from oracle import model as M


def spec_of(shape):
    return M.Spec(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                  shape.d_ffn, shape.vocab, shape.rope_base, shape.rms_eps)


TINY_GQA = I.ModelShape("tiny-gqa", 2, 64, 4, 2, 16, 96, 50, "f32")


def _model(shape=TINY_GQA, lora_rank=0):
    w = I.weights_numpy(shape, seed=11)
    lora = I.lora_numpy(shape, lora_rank, seed=12) if lora_rank else None
    return M.Model(spec_of(shape), w, lora)


# ---------------------------------------------------------------- attention
def _sdpa_ref(q, k, v, q_pos, k_pos):
    """torch SDPA in float64 with an explicit visibility mask and GQA."""
    qt = torch.tensor(q, dtype=torch.float64).permute(1, 0, 2)[None]
    kt = torch.tensor(k, dtype=torch.float64).permute(1, 0, 2)[None]
    vt = torch.tensor(v, dtype=torch.float64).permute(1, 0, 2)[None]
    mask = torch.tensor(np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None])
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("Hq,Hkv,L,R", [(4, 4, 0, 5), (8, 2, 37, 7), (32, 8, 130, 7), (6, 3, 16, 1)])
def test_attention_matches_sdpa(Hq, Hkv, L, R):
    g = np.random.default_rng(0)
    hd = 16
    q = g.standard_normal((R, Hq, hd)).astype(np.float32)
    k = g.standard_normal((L + R, Hkv, hd)).astype(np.float32)
    v = g.standard_normal((L + R, Hkv, hd)).astype(np.float32)
    q_pos = L + np.arange(R)
    k_pos = np.arange(L + R)
    got = M.causal_attention(q, k, v, q_pos, k_pos, Hq // Hkv)
    ref = _sdpa_ref(q, k, v, q_pos, k_pos)
    np.testing.assert_allclose(got, ref, atol=2e-6, rtol=2e-5)


def test_attention_closed_forms():
    g = np.random.default_rng(1)
    hd, Hq, Hkv = 8, 4, 2
    k = g.standard_normal((9, Hkv, hd)).astype(np.float32)
    v = g.standard_normal((9, Hkv, hd)).astype(np.float32)
    q = g.standard_normal((1, Hq, hd)).astype(np.float32)
    # only key 0 visible -> output is v[0] of the head's group
    o = M.causal_attention(q, k, v, np.array([0]), np.arange(9), 2)
    np.testing.assert_allclose(o[0], v[0, np.arange(Hq) // 2], atol=1e-6)
    # zero query -> uniform weights over the visible keys
    o = M.causal_attention(np.zeros_like(q), k, v, np.array([4]), np.arange(9), 2)
    np.testing.assert_allclose(o[0], v[:5, np.arange(Hq) // 2].mean(axis=0), atol=1e-6)


def test_paged_gather_matches_dense():
    g = np.random.default_rng(2)
    P, Hkv, hd, L = 4, 2, 8, 23
    n_pages = 12
    pool = g.standard_normal((n_pages, Hkv, P, hd)).astype(np.float32)
    table = g.permutation(n_pages)[: -(-L // P)]
    dense = np.concatenate([pool[p].transpose(1, 0, 2) for p in table])[:L]
    np.testing.assert_array_equal(M.gather_pages(pool, table, L, P), dense)
    # token j is at page table[j//P], slot j%P
    j = 13
    np.testing.assert_array_equal(M.gather_pages(pool, table, L, P)[j], pool[table[j // P], :, j % P])


# ---------------------------------------------------------------- norm / rope
def test_rmsnorm_matches_torch():
    g = np.random.default_rng(3)
    x = g.standard_normal((5, 64)).astype(np.float32) * 3
    w = g.standard_normal(64).astype(np.float32)
    ref = F.rms_norm(torch.tensor(x, dtype=torch.float64), (64,), torch.tensor(w, dtype=torch.float64), eps=1e-6)
    np.testing.assert_allclose(M.rmsnorm(x, w, 1e-6), ref.numpy(), rtol=1e-5, atol=1e-6)


def _rope_complex(x, pos, base):
    """RoPE as multiplication of (x_i + i x_{i+hd/2}) by exp(i pos base^(-2i/hd))."""
    hd = x.shape[-1]
    half = hd // 2
    xt = torch.tensor(x, dtype=torch.float64)
    z = torch.complex(xt[..., :half], xt[..., half:])
    inv = torch.tensor(float(base), dtype=torch.float64) ** (-2.0 * torch.arange(half, dtype=torch.float64) / hd)
    ang = torch.tensor(pos, dtype=torch.float64)[:, None] * inv[None]
    z = z * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    return torch.cat([z.real, z.imag], dim=-1).numpy()


def test_rope_matches_complex_rotation():
    g = np.random.default_rng(4)
    x = g.standard_normal((6, 3, 32)).astype(np.float32)
    pos = np.array([0, 1, 2, 100, 4095, 6150])
    np.testing.assert_allclose(M.apply_rope(x, pos, 10000.0), _rope_complex(x, pos, 10000.0), atol=2e-6)


def test_rope_relative_position():
    g = np.random.default_rng(5)
    q = g.standard_normal((1, 1, 64)).astype(np.float32)
    k = g.standard_normal((1, 1, 64)).astype(np.float32)
    d1 = (M.apply_rope(q, [50], 1e4) * M.apply_rope(k, [20], 1e4)).sum()
    d2 = (M.apply_rope(q, [130], 1e4) * M.apply_rope(k, [100], 1e4)).sum()
    assert abs(d1 - d2) < 1e-4
    np.testing.assert_allclose(np.linalg.norm(M.apply_rope(q, [77], 1e4)), np.linalg.norm(q), rtol=1e-6)


# ---------------------------------------------------------------- whole model
def _torch_forward(spec, w, ids, lora=None, is_mask=None):
    """float64 forward composed from torch library routines (independent formulation)."""
    t = lambda a: torch.tensor(M.f32(a), dtype=torch.float64)
    R = len(ids)
    x = t(w["embed"])[torch.tensor(ids)]
    qd, kd = spec.n_q_heads * spec.head_dim, spec.n_kv_heads * spec.head_dim
    pos = np.arange(R)
    msk = torch.tensor(is_mask if is_mask is not None else np.zeros(R, bool))[:, None]
    for li, L in enumerate(w["layers"]):
        def lin(h, wt, tgt):
            y = F.linear(h, wt)
            if lora is not None:
                a, b = lora[li][tgt]
                y = y + torch.where(msk, F.linear(F.linear(h, t(a)), t(b)), torch.zeros_like(y))
            return y
        h = F.rms_norm(x, (spec.d_model,), t(L["attn_norm"]), eps=spec.rms_eps)
        wqkv = t(L["wqkv"])
        q = lin(h, wqkv[:qd], "q").reshape(R, spec.n_q_heads, spec.head_dim)
        k = lin(h, wqkv[qd:qd + kd], "k").reshape(R, spec.n_kv_heads, spec.head_dim)
        v = lin(h, wqkv[qd + kd:], "v").reshape(R, spec.n_kv_heads, spec.head_dim)
        q = torch.tensor(_rope_complex(q.numpy(), pos, spec.rope_base))
        k = torch.tensor(_rope_complex(k.numpy(), pos, spec.rope_base))
        o = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], k.permute(1, 0, 2)[None],
                                           v.permute(1, 0, 2)[None], is_causal=True, enable_gqa=True)
        o = o[0].permute(1, 0, 2).reshape(R, qd)
        x = x + lin(o, t(L["wo"]), "o")
        h2 = F.rms_norm(x, (spec.d_model,), t(L["ffn_norm"]), eps=spec.rms_eps)
        x = x + lin(F.silu(lin(h2, t(L["wg"]), "g")) * lin(h2, t(L["wu"]), "u"), t(L["wd"]), "d")
    x = F.rms_norm(x, (spec.d_model,), t(w["final_norm"]), eps=spec.rms_eps)
    return F.linear(x, t(w["lm_head"])).numpy()


def test_model_matches_torch_composition():
    m = _model()
    ids = I.prompts(1, 19, m.spec.vocab, seed=5)[0]
    logits, _ = m.forward(ids, np.arange(len(ids)), M.empty_cache(m.spec))
    ref = _torch_forward(m.spec, m.w, ids)
    np.testing.assert_allclose(logits, ref, atol=2e-5, rtol=1e-4)


def test_model_with_lora_matches_torch_composition():
    m = _model(lora_rank=8)
    ids = I.prompts(1, 11, m.spec.vocab, seed=6)[0]
    is_mask = np.zeros(len(ids), bool)
    is_mask[[3, 7, 8]] = True
    logits, _ = m.forward(ids, np.arange(len(ids)), M.empty_cache(m.spec), is_mask=is_mask)
    ref = _torch_forward(m.spec, m.w, ids, lora=m.lora, is_mask=is_mask)
    np.testing.assert_allclose(logits, ref, atol=2e-5, rtol=1e-4)


def test_kv_cache_incremental_equals_one_shot():
    m = _model()
    ids = I.prompts(1, 23, m.spec.vocab, seed=7)[0]
    full, kv_full = m.forward(ids, np.arange(23), M.empty_cache(m.spec))
    a, kv_a = m.forward(ids[:15], np.arange(15), M.empty_cache(m.spec))
    cache = M.extend_cache(M.empty_cache(m.spec), kv_a, 15)
    b, kv_b = m.forward(ids[15:], np.arange(15, 23), cache)
    np.testing.assert_allclose(np.concatenate([a, b]), full, atol=1e-5)
    for (k1, v1), (k2, v2) in zip(kv_full, kv_b):
        np.testing.assert_allclose(k1[15:], k2, atol=1e-5)
        np.testing.assert_allclose(v1[15:], v2, atol=1e-5)


def test_causality_future_tokens_do_not_leak():
    m = _model()
    ids = I.prompts(1, 12, m.spec.vocab, seed=8)[0]
    ids2 = ids.copy()
    ids2[9] = (ids2[9] + 1) % m.spec.vocab
    a, _ = m.forward(ids, np.arange(12), M.empty_cache(m.spec))
    b, _ = m.forward(ids2, np.arange(12), M.empty_cache(m.spec))
    np.testing.assert_array_equal(a[:9], b[:9])
    assert np.abs(a[9:] - b[9:]).max() > 1e-3


def test_position_shift_invariance():
    m = _model()
    ids = I.prompts(1, 10, m.spec.vocab, seed=9)[0]
    a, _ = m.forward(ids, np.arange(10), M.empty_cache(m.spec))
    b, _ = m.forward(ids, 300 + np.arange(10), M.empty_cache(m.spec))
    np.testing.assert_allclose(a, b, atol=5e-4)


def test_lora_gating_clean_rows_bit_identical_and_mask_rows_merged():
    m = _model(lora_rank=8)
    base = M.Model(m.spec, m.w, None)
    ids = np.array(list(I.prompts(1, 6, m.spec.vocab, seed=10)[0]) + [m.spec.mask_id] * 3)
    is_mask = ids == m.spec.mask_id
    got, _ = m.forward(ids, np.arange(9), M.empty_cache(m.spec), is_mask=is_mask)
    ref, _ = base.forward(ids, np.arange(9), M.empty_cache(m.spec))
    np.testing.assert_array_equal(got[:6], ref[:6])        # verify rows: base weights only
    assert np.abs(got[6:] - ref[6:]).max() > 1e-3
    # MASK rows see the merged weights W + B A (closed form of the low-rank update)
    merged = {"embed": m.w["embed"], "final_norm": m.w["final_norm"], "lm_head": m.w["lm_head"], "layers": []}
    qd, kd = m.spec.n_q_heads * m.spec.head_dim, m.spec.n_kv_heads * m.spec.head_dim
    for L, lo in zip(m.w["layers"], m.lora):
        dw = {t: M.f32(lo[t][1]) @ M.f32(lo[t][0]) for t in lo}
        Lm = dict(L)
        Lm["wqkv"] = M.f32(L["wqkv"]) + np.concatenate([dw["q"], dw["k"], dw["v"]])
        for t, key in (("o", "wo"), ("g", "wg"), ("u", "wu"), ("d", "wd")):
            Lm[key] = M.f32(L[key]) + dw[t]
        merged["layers"].append(Lm)
    # an all-MASK block under merged weights equals the gated model's all-MASK block
    allmask = np.full(4, m.spec.mask_id)
    g2, _ = m.forward(allmask, np.arange(4), M.empty_cache(m.spec), is_mask=np.ones(4, bool))
    r2, _ = M.Model(m.spec, merged, None).forward(allmask, np.arange(4), M.empty_cache(m.spec))
    np.testing.assert_allclose(g2, r2, atol=2e-5, rtol=1e-4)


def test_round_bf16_is_nearest_even():
    """The precision model's rounding: ties to even on hand-made halfway cases, and torch's
    float32 -> bfloat16 conversion on random values over many binades."""
    h = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 3 * 2 ** -8)], np.float32)
    want = np.array([1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, -(1 + 2 ** -6)], np.float32)
    np.testing.assert_array_equal(M.round_bf16(h), want)
    g = np.random.default_rng(5)
    x = (g.standard_normal(100000) * np.exp2(g.integers(-40, 40, 100000))).astype(np.float32)
    np.testing.assert_array_equal(M.round_bf16(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_act_bf16_mode_rounds_stored_activations():
    """act_bf16 = True: the attention outputs it reports are bfloat16 values, the KV it returns
    too, and the logits stay within the bf16 storage error of the fp32 forward."""
    shape = I.SMALL_BF16
    w = I.weights_numpy(shape, seed=0)
    spec = M.Spec(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.d_ffn,
                  shape.vocab, shape.rope_base, shape.rms_eps)
    ids = I.ragged_prompts([9], shape.vocab, seed=4)[0]
    pos = np.arange(len(ids))
    l32, _ = M.Model(spec, w).forward(ids, pos, M.empty_cache(spec))
    l16, kv, att = M.Model(spec, w, act_bf16=True).forward(ids, pos, M.empty_cache(spec), return_hidden=True)
    for a in att + [t for pair in kv for t in pair]:
        assert not (np.ascontiguousarray(a, np.float32).view(np.uint32) & 0xFFFF).any()
    err = np.abs(l16 - l32).max() / np.abs(l32).max()
    assert 0 < err < 2e-2, err
