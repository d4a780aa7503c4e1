"""fp32 causal transformer of the ISD decode step (oracle; test infrastructure only).

What the pages fix: the model keeps *strict causal attention* and the *logit shift*
(the output at position i predicts the token at i+1), so one forward pass over a
block of rows appended to a KV cache is an ordinary causal decoder pass (wiki note
"Introspective Diffusion Language Models", sections *TL;DR* and *Method*; Agentic
Commons post, section *Introspective Consistency*).  R-ISD adds a gated LoRA that
is active only at MASK positions while verify positions use the base weights
(wiki note, *Key claims* and *Method*; GeekNews, *Lossless R-ISD*).

The pages give no architecture; the configurations name a Qwen3-shaped pre-norm
decoder, read here as (no biases, untied LM head, no QK-norm):

    h  = x + Wo * Attn(RoPE(Wq n(x)), RoPE(Wk n(x)), Wv n(x)),   n = RMSNorm
    x' = h + Wd (silu(Wg n(h)) * Wu n(h))
    logits = Wlm RMSNorm(x_last)

RMSNorm(x) = g * x / sqrt(mean(x^2) + eps).  RoPE is the rotate-half form with
angle pos * base^(-2i/hd), i < hd/2; the cos/sin values are computed in float64
and rounded to float32.  Grouped-query attention: query head h reads KV head
h // (Hq/Hkv); scores are scaled by 1/sqrt(hd).  The MASK token id equals the
vocabulary size V and indexes row V of the (V+1)-row embedding table, so the LM
head (V columns) can never emit it.

Weight layout (each matrix stored out x in, y = x @ W.T):
    embed [V+1, d], final_norm [d], lm_head [V, d]
    per layer: attn_norm [d], wqkv [(Hq+2Hkv)*hd, d] (q rows, then k, then v),
               wo [d, Hq*hd], ffn_norm [d], wg [F, d], wu [F, d], wd [d, F]
LoRA per layer and target m in (q, k, v, o, g, u, d):
    a[m] [r, d_in], b[m] [d_out, r];  y_m += is_mask * (x @ a[m].T) @ b[m].T

Matrices may be float32 arrays or bf16 bit patterns (uint16); the latter are
widened to float32 (exactly) before use, so the oracle computes in fp32 on the
same values the bf16 GPU path stores.

Model(..., act_bf16=True) is a precision model of that path, not a second reference:
activations are rounded to bfloat16 (nearest, ties to even) where the bf16 path stores
them between kernels (the two RMSNorm outputs of a layer and the final one, q/k/v after
RoPE and hence the KV cache, the attention output, the SwiGLU product); everything else
stays fp32.  Its distance from the fp32 forward is the error that bf16 storage alone
causes, the yardstick for the GPU path's deviation at depth.
"""
from dataclasses import dataclass

import numpy as np

LORA_TARGETS = ("q", "k", "v", "o", "g", "u", "d")


@dataclass(frozen=True)
class Spec:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    rope_base: float = 10000.0
    rms_eps: float = 1e-6

    @property
    def mask_id(self):
        return self.vocab

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads


def f32(a):
    """float32 view of a weight: float arrays are cast, uint16 arrays are bf16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return a.astype(np.float32, copy=False)


def round_bf16(x):
    """float32 -> the nearest bfloat16 value (ties to even), returned as float32 (finite x)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def rmsnorm(x, g, eps):
    x = x.astype(np.float32, copy=False)
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=np.float32)
    return (x / np.sqrt(ms + np.float32(eps))) * f32(g)


def rope_tables(positions, head_dim, base):
    """cos, sin [len(positions), head_dim/2] float32 (computed in float64, then rounded)."""
    half = head_dim // 2
    inv_freq = np.power(float(base), -2.0 * np.arange(half, dtype=np.float64) / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def apply_rope(x, positions, base):
    """x [R, H, hd] float32, rotate-half RoPE at the given absolute positions."""
    hd = x.shape[-1]
    half = hd // 2
    cos, sin = rope_tables(positions, hd, base)
    cos = cos[:, None, :]
    sin = sin[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1).astype(np.float32)


def silu(x):
    return x / (np.float32(1.0) + np.exp(-x))


def causal_attention(q, k_all, v_all, q_pos, k_pos, group):
    """Dense causal attention.

    q [R, Hq, hd]; k_all, v_all [Lk, Hkv, hd]; q_pos [R]; k_pos [Lk].
    Row r attends to every key j with k_pos[j] <= q_pos[r].  Returns [R, Hq, hd].
    """
    R, Hq, hd = q.shape
    kv_head = np.arange(Hq) // group
    k = k_all[:, kv_head, :]                      # [Lk, Hq, hd]
    v = v_all[:, kv_head, :]
    scores = np.einsum("rhd,khd->hrk", q, k) / np.float32(np.sqrt(hd))
    visible = k_pos[None, :] <= q_pos[:, None]    # [R, Lk]
    scores = np.where(visible[None], scores, -np.inf)
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - m)
    pr = e / e.sum(axis=-1, keepdims=True)
    return np.einsum("hrk,khd->rhd", pr.astype(np.float32), v).astype(np.float32)


def gather_pages(pool, page_table, length, page_size):
    """Dense [length, Hkv, hd] view of a paged cache.

    pool [n_pages, Hkv, page_size, hd]; page_table [n_logical] page ids.
    Token j lives in page page_table[j // page_size], slot j % page_size.
    """
    n_log = -(-length // page_size)
    pages = pool[np.asarray(page_table[:n_log], dtype=np.int64)]   # [n_log, Hkv, P, hd]
    dense = pages.transpose(0, 2, 1, 3).reshape(n_log * page_size, pool.shape[1], pool.shape[3])
    return dense[:length]


def paged_attention(q, pool_k, pool_v, page_table, ctx_len, q_pos, group, page_size):
    """Attention of a block of query rows against a paged cache holding ctx_len tokens.

    The block's own keys are already in the pages (positions ctx_len - R .. ctx_len - 1
    for a block of R rows), as a paged-only kernel sees them.
    """
    k = f32(gather_pages(pool_k, page_table, ctx_len, page_size))
    v = f32(gather_pages(pool_v, page_table, ctx_len, page_size))
    return causal_attention(q.astype(np.float32), k, v, np.asarray(q_pos), np.arange(ctx_len), group)


def _lin(x, w, lora_a=None, lora_b=None, row_mask=None):
    y = x @ f32(w).T
    if lora_a is not None and row_mask is not None and np.any(row_mask):
        d = (x @ f32(lora_a).T) @ f32(lora_b).T
        y = y + np.where(row_mask[:, None], d, np.float32(0.0)).astype(np.float32)
    return y.astype(np.float32)


def layer_forward(spec, L, x, positions, ck, cv, lo=None, is_mask=None, rd=None):
    """One pre-norm decoder layer over a block of rows of one sequence.

    L: the layer's weights (attn_norm, wqkv, wo, ffn_norm, wg, wu, wd); x [R, d] float32 the
    residual stream entering the layer; positions [R]; ck, cv [Lc, Hkv, hd] the cached keys and
    values of positions 0 .. Lc-1; lo: None or the layer's LoRA {m: (a, b)}, applied on the
    rows of is_mask; rd: the activation rounding of the bf16 precision model (None = none).
    Returns (x_out [R, d], (k, v) of the block [R, Hkv, hd], attention output [R, Hq, hd]).
    """
    s = spec
    rd = rd if rd is not None else (lambda a: a)
    R = x.shape[0]
    if is_mask is None:
        is_mask = np.zeros(R, dtype=bool)
    qd, kd = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim

    def lin(inp, w, tgt):
        if lo is None:
            return _lin(inp, w)
        a, b = lo[tgt]
        return _lin(inp, w, a, b, is_mask)

    h = rd(rmsnorm(x, L["attn_norm"], s.rms_eps))
    wqkv = f32(L["wqkv"])
    q = lin(h, wqkv[:qd], "q").reshape(R, s.n_q_heads, s.head_dim)
    k = lin(h, wqkv[qd:qd + kd], "k").reshape(R, s.n_kv_heads, s.head_dim)
    v = lin(h, wqkv[qd + kd:], "v").reshape(R, s.n_kv_heads, s.head_dim)
    q = rd(apply_rope(q, positions, s.rope_base))
    k = rd(apply_rope(k, positions, s.rope_base))
    v = rd(v)
    k_all = np.concatenate([ck, k], axis=0)
    v_all = np.concatenate([cv, v], axis=0)
    k_pos = np.concatenate([np.arange(len(ck)), positions])
    o = rd(causal_attention(q, k_all, v_all, positions, k_pos, s.group))
    x = x + lin(o.reshape(R, qd), L["wo"], "o")
    h2 = rd(rmsnorm(x, L["ffn_norm"], s.rms_eps))
    g = lin(h2, L["wg"], "g")
    u = lin(h2, L["wu"], "u")
    x = x + lin(rd((silu(g) * u).astype(np.float32)), L["wd"], "d")
    return x, (k, v), o


class Model:
    """fp32 forward of a block of rows of ONE sequence on top of its KV cache.

    weights: dict with the keys listed in the module docstring; per-layer tensors in
    weights["layers"][l].  lora: None or list (per layer) of dicts {m: (a, b)}.
    """

    def __init__(self, spec, weights, lora=None, act_bf16=False):
        self.spec = spec
        self.w = weights
        self.lora = lora
        self.rd = round_bf16 if act_bf16 else (lambda a: a)

    def embed(self, ids):
        return f32(self.w["embed"])[np.asarray(ids, dtype=np.int64)].astype(np.float32)

    def forward(self, ids, positions, cache, is_mask=None, return_hidden=False):
        """Forward a block.

        ids, positions: [R] ints (positions need not start at len(cache) for tests, but
        the decode step uses consecutive positions L..L+R-1).
        cache: list per layer of (K [L, Hkv, hd], V [L, Hkv, hd]) float32, positions 0..L-1.
        is_mask: [R] bool selecting the rows where the LoRA is active.
        Returns (logits [R, V] float32, block_kv list per layer of (K [R,...], V [R,...]),
        and the per-layer attention outputs when return_hidden).
        """
        s = self.spec
        ids = np.asarray(ids, dtype=np.int64)
        positions = np.asarray(positions, dtype=np.int64)
        R = len(ids)
        if is_mask is None:
            is_mask = np.zeros(R, dtype=bool)
        x = self.embed(ids)
        block_kv = []
        attn_out = []
        for li, L in enumerate(self.w["layers"]):
            lo = self.lora[li] if self.lora is not None else None
            if cache is not None:
                ck, cv = cache[li]
            else:
                ck = cv = np.zeros((0, s.n_kv_heads, s.head_dim), np.float32)
            x, kv, o = layer_forward(s, L, x, positions, ck, cv, lo, is_mask, self.rd)
            block_kv.append(kv)
            attn_out.append(o)
        logits = self.rd(rmsnorm(x, self.w["final_norm"], s.rms_eps)) @ f32(self.w["lm_head"]).T
        logits = logits.astype(np.float32)
        if return_hidden:
            return logits, block_kv, attn_out
        return logits, block_kv


def empty_cache(spec):
    z = np.zeros((0, spec.n_kv_heads, spec.head_dim), np.float32)
    return [(z, z) for _ in range(spec.n_layers)]


def extend_cache(cache, block_kv, keep):
    """Append the first `keep` rows of a block's K/V to the cache (per layer)."""
    return [(np.concatenate([ck, bk[:keep]]), np.concatenate([cv, bv[:keep]]))
            for (ck, cv), (bk, bv) in zip(cache, block_kv)]
