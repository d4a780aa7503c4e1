"""Seeded synthetic inputs shared by the oracle-side tests, the GPU tests and the bench.

This module holds the workload recipes (model shapes, batch/prompt/stride settings)
and the seeded generators of weights, prompts and kernel-level inputs.  It contains
none of the decoding method's arithmetic: no forward pass, no softmax, no sampling
rule.  Neither the oracle nor the HIP library depends on the other; both may take
their inputs from here.

Seeds: weights 0, Philox stream 1, LoRA 2, prompts / context lengths / page shuffles 3.
Weights are N(0, 0.02) for every matrix (embedding, projections, LM head, LoRA A and B);
norm gains are 1.  The pages' trained checkpoints and evaluation prompts are not
available, so random weights and uniformly random prompt ids stand in for them.
"""
from dataclasses import dataclass, replace

import numpy as np

SEED_WEIGHTS = 0
SEED_PHILOX = 1
SEED_LORA = 2
SEED_DATA = 3
INIT_STD = 0.02
LORA_TARGETS = ("q", "k", "v", "o", "g", "u", "d")


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    dtype: str                 # "f32" or "bf16": the storage / compute type of the GPU path
    rope_base: float = 10000.0
    rms_eps: float = 1e-6

    @property
    def qkv_rows(self):
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def n_params(self):
        d, F, V = self.d_model, self.d_ffn, self.vocab
        per_layer = self.qkv_rows * d + d * self.n_q_heads * self.head_dim + 3 * F * d + 2 * d
        return (V + 1) * d + self.n_layers * per_layer + d + V * d


# Tiny end-to-end model: 2 layers, d 128, 4 heads x 32 (no KV-head count is given, so MHA),
# SwiGLU 512, vocab 1024, fp32.
TINY = ModelShape("tiny", 2, 128, 4, 4, 32, 512, 1024, "f32")
# Small bf16 model used for bf16-path parity at oracle-friendly sizes (same head_dim and
# grouping as the 8B shape, so the same kernels run).
SMALL_BF16 = ModelShape("small-bf16", 2, 512, 8, 2, 128, 1024, 4096, "bf16")
QWEN3_8B = ModelShape("qwen3-8b-shape", 36, 4096, 32, 8, 128, 12288, 151936, "bf16")
QWEN3_32B = ModelShape("qwen3-32b-shape", 64, 5120, 64, 8, 128, 25600, 151936, "bf16")


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape
    batch: int
    prompt_len: int
    max_new: int
    stride: int
    temperature: float
    propose: str               # "sample" or "argmax"
    lora_rank: int = 0
    page_size: int = 16


TINY_E2E = Workload("tiny-e2e", TINY, 2, 32, 32, 2, 1.0, "sample")
QWEN3_8B_DECODE = Workload("qwen3-8b-isd-b64", QWEN3_8B, 64, 1024, 1024, 4, 1.0, "argmax")
QWEN3_8B_SWEEP = tuple(replace(QWEN3_8B_DECODE, name=f"qwen3-8b-isd-b{b}", batch=b) for b in (1, 8, 32, 64))
RISD_8B = Workload("qwen3-8b-risd-b16", QWEN3_8B, 16, 512, 512, 4, 0.0, "argmax", lora_rank=128)
QWEN3_32B_DECODE = Workload("qwen3-32b-isd-b64", QWEN3_32B, 64, 4096, 2048, 4, 1.0, "sample")


# Attention + acceptance microbench: batch 64, 32 q / 8 kv heads x 128, bf16 KV in 16-token
# pages with a shuffled page table, contexts uniform in [512, 4096], 2N-1 = 7 query rows
# (N = 4), vocab 151936, p-logits ~ N(0, 3^2), q-logits = p + N(0, 0.3^2).
@dataclass(frozen=True)
class AttnSamplerMicro:
    batch: int = 64
    n_q_heads: int = 32
    n_kv_heads: int = 8
    head_dim: int = 128
    page_size: int = 16
    ctx_lo: int = 512
    ctx_hi: int = 4096
    stride: int = 4
    vocab: int = 151936
    p_std: float = 3.0
    q_noise_std: float = 0.3


ATTN_SAMPLER_MICRO = AttnSamplerMicro()


# --------------------------------------------------------------------------------------
def bf16_bits(x):
    """Round float32 to bfloat16 (nearest-even) and return the bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def _rng(seed, index):
    return np.random.Generator(np.random.PCG64([int(seed), int(index)]))


def weight_names(shape):
    """Declared tensor order; the generator index of a tensor is its position here."""
    names = ["embed"]
    for l in range(shape.n_layers):
        names += [f"layers.{l}.{n}" for n in ("attn_norm", "wqkv", "wo", "ffn_norm", "wg", "wu", "wd")]
    names += ["final_norm", "lm_head"]
    return names


def weight_shape(shape, name):
    d, F, V = shape.d_model, shape.d_ffn, shape.vocab
    leaf = name.split(".")[-1]
    return {
        "embed": (V + 1, d), "final_norm": (d,), "lm_head": (V, d),
        "attn_norm": (d,), "ffn_norm": (d,),
        "wqkv": (shape.qkv_rows, d), "wo": (d, shape.n_q_heads * shape.head_dim),
        "wg": (F, d), "wu": (F, d), "wd": (d, F),
    }[leaf]


def _nest(shape, flat):
    w = {"embed": flat["embed"], "final_norm": flat["final_norm"], "lm_head": flat["lm_head"],
         "layers": []}
    for l in range(shape.n_layers):
        w["layers"].append({n: flat[f"layers.{l}.{n}"] for n in
                            ("attn_norm", "wqkv", "wo", "ffn_norm", "wg", "wu", "wd")})
    return w


def weights_numpy(shape, seed=SEED_WEIGHTS, scale=1.0, sticky=None):
    """Weights on the host: float32 arrays for f32 shapes, bf16 bit patterns (uint16) for bf16.

    Each tensor has its own generator PCG64([seed, index]); norm gains are exactly 1.
    Test-only variants (the configurations themselves use scale=1, sticky=None):
      scale   multiplies the embedding and LM head, making distributions peaky;
      sticky  (alpha, beta, gamma, token): adds alpha*c to every embedding row, sets the
              MASK row to gamma*c and adds beta*c to the LM-head row of `token`, c a random
              unit vector (PCG64([seed, 10**6])), so that greedy MASK-row proposals are
              accepted part of the time.
    """
    flat = {}
    names = weight_names(shape)
    for i, name in enumerate(names):
        shp = weight_shape(shape, name)
        if name.endswith("norm"):
            a = np.ones(shp, np.float32)
        else:
            a = (_rng(seed, i).standard_normal(shp, dtype=np.float32) * np.float32(INIT_STD))
            if name in ("embed", "lm_head") and scale != 1.0:
                a = a * np.float32(scale)
        flat[name] = a
    if sticky is not None:
        alpha, beta, gamma, tok = sticky
        c = _rng(seed, 10 ** 6).standard_normal(shape.d_model).astype(np.float32)
        c /= np.linalg.norm(c)
        flat["embed"] = flat["embed"] + np.float32(alpha) * c
        flat["embed"][shape.vocab] = np.float32(gamma) * c
        flat["lm_head"][tok] += np.float32(beta) * c
    if shape.dtype == "bf16":
        flat = {k: bf16_bits(v) for k, v in flat.items()}
    return _nest(shape, flat)


def lora_shapes(shape, rank):
    """{target: (a_shape [r, d_in], b_shape [d_out, r])} per layer."""
    d, F = shape.d_model, shape.d_ffn
    qd, kd = shape.n_q_heads * shape.head_dim, shape.n_kv_heads * shape.head_dim
    io = {"q": (d, qd), "k": (d, kd), "v": (d, kd), "o": (qd, d), "g": (d, F), "u": (d, F), "d": (F, d)}
    return {m: ((rank, io[m][0]), (io[m][1], rank)) for m in LORA_TARGETS}


def lora_numpy(shape, rank, seed=SEED_LORA, scale=1.0):
    """Per layer {target: (A [r, d_in], B [d_out, r])}, generator PCG64([seed, index]).

    scale (test-only) multiplies A and B, so that the adapter's contribution is of the order
    of the base projection's and a wrong delta cannot hide inside a tolerance."""
    out = []
    idx = 0
    shp = lora_shapes(shape, rank)
    for _ in range(shape.n_layers):
        layer = {}
        for m in LORA_TARGETS:
            pair = []
            for s in shp[m]:
                a = _rng(seed, idx).standard_normal(s, dtype=np.float32) * np.float32(INIT_STD * scale)
                idx += 1
                pair.append(bf16_bits(a) if shape.dtype == "bf16" else a)
            layer[m] = tuple(pair)
        out.append(layer)
    return out


def weights_torch(shape, device, seed=SEED_WEIGHTS, lora_rank=0, lora_seed=SEED_LORA):
    """Weights generated with torch on `device` (fast path for the 8B / 32B shapes).

    Tensor i uses torch.Generator(device).manual_seed(seed * 1_000_003 + i); matrices are
    drawn in float32 and rounded to bfloat16 by torch.  Returns (weights, lora) nested like
    weights_numpy / lora_numpy but holding torch tensors.
    """
    import torch
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    flat = {}
    for i, name in enumerate(weight_names(shape)):
        shp = weight_shape(shape, name)
        if name.endswith("norm"):
            flat[name] = torch.ones(shp, dtype=dt, device=device)
        else:
            g = torch.Generator(device=device).manual_seed(seed * 1_000_003 + i)
            t = torch.empty(shp, dtype=torch.float32, device=device)
            t.normal_(0.0, INIT_STD, generator=g)
            flat[name] = t.to(dt)
            del t
    lora = None
    if lora_rank:
        lora = []
        idx = 0
        shp = lora_shapes(shape, lora_rank)
        for _ in range(shape.n_layers):
            layer = {}
            for m in LORA_TARGETS:
                pair = []
                for s in shp[m]:
                    g = torch.Generator(device=device).manual_seed(lora_seed * 1_000_003 + idx)
                    idx += 1
                    t = torch.empty(s, dtype=torch.float32, device=device)
                    t.normal_(0.0, INIT_STD, generator=g)
                    pair.append(t.to(dt))
                layer[m] = tuple(pair)
            lora.append(layer)
    return _nest(shape, flat), lora


def prompts(batch, length, vocab, seed=SEED_DATA):
    """Uniformly random prompt ids [batch, length] int32 (one generator for the batch)."""
    return _rng(seed, 0).integers(0, vocab, size=(batch, length), dtype=np.int64).astype(np.int32)


def ragged_prompts(lengths, vocab, seed=SEED_DATA):
    g = _rng(seed, 1)
    return [g.integers(0, vocab, size=int(n), dtype=np.int64).astype(np.int32) for n in lengths]


def attn_micro(cfg=ATTN_SAMPLER_MICRO, seed=SEED_DATA, batch=None, ctx_lo=None, ctx_hi=None):
    """Inputs of the paged-attention microbench (numpy).

    Returns dict with
      ctx      int32 [B]      context length per sequence (includes the 2N-1 block rows)
      q        uint16 [B, R, Hq, hd]   bf16 bits, N(0,1)
      k_pages  uint16 [n_pages, Hkv, P, hd]   bf16 bits, N(0,1) (logical token-major)
      v_pages  uint16 [n_pages, Hkv, P, hd]
      page_table int32 [B, max_pages]  a random permutation of the pool, -1 padded
    """
    B = cfg.batch if batch is None else batch
    lo = cfg.ctx_lo if ctx_lo is None else ctx_lo
    hi = cfg.ctx_hi if ctx_hi is None else ctx_hi
    R = 2 * cfg.stride - 1
    g = _rng(seed, 2)
    ctx = g.integers(lo, hi + 1, size=B).astype(np.int32)
    npg = [-(-int(c) // cfg.page_size) for c in ctx]
    n_pages = int(sum(npg))
    perm = g.permutation(n_pages).astype(np.int32)
    width = max(npg)
    pt = np.full((B, width), -1, np.int32)
    off = 0
    for b in range(B):
        pt[b, :npg[b]] = perm[off:off + npg[b]]
        off += npg[b]
    q = bf16_bits(g.standard_normal((B, R, cfg.n_q_heads, cfg.head_dim), dtype=np.float32))
    k = bf16_bits(g.standard_normal((n_pages, cfg.n_kv_heads, cfg.page_size, cfg.head_dim), dtype=np.float32))
    v = bf16_bits(g.standard_normal((n_pages, cfg.n_kv_heads, cfg.page_size, cfg.head_dim), dtype=np.float32))
    return dict(ctx=ctx, q=q, k_pages=k, v_pages=v, page_table=pt)


def sampler_micro(cfg=ATTN_SAMPLER_MICRO, seed=SEED_DATA, batch=None, vocab=None):
    """Logits of the acceptance microbench (numpy float32).

    p_logits [B, 2N-1, V] ~ N(0, p_std^2); q_logits [B, N-1, V] = p_logits[:, i-1] + N(0, q_noise^2)
    is the proposal distribution of pending token i (the previous pass's MASK row).
    """
    B = cfg.batch if batch is None else batch
    V = cfg.vocab if vocab is None else vocab
    R = 2 * cfg.stride - 1
    g = _rng(seed, 4)
    p = g.standard_normal((B, R, V), dtype=np.float32) * np.float32(cfg.p_std)
    q = p[:, :cfg.stride - 1, :] + g.standard_normal((B, cfg.stride - 1, V), dtype=np.float32) * np.float32(cfg.q_noise_std)
    return dict(p_logits=p, q_logits=q.astype(np.float32))
