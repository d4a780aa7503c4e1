"""GPU parity: paged causal attention kernel (isd_attn_paged) vs the oracle's dense
causal attention over the gathered pages.

Inputs are the attention microbench recipe (isd_inputs.attn_micro): bf16 Q/K/V ~ N(0,1),
32 query / 8 KV heads x 128, 16-token pages with a shuffled page table.  Tolerance: the
bf16 path bar, max|gpu - oracle| <= 2e-2 * max|oracle| per sequence.
"""
import numpy as np
import pytest
import torch

import isd_inputs as I
from oracle import model as M

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def _run(inp, q_len, n_kv=8):
    from strided_decoding_amd import attn_paged
    q = _bf16_tensor(inp["q"]).to(DEV)
    kp = _bf16_tensor(inp["k_pages"]).to(DEV)
    # library layout: V transposed inside each page -> [n_pages, Hkv, hd, P]
    vp = _bf16_tensor(inp["v_pages"]).to(DEV).transpose(2, 3).contiguous()
    pt = torch.from_numpy(inp["page_table"]).to(DEV)
    ctx = torch.from_numpy(inp["ctx"]).to(DEV)
    ql = torch.from_numpy(np.asarray(q_len, np.int32)).to(DEV)
    print(f"attn case B={q.shape[0]} ctx_max={int(inp['ctx'].max())}", flush=True)
    out, _, _ = attn_paged(q, kp, vp, pt, ctx, ql, n_kv)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _oracle(inp, b, q_len, group=4):
    R = inp["q"].shape[1]
    q = M.f32(inp["q"][b])
    ctx = int(inp["ctx"][b])
    n = int(q_len[b])
    pos = ctx - n + np.arange(n)
    o = M.paged_attention(q[:n], inp["k_pages"], inp["v_pages"], inp["page_table"][b], ctx, pos, group, 16)
    full = np.zeros((R,) + o.shape[1:], np.float32)
    full[:n] = o
    return full


def _check(inp, q_len, out, group=4):
    for b in range(out.shape[0]):
        ref = _oracle(inp, b, q_len, group)
        scale = max(np.abs(ref).max(), 1e-6)
        err = np.abs(out[b] - ref).max()
        assert err <= 2e-2 * scale, (b, err, scale)
        n = int(q_len[b])
        assert np.all(out[b, n:] == 0)


@pytest.mark.parametrize("lo,hi", [(8, 31), (17, 300), (480, 1100)])
def test_attention_small_batches(lo, hi):
    inp = I.attn_micro(batch=6, ctx_lo=lo, ctx_hi=hi, seed=11 + lo)
    q_len = np.full(6, 7, np.int32)
    _check(inp, q_len, _run(inp, q_len))


def test_attention_ragged_query_lengths():
    inp = I.attn_micro(batch=8, ctx_lo=40, ctx_hi=700, seed=5)
    q_len = np.array([7, 4, 1, 0, 7, 2, 6, 3], np.int32)
    _check(inp, q_len, _run(inp, q_len))


def test_attention_full_microbench_shape():
    inp = I.attn_micro()        # batch 64, contexts in [512, 4096]
    q_len = np.full(64, 7, np.int32)
    _check(inp, q_len, _run(inp, q_len))


def test_attention_row_invariance():
    """A row's output does not depend on how many later rows share its block."""
    inp = I.attn_micro(batch=4, ctx_lo=300, ctx_hi=900, seed=9)
    full = _run(inp, np.full(4, 7, np.int32))
    # the same first row alone: context shortened so that it sits at the same position
    inp1 = dict(inp)
    inp1["ctx"] = inp["ctx"] - 6
    one = _run(inp1, np.ones(4, np.int32))
    np.testing.assert_array_equal(one[:, 0], full[:, 0])


@pytest.mark.parametrize("batch,lo,hi", [(8, 300, 2500), (64, 512, 4096)])
def test_attention_32b_head_grouping(batch, lo, hi):
    """The 32B shape's heads: 64 query heads over 8 KV heads (8 per group, so a block's 7 rows
    x 8 heads take the four-wave workgroup), small and full batches, ragged query lengths."""
    import dataclasses
    cfg = dataclasses.replace(I.ATTN_SAMPLER_MICRO, n_q_heads=64, n_kv_heads=8)
    inp = I.attn_micro(cfg, batch=batch, ctx_lo=lo, ctx_hi=hi, seed=31 + batch)
    q_len = np.random.default_rng(batch).integers(0, 8, size=batch).astype(np.int32)
    q_len[0] = 7
    _check(inp, q_len, _run(inp, q_len, n_kv=8), group=8)


def test_attention_one_split_past_2048_keys():
    """64 slots with contexts a little past 2048 keys take a single 2560-key split per (slot, KV
    head): every row is final in the attention kernel, and each workgroup reloads its window of
    page ids (128 pages, 2048 keys) once inside its key range."""
    inp = I.attn_micro(batch=64, ctx_lo=2049, ctx_hi=2560, seed=41)
    assert int(inp["ctx"].max()) > 2048 + 16
    q_len = np.random.default_rng(41).integers(1, 8, size=64).astype(np.int32)
    _check(inp, q_len, _run(inp, q_len))


def test_attention_merge_of_many_splits():
    """Two slots with contexts of 3000..4096 keys take 128-key splits: rows span 24..32 splits,
    so the merge runs its multi-group path (16 splits a group, the maxima of every group
    first); ragged query lengths put rows of one block on both sides of a split boundary."""
    inp = I.attn_micro(batch=2, ctx_lo=3000, ctx_hi=4096, seed=43)
    q_len = np.array([7, 5], np.int32)
    _check(inp, q_len, _run(inp, q_len))
