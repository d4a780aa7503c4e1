"""GPU properties that hold at any size, checked GPU against GPU through the C ABI:

* R-ISD lossless claim (wiki note, Key claims and Method; GeekNews, Lossless R-ISD):
  greedy ISD with the MASK-gated LoRA commits exactly the tokens of greedy AR decoding
  (N = 1) of the same base weights, bit for bit;
* the KV cache after decode passes equals a fresh prefill of the committed tokens
  (first-rejection rollback and logit shift).
"""
import numpy as np
import pytest
import torch

import isd_inputs as I

pytestmark = pytest.mark.gpu


def _engine(shape, w, N, T, B, max_seq, lora=None, propose="argmax"):
    from strided_decoding_amd import Engine
    return Engine(shape, w, stride=N, temperature=T, propose=propose, seed=1, max_batch=B, max_seq_len=max_seq,
                  lora=lora)


def _generate(eng, prompts, max_new, max_steps=10_000):
    B = len(prompts)
    first = eng.prefill(list(range(B)), prompts, max_new).cpu().numpy()
    out = [[int(first[b])] for b in range(B)]
    acc = ver = steps = 0
    while steps < max_steps:
        tok, nc, na = eng.step()
        steps += 1
        tok, nc, na = tok.cpu().numpy(), nc.cpu().numpy(), na.cpu().numpy()
        for b in range(B):
            out[b] += [int(x) for x in tok[b, :nc[b]]]
        acc += int(na.sum())
        if all(len(o) >= m for o, m in zip(out, max_new)):
            break
    st = eng.slots_host()
    ver = sum(s["verified"] for s in st[:B])
    return out, steps, acc, ver


@pytest.mark.parametrize("sticky", [None, (0.0, 20.0, 4.0, 7)])
def test_risd_greedy_equals_ar_greedy_bf16(sticky):
    shape = I.SMALL_BF16
    w = I.weights_numpy(shape, seed=0, scale=20.0, sticky=sticky)
    lora = I.lora_numpy(shape, 128)
    prompts = I.ragged_prompts([37, 64, 5, 100], shape.vocab, seed=8)
    max_new = [40, 33, 48, 25]
    print(f"risd vs ar sticky={sticky}", flush=True)
    ar, ar_steps, _, _ = _generate(_engine(shape, w, 1, 0.0, 4, 200), prompts, max_new)
    isd, isd_steps, acc, ver = _generate(_engine(shape, w, 4, 0.0, 4, 200, lora=lora), prompts, max_new)
    print(f"AR passes {ar_steps}, R-ISD passes {isd_steps}, accepted {acc}/{ver}", flush=True)
    for b in range(4):
        assert isd[b][:max_new[b]] == ar[b][:max_new[b]], b
    if sticky is not None:
        assert acc > 0 and isd_steps < ar_steps


def test_isd_greedy_equals_ar_greedy_fp32():
    shape = I.ModelShape("tiny-gqa", 2, 128, 4, 2, 32, 256, 512, "f32")
    w = I.weights_numpy(shape, seed=4, scale=8.0, sticky=(0.0, 10.0, 2.0, 7))
    prompts = I.ragged_prompts([9, 30], shape.vocab, seed=2)
    ar, _, _, _ = _generate(_engine(shape, w, 1, 0.0, 2, 128), prompts, [50, 50])
    isd, _, acc, _ = _generate(_engine(shape, w, 3, 0.0, 2, 128), prompts, [50, 50])
    assert isd == ar


def _gather(eng, b, L):
    kp, vp = eng.kv_pools()
    pt = eng.page_table()[b].cpu().numpy()
    P = eng.cfg.page_size
    n = -(-L // P)
    pages = torch.from_numpy(pt[:n]).long().to(kp.device)
    k = kp[:, pages].permute(0, 1, 3, 2, 4).reshape(kp.shape[0], n * P, kp.shape[2], kp.shape[4])[:, :L]
    v = vp[:, pages].permute(0, 1, 4, 2, 3).reshape(vp.shape[0], n * P, vp.shape[2], vp.shape[3])[:, :L]
    return k.float().cpu().numpy(), v.float().cpu().numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kv_cache_equals_fresh_prefill(dtype):
    if dtype == "f32":
        shape = I.ModelShape("tiny-gqa", 2, 128, 4, 2, 32, 256, 512, "f32")
        w = I.weights_numpy(shape, seed=4, scale=8.0)
        tol = 2e-5
    else:
        shape = I.SMALL_BF16
        w = I.weights_numpy(shape, seed=0, scale=20.0)
        tol = 2e-2
    prompts = I.ragged_prompts([21, 50], shape.vocab, seed=12)
    eng = _engine(shape, w, 3, 1.0, 2, 160, propose="sample")
    out, _, _, _ = _generate(eng, prompts, [60, 60], max_steps=12)
    st = eng.slots_host()
    for b in range(2):
        L = st[b]["L"]
        committed = list(prompts[b]) + out[b]
        assert st[b]["c"] == committed[L]
        fresh = _engine(shape, w, 3, 1.0, 1, 160, propose="sample")
        fresh.prefill([0], [np.array(committed[:L], np.int32)], [2])
        k1, v1 = _gather(eng, b, L)
        k2, v2 = _gather(fresh, 0, L)
        for a, r in ((k1, k2), (v1, v2)):
            err = np.abs(a - r).max() / max(np.abs(r).max(), 1e-6)
            assert err <= tol, (b, err)
