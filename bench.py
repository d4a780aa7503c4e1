#!/usr/bin/env python
"""ISD decode benchmark on one MI355X.

Workload: Qwen3-8B-shaped random-init bf16 model (36 layers, d 4096, 32/8 heads x 128,
SwiGLU 12288, vocab 151936), batch 64, stride N = 4, argmax proposals, temperature 1,
1024-token uniformly random prompts (synthetic stand-ins for the pages' prompts and
trained weights, which are not available).  A step is one isd_step: one ISD pass over
all 64 slots (block assembly, page reservation, 36 layers, LM head, acceptance /
resample / proposals, KV truncation).  `value` is committed tokens per second over the
timed steps, with everything resident in HBM before the timed region starts.

Prints one JSON line; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "committed tokens/s on 1 MI355X (8B-shape, batch 64, N=4); ISD-step HBM GB/s"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--batch", type=int, default=64)
    p.add_argument("--prompt-len", type=int, default=1024)
    p.add_argument("--gen", type=int, default=1024)
    p.add_argument("--profile-steps", type=int, default=6)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--out", default=None, help="also write the JSON line to this file")
    return p.parse_args()


def kernel_model(shape, M, N, ctx_rows, attn_keys):
    """Algorithmic bytes and flops of one launch of each kernel of a decode pass.

    M rows (batch x (2N-1)); ctx_rows: sum over slots of keys in the pages this pass
    (L + q_len); attn_keys: sum over live query rows of visible keys.  Weights are read
    once per pass; activations are counted once in and once out.
    """
    d, F, V = shape.d_model, shape.d_ffn, shape.vocab
    qd = shape.n_q_heads * shape.head_dim
    kd = shape.n_kv_heads * shape.head_dim
    qkvw = qd + 2 * kd
    kv_tok = 2 * kd * 2                       # K and V bytes per token per layer
    g = {
        "gemm_qkv": (qkvw * d * 2 + M * d * 2 + M * qkvw * 2, 2.0 * M * qkvw * d),
        "gemm_o": (d * qd * 2 + M * qd * 2 + M * d * 8, 2.0 * M * d * qd),
        "gemm_gate_up": (2 * F * d * 2 + M * d * 2 + M * F * 2, 2.0 * M * 2 * F * d),
        "gemm_down": (d * F * 2 + M * F * 2 + M * d * 8, 2.0 * M * d * F),
        "lm_head": (V * d * 2 + M * d * 2 + M * V * 4, 2.0 * M * V * d),
        "attention": (ctx_rows * kv_tok + 2 * M * qd * 2, 4.0 * attn_keys * shape.n_q_heads * shape.head_dim),
        "row_stats": (M * V * 4, 0.0),
    }
    return g


def step_bytes(shape, M, ctx_rows):
    """Algorithmic HBM bytes of one pass: weights once, KV of every slot, logits out and in."""
    L = shape.n_layers
    d, F, V = shape.d_model, shape.d_ffn, shape.vocab
    qd = shape.n_q_heads * shape.head_dim
    kd = shape.n_kv_heads * shape.head_dim
    w = L * ((qd + 2 * kd) * d + d * qd + 3 * F * d) * 2 + V * d * 2
    kv = ctx_rows * 2 * kd * 2 * L
    return w + kv + 2 * M * V * 4


def cpu_baseline(shape, weights, eng, B, N, T):
    """The oracle timed on this host: one ISD pass of one slot of the same workload.

    The slot's block rows and context length are taken from the GPU run; its KV cache is
    synthetic (random values of the right shape), since an oracle prefill of 1024 tokens
    at this shape would take many minutes.
    """
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import isd as OI
    from oracle import model as M

    log("cpu baseline: copying weights to host")
    t0 = time.perf_counter()

    def host(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    w = {k: host(weights[k]) for k in ("embed", "final_norm", "lm_head")}
    w["layers"] = [{k: host(v) for k, v in layer.items()} for layer in weights["layers"]]
    log(f"cpu baseline: weights on host in {time.perf_counter() - t0:.1f}s")
    spec = M.Spec(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.d_ffn,
                  shape.vocab, shape.rope_base, shape.rms_eps)
    model = M.Model(spec, w)
    st = eng.slots_host()[0]
    L = st["L"]
    state = {1: "A", 2: "B"}.get(st["state"], "B")
    pending = [st[f"pending{j}"] for j in range(N - 1)] if state == "A" else []
    ids = [st["c"]] + pending + [shape.vocab] * (N - 1)
    rng = np.random.default_rng(0)
    cache = [(rng.standard_normal((L, shape.n_kv_heads, shape.head_dim), dtype=np.float32),
              rng.standard_normal((L, shape.n_kv_heads, shape.head_dim), dtype=np.float32))
             for _ in range(shape.n_layers)]
    threads = sum(x.get("num_threads", 0) for x in threadpool_info() if x.get("user_api") == "blas") or 1
    log(f"cpu baseline: oracle pass of slot 0 ({state}, {len(ids)} rows, context {L}) on {threads} threads")
    t0 = time.perf_counter()
    logits, _ = model.forward(ids, L + np.arange(len(ids)), cache)
    out = OI.decide(state, L, st["t"], 0, pending, [None] * len(pending), logits, N, T, "argmax", 1)
    dt = time.perf_counter() - t0
    n_tok = len(out.tokens)
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"one ISD pass of one slot (1 of {B}): {len(ids)} rows over a {L}-token synthetic KV "
                      f"cache, 36 layers + LM head + decisions, fp32 numpy; committed {n_tok} token(s) "
                      f"in {dt:.1f}s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1"}))
        sys.exit(2)
    import torch

    import isd_inputs as I
    from strided_decoding_amd import Engine

    wl = I.QWEN3_8B_DECODE
    shape = wl.model
    B, N, T = args.batch, wl.stride, wl.temperature
    R = 2 * N - 1
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    weights, _ = I.weights_torch(shape, dev)
    torch.cuda.synchronize()
    log(f"weights generated in {time.perf_counter() - t0:.1f}s")
    max_seq = args.prompt_len + args.gen + 2 * N + 8
    chunk = 16
    eng = Engine(shape, weights, stride=N, temperature=T, propose=wl.propose, seed=I.SEED_PHILOX, max_batch=B,
                 max_seq_len=max_seq, max_prefill_tokens=chunk * args.prompt_len, device=dev)
    log(f"engine: kv pool {eng.sizes[0] / 2**30:.1f} GiB, workspace {eng.sizes[1] / 2**30:.2f} GiB")
    prompts = I.prompts(B, args.prompt_len, shape.vocab)
    t0 = time.perf_counter()
    for s0 in range(0, B, chunk):
        sl = list(range(s0, min(B, s0 + chunk)))
        eng.prefill(sl, [prompts[b] for b in sl], [args.gen] * len(sl))
        torch.cuda.synchronize()
        log(f"prefilled slots {sl[0]}..{sl[-1]}")
    log(f"prefill {B}x{args.prompt_len} in {time.perf_counter() - t0:.1f}s")

    for _ in range(args.warmup):
        eng.step()
    torch.cuda.synchronize()
    st0 = eng.slots_host()
    tot = torch.zeros((), dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        _, nc, _ = eng.step()
        tot += nc.sum()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    committed = int(tot.item())
    st1 = eng.slots_host()
    passes = sum(s1["passes"] - s0["passes"] for s0, s1 in zip(st0, st1))
    verified = sum(s1["verified"] - s0["verified"] for s0, s1 in zip(st0, st1))
    accepted = sum(s1["accepted"] - s0["accepted"] for s0, s1 in zip(st0, st1))
    live = sum(1 for s in st1 if s["state"] in (1, 2))
    ms = 1e3 * elapsed / args.steps
    log(f"timed {args.steps} steps: {ms:.3f} ms/step, {committed} tokens, live slots {live}")

    # kernel timings: a separate phase with event pairs around every launch
    ctx_rows = attn_keys = 0
    eng.profile(True)
    for _ in range(args.profile_steps):
        before = eng.slots_host()
        for s in before:
            q = R if s["state"] == 1 else (N if s["state"] == 2 else 0)
            if q:
                ctx_rows += s["L"] + q
                attn_keys += sum(s["L"] + i + 1 for i in range(q))
        eng.step()
    rep = eng.profile_report()
    eng.profile(False)
    P = max(1, args.profile_steps)
    model = kernel_model(shape, B * R, N, ctx_rows / P, attn_keys / P)
    kernels = {}
    for name, (n, tot_ms) in rep.items():
        per_pass = n / P
        e = {"launches_per_step": per_pass, "avg_us": 1e3 * tot_ms / n, "ms_per_step": tot_ms / P}
        if name in model:
            b, f = model[name]
            e["GBps"] = b / (e["avg_us"] * 1e-6) / 1e9
            e["TFLOPs"] = f / (e["avg_us"] * 1e-6) / 1e12
        kernels[name] = e
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    d = kernels[dom]
    b, f = model.get(dom, (0.0, 0.0))
    intensity = f / b if b else 0.0
    if dom in model and intensity > MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": d["TFLOPs"], "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": d["TFLOPs"] / MFMA_BF16_PEAK_TFS, "traffic": None}
    else:
        gbs = d.get("GBps", 0.0)
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "traffic": None}
    roof["kernel"] = dom
    roof["per_launch"] = {"bytes": b, "flops": f, "avg_us": d["avg_us"]}
    sb = step_bytes(shape, B * R, ctx_rows / P)
    out = {
        "metric": METRIC, "value": committed / elapsed, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random-init weights N(0,0.02), uniformly random prompt ids)",
        "config": {"workload": wl.name, "batch": B, "stride": N, "prompt_len": args.prompt_len,
                   "max_new": args.gen, "propose": wl.propose, "temperature": T, "parallelism": "single GPU"},
        "isd_steps_per_s": args.steps / elapsed,
        "tokens_per_forward": committed / max(1, passes),
        "acceptance": accepted / max(1, verified),
        "step_hbm_GBps": sb / (ms * 1e-3) / 1e9,
        "step_hbm_frac": sb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "step_algorithmic_bytes": sb,
        "projected_tokens_per_s_at_p0.9": args.steps / elapsed * B * 2.919,
        "roofline": roof,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shape, weights, eng, B, N, T)
    line = json.dumps(out)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
