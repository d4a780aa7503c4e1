#!/usr/bin/env python
"""ISD decode benchmark on one MI355X.

Workload: Qwen3-8B-shaped random-init bf16 model (36 layers, d 4096, 32/8 heads x 128,
SwiGLU 12288, vocab 151936), batch 64, stride N = 4, argmax proposals, temperature 1,
1024-token uniformly random prompts (synthetic stand-ins for the pages' prompts and
trained weights, which are not available).  A step is one ISD pass over all 64 slots
(block assembly, page reservation, 36 layers, LM head, acceptance / resample / proposals,
KV truncation), launched as isd_step_n runs of passes (one HIP graph launch each).  `value`
is committed tokens per second over the timed steps, with everything resident in HBM
before the timed region starts.  The default 10 + 1000 passes walk the slots' contexts from
1034 to 2034 tokens, so the timed window averages the 1024 + 1024 workload's mean context.

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
    p.add_argument("--steps", type=int, default=None,
                   help="timed passes (default: 1000 for the 8B isd workload, the whole generation window; "
                        "200 for the 32B shape, R-ISD and the microbench; 100 for the meter)")
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", choices=("isd", "risd", "meter", "micro"), default="isd",
                   help="isd: decode throughput (default); risd: R-ISD == AR check and overhead factor; "
                        "meter: introspective acceptance rate of the model's own proposals (teacher-forced); "
                        "micro: the attention + acceptance kernel microbench (64 slots, contexts U[512, 4096], "
                        "7 query rows, vocab 151936) with the oracle timed beside it")
    p.add_argument("--passes-per-launch", type=int, default=8,
                   help="passes per isd_step_n call (one graph launch each; 1 = isd_step)")
    p.add_argument("--model", choices=("8b", "32b"), default="8b", help="model shape of the isd workload")
    p.add_argument("--batch", type=int, default=None, help="slots (default: the workload's)")
    p.add_argument("--stride", type=int, default=None, help="ISD stride N (default: the workload's, 4)")
    p.add_argument("--active", type=int, default=None,
                   help="isd workload: prefill only slots 0..K-1 of the batch and step them as the active "
                        "prefix (isd_step_active)")
    p.add_argument("--prompt-len", type=int, default=None)
    p.add_argument("--gen", type=int, default=None)
    p.add_argument("--profile-steps", type=int, default=6)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ar-check", action="store_true",
                   help="R-ISD workload: skip the comparison with plain autoregressive greedy decoding")
    p.add_argument("--no-graphs", action="store_true", help="launch every pass eagerly (no HIP graph replay)")
    p.add_argument("--out", default=None, help="also write the JSON line to this file")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB (counter calibration) and exit")
    p.add_argument("--trace-summary", default=None, metavar="DIR",
                   help="only summarise a rocprofv3 --kernel-trace csv output directory (no GPU) and exit")
    p.add_argument("--pmc-summary", default=None, metavar="DIR",
                   help="only summarise rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (no GPU) and exit")
    p.add_argument("--counter-summary", default=None, metavar="DIR",
                   help="only print the mean of every counter per decode op of a rocprofv3 --pmc run (no GPU) "
                        "and exit")
    return p.parse_args()


def kernel_model(shape, M, N, ctx_rows, attn_keys):
    """Algorithmic bytes and flops of one launch of each kernel of a decode pass.

    M live rows (2N-1 per A-state slot, N per B-state slot); ctx_rows: sum over slots of keys in the pages this pass
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


def tpf_projection(p, N):
    """Tokens per forward of the ISD state machine at a per-token acceptance p (a projection for
    trained weights; random-init weights accept almost nothing).  N = 1 is plain AR."""
    if N == 1:
        return 1.0
    return (2 + sum(p ** k for k in range(1, N - 1))) / (2 - p ** (N - 1))


def step_bytes(shape, M, ctx_rows):
    """Algorithmic HBM bytes of one pass: weights once, KV of every slot, logits out and in."""
    L = shape.n_layers
    d, F, V = shape.d_model, shape.d_ffn, shape.vocab
    qd = shape.n_q_heads * shape.head_dim
    kd = shape.n_kv_heads * shape.head_dim
    w = L * ((qd + 2 * kd) * d + d * qd + 3 * F * d) * 2 + V * d * 2
    kv = ctx_rows * 2 * kd * 2 * L
    return w + kv + 2 * M * V * 4


# Kernel (demangled-name pattern) behind each profiled operation whose traffic can be read from
# rocprofv3 counters: the decode launches are the most frequent grid of that kernel in a run.
# o and down run the same kernel with the same grid, in turn (o of a layer, then its down):
# (period, index) selects every period-th of those dispatches in dispatch order.
OP_KERNELS = {
    "gemm_gate_up": (r"gemm_bf16_big_kernel<3, false, false, 3>", ("gemm_tile.h", "k_gemm_big_swiglu.hip")),
    "gemm_qkv": (r"gemm_bf16_big_kernel<1, true, false, 3>", ("gemm_tile.h", "k_gemm_big_store_f32.hip")),
    "gemm_o": (r"gemm_bf16_big_kernel<2, true, false, 4>", ("gemm_tile.h", "k_gemm_big_resid.hip"), (2, 0)),
    "gemm_down": (r"gemm_bf16_big_kernel<2, true, false, 4>", ("gemm_tile.h", "k_gemm_big_resid.hip"), (2, 1)),
    "splitk_resid_norm": (r"splitk_resid_norm_kernel", ("k_gemm.hip",)),
    "rope_append": (r"rope_append_kernel<", ("k_block.hip",)),
    # the LM head's kernel instance is also the prefill's (fp32) QKV projection: at this
    # workload the decode LM head is the grid of 2 row tiles x 600 (8-aligned) column tiles of
    # four-wave workgroups
    "lm_head": (r"gemm_bf16_big_kernel<1, false, false, 4>", ("gemm_tile.h", "k_gemm_big_store_f32.hip"), None,
                2 * 600 * 256),
    "attention": (r"attn_bf16_kernel<", ("k_attn.hip",)),
    "attn_combine": (r"attn_combine_kernel", ("k_attn.hip",)),
    "row_stats": (r"row_stats_kernel", ("k_sampler.hip",)),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_qwen3_8b_b64.md")
COPY_KERNEL = r"neg_kernel"


def kernel_source_sha(files):
    import hashlib
    h = hashlib.sha256()
    for f in files + ("isd_common.h",):
        with open(os.path.join(ROOT, "strided_decoding_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _csv_rows(root, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(root, "**", "*" + suffix), recursive=True)):
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {root}")
    return rows


def _col(row, *names):
    low = {k.lower(): v for k, v in row.items()}
    for n in names:
        if n.lower() in low:
            return low[n.lower()]
    raise KeyError(names)


def _grid(row):
    try:
        return int(_col(row, "Grid_Size"))
    except KeyError:
        return int(_col(row, "Grid_Size_X")) * int(_col(row, "Grid_Size_Y")) * int(_col(row, "Grid_Size_Z"))


def _short(name, n=90):
    name = name.replace("isd::(anonymous namespace)::", "").replace("(isd::EpiMode)", "")
    return name if len(name) <= n else name[:n - 3] + "..."


def trace_summary(root):
    """Per (kernel, grid) dispatch count and durations from a rocprofv3 --kernel-trace csv run."""
    rows = _csv_rows(root, "kernel_trace.csv")
    acc = {}
    for r in rows:
        k = (_col(r, "Kernel_Name"), _grid(r))
        ns = int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))
        e = acc.setdefault(k, [0, 0, float("inf"), 0])
        e[0] += 1
        e[1] += ns
        e[2] = min(e[2], ns)
        e[3] = max(e[3], ns)
    tot = sum(e[1] for e in acc.values())
    print("| kernel | grid (threads) | dispatches | avg us | min us | max us | % time |")
    print("|---|---|---|---|---|---|---|")
    for (name, grid), e in sorted(acc.items(), key=lambda kv: -kv[1][1])[:30]:
        print(f"| `{_short(name)}` | {grid} | {e[0]} | {e[1] / e[0] / 1e3:.1f} | {e[2] / 1e3:.1f} | "
              f"{e[3] / 1e3:.1f} | {100 * e[1] / tot:.1f} |")
    # decode ops: the most frequent grid of each op's kernel (o and down split by dispatch order)
    import re
    print("\n| op | kernel | grid (threads) | dispatches | avg us |")
    print("|---|---|---|---|---|")
    for op, (pat, _files, *sel) in OP_KERNELS.items():
        nth = sel[0] if sel else None
        per = {}
        for r in rows:
            if re.search(pat, _col(r, "Kernel_Name")):
                ns = int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))
                per.setdefault(_grid(r), []).append((int(_col(r, "Start_Timestamp")), ns))
        grid = sel[1] if len(sel) > 1 else (max(per, key=lambda g: len(per[g])) if per else None)
        if grid not in per:
            continue
        v = [ns for _, ns in sorted(per[grid])]
        if nth:
            v = v[nth[1]::nth[0]]
        print(f"| {op} | `{_short(pat)}` | {grid} | {len(v)} | {sum(v) / len(v) / 1e3:.1f} |")


def _counter_by_grid(root, counter, pattern, nth=None, grid=None):
    """(grid, dispatches, mean value) of a counter over the most frequent grid (or the given
    one) of the kernels matching pattern; nth = (period, index) keeps every period-th dispatch
    in dispatch order."""
    import re
    per = {}
    for r in _csv_rows(root, "counter_collection.csv"):
        if _col(r, "Counter_Name") != counter or not re.search(pattern, _col(r, "Kernel_Name")):
            continue
        try:
            order = int(_col(r, "Dispatch_Id"))
        except KeyError:
            order = len(per.get(_grid(r), []))
        per.setdefault(_grid(r), []).append((order, float(_col(r, "Counter_Value"))))
    if not per:
        raise SystemExit(f"no {counter} records for /{pattern}/ under {root}")
    if grid is None:
        grid = max(per, key=lambda g: len(per[g]))
    elif grid not in per:
        raise SystemExit(f"no {counter} records of grid {grid} for /{pattern}/ under {root}")
    v = [x for _, x in sorted(per[grid])]
    if nth:
        v = v[nth[1]::nth[0]]
    return grid, len(v), sum(v) / len(v)


def pmc_summary(root):
    """HBM traffic per decode launch of each kernel in OP_KERNELS, calibrated on a plain copy.

    root holds four rocprofv3 --pmc runs: fetch_bench and write_bench (FETCH_SIZE resp.
    WRITE_SIZE over the benchmark), fetch_copy and write_copy (the same counters over
    --copy-probe-mib, whose kernel reads and writes a known number of bytes), and
    copy_probe.log, the probe's own output.
    """
    import re
    copy_bytes = None
    for line in open(os.path.join(root, "copy_probe.log")):
        m = re.match(r"(\d+) bytes read and", line)
        if m:
            copy_bytes = int(m.group(1))
    _, _, cf = _counter_by_grid(os.path.join(root, "fetch_copy"), "FETCH_SIZE", COPY_KERNEL)
    _, _, cw = _counter_by_grid(os.path.join(root, "write_copy"), "WRITE_SIZE", COPY_KERNEL)
    kf, kw = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    print(f"copy calibration: {copy_bytes} bytes each way; FETCH_SIZE {cf:.0f} KiB -> factor {kf:.4f}; "
          f"WRITE_SIZE {cw:.0f} KiB -> factor {kw:.4f}\n")
    print("| op | kernel | grid | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | traffic bytes (calibrated) |")
    print("|---|---|---|---|---|---|---|")
    rec = {}
    for op, (pat, files, *sel) in OP_KERNELS.items():
        nth = sel[0] if sel else None
        grid = sel[1] if len(sel) > 1 else None
        try:
            g, n, f = _counter_by_grid(os.path.join(root, "fetch_bench"), "FETCH_SIZE", pat, nth, grid)
            g2, _, w = _counter_by_grid(os.path.join(root, "write_bench"), "WRITE_SIZE", pat, nth, grid)
        except SystemExit:
            continue
        t = f * 1024 * kf + w * 1024 * kw
        rec[op] = {"grid": g, "traffic_bytes": t, "fetch_kib": f, "write_kib": w,
                   "source_sha": kernel_source_sha(files)}
        print(f"| {op} | `{pat}` | {g}/{g2} | {n} | {f:.0f} | {w:.0f} | {t:.4g} |")
    print("\n```json\n" + json.dumps({"calibration": {"fetch": kf, "write": kw}, "ops": rec}, indent=1) + "\n```")


def counter_summary(root):
    """Mean value per dispatch of every counter of a rocprofv3 --pmc run, for each decode op of
    OP_KERNELS (its decode grid, o and down told apart by dispatch order)."""
    names = sorted({_col(r, "Counter_Name") for r in _csv_rows(root, "counter_collection.csv")})
    print("| op | grid | dispatches | " + " | ".join(names) + " |")
    print("|---|---|---|" + "---|" * len(names))
    for op, (pat, _files, *sel) in OP_KERNELS.items():
        nth = sel[0] if sel else None
        grid = sel[1] if len(sel) > 1 else None
        vals = []
        try:
            for c in names:
                g, n, v = _counter_by_grid(root, c, pat, nth, grid)
                vals.append(v)
        except SystemExit:
            continue
        print(f"| {op} | {g} | {n} | " + " | ".join(f"{v:.4g}" for v in vals) + " |")


def load_traffic(op):
    """Calibrated HBM bytes per launch of op from the committed counter summary, or None when
    there is none or the kernel's source has changed since the counters were taken."""
    import re
    if not os.path.exists(TRAFFIC_FILE) or op not in OP_KERNELS:
        return None
    m = re.search(r"```json\n(.*?)\n```", open(TRAFFIC_FILE).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))["ops"].get(op)
    if not rec or rec["source_sha"] != kernel_source_sha(OP_KERNELS[op][1]):
        return None
    return rec["traffic_bytes"]


def copy_probe(mib):
    """A plain device copy of a known size: the counters' calibration kernel."""
    import torch
    n = mib * 2**20 // 4
    x = torch.randn(n, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(5):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(f"{n * 4} bytes read and {n * 4} bytes written per torch.neg launch", flush=True)


def cpu_baseline(shape, weights, eng, B, N, T, min_seconds=10.0, max_slots=8):
    """The oracle timed on this host: one ISD pass of each of the first slots of the same
    workload, slot after slot until about min_seconds of work (at most max_slots slots).

    Each slot's block rows and context length are taken from the GPU run; its KV cache is
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
    slots = eng.slots_host()
    threads = sum(x.get("num_threads", 0) for x in threadpool_info() if x.get("user_api") == "blas") or 1
    rng = np.random.default_rng(0)
    n_tok, rows, ctx, dt, b = 0, 0, 0, 0.0, 0
    while b < min(B, max_slots) and (b == 0 or dt < min_seconds):
        st = slots[b]
        L = st["L"]
        state = {1: "A", 2: "B"}.get(st["state"], "B")
        pending = [st[f"pending{j}"] for j in range(N - 1)] if state == "A" else []
        ids = [st["c"]] + pending + [shape.vocab] * (N - 1)
        cache = [(rng.standard_normal((L, shape.n_kv_heads, shape.head_dim), dtype=np.float32),
                  rng.standard_normal((L, shape.n_kv_heads, shape.head_dim), dtype=np.float32))
                 for _ in range(shape.n_layers)]
        log(f"cpu baseline: oracle pass of slot {b} ({state}, {len(ids)} rows, context {L}) on {threads} threads")
        t0 = time.perf_counter()
        logits, _ = model.forward(ids, L + np.arange(len(ids)), cache)
        out = OI.decide(state, L, st["t"], b, pending, [None] * len(pending), logits, N, T, "argmax", 1)
        dt += time.perf_counter() - t0
        n_tok += len(out.tokens)
        rows += len(ids)
        ctx += L
        b += 1
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle", "host": host_info(),
            "sample": f"one ISD pass of each of slots 0..{b - 1} ({b} of {B}): {rows} rows over synthetic KV caches "
                      f"of {ctx // b} tokens on average, {shape.n_layers} layers + LM head + decisions each, fp32 "
                      f"numpy; committed {n_tok} token(s) in {dt:.1f}s"}


def prefill_engine(I, Engine, torch, shape, weights, dev, B, N, T, propose, prompt_len, gen, lora=None, chunk=16,
                   live=None, max_seq=None, engine=None):
    """An engine with B slots, the first `live` (default all) prefilled with uniformly random
    prompts (16 slots per call); `engine`: prefill that one's slots again instead."""
    max_seq = max_seq or prompt_len + gen + 2 * N + 8
    eng = engine
    if eng is None:
        eng = Engine(shape, weights, stride=N, temperature=T, propose=propose, seed=I.SEED_PHILOX, max_batch=B,
                     max_seq_len=max_seq, max_prefill_tokens=chunk * prompt_len, lora=lora, device=dev)
        log(f"engine N={N} lora={'yes' if lora else 'no'}: kv pool {eng.sizes[0] / 2**30:.1f} GiB, "
            f"workspace {eng.sizes[1] / 2**30:.2f} GiB")
    prompts = I.prompts(B, prompt_len, shape.vocab)
    t0 = time.perf_counter()
    first = []
    for s0 in range(0, live or B, chunk):
        sl = list(range(s0, min(live or B, s0 + chunk)))
        first += eng.prefill(sl, [prompts[b] for b in sl], [gen] * len(sl)).cpu().tolist()
        torch.cuda.synchronize()
    log(f"prefill {B}x{prompt_len} in {time.perf_counter() - t0:.1f}s")
    return eng, first


def run_passes(eng, n, n_active, per_launch):
    """n passes: isd_step_n runs of per_launch passes (then single passes for the rest), or
    isd_step / isd_step_active one at a time; returns the host seconds spent in the calls."""
    h = 0.0
    done = 0
    while done < n:
        t = time.perf_counter()
        if n_active is None and per_launch > 1 and n - done >= per_launch:
            eng.step_n(per_launch)
            done += per_launch
        else:
            eng.step(n_active)
            done += 1
        h += time.perf_counter() - t
    return h


def timed_steps(eng, torch, steps, warmup, graphs, n_active=None, per_launch=1):
    """Warm-up steps, then `steps` steps between two synchronizations; slot records around them.
    Also returns the host time spent enqueuing the timed passes."""
    eng.set_graphs(graphs)
    run_passes(eng, warmup, n_active, per_launch)
    torch.cuda.synchronize()
    st0 = eng.slots_host()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    host = run_passes(eng, steps, n_active, per_launch)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timed_steps.host_seconds = host
    return elapsed, st0, eng.slots_host()


def delta(st0, st1, field):
    return sum(s1[field] - s0[field] for s0, s1 in zip(st0, st1))


def kernel_profile(eng, shape, B, N, steps, n_active=None):
    """Per-op launch counts and durations (HIP events on the launch stream) over `steps` passes,
    with the algorithmic bytes / flops of the same passes."""
    R = 2 * N - 1
    ctx_rows = attn_keys = live_rows = 0
    eng.profile(True)
    for _ in range(steps):
        for s in eng.slots_host():
            q = R if s["state"] == 1 else (N if s["state"] == 2 else 0)
            if q:
                ctx_rows += s["L"] + q
                attn_keys += sum(s["L"] + i + 1 for i in range(q))
                live_rows += q
        eng.step(n_active)
    rep = eng.profile_report()
    eng.profile(False)
    P = max(1, steps)
    # a pass computes its live rows only (packed: 2N-1 per A-state slot, N per B-state slot)
    kernel_profile.live_rows = live_rows / P
    model = kernel_model(shape, live_rows / P, N, ctx_rows / P, attn_keys / P)
    kernels = {}
    for name, (n, tot_ms) in rep.items():
        e = {"launches_per_step": n / P, "avg_us": 1e3 * tot_ms / n, "ms_per_step": tot_ms / P}
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
                "frac": d["TFLOPs"] / MFMA_BF16_PEAK_TFS}
    else:
        gbs = d.get("GBps", 0.0)
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}
    roof["traffic"] = load_traffic(dom)
    roof["kernel"] = dom
    roof["per_launch"] = {"bytes": b, "flops": f, "avg_us": d["avg_us"]}
    return kernels, roof, ctx_rows / P


def window_ctx_rows(st0, st1, N):
    """Mean keys in the pages per pass (sum over live slots of L + q_len) over a timed window,
    from the slot records at its two ends (L grows steadily; q_len alternates between the
    B-state N rows and the A-state 2N-1 rows with random weights)."""
    rows = 0.0
    for s0, s1 in zip(st0, st1):
        if s0["state"] in (1, 2):
            rows += 0.5 * (s0["L"] + s1["L"]) + 0.5 * (N + 2 * N - 1)
    return rows


def report(args, wl_name, shape, B, N, T, propose, prompt_len, gen, elapsed, st0, st1, kernels, roof, ctx_rows,
           metric=METRIC):
    committed = delta(st0, st1, "committed")
    ms = 1e3 * elapsed / args.steps
    ctx_rows = window_ctx_rows(st0, st1, N) or ctx_rows
    sb = step_bytes(shape, getattr(kernel_profile, "live_rows", B * (2 * N - 1)), ctx_rows)
    live0 = [s["L"] for s in st0 if s["state"] in (1, 2)] or [0]
    live1 = [s["L"] for s in st1 if s["state"] in (1, 2)] or [0]
    per_launch = 1 if args.no_graphs else args.passes_per_launch
    return {
        "metric": metric, "value": committed / elapsed, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random-init weights N(0,0.02), uniformly random prompt ids)",
        "config": {"workload": wl_name, "batch": B, "stride": N, "prompt_len": prompt_len, "max_new": gen,
                   "propose": propose, "temperature": T, "parallelism": "single GPU",
                   "hip_graphs": not args.no_graphs, "passes_per_graph_launch": per_launch,
                   "timed_context": [min(live0), max(live1)]},
        "host_enqueue_ms_per_step": 1e3 * getattr(timed_steps, "host_seconds", 0.0) / args.steps,
        "isd_steps_per_s": args.steps / elapsed,
        "tokens_per_forward": committed / max(1, delta(st0, st1, "passes")),
        "acceptance": delta(st0, st1, "accepted") / max(1, delta(st0, st1, "verified")),
        "step_hbm_GBps": sb / (ms * 1e-3) / 1e9,
        "step_hbm_frac": sb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "step_algorithmic_bytes": sb,
        "tpf_formula_at_measured_acceptance": tpf_projection(
            delta(st0, st1, "accepted") / max(1, delta(st0, st1, "verified")), N),
        "projected_tokens_per_s_at_p0.9": args.steps / elapsed * B * tpf_projection(0.9, N),
        "stride_efficiency_at_p0.9": tpf_projection(0.9, N) ** 2 / (2 * N - 1),
        "roofline": roof,
        "live_rows_per_pass": getattr(kernel_profile, "live_rows", None),
        "kernels": kernels,
    }


def emit(args, out):
    line = json.dumps(out)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


def generate(eng, torch, B):
    """Decode every slot to completion; the committed tokens of each slot (prefill's first one
    not included)."""
    toks = [[] for _ in range(B)]
    n = 0
    while True:
        st = eng.slots_host()
        if not any(s["state"] in (1, 2) for s in st):
            return toks, n
        tok, nc, _ = eng.step()
        n += 1
        t, c = tok.cpu().numpy(), nc.cpu().numpy()
        for b in range(B):
            toks[b] += t[b, :c[b]].tolist()


def run_risd(args, I, Engine, torch, dev):
    """R-ISD on the 8B shape: greedy R-ISD (gated rank-128 LoRA on the MASK rows) must commit
    exactly the tokens of greedy AR decoding (N = 1) with the base weights; the overhead factor
    alpha is the R-ISD step time over the step time of ISD without the adapter (same shapes)."""
    wl = I.RISD_8B
    shape, N, T, propose = wl.model, args.stride or wl.stride, wl.temperature, wl.propose
    B = args.batch or wl.batch
    pl = args.prompt_len or wl.prompt_len
    gen = args.gen or wl.max_new
    t0 = time.perf_counter()
    weights, lora = I.weights_torch(shape, dev, lora_rank=wl.lora_rank)
    torch.cuda.synchronize()
    log(f"weights + rank-{wl.lora_rank} adapter generated in {time.perf_counter() - t0:.1f}s")
    seqs = {}
    for name, n, lo in (() if args.no_ar_check else (("risd", N, lora), ("ar", 1, None))):
        eng, first = prefill_engine(I, Engine, torch, shape, weights, dev, B, n, T, propose, pl, gen, lora=lo)
        eng.set_graphs(not args.no_graphs)
        t0 = time.perf_counter()
        toks, steps = generate(eng, torch, B)
        seqs[name] = [[f] + t for f, t in zip(first, toks)]
        log(f"{name}: {steps} passes, {sum(len(t) for t in toks)} tokens in {time.perf_counter() - t0:.1f}s")
        del eng
        torch.cuda.empty_cache()
    same = seqs["risd"] == seqs["ar"] if seqs else None
    n_cmp = sum(len(t) for t in seqs["ar"]) if seqs else 0
    first_diff = None
    if seqs and not same:
        for b, (x, y) in enumerate(zip(seqs["risd"], seqs["ar"])):
            if x != y:
                first_diff = {"slot": b, "index": next(i for i, (u, v) in enumerate(zip(x, y)) if u != v)}
                break
    log(f"R-ISD greedy == AR greedy: {same} ({n_cmp} tokens)")
    res = {}
    for name, lo in (("isd", None), ("risd", lora)):
        eng, _ = prefill_engine(I, Engine, torch, shape, weights, dev, B, N, T, propose, pl, gen, lora=lo)
        elapsed, st0, st1 = timed_steps(eng, torch, args.steps, args.warmup, not args.no_graphs)
        log(f"{name}: {1e3 * elapsed / args.steps:.3f} ms/step")
        if name == "risd":
            kernels, roof, ctx = kernel_profile(eng, shape, B, N, args.profile_steps)
        res[name] = (elapsed, st0, st1)
        del eng
        torch.cuda.empty_cache()
    elapsed, st0, st1 = res["risd"]
    out = report(args, wl.name, shape, B, N, T, propose, pl, gen, elapsed, st0, st1, kernels, roof, ctx,
                 metric="committed tokens/s on 1 MI355X (8B-shape R-ISD, batch 16, N=4, greedy)")
    out["config"]["lora_rank"] = wl.lora_rank
    out["risd_alpha"] = res["risd"][0] / res["isd"][0]
    out["isd_no_adapter_ms_per_step"] = 1e3 * res["isd"][0] / args.steps
    out["risd_equals_ar_greedy"] = same
    out["ar_tokens_compared"] = n_cmp
    if first_diff:
        out["first_difference"] = first_diff
    emit(args, out)


def run_meter(args, I, Engine, torch, dev):
    """Introspective acceptance meter on the 8B shape: every pending token (the model's own
    MASK-row proposal) is committed untested and re-scored by the next pass's anchor; the
    rate is the mean acceptance probability (p(x) for argmax proposals at T = 1)."""
    wl = I.QWEN3_8B_DECODE
    shape, N, T, propose = wl.model, args.stride or wl.stride, wl.temperature, wl.propose
    B = args.batch or wl.batch
    pl = args.prompt_len or wl.prompt_len
    gen = args.gen or wl.max_new
    weights, _ = I.weights_torch(shape, dev)
    eng, _ = prefill_engine(I, Engine, torch, shape, weights, dev, B, N, T, propose, pl, gen)
    eng.set_meter(True)
    elapsed, st0, st1 = timed_steps(eng, torch, args.steps, args.warmup, not args.no_graphs)
    s_sum = sum(s["meter_sum"] for s in st1) - sum(s["meter_sum"] for s in st0)
    s_n = delta(st0, st1, "meter_n")
    rate = s_sum / max(1, s_n)
    log(f"meter: {s_n} re-scored tokens, introspective acceptance {rate:.6f}, "
        f"{1e3 * elapsed / args.steps:.3f} ms/step")
    out = {
        "metric": f"introspective acceptance rate (8B-shape, batch {B}, N={N}, {propose} proposals, T={T}; "
                  "teacher-forced re-scoring of the model's own proposals)",
        "value": rate, "unit": "probability", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random-init weights N(0,0.02), uniformly random prompt ids)",
        "config": {"workload": f"qwen3-8b-meter-b{B}", "batch": B, "stride": N, "prompt_len": pl,
                   "max_new": gen, "propose": propose, "temperature": T, "parallelism": "single GPU",
                   "hip_graphs": not args.no_graphs},
        "rescored_tokens": s_n,
    }
    emit(args, out)


def host_info():
    """CPU model (lscpu) and the BLAS library numpy uses (threadpoolctl)."""
    import subprocess
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
    except Exception:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [x for x in threadpool_info() if x.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas, "nproc": os.cpu_count()}


def run_micro(args, I, torch, dev):
    """The attention + acceptance kernel microbench: one paged-attention launch over 64 slots
    (32 query / 8 KV heads x 128, bf16 KV in 16-token pages under a shuffled page table, contexts
    uniform in [512, 4096], 7 query rows) and one acceptance step over 64 x 7 rows of 151936
    logits, with fresh logits every pass (p ~ N(0, 3^2); a pending token's verify row is its
    proposing row + N(0, 0.3^2)).  A step is one attention launch plus one acceptance step.
    The oracle computes the same attention and decisions on the host beside it."""
    import numpy as np

    from strided_decoding_amd import attn_paged, sample
    cfg = I.ATTN_SAMPLER_MICRO
    B, N, V = cfg.batch, cfg.stride, cfg.vocab
    R = 2 * N - 1
    steps, warm = args.steps, args.warmup
    a = I.attn_micro(cfg)
    ctx = a["ctx"]

    def bf(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    q = bf(a["q"])
    kp = bf(a["k_pages"])
    vp = bf(a["v_pages"]).permute(0, 1, 3, 2).contiguous()          # pages hold V transposed
    pt = torch.from_numpy(a["page_table"]).to(dev)
    ctx_t = torch.from_numpy(ctx).to(dev)
    qlen = torch.full((B,), R, dtype=torch.int32, device=dev)
    out, ws, _ = attn_paged(q, kp, vp, pt, ctx_t, qlen, cfg.n_kv_heads)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(warm):
        attn_paged(q, kp, vp, pt, ctx_t, qlen, cfg.n_kv_heads, out=out, workspace=ws)
    ev[0].record()
    for _ in range(steps):
        attn_paged(q, kp, vp, pt, ctx_t, qlen, cfg.n_kv_heads, out=out, workspace=ws)
    ev[1].record()
    torch.cuda.synchronize()
    attn_us = 1e3 * ev[0].elapsed_time(ev[1]) / steps
    kd = cfg.n_kv_heads * cfg.head_dim
    attn_bytes = int(ctx.sum()) * 2 * kd * 2 + 2 * B * R * cfg.n_q_heads * cfg.head_dim * 2
    attn_flops = 4.0 * sum(sum(int(c) - R + i + 1 for i in range(R)) for c in ctx) * cfg.n_q_heads * cfg.head_dim
    log(f"micro: attention {attn_us:.1f} us per launch, {attn_bytes / attn_us / 1e3:.0f} GB/s")

    # acceptance steps with fresh logits (the state machine runs on; q rows from the previous pass)
    g = torch.Generator(device=dev).manual_seed(7)
    slots = torch.zeros((B, 32), dtype=torch.int32, device=dev)
    slots[:, 0], slots[:, 1], slots[:, 3], slots[:, 5] = 2, 100, 1, 1 << 30
    slots[:, 8:22] = -1
    bufs = [torch.empty((B, R, V), dtype=torch.float32, device=dev) for _ in range(2)]
    bufs[1].normal_(0.0, cfg.p_std, generator=g)
    tok = torch.empty((B, N), dtype=torch.int32, device=dev)
    nc = torch.empty(B, dtype=torch.int32, device=dev)
    na = torch.empty(B, dtype=torch.int32, device=dev)
    sws = None
    samp_ms = 0.0
    evs = []
    for it in range(warm + steps):
        cur, prev = bufs[it & 1], bufs[(it & 1) ^ 1]
        cur.normal_(0.0, cfg.p_std, generator=g)
        q_row = slots[:, 15:15 + N - 1].long().clamp(min=0)
        src = prev.view(B * R, V)[q_row.reshape(-1)].view(B, N - 1, V)
        noisy = src + cfg.q_noise_std * torch.randn(src.shape, generator=g, device=dev)
        cur[:, :N - 1] = torch.where((slots[:, 0] == 1)[:, None, None], noisy, cur[:, :N - 1])
        if it == warm:
            st0 = slots.cpu().numpy().copy()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        sws = sample(slots, cur, prev.view(B * R, V), N, 1.0, "sample", I.SEED_PHILOX, tok, nc, na, workspace=sws)
        e[1].record()
        if it >= warm:
            evs.append(e)
    torch.cuda.synchronize()
    samp_ms = sum(e[0].elapsed_time(e[1]) for e in evs)
    samp_us = 1e3 * samp_ms / steps
    st1 = slots.cpu().numpy()
    d = st1 - st0
    acc = d[:, 23].sum() / max(1, d[:, 24].sum())
    tpf = d[:, 25].sum() / max(1, d[:, 22].sum())
    samp_bytes = B * R * V * 4 * 2          # the pass's rows once for the statistics, the previous rows once
    log(f"micro: acceptance step {samp_us:.1f} us, acceptance {acc:.4f}, tokens per forward {tpf:.4f} "
        f"(closed form at that acceptance {tpf_projection(acc, N):.4f})")

    # the oracle on the same inputs: attention of every slot, decisions of every slot
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import isd as OI
        from oracle import model as M
        threads = sum(x.get("num_threads", 0) for x in threadpool_info() if x.get("user_api") == "blas") or 1
        k_np = M.f32(a["k_pages"])
        v_np = M.f32(a["v_pages"])
        q_np = M.f32(a["q"])
        t0 = time.perf_counter()
        for b in range(B):
            c = int(ctx[b])
            M.paged_attention(q_np[b], k_np, v_np, a["page_table"][b], c, c - R + np.arange(R),
                              cfg.n_q_heads // cfg.n_kv_heads, cfg.page_size)
        t_attn = time.perf_counter() - t0
        lg = I.sampler_micro(cfg)
        t0 = time.perf_counter()
        for b in range(B):
            OI.decide("B", 100, 1, b, [], [], lg["p_logits"][b], N, 1.0, "sample", I.SEED_PHILOX)
        t_samp = time.perf_counter() - t0
        cpu = {"value": 1e6 * (t_attn + t_samp), "unit": "us per step", "cores": threads, "kind": "oracle",
               "sample": f"the whole step: attention of all {B} slots (contexts {int(ctx.min())}..{int(ctx.max())}) "
                         f"{t_attn:.2f}s and the B-state decisions of all {B} slots on the recipe's logits "
                         f"{t_samp:.2f}s, fp32/fp64 numpy",
               "host": host_info()}
    us = attn_us + samp_us
    out = {
        "metric": "attention + acceptance microbench time per step (64 slots, N=4, contexts U[512,4096], "
                  "vocab 151936)",
        "value": us, "unit": "us", "n_gpus": 1, "steps": steps, "warmup": warm, "ms_per_step": us / 1e3,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16 attention, fp32 logits",
        "data": "synthetic (N(0,1) bf16 Q/K/V, shuffled page table; N(0,3^2) logits with N(0,0.3^2) proposal noise)",
        "config": {"workload": "attn-accept-micro-b64", "batch": B, "stride": N, "ctx": [cfg.ctx_lo, cfg.ctx_hi],
                   "vocab": V},
        "attention_us": attn_us, "attention_GBps": attn_bytes / attn_us / 1e3,
        "acceptance_step_us": samp_us, "acceptance_step_GBps": samp_bytes / samp_us / 1e3,
        "acceptance": acc, "tokens_per_forward": tpf, "tpf_formula_at_measured_acceptance": tpf_projection(acc, N),
        "roofline": {"bound": "hbm", "achieved": attn_bytes / attn_us / 1e3, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": attn_bytes / attn_us / 1e3 / HBM_PEAK_GBS, "traffic": None, "kernel": "attention",
                     "per_launch": {"bytes": attn_bytes, "flops": attn_flops, "avg_us": attn_us}},
    }
    if cpu:
        out["cpu_baseline"] = cpu
    emit(args, out)


def main():
    args = parse()
    if args.trace_summary:
        return trace_summary(args.trace_summary)
    if args.pmc_summary:
        return pmc_summary(args.pmc_summary)
    if args.counter_summary:
        return counter_summary(args.counter_summary)
    if args.copy_probe_mib:
        return copy_probe(args.copy_probe_mib)
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on exactly one GPU; --gpus must be 1"}))
        sys.exit(2)
    import torch

    import isd_inputs as I
    from strided_decoding_amd import Engine

    dev = torch.device("cuda:0")
    if args.steps is None:
        args.steps = {"risd": 200, "meter": 100, "micro": 200}.get(args.workload,
                                                                   200 if args.model == "32b" else 1000)
    if args.workload == "micro":
        return run_micro(args, I, torch, dev)
    if args.workload == "risd":
        return run_risd(args, I, Engine, torch, dev)
    if args.workload == "meter":
        return run_meter(args, I, Engine, torch, dev)
    wl = I.QWEN3_32B_DECODE if args.model == "32b" else I.QWEN3_8B_DECODE
    shape, N, T, propose = wl.model, args.stride or wl.stride, wl.temperature, wl.propose
    B = args.batch or wl.batch
    pl = args.prompt_len or wl.prompt_len
    gen = args.gen or wl.max_new
    t0 = time.perf_counter()
    weights, _ = I.weights_torch(shape, dev)
    torch.cuda.synchronize()
    log(f"weights generated in {time.perf_counter() - t0:.1f}s")
    K = args.active
    if K is not None and not 1 <= K <= B:
        raise SystemExit(f"--active must be in 1..{B}")
    eng, _ = prefill_engine(I, Engine, torch, shape, weights, dev, B, N, T, propose, pl, gen, live=K)
    elapsed, st0, st1 = timed_steps(eng, torch, args.steps, args.warmup, not args.no_graphs, n_active=K,
                                    per_launch=1 if args.no_graphs else args.passes_per_launch)
    live = sum(1 for s in st1 if s["state"] in (1, 2))
    log(f"timed {args.steps} steps: {1e3 * elapsed / args.steps:.3f} ms/step, "
        f"{delta(st0, st1, 'committed')} tokens, live slots {live}")
    # per-kernel figures at the timed window's mean context: the live slots are prefilled again
    # with prompts of that length (the timed passes moved every context through the window)
    prof_ctx = int(round(window_ctx_rows(st0, st1, N) / max(1, live) - 0.5 * (3 * N - 1)))
    prof_ctx = max(1, min(prof_ctx, pl + gen - 64))

    def reprefill():
        prefill_engine(I, Engine, torch, shape, weights, dev, B, N, T, propose, prof_ctx, pl + gen - prof_ctx,
                       live=K, chunk=8, engine=eng)

    reprefill()
    graph_ab = None
    if K is None and not args.no_graphs:
        graph_ab = {}
        for per in (1, args.passes_per_launch):
            run_passes(eng, 2 * per, None, per)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            run_passes(eng, 4 * per, None, per)
            torch.cuda.synchronize()
            graph_ab[f"passes_per_launch_{per}_ms_per_step"] = 1e3 * (time.perf_counter() - t0) / (4 * per)
            reprefill()
        log(f"graph launches: {graph_ab}")
    kernels, roof, ctx = kernel_profile(eng, shape, B, N, args.profile_steps, n_active=K)
    name = wl.name if B == wl.batch else wl.name.rsplit("-b", 1)[0] + f"-b{B}"
    if N != wl.stride:
        name += f"-n{N}"
    if K is not None:
        name += f"-active{K}"
    metric = METRIC if wl is I.QWEN3_8B_DECODE and N == wl.stride and K is None else \
        f"committed tokens/s on 1 MI355X ({'8B' if wl is I.QWEN3_8B_DECODE else '32B'}-shape, batch {B}, N={N}" + \
        (f", {K} live slots stepped as the active prefix)" if K is not None else ")")
    out = report(args, name, shape, K or B, N, T, propose, pl, gen, elapsed, st0, st1, kernels, roof, ctx, metric)
    out["kernel_profile_context"] = prof_ctx
    if graph_ab:
        out["graph_launch_ab"] = graph_ab
    if K is not None:
        out["config"]["batch"] = B
        out["config"]["active_slots"] = K
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shape, weights, eng, B, N, T)
    emit(args, out)


if __name__ == "__main__":
    main()
