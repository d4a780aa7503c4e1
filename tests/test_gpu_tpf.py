"""Tokens per forward measured on the GPU against the pages' closed form (wiki note, Method;
GeekNews, Speedup Factor Explorer): TPF = (2 + p + ... + p^(N-2)) / (2 - p^(N-1)) for
acceptance rate p.

isd_sample_step runs the A/B state machine of 64 slots over 10^4 consecutive passes with
fresh logits of the attention + acceptance microbench recipe every pass: every row ~ N(0, 3^2)
over the 151936-token vocabulary, except that a pending token's verify row is the logits row
that proposed it in the previous pass plus N(0, 0.3^2) noise (so p and q differ as in the
recipe, acceptance ~ 0.876).  Acceptance events are then independent across positions and
passes, and the measured tokens per pass must equal the closed form at the measured
acceptance, within the Monte Carlo error (slots are independent chains: the standard error
comes from the spread of the 64 per-slot rates).
"""
import numpy as np
import pytest
import torch

import isd_inputs as I
from oracle import tpf as TPF

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("N", [2, 3, 4, 8])
def test_measured_tpf_matches_closed_form(N):
    from strided_decoding_amd import sample
    cfg = I.ATTN_SAMPLER_MICRO
    B, V, R = cfg.batch, cfg.vocab, 2 * N - 1
    n_passes = 10_000
    g = torch.Generator(device=DEV).manual_seed(1000 + N)
    slots = torch.zeros((B, 32), dtype=torch.int32, device=DEV)
    slots[:, 0] = 2                          # state B: the first pass proposes
    slots[:, 1] = 100                        # L
    slots[:, 3] = 1                          # t
    slots[:, 5] = 1 << 30                    # max_new: no slot finishes
    slots[:, 8:22] = -1
    bufs = [torch.empty((B, R, V), dtype=torch.float32, device=DEV) for _ in range(2)]
    bufs[1].normal_(0.0, cfg.p_std, generator=g)
    tok = torch.empty((B, N), dtype=torch.int32, device=DEV)
    nc = torch.empty(B, dtype=torch.int32, device=DEV)
    na = torch.empty(B, dtype=torch.int32, device=DEV)
    ws = None
    rows_b = torch.arange(B, device=DEV)[:, None]
    print(f"tpf N={N}: {n_passes} passes of {B} slots", flush=True)
    for it in range(n_passes):
        cur, prev = bufs[it & 1], bufs[(it & 1) ^ 1]
        cur.normal_(0.0, cfg.p_std, generator=g)
        if N > 1:
            # A-state slots: verify row i-1 = the previous pass's proposing row + N(0, 0.3^2)
            q_row = slots[:, 15:15 + N - 1].long().clamp(min=0)
            src = prev.view(B * R, V)[q_row.reshape(-1)].view(B, N - 1, V)
            noisy = src + cfg.q_noise_std * torch.randn(src.shape, generator=g, device=DEV)
            is_a = (slots[:, 0] == 1)[:, None, None]
            cur[:, :N - 1] = torch.where(is_a, noisy, cur[:, :N - 1])
        ws = sample(slots, cur, prev.view(B * R, V), N, 1.0, "sample", I.SEED_PHILOX, tok, nc, na, workspace=ws)
        if (it + 1) % 2500 == 0:
            torch.cuda.synchronize()
            print(f"tpf N={N}: {it + 1} passes", flush=True)
    s = slots.cpu().numpy()
    passes, accepted, verified, committed = s[:, 22], s[:, 23], s[:, 24], s[:, 25]
    assert np.all(passes == n_passes) and np.all(s[:, 7] == 0)
    p_hat = accepted.sum() / verified.sum()
    per_slot = committed / passes
    tpf = per_slot.mean()
    se = per_slot.std(ddof=1) / np.sqrt(B)
    ref = TPF.tpf_closed_form(p_hat, N)
    print(f"tpf N={N}: acceptance {p_hat:.4f}, measured TPF {tpf:.4f} +- {se:.4f}, closed form {ref:.4f}, "
          f"efficiency TPF^2/(2N-1) {TPF.efficiency(tpf, R):.3f}", flush=True)
    assert 0.84 < p_hat < 0.91                 # the recipe's acceptance, sum_x min(p, q) ~ 0.876
    assert abs(tpf - ref) <= 4 * se + 1e-3, (tpf, ref, se)
