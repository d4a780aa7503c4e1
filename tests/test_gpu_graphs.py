"""isd_set_graphs / isd_step_n: replaying decode passes from captured HIP graphs gives exactly
the eager results.  Two contexts with the same weights and prompts, one launching eagerly and one
replaying graphs, are stepped side by side (with eager torch work and synchronizations
between the replays), and every pass's tokens, counts, logits, slot records and page tables
are compared bit for bit; a prefill that recycles a slot between replays, profiling (which
launches eagerly) and switching graphs off are exercised on the way.
"""
import numpy as np
import pytest
import torch

import isd_inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _engine(shape, w, prompts, max_new, N=4, T=1.0, propose="sample", lora=None, graphs=False):
    from strided_decoding_amd import Engine
    max_seq = max(len(p) for p in prompts) + 64
    eng = Engine(shape, w, stride=N, temperature=T, propose=propose, seed=1, max_batch=len(prompts),
                 max_seq_len=max_seq, lora=lora, graphs=graphs)
    eng.prefill(list(range(len(prompts))), prompts, max_new)
    return eng


def _same(a, b, step):
    ta, na, aa = [t.cpu().numpy() for t in a[0]]
    tb, nb, ab = [t.cpu().numpy() for t in b[0]]
    np.testing.assert_array_equal(na, nb, err_msg=f"n_commit, step {step}")
    np.testing.assert_array_equal(aa, ab, err_msg=f"n_accept, step {step}")
    for s in range(len(na)):
        np.testing.assert_array_equal(ta[s, :na[s]], tb[s, :nb[s]], err_msg=f"tokens, step {step}")
    assert torch.equal(a[1], b[1]), f"logits differ at step {step}"
    assert torch.equal(a[2], b[2]), f"page tables differ at step {step}"
    assert a[3] == b[3], f"slot records differ at step {step}"


def _snap(eng, out):
    torch.cuda.synchronize()
    return ([t.clone() for t in out], eng.logits().clone(), eng.page_table().clone(), eng.slots_host())


@pytest.mark.parametrize("propose,T", [("sample", 1.0), ("argmax", 0.0)])
def test_graph_replay_equals_eager(propose, T):
    shape = I.SMALL_BF16
    w = I.weights_numpy(shape, seed=0, scale=20.0, sticky=(0.0, 20.0, 4.0, 7))
    prompts = I.ragged_prompts([37, 5, 90, 16], shape.vocab, seed=12)
    max_new = [40, 25, 33, 40]
    print(f"graphs {propose} T={T}", flush=True)
    eager = _engine(shape, w, prompts, max_new, T=T, propose=propose)
    graph = _engine(shape, w, prompts, max_new, T=T, propose=propose, graphs=True)
    scratch = torch.randn(1 << 20, device=DEV)
    for step in range(14):
        a = _snap(eager, eager.step())
        b = _snap(graph, graph.step())
        _same(a, b, step)
        scratch.mul_(0.5).add_(1.0)             # the program's own eager work between replays
        torch.cuda.synchronize()
        if step == 5:                            # recycle slot 1 in both contexts
            p = [I.ragged_prompts([21], shape.vocab, seed=13)[0]]
            eager.prefill([1], p, [30])
            graph.prefill([1], p, [30])
        if step == 8:                            # profiled passes launch eagerly
            graph.profile(True)
        if step == 10:
            graph.profile(False)
            graph.profile_report()
        if step == 12:
            graph.set_graphs(False)


def test_graph_replay_equals_eager_with_adapter():
    """The MASK-row adapter under graph replay: at d_model 2048 the shrinks run as k-splits whose
    arrival counters every launch leaves at zero, so each replay sums its partials exactly as
    the eager launches do."""
    shape = I.ModelShape("mid-bf16", 1, 2048, 16, 4, 128, 4096, 4096, "bf16")
    w = I.weights_numpy(shape, seed=2, scale=20.0)
    lora = I.lora_numpy(shape, 64, scale=3.0)
    prompts = I.ragged_prompts([19, 33, 8], shape.vocab, seed=15)
    max_new = [30, 30, 30]
    eager = _engine(shape, w, prompts, max_new, lora=lora)
    graph = _engine(shape, w, prompts, max_new, lora=lora, graphs=True)
    scratch = torch.randn(1 << 20, device=DEV)
    for step in range(8):
        a = _snap(eager, eager.step())
        b = _snap(graph, graph.step())
        _same(a, b, step)
        scratch.mul_(0.5).add_(1.0)
        torch.cuda.synchronize()


@pytest.mark.parametrize("n_passes", [2, 3, 8])
def test_multi_pass_graph_equals_single_passes(n_passes):
    """isd_step_n: n passes in one graph launch commit exactly what n eager isd_step calls
    commit, pass by pass (odd counts leave the logits-buffer parity flipped for the next call)."""
    shape = I.SMALL_BF16
    w = I.weights_numpy(shape, seed=0, scale=20.0, sticky=(0.0, 20.0, 4.0, 7))
    prompts = I.ragged_prompts([37, 5, 90, 16], shape.vocab, seed=12)
    max_new = [60, 45, 53, 60]
    print(f"multi-pass graph n={n_passes}", flush=True)
    eager = _engine(shape, w, prompts, max_new)
    multi = _engine(shape, w, prompts, max_new, graphs=True)
    for call in range(3):
        t, c, a = [x.clone() for x in multi.step_n(n_passes)]
        torch.cuda.synchronize()
        for i in range(n_passes):
            et, ec, ea = eager.step()
            torch.cuda.synchronize()
            assert torch.equal(ec, c[i]) and torch.equal(ea, a[i]), (call, i)
            for b in range(len(prompts)):
                n = int(ec[b])
                assert torch.equal(et[b, :n], t[i, b, :n]), (call, i, b)
        assert torch.equal(eager.logits(), multi.logits()), call
        assert eager.slots_host() == multi.slots_host(), call
        assert torch.equal(eager.page_table(), multi.page_table()), call
