"""isd_sample_step_noalloc (the acceptance step with its statistics in the library's fixed
scratch array) against isd_sample_step with a caller workspace, through the C ABI: identical
slot records, tokens, counts and decision records, bit for bit, on two calls in a row (the
second smaller than the first, so that it reads no statistics the first one left behind)."""
import ctypes as C

import numpy as np
import pytest
import torch

from strided_decoding_amd import _abi as A

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(B, N, V, seed):
    R = 2 * N - 1
    g = torch.Generator(device=DEV).manual_seed(seed)
    logits = torch.randn((B, R, V), generator=g, device=DEV) * 3.0
    q = torch.randn((B * R, V), generator=g, device=DEV) * 3.0
    slots = torch.zeros((B, 32), dtype=torch.int32, device=DEV)
    states = torch.tensor([1, 2, 1, 3] * (B // 4) + [1] * (B % 4), dtype=torch.int32)
    slots[:, 0] = states.to(DEV)
    slots[:, 1] = 200
    slots[:, 3] = 5
    slots[:, 4] = 1
    slots[:, 5] = 1 << 20
    slots[:, 8:22] = -1
    slots[:, 8:8 + N - 1] = torch.randint(0, V, (B, N - 1), generator=g, device=DEV).int()
    slots[:, 15:15 + N - 1] = (torch.arange(B, device=DEV)[:, None] * R + N +
                               torch.arange(N - 1, device=DEV)[None, :]).int()
    return slots, logits, q


def _call(lib, fn, slots, logits, q, N, workspace=None):
    B, R, V = logits.shape
    out = dict(slots=slots.clone(), tok=torch.full((B, N), -7, dtype=torch.int32, device=DEV),
               nc=torch.full((B,), -7, dtype=torch.int32, device=DEV),
               na=torch.full((B,), -7, dtype=torch.int32, device=DEV),
               margins=torch.zeros((B, 2 * N), dtype=torch.float64, device=DEV),
               kinds=torch.zeros((B, 2 * N), dtype=torch.int32, device=DEV))
    args = A.SampleArgs(B, N, V, A.ISD_PROPOSE_SAMPLE, q.shape[0], 1.0, 1, out["slots"].data_ptr(),
                        logits.data_ptr(), q.data_ptr(), out["tok"].data_ptr(), out["nc"].data_ptr(),
                        out["na"].data_ptr(), 0 if workspace is None else workspace.data_ptr(), 0,
                        out["margins"].data_ptr(), out["kinds"].data_ptr())
    rc = getattr(lib, fn)(C.byref(args), C.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc, out


def test_noalloc_sample_step_equals_workspace_version():
    lib = A.load()
    for B, N, V, seed in ((64, 4, 151936, 1), (12, 3, 5000, 2)):
        print(f"no-alloc acceptance step B={B} N={N} V={V}", flush=True)
        slots, logits, q = _inputs(B, N, V, seed)
        R = 2 * N - 1
        ws = torch.empty(lib.isd_sample_step_workspace_bytes(B, R, V, q.shape[0]), dtype=torch.uint8, device=DEV)
        rc_ref, ref = _call(lib, "isd_sample_step", slots, logits, q, N, workspace=ws)
        rc, got = _call(lib, "isd_sample_step_noalloc", slots, logits, q, N)
        torch.cuda.synchronize()
        assert rc_ref == A.ISD_OK and rc == A.ISD_OK
        for k in ref:
            assert torch.equal(ref[k], got[k]), (B, k)
        assert int(ref["nc"].min()) >= 0 and int((ref["slots"][:, 22] == 1).sum()) == int((slots[:, 0] != 3).sum())


def test_noalloc_sample_step_refusals():
    """Host-side refusals (nothing is launched): a workspace passed in, and a call whose
    statistics would not fit the scratch."""
    lib = A.load()
    slots, logits, q = _inputs(8, 4, 5000, 3)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    rc, _ = _call(lib, "isd_sample_step_noalloc", slots, logits, q, 4, workspace=ws)
    assert rc == A.ISD_E_ARG
    big = A.SampleArgs(4096, 8, 151936, A.ISD_PROPOSE_SAMPLE, 4096 * 15, 1.0, 1, slots.data_ptr(),
                       logits.data_ptr(), q.data_ptr(), slots.data_ptr(), slots.data_ptr(), slots.data_ptr(), 0, 0,
                       0, 0)
    assert lib.isd_sample_step_noalloc(C.byref(big), None) == A.ISD_E_CAPACITY
