"""CPU checks of the C ABI: libisd.so loads, exports every function include/isd.h declares,
and the host-side size query / configuration validation behaves as documented.  No GPU
work is launched (a size query touches no HIP API)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "isd.h")


def _lib():
    from strided_decoding_amd import _abi as A
    if not os.path.exists(A.LIB_PATH):
        from strided_decoding_amd import build
        build.build(verbose=False)
    return A, A.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b((?:isd|attn)_[a-z_0-9]+)\s*\(", src)))


def test_header_declarations_match_binding():
    A, _ = _lib()
    assert set(_declared()) == set(A.EXPORTS)


def test_library_exports_every_declared_symbol():
    _, lib = _lib()
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.isd_version().startswith(b"isd-mi355x")


def _cfg(A, **kw):
    base = dict(n_layers=36, d_model=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, d_ffn=12288, vocab=151936,
                rope_base=1e4, rms_eps=1e-6, dtype=A.ISD_BF16, stride_n=4, page_size=16, max_batch=64,
                max_seq_len=2048 + 16, n_pages=64 * 130, max_prefill_tokens=16384, lora_rank=0,
                propose=A.ISD_PROPOSE_ARGMAX, temperature=1.0, seed=1)
    base.update(kw)
    return A.Config(**base)


def _query(A, lib, cfg):
    sizes = A.Sizes()
    ctx = C.c_void_p(1)
    rc = lib.isd_init(C.byref(cfg), None, None, None, C.byref(sizes), C.byref(ctx), None)
    return rc, sizes, ctx


def test_size_query_qwen3_8b_shape():
    A, lib = _lib()
    rc, sizes, ctx = _query(A, lib, _cfg(A))
    assert rc == A.ISD_OK and ctx.value is None
    # KV pool: 2 (K,V) x 36 layers x pages x 8 heads x 16 tokens x 128 dims x 2 bytes
    assert sizes.kv_pool_bytes == 2 * 36 * 64 * 130 * 8 * 16 * 128 * 2
    # workspace holds at least the double-buffered logits of 64 x 7 rows
    assert sizes.workspace_bytes > 2 * 64 * 7 * 151936 * 4
    assert sizes.workspace_bytes < 64 << 30


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 64, "ISD_E_SHAPE"),           # bf16 kernels are built for head_dim 128
    ("page_size", 32, "ISD_E_SHAPE"),
    ("n_kv_heads", 7, "ISD_E_SHAPE"),          # Hq not a multiple of Hkv
    ("stride_n", 0, "ISD_E_ARG"),
    ("stride_n", 9, "ISD_E_ARG"),
    ("dtype", 5, "ISD_E_ARG"),
    ("temperature", -1.0, "ISD_E_ARG"),
    ("lora_rank", 100, "ISD_E_SHAPE"),
    ("propose", 3, "ISD_E_ARG"),
])
def test_config_validation(field, value, code):
    A, lib = _lib()
    rc, _, _ = _query(A, lib, _cfg(A, **{field: value}))
    assert rc == getattr(A, code)


def test_fp32_config_accepts_small_head_dim():
    A, lib = _lib()
    rc, sizes, _ = _query(A, lib, _cfg(A, dtype=A.ISD_F32, head_dim=32, n_layers=2, d_model=128, n_q_heads=4,
                                       n_kv_heads=4, d_ffn=512, vocab=1024, max_batch=2, max_seq_len=96,
                                       n_pages=16, max_prefill_tokens=64))
    assert rc == A.ISD_OK and sizes.kv_pool_bytes == 2 * 2 * 16 * 4 * 16 * 32 * 4


def test_null_arguments_rejected():
    A, lib = _lib()
    sizes = A.Sizes()
    ctx = C.c_void_p()
    assert lib.isd_init(None, None, None, None, C.byref(sizes), C.byref(ctx), None) == A.ISD_E_ARG
    assert lib.isd_step(None, None, None, None, None, None) == A.ISD_E_ARG
    assert lib.isd_step_n(None, 2, None, None, None, None) == A.ISD_E_ARG
    assert lib.isd_release(None) == A.ISD_E_ARG
