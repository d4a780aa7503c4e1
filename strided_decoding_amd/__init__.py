"""MI355X (gfx950) Introspective Strided Decoding: HIP kernels behind a C ABI (libisd.so).

`Engine` wraps one decoding context (isd_init / isd_prefill / isd_step); `attn_paged` and
`sample` call the kernel-level entry points.  The HIP library is required; there is no
CPU fallback.
"""
from ._abi import EXPORTS, LIB_PATH, IsdError, load  # noqa: F401


def __getattr__(name):
    if name in ("Engine", "attn_paged", "sample", "gemm", "pack_weight", "PackedWeight"):
        from . import engine
        return getattr(engine, name)
    raise AttributeError(name)
