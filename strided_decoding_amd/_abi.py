"""ctypes mirror of include/isd.h and the loader of libisd.so.

The library is required: importing this module on a machine without the built
libisd.so raises, there is no fallback implementation.
"""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libisd.so")

ISD_MAX_STRIDE = 8
ISD_OK, ISD_E_ARG, ISD_E_SHAPE, ISD_E_CAPACITY, ISD_E_STATE, ISD_E_HIP, ISD_E_NONFINITE = 0, -1, -2, -3, -4, -5, -6
STATUS_NAMES = {0: "ISD_OK", -1: "ISD_E_ARG", -2: "ISD_E_SHAPE", -3: "ISD_E_CAPACITY", -4: "ISD_E_STATE",
                -5: "ISD_E_HIP", -6: "ISD_E_NONFINITE"}
ISD_F32, ISD_BF16 = 0, 1
ISD_PROPOSE_SAMPLE, ISD_PROPOSE_ARGMAX = 0, 1
ISD_SLOT_EMPTY, ISD_SLOT_A, ISD_SLOT_B, ISD_SLOT_DONE = 0, 1, 2, 3
ISD_DEC_ACCEPT, ISD_DEC_RESID, ISD_DEC_Z1, ISD_DEC_PROPOSE = 0, 1, 2, 3
DEC_NAMES = {ISD_DEC_ACCEPT: "accept", ISD_DEC_RESID: "resid", ISD_DEC_Z1: "z1", ISD_DEC_PROPOSE: "propose"}
ISD_DEBUG_MAX_ROWS = 64
# a status only the device reports (an enqueuing call returns it as the context's sticky
# status); ISD_E_CAPACITY and ISD_E_STATE are also host refusals (isd_get_status tells them apart)
DEVICE_STATUSES = (-6,)

# symbols the header declares (checked by the CPU test-suite)
EXPORTS = ("isd_init", "isd_prefill", "isd_step", "isd_step_active", "isd_step_n", "isd_get_buffers",
           "isd_get_status", "isd_release", "attn_paged_decode_workspace_bytes", "attn_paged_decode",
           "isd_sample_step_workspace_bytes", "isd_sample_step", "isd_version", "isd_profile",
           "isd_profile_report", "isd_gemm", "isd_gemm_splits", "isd_set_graphs", "isd_packed_weight_bytes",
           "isd_pack_weights", "isd_set_meter", "isd_sample_step_noalloc")

ISD_GEMM_STORE, ISD_GEMM_STORE_F32, ISD_GEMM_RESID, ISD_GEMM_SWIGLU = 0, 1, 2, 3


class GemmArgs(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("mode", C.c_int32), ("M", C.c_int32), ("N", C.c_int32), ("K", C.c_int32),
                ("splits", C.c_int32), ("X", C.c_void_p), ("W", C.c_void_p), ("W2", C.c_void_p), ("Y", C.c_void_p),
                ("R", C.c_void_p), ("workspace", C.c_void_p), ("norm_g", C.c_void_p), ("norm_out", C.c_void_p),
                ("norm_eps", C.c_float), ("path", C.c_int32)]


class ProfEntry(C.Structure):
    _fields_ = [("name", C.c_char * 32), ("launches", C.c_int32), ("total_ms", C.c_double)]


class IsdError(RuntimeError):
    def __init__(self, where, code):
        super().__init__(f"{where} failed: {STATUS_NAMES.get(code, code)}")
        self.code = code


class Config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("d_ffn", C.c_int32), ("vocab", C.c_int32),
                ("rope_base", C.c_float), ("rms_eps", C.c_float), ("dtype", C.c_int32), ("stride_n", C.c_int32),
                ("page_size", C.c_int32), ("max_batch", C.c_int32), ("max_seq_len", C.c_int32),
                ("n_pages", C.c_int32), ("max_prefill_tokens", C.c_int32), ("lora_rank", C.c_int32),
                ("propose", C.c_int32), ("temperature", C.c_float), ("seed", C.c_uint64)]


PP = C.POINTER(C.c_void_p)


class Weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p), ("lm_head", C.c_void_p),
                ("attn_norm", PP), ("wqkv", PP), ("wo", PP), ("ffn_norm", PP), ("wg", PP), ("wu", PP),
                ("wd", PP), ("lora_a", PP), ("lora_b", PP)]


class Sizes(C.Structure):
    _fields_ = [("kv_pool_bytes", C.c_size_t), ("workspace_bytes", C.c_size_t)]


SLOT_INTS = 32   # isd_slot is 32 int32 words
SLOT_FIELDS = ["state", "L", "c", "t", "n_gen", "max_new", "n_pages", "status"] + \
    [f"pending{i}" for i in range(ISD_MAX_STRIDE - 1)] + [f"q_row{i}" for i in range(ISD_MAX_STRIDE - 1)] + \
    ["passes", "accepted", "verified", "committed", "meter_sum_lo", "meter_sum_hi", "meter_n"] + \
    [f"pad{i}" for i in range(3)]
METER_SUM_WORD = 26   # meter_sum: a double in words 26-27


class Buffers(C.Structure):
    _fields_ = [("slots", C.c_void_p), ("page_table", C.c_void_p), ("max_pages_per_slot", C.c_int32),
                ("free_stack", C.c_void_p), ("n_free", C.c_void_p), ("logits", C.c_void_p),
                ("rows_per_slot", C.c_int32), ("row_token", C.c_void_p), ("row_pos", C.c_void_p),
                ("k_pool", C.c_void_p), ("v_pool", C.c_void_p), ("attn_out", C.c_void_p),
                ("prefill_logits", C.c_void_p), ("row_off", C.c_void_p), ("row_len", C.c_void_p)]


class Debug(C.Structure):
    _fields_ = [("n_rows", C.c_int32), ("rows", C.c_void_p), ("layer_in", C.c_void_p), ("layer_attn", C.c_void_p),
                ("final_normed", C.c_void_p), ("margins", C.c_void_p), ("kinds", C.c_void_p)]


class AttnArgs(C.Structure):
    _fields_ = [("batch", C.c_int32), ("rows", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("page_size", C.c_int32), ("max_pages", C.c_int32),
                ("max_ctx", C.c_int32), ("q", C.c_void_p), ("k_pool", C.c_void_p), ("v_pool", C.c_void_p),
                ("page_table", C.c_void_p), ("ctx_len", C.c_void_p), ("q_len", C.c_void_p), ("out", C.c_void_p),
                ("workspace", C.c_void_p)]


class SampleArgs(C.Structure):
    _fields_ = [("batch", C.c_int32), ("stride_n", C.c_int32), ("vocab", C.c_int32), ("propose", C.c_int32),
                ("q_rows", C.c_int32), ("temperature", C.c_float), ("seed", C.c_uint64), ("slots", C.c_void_p),
                ("logits", C.c_void_p), ("q_logits", C.c_void_p), ("tokens", C.c_void_p),
                ("n_commit", C.c_void_p), ("n_accept", C.c_void_p), ("workspace", C.c_void_p), ("meter", C.c_int32),
                ("margins", C.c_void_p), ("kinds", C.c_void_p)]


_lib = None


def load(path=LIB_PATH):
    """Load libisd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m strided_decoding_amd.build` "
                          "(hipcc, gfx950); there is no fallback implementation")
    lib = C.CDLL(path)
    lib.isd_init.argtypes = [C.POINTER(Config), C.POINTER(Weights), C.c_void_p, C.c_void_p, C.POINTER(Sizes),
                             C.POINTER(C.c_void_p), C.c_void_p]
    lib.isd_prefill.argtypes = [C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.c_void_p, C.POINTER(C.c_int32),
                                C.POINTER(C.c_int32), C.c_void_p, C.c_void_p]
    lib.isd_step.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(Debug), C.c_void_p]
    lib.isd_step_n.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
    lib.isd_step_active.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
    lib.isd_get_buffers.argtypes = [C.c_void_p, C.POINTER(Buffers)]
    lib.isd_get_status.argtypes = [C.c_void_p, C.c_void_p]
    lib.isd_release.argtypes = [C.c_void_p]
    lib.attn_paged_decode_workspace_bytes.argtypes = [C.POINTER(AttnArgs)]
    lib.attn_paged_decode_workspace_bytes.restype = C.c_size_t
    lib.attn_paged_decode.argtypes = [C.POINTER(AttnArgs), C.c_void_p]
    lib.isd_sample_step_workspace_bytes.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_int32]
    lib.isd_sample_step_workspace_bytes.restype = C.c_size_t
    lib.isd_sample_step.argtypes = [C.POINTER(SampleArgs), C.c_void_p]
    lib.isd_sample_step_noalloc.argtypes = [C.POINTER(SampleArgs), C.c_void_p]
    lib.isd_version.restype = C.c_char_p
    lib.isd_gemm.argtypes = [C.POINTER(GemmArgs), C.c_void_p]
    lib.isd_gemm.restype = C.c_int
    lib.isd_gemm_splits.argtypes = [C.c_int32, C.c_int32, C.c_int32]
    lib.isd_gemm_splits.restype = C.c_int32
    lib.isd_packed_weight_bytes.argtypes = [C.c_int32, C.c_int32]
    lib.isd_packed_weight_bytes.restype = C.c_size_t
    lib.isd_pack_weights.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p]
    lib.isd_set_meter.argtypes = [C.c_void_p, C.c_int32]
    lib.isd_profile.argtypes = [C.c_void_p, C.c_int32]
    lib.isd_set_graphs.argtypes = [C.c_void_p, C.c_int32]
    lib.isd_profile_report.argtypes = [C.c_void_p, C.POINTER(ProfEntry), C.c_int32, C.POINTER(C.c_int32)]
    for f in ("isd_init", "isd_prefill", "isd_step", "isd_step_active", "isd_step_n", "isd_get_buffers",
              "isd_get_status", "isd_release", "attn_paged_decode", "isd_sample_step", "isd_profile",
              "isd_profile_report", "isd_set_graphs", "isd_set_meter", "isd_pack_weights",
              "isd_sample_step_noalloc"):
        getattr(lib, f).restype = C.c_int
    _lib = lib
    return lib


def check(where, code):
    if code != ISD_OK:
        raise IsdError(where, code)
