"""Thin Python front of libisd: torch provides device memory and streams, every step of
the decode path runs in the library's HIP kernels.
"""
import ctypes as C

import numpy as np
import torch

from . import _abi as A

LORA_ORDER = ("q", "k", "v", "o", "g", "u", "d")


def _dt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_device(a, dtype, device):
    """numpy float32 array or uint16 bf16-bit array -> contiguous device tensor of `dtype`."""
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=_dt(dtype)).contiguous()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a.astype(np.float32))
    return t.to(device=device, dtype=_dt(dtype)).contiguous()


class PackedWeight:
    """A bf16 weight [rows, cols] in the packed MFMA-operand layout of the bf16 GEMMs (see
    isd_pack_weights); `data` is the device buffer, rows padded to a multiple of 32."""

    def __init__(self, data, rows, cols):
        self.data, self.rows, self.cols = data, rows, cols

    def data_ptr(self):
        return self.data.data_ptr()


def pack_weight(W, stream=None):
    """Row-major bf16 device tensor [rows, cols] -> PackedWeight (isd_pack_weights)."""
    lib = A.load()
    if W.dtype != torch.bfloat16 or W.dim() != 2:
        raise TypeError("pack_weight takes a 2-D bfloat16 device tensor")
    W = W.contiguous()
    rows, cols = W.shape
    nbytes = lib.isd_packed_weight_bytes(rows, cols)
    if nbytes == 0:
        raise ValueError(f"cannot pack a [{rows}, {cols}] weight (cols must be a positive multiple of 16)")
    out = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=W.device)
    stream = stream if stream is not None else torch.cuda.current_stream(W.device)
    A.check("isd_pack_weights", lib.isd_pack_weights(W.data_ptr(), out.data_ptr(), rows, cols,
                                                     C.c_void_p(stream.cuda_stream)))
    return PackedWeight(out, rows, cols)


PACKED = ("wqkv", "wo", "wg", "wu", "wd")


class Engine:
    """One decoding context: weights, KV pool and workspace resident on `device`.

    shape: isd_inputs.ModelShape; weights / lora: nested like isd_inputs.weights_numpy /
    lora_numpy (numpy or torch tensors).
    """

    def __init__(self, shape, weights, *, stride, temperature, propose="sample", seed=1, max_batch=1,
                 max_seq_len=256, n_pages=None, max_prefill_tokens=None, lora=None, page_size=16,
                 device="cuda:0", stream=None, graphs=None):
        self.lib = A.load()
        self.shape = shape
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        dt = shape.dtype
        self.N = stride
        self.R = 2 * stride - 1
        self.max_batch = max_batch
        lora_rank = 0 if lora is None else int(lora[0]["q"][0].shape[0])
        if n_pages is None:
            n_pages = max_batch * (-(-(max_seq_len + 2 * stride) // page_size))
        if max_prefill_tokens is None:
            max_prefill_tokens = max_batch * max_seq_len
        cfg = A.Config(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                       shape.d_ffn, shape.vocab, shape.rope_base, shape.rms_eps,
                       A.ISD_BF16 if dt == "bf16" else A.ISD_F32, stride, page_size, max_batch, max_seq_len,
                       n_pages, max_prefill_tokens, lora_rank,
                       A.ISD_PROPOSE_ARGMAX if propose == "argmax" else A.ISD_PROPOSE_SAMPLE,
                       float(temperature), int(seed))
        self.cfg = cfg
        # weights (kept alive by this object)
        dev = self.device
        bf = dt == "bf16"
        # bf16 projection weights go to the library in the packed operand layout
        pk = (lambda t: pack_weight(t, self.stream).data) if bf else (lambda t: t)
        self.w = {k: to_device(weights[k], dt, dev) for k in ("embed", "final_norm")}
        self.w["lm_head"] = pk(to_device(weights["lm_head"], dt, dev))
        self.wl = [{k: pk(to_device(v, dt, dev)) if k in PACKED else to_device(v, dt, dev) for k, v in layer.items()}
                   for layer in weights["layers"]]
        self.lora = None
        if lora is not None:
            # stacked per layer: A of (q, k, v) and of (gate, up) contiguous, and likewise B, so
            # that the library runs each group's shrink (and expand) as one product
            self.lora = []
            for layer in lora:
                ent = {}
                for group in (("q", "k", "v"), ("o",), ("g", "u"), ("d",)):
                    for which in (0, 1):
                        parts = [to_device(layer[m][which], dt, dev) for m in group]
                        flat = torch.cat([pk(t).reshape(-1) for t in parts])
                        off = 0
                        for m, t in zip(group, parts):
                            view = flat[off:off + t.numel()].view(t.shape)
                            off += t.numel()
                            ent.setdefault(m, [None, None])[which] = view
                self.lora.append({m: tuple(v) for m, v in ent.items()})

        def arr(name):
            return (C.c_void_p * len(self.wl))(*[t[name].data_ptr() for t in self.wl])

        self._arrs = {n: arr(n) for n in ("attn_norm", "wqkv", "wo", "ffn_norm", "wg", "wu", "wd")}
        la = lb = None
        if self.lora is not None:
            la = (C.c_void_p * (7 * len(self.lora)))(*[l[m][0].data_ptr() for l in self.lora for m in LORA_ORDER])
            lb = (C.c_void_p * (7 * len(self.lora)))(*[l[m][1].data_ptr() for l in self.lora for m in LORA_ORDER])
        self._la, self._lb = la, lb
        cast = lambda x: C.cast(x, A.PP) if x is not None else None
        self.cw = A.Weights(self.w["embed"].data_ptr(), self.w["final_norm"].data_ptr(),
                            self.w["lm_head"].data_ptr(), *[cast(self._arrs[n]) for n in
                                                            ("attn_norm", "wqkv", "wo", "ffn_norm", "wg", "wu", "wd")],
                            cast(la), cast(lb))
        sizes = A.Sizes()
        ctx = C.c_void_p()
        A.check("isd_init(size query)", self.lib.isd_init(C.byref(cfg), C.byref(self.cw), None, None,
                                                          C.byref(sizes), C.byref(ctx), None))
        self.sizes = (sizes.kv_pool_bytes, sizes.workspace_bytes)
        self.kv_pool = torch.empty(sizes.kv_pool_bytes, dtype=torch.uint8, device=dev)
        self.workspace = torch.empty(sizes.workspace_bytes, dtype=torch.uint8, device=dev)
        A.check("isd_init", self.lib.isd_init(C.byref(cfg), C.byref(self.cw), self.kv_pool.data_ptr(),
                                              self.workspace.data_ptr(), C.byref(sizes), C.byref(ctx),
                                              self._s()))
        self.ctx = ctx
        self.tokens = torch.full((max_batch, stride), -1, dtype=torch.int32, device=dev)
        self.n_commit = torch.zeros(max_batch, dtype=torch.int32, device=dev)
        self.n_accept = torch.zeros(max_batch, dtype=torch.int32, device=dev)
        b = A.Buffers()
        A.check("isd_get_buffers", self.lib.isd_get_buffers(self.ctx, C.byref(b)))
        self._buf = b
        self._prefilled = False
        self.device_status = A.ISD_OK     # the sticky device status the last call returned
        self._multi = {}
        if graphs is not None:
            self.set_graphs(graphs)

    def _s(self):
        return C.c_void_p(self.stream.cuda_stream)

    def __del__(self):
        try:
            if getattr(self, "ctx", None) is not None and self.ctx.value:
                self.lib.isd_release(self.ctx)
                self.ctx = None
        except Exception:
            pass

    # ------------------------------------------------------------------ calls
    def _enqueued(self, where, rc):
        """A call's return: host-side errors raise; after the work was enqueued the call returns
        the context's sticky device status, kept in self.device_status."""
        if rc in A.DEVICE_STATUSES:
            self.device_status = rc
            return rc
        A.check(where, rc)
        self.device_status = rc
        return rc

    def prefill(self, slots, prompts, max_new):
        n = len(slots)
        lens = [len(p) for p in prompts]
        offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        ids = torch.from_numpy(np.concatenate([np.asarray(p, np.int32) for p in prompts])).to(self.device)
        self._prompt_ids = ids
        first = torch.empty(n, dtype=torch.int32, device=self.device)
        cs = (C.c_int32 * n)(*slots)
        co = (C.c_int32 * (n + 1))(*offs.tolist())
        cm = (C.c_int32 * n)(*max_new)
        self._enqueued("isd_prefill", self.lib.isd_prefill(self.ctx, n, cs, ids.data_ptr(), co, cm,
                                                           first.data_ptr(), self._s()))
        self._prefilled = True
        return first

    def step(self, n_active=None, debug=None):
        """One ISD pass over every slot, or over slots 0 .. n_active-1 (isd_step_active).
        debug: an isd_debug record (make_debug) filled by the pass."""
        if n_active is None:
            self._enqueued("isd_step", self.lib.isd_step(self.ctx, self.tokens.data_ptr(), self.n_commit.data_ptr(),
                                                         self.n_accept.data_ptr(),
                                                         C.byref(debug.c) if debug is not None else None, self._s()))
        else:
            assert debug is None, "isd_step_active takes no debug record"
            self._enqueued("isd_step_active", self.lib.isd_step_active(self.ctx, int(n_active), self.tokens.data_ptr(),
                                                                       self.n_commit.data_ptr(),
                                                                       self.n_accept.data_ptr(), self._s()))
        return self.tokens, self.n_commit, self.n_accept

    def step_n(self, n_passes):
        """n_passes consecutive passes (isd_step_n: one graph launch with graphs on).  Returns
        (tokens [n, B, N], n_commit [n, B], n_accept [n, B]) device tensors."""
        if n_passes not in self._multi:
            B, N, dev = self.max_batch, self.N, self.device
            self._multi[n_passes] = (torch.full((n_passes, B, N), -1, dtype=torch.int32, device=dev),
                                     torch.zeros((n_passes, B), dtype=torch.int32, device=dev),
                                     torch.zeros((n_passes, B), dtype=torch.int32, device=dev))
        t, c, a = self._multi[n_passes]
        self._enqueued("isd_step_n", self.lib.isd_step_n(self.ctx, int(n_passes), t.data_ptr(), c.data_ptr(),
                                                         a.data_ptr(), self._s()))
        return t, c, a

    def make_debug(self, rows, layers=True, decisions=True):
        """An isd_debug record following the pass rows `rows` (slot b's block row i is
        b*(2N-1)+i): per-layer inputs and attention outputs and the LM head input when
        `layers`, every slot's decision kinds and margins when `decisions`."""
        return DebugRecord(self, rows, layers, decisions)

    def status(self):
        """isd_get_status: synchronizes and returns the sticky device status."""
        return self.lib.isd_get_status(self.ctx, self._s())

    def profile(self, enable):
        A.check("isd_profile", self.lib.isd_profile(self.ctx, 1 if enable else 0))

    def set_meter(self, enable):
        """Introspective acceptance meter (isd_set_meter): pending tokens are committed untested
        and their acceptance probabilities accumulate in the slot records (meter_sum, meter_n)."""
        A.check("isd_set_meter", self.lib.isd_set_meter(self.ctx, 1 if enable else 0))

    def set_graphs(self, enable):
        """Replay isd_step from captured HIP graphs (see isd_set_graphs)."""
        A.check("isd_set_graphs", self.lib.isd_set_graphs(self.ctx, 1 if enable else 0))

    def profile_report(self):
        """{kernel name: (launches, total milliseconds)} since the last report (synchronizes)."""
        cap = 64
        arr = (A.ProfEntry * cap)()
        n = C.c_int32()
        A.check("isd_profile_report", self.lib.isd_profile_report(self.ctx, arr, cap, C.byref(n)))
        return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(min(n.value, cap))}

    # ------------------------------------------------------------------ views
    def _view(self, ptr, nbytes, dtype, shape):
        off = ptr - self.workspace.data_ptr()
        return self.workspace[off:off + nbytes].view(dtype).view(shape)

    def slots_view(self):
        return self._view(self._buf.slots, self.max_batch * A.SLOT_INTS * 4, torch.int32,
                          (self.max_batch, A.SLOT_INTS))

    def slots_host(self):
        """Per-slot state as a list of dicts (synchronizes)."""
        torch.cuda.synchronize(self.device)
        a = np.ascontiguousarray(self.slots_view().cpu().numpy())
        out = [dict(zip(A.SLOT_FIELDS, row.tolist())) for row in a]
        msum = a[:, A.METER_SUM_WORD:A.METER_SUM_WORD + 2].copy().view(np.float64)[:, 0]
        for d, m in zip(out, msum):
            d["meter_sum"] = float(m)
        return out

    def page_table(self):
        mp = self._buf.max_pages_per_slot
        return self._view(self._buf.page_table, self.max_batch * mp * 4, torch.int32, (self.max_batch, mp))

    def free_stack(self):
        n = int(self._view(self._buf.n_free, 4, torch.int32, (1,)).item())
        return self._view(self._buf.free_stack, self.cfg.n_pages * 4, torch.int32, (self.cfg.n_pages,))[:n]

    def _slot_rows(self):
        """Packed row of each slot's block row [max_batch, 2N-1] of the last pass (host int64;
        rows past a slot's live rows repeat its first row), synchronizes."""
        torch.cuda.synchronize(self.device)
        n = self.max_batch * self.R
        off = self._view(self._buf.row_off, self.max_batch * 4, torch.int32, (self.max_batch,)).cpu().numpy()
        ln = self._view(self._buf.row_len, self.max_batch * 4, torch.int32, (self.max_batch,)).cpu().numpy()
        i = np.arange(self.R)[None, :]
        idx = np.where(i < ln[:, None], off[:, None] + i, off[:, None])
        return np.clip(idx, 0, n - 1).astype(np.int64)

    def row_offsets(self):
        """First packed row of each slot's block in the last pass [max_batch] (host int array):
        a slot's q_row entries name packed rows of the pass that proposed them."""
        torch.cuda.synchronize(self.device)
        return self._view(self._buf.row_off, self.max_batch * 4, torch.int32, (self.max_batch,)).cpu().numpy()

    def logits(self):
        """Logits of the last decode pass per slot block row [max_batch, 2N-1, V] (float32; a
        copy gathered from the packed rows; rows past a slot's live rows are not meaningful)."""
        b = A.Buffers()          # the logits buffer alternates between passes: query it now
        A.check("isd_get_buffers", self.lib.isd_get_buffers(self.ctx, C.byref(b)))
        V = self.shape.vocab
        n = self.max_batch * self.R
        flat = self._view(b.logits, n * V * 4, torch.float32, (n, V))
        idx = torch.from_numpy(self._slot_rows().reshape(-1)).to(self.device)
        return flat.index_select(0, idx).view(self.max_batch, self.R, V)

    def prefill_logits(self, n):
        """Logits of the last prompt row of each slot of the last isd_prefill call [n, V]
        (valid until the next pass)."""
        b = A.Buffers()
        A.check("isd_get_buffers", self.lib.isd_get_buffers(self.ctx, C.byref(b)))
        V = self.shape.vocab
        return self._view(b.prefill_logits, n * V * 4, torch.float32, (n, V))

    def rows(self):
        """(token, position) of each slot's block rows in the last pass [max_batch, 2N-1]
        (gathered from the packed rows; -1 positions past a slot's live rows)."""
        n = self.max_batch * self.R
        idx = self._slot_rows()
        ln = self._view(self._buf.row_len, self.max_batch * 4, torch.int32, (self.max_batch,)).cpu().numpy()
        tok = self._view(self._buf.row_token, n * 4, torch.int32, (n,)).cpu().numpy()[idx]
        pos = self._view(self._buf.row_pos, n * 4, torch.int32, (n,)).cpu().numpy()[idx]
        pos = np.where(np.arange(self.R)[None, :] < ln[:, None], pos, -1)
        return torch.from_numpy(tok), torch.from_numpy(pos)

    def kv_pools(self):
        """(K, V) pools: K [L, n_pages, Hkv, P, hd], V [L, n_pages, Hkv, hd, P] (act dtype)."""
        s = self.shape
        dt = _dt(s.dtype)
        el = self.kv_pool.numel() // 2
        kp = self.kv_pool[:el].view(dt).view(s.n_layers, self.cfg.n_pages, s.n_kv_heads, self.cfg.page_size,
                                              s.head_dim)
        vp = self.kv_pool[el:].view(dt).view(s.n_layers, self.cfg.n_pages, s.n_kv_heads, s.head_dim,
                                              self.cfg.page_size)
        return kp, vp


class DebugRecord:
    """Device buffers of one isd_debug record (see isd.h) and their torch views."""

    def __init__(self, eng, rows, layers, decisions):
        s, dev = eng.shape, eng.device
        rows = [int(r) for r in rows]
        if len(rows) > A.ISD_DEBUG_MAX_ROWS:
            raise ValueError(f"at most {A.ISD_DEBUG_MAX_ROWS} rows")
        n = len(rows)
        act = _dt(s.dtype)
        qd = s.n_q_heads * s.head_dim
        self.rows = torch.tensor(rows, dtype=torch.int32, device=dev)
        self.layer_in = self.layer_attn = self.final_normed = self.margins = self.kinds = None
        if layers:
            self.layer_in = torch.zeros((s.n_layers + 1, n, s.d_model), dtype=torch.float32, device=dev)
            self.layer_attn = torch.zeros((s.n_layers, n, qd), dtype=act, device=dev)
            self.final_normed = torch.zeros((n, s.d_model), dtype=act, device=dev)
        if decisions:
            self.margins = torch.zeros((eng.max_batch, 2 * eng.N), dtype=torch.float64, device=dev)
            self.kinds = torch.zeros((eng.max_batch, 2 * eng.N), dtype=torch.int32, device=dev)
        ptr = lambda t: 0 if t is None else t.data_ptr()
        self.c = A.Debug(n, self.rows.data_ptr(), ptr(self.layer_in), ptr(self.layer_attn), ptr(self.final_normed),
                         ptr(self.margins), ptr(self.kinds))


def attn_paged(q, k_pool, v_pool, page_table, ctx_len, q_len, n_kv_heads, out=None, workspace=None, stream=None):
    """Kernel-level paged attention (see attn_paged_decode).  q [B, R, Hq, hd] bf16 on device."""
    lib = A.load()
    B, R, Hq, hd = q.shape
    P = k_pool.shape[2]
    args = A.AttnArgs(B, R, Hq, n_kv_heads, hd, P, page_table.shape[1], int(ctx_len.max().item()),
                      q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), page_table.data_ptr(),
                      ctx_len.data_ptr(), q_len.data_ptr(), 0, 0)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = torch.empty(lib.attn_paged_decode_workspace_bytes(C.byref(args)), dtype=torch.uint8,
                                device=q.device)
    args.out = out.data_ptr()
    args.workspace = workspace.data_ptr()
    stream = stream if stream is not None else torch.cuda.current_stream(q.device)
    A.check("attn_paged_decode", lib.attn_paged_decode(C.byref(args), C.c_void_p(stream.cuda_stream)))
    return out, workspace, args


GEMM_PATHS = {"auto": 0, "tiled": 1, "skinny": 2, "tiled4": 3, "tiled3": 4, "tiled2": 5}


def gemm(X, W, mode="store", W2=None, out=None, R=None, splits=0, workspace=None, stream=None,
         norm_g=None, norm_out=None, norm_eps=1e-6, path="auto"):
    """Kernel-level projection (see isd_gemm): X [M, K]; W [N, K] a PackedWeight for bf16
    (pack_weight) or a float32 device tensor.

    mode "resid" with norm_g / norm_out also writes RMSNorm(R) * norm_g into norm_out.
    path: "auto", "tiled", "skinny" (bf16 kernel choice; M <= 128 for skinny) or "tiled4",
    "tiled3", "tiled2" (the tiled kernel with that many waves per workgroup)."""
    lib = A.load()
    M, K = X.shape
    bf = X.dtype == torch.bfloat16
    if bf != isinstance(W, PackedWeight) or (W2 is not None and bf != isinstance(W2, PackedWeight)):
        raise TypeError("bf16 products take PackedWeight operands (pack_weight), float32 ones plain tensors")
    N = W.rows if bf else W.shape[0]
    modes = {"store": A.ISD_GEMM_STORE, "store_f32": A.ISD_GEMM_STORE_F32, "resid": A.ISD_GEMM_RESID,
             "swiglu": A.ISD_GEMM_SWIGLU}
    md = modes[mode]
    if out is None and md != A.ISD_GEMM_RESID:
        out = torch.empty((M, N), dtype=torch.float32 if md == A.ISD_GEMM_STORE_F32 else X.dtype, device=X.device)
    S = splits or (lib.isd_gemm_splits(N, K, 1 if md == A.ISD_GEMM_SWIGLU else 0) if bf else 1)
    if bf and S > 1 and workspace is None:
        workspace = torch.empty(S * M * N * (2 if md == A.ISD_GEMM_SWIGLU else 1), dtype=torch.float32,
                                device=X.device)
    args = A.GemmArgs(A.ISD_BF16 if bf else A.ISD_F32, md, M, N, K, splits, X.data_ptr(), W.data_ptr(),
                      0 if W2 is None else W2.data_ptr(), 0 if out is None else out.data_ptr(),
                      0 if R is None else R.data_ptr(), 0 if workspace is None else workspace.data_ptr(),
                      0 if norm_g is None else norm_g.data_ptr(), 0 if norm_out is None else norm_out.data_ptr(),
                      float(norm_eps), GEMM_PATHS[path])
    stream = stream if stream is not None else torch.cuda.current_stream(X.device)
    A.check("isd_gemm", lib.isd_gemm(C.byref(args), C.c_void_p(stream.cuda_stream)))
    return out if md != A.ISD_GEMM_RESID else R


def sample(slots, logits, q_logits, stride, temperature, propose, seed, tokens, n_commit, n_accept,
           workspace=None, stream=None, meter=False, margins=None, kinds=None):
    """Kernel-level acceptance step (see isd_sample_step).  slots: int32 [B, 32] device tensor
    (in/out); meter: the introspective acceptance meter mode (see isd_set_meter); margins
    (float64) / kinds (int32) [B, 2N]: optional decision record."""
    lib = A.load()
    B, R, V = logits.shape
    q_rows = 0 if q_logits is None else q_logits.shape[0]
    if workspace is None:
        workspace = torch.empty(lib.isd_sample_step_workspace_bytes(B, R, V, q_rows), dtype=torch.uint8,
                                device=logits.device)
    args = A.SampleArgs(B, stride, V, A.ISD_PROPOSE_ARGMAX if propose == "argmax" else A.ISD_PROPOSE_SAMPLE,
                        q_rows, float(temperature), int(seed), slots.data_ptr(), logits.data_ptr(),
                        0 if q_logits is None else q_logits.data_ptr(), tokens.data_ptr(), n_commit.data_ptr(),
                        n_accept.data_ptr(), workspace.data_ptr(), 1 if meter else 0,
                        0 if margins is None else margins.data_ptr(), 0 if kinds is None else kinds.data_ptr())
    stream = stream if stream is not None else torch.cuda.current_stream(logits.device)
    A.check("isd_sample_step", lib.isd_sample_step(C.byref(args), C.c_void_p(stream.cuda_stream)))
    return workspace
