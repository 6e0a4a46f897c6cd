"""ctypes binding of libsparse_attn.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  torch provides device memory (outputs and
workspace) and the current HIP stream.  There is no fallback: if the shared
library is missing, importing any entry point raises.

The names mirror the C ABI of ``include/sparse_attn.h``; ``forward`` is the
convenience wrapper that allocates outputs and workspace and calls
``sparse_attn_fwd`` on torch's current stream.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
# SPARSE_ATTN_LIB: load another build of the library (e.g. a sanitizer build)
LIB_PATH = os.environ.get("SPARSE_ATTN_LIB") or os.path.join(HERE, "libsparse_attn.so")

SA_BF16, SA_F32, SA_FP8 = 0, 1, 2
SA_GATE_MEAN, SA_GATE_MINMAX = 0, 1
SA_OK = 0
ERROR_CODES = {
    -1: "SA_E_INVALID_ARG", -2: "SA_E_SHAPE", -3: "SA_E_UNSUPPORTED_HEAD_DIM",
    -4: "SA_E_NO_SELF", -5: "SA_E_ALIGNMENT", -6: "SA_E_WORKSPACE_TOO_SMALL",
    -7: "SA_E_HIP", -8: "SA_E_UNSUPPORTED", -9: "SA_E_SCRATCH_LIMIT", -10: "SA_E_CHECK",
}
# Every symbol the C header declares.
EXPORTS = ("sparse_attn_workspace_bytes", "sparse_attn_fwd", "sparse_attn_block_pool",
           "sparse_attn_strerror", "sparse_attn_set_timing", "sparse_attn_stage_times",
           "sparse_attn_bwd_workspace_bytes", "sparse_attn_bwd", "sparse_attn_fwd_noalloc",
           "sparse_attn_check_far_lists", "sparse_attn_set_checks")


class SparseAttnCfg(ctypes.Structure):
    """Mirror of ``sparse_attn_cfg``."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("window", ctypes.c_int32), ("token_top_k", ctypes.c_int32),
        ("index_dim", ctypes.c_int32),
        ("idx_q", ctypes.c_void_p), ("idx_k", ctypes.c_void_p),
        ("sink", ctypes.c_void_p), ("softmax_scale", ctypes.c_float),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("block_sel_out", ctypes.c_void_p), ("token_sel_out", ctypes.c_void_p),
        ("stream", ctypes.c_void_p),
        ("kv_len", ctypes.c_int32),
        ("gate_repr", ctypes.c_int32), ("gate_shared", ctypes.c_int32),
        ("gate_first", ctypes.c_int32), ("cmp_block", ctypes.c_int32),
        ("block_means", ctypes.c_void_p),
    ]


class SparseAttnFarLists(ctypes.Structure):
    """Mirror of ``sparse_attn_far_lists``."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("n_blocks", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("span", ctypes.c_int32), ("kslots", ctypes.c_int32), ("rows_per_chunk", ctypes.c_int32),
        ("ordered", ctypes.c_int32), ("n_chunks", ctypes.c_int32),
        ("max_entries", ctypes.c_int64), ("max_chunks", ctypes.c_int32),
        ("sel", ctypes.c_void_p), ("list_off", ctypes.c_void_p), ("list_ch", ctypes.c_void_p),
        ("chunk_list", ctypes.c_void_p), ("chunk_start", ctypes.c_void_p),
        ("entries", ctypes.c_void_p),
        ("detail", ctypes.c_char_p), ("detail_bytes", ctypes.c_size_t),
    ]


class SparseAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {ERROR_CODES.get(code, code)} ({sparse_attn_strerror(code)})")


_lib = None


def load_library():
    """Load libsparse_attn.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sliding_window_long_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.sparse_attn_workspace_bytes.argtypes = [P(SparseAttnCfg), P(ctypes.c_size_t)]
    lib.sparse_attn_workspace_bytes.restype = ctypes.c_int
    lib.sparse_attn_fwd.argtypes = [ctypes.c_void_p] * 3 + [P(SparseAttnCfg), ctypes.c_void_p,
                                                            ctypes.c_void_p]
    lib.sparse_attn_fwd.restype = ctypes.c_int
    lib.sparse_attn_fwd_noalloc.argtypes = lib.sparse_attn_fwd.argtypes
    lib.sparse_attn_fwd_noalloc.restype = ctypes.c_int
    lib.sparse_attn_block_pool.argtypes = [ctypes.c_void_p, P(SparseAttnCfg), ctypes.c_void_p]
    lib.sparse_attn_block_pool.restype = ctypes.c_int
    lib.sparse_attn_strerror.argtypes = [ctypes.c_int]
    lib.sparse_attn_strerror.restype = ctypes.c_char_p
    lib.sparse_attn_set_timing.argtypes = [ctypes.c_int]
    lib.sparse_attn_set_timing.restype = ctypes.c_int
    lib.sparse_attn_stage_times.argtypes = [P(ctypes.c_int32), P(ctypes.c_char_p),
                                            P(ctypes.c_float), ctypes.c_int32]
    lib.sparse_attn_stage_times.restype = ctypes.c_int
    lib.sparse_attn_bwd_workspace_bytes.argtypes = [P(SparseAttnCfg), P(ctypes.c_size_t)]
    lib.sparse_attn_bwd_workspace_bytes.restype = ctypes.c_int
    lib.sparse_attn_bwd.argtypes = [ctypes.c_void_p] * 6 + [P(SparseAttnCfg)] + [ctypes.c_void_p] * 4
    lib.sparse_attn_bwd.restype = ctypes.c_int
    lib.sparse_attn_check_far_lists.argtypes = [P(SparseAttnFarLists)]
    lib.sparse_attn_check_far_lists.restype = ctypes.c_int
    lib.sparse_attn_set_checks.argtypes = [ctypes.c_int]
    lib.sparse_attn_set_checks.restype = ctypes.c_int
    _lib = lib
    return lib


@dataclass
class Params:
    """Shape and method parameters of one call (see the C header)."""
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_len: int
    head_dim: int
    dtype: int = SA_BF16
    block_size: int = 0
    top_k: int = 0
    window: int = 0
    token_top_k: int = 0
    index_dim: int = 0
    softmax_scale: float = 0.0
    kv_len: int = 0           # > seq_len: decode/append step over a cached history
    gate_repr: int = SA_GATE_MEAN   # block summary: SA_GATE_MEAN or SA_GATE_MINMAX
    gate_shared: int = 0      # 1: one block selection per kv group
    gate_first: int = 0       # 1: block 0 always kept (takes a slot)
    cmp_block: int = 0        # tokens per compressed key/value; 0 = no compressed branch

    def cfg(self) -> SparseAttnCfg:
        c = SparseAttnCfg()
        c.struct_size = ctypes.sizeof(SparseAttnCfg)
        for f in ("batch", "n_q_heads", "n_kv_heads", "seq_len", "head_dim", "dtype",
                  "block_size", "top_k", "window", "token_top_k", "index_dim", "kv_len",
                  "gate_repr", "gate_shared", "gate_first", "cmp_block"):
            setattr(c, f, int(getattr(self, f)))
        c.softmax_scale = float(self.softmax_scale)
        return c


def sparse_attn_strerror(code: int) -> str:
    return load_library().sparse_attn_strerror(int(code)).decode()


def _check(rc: int, where: str):
    if rc != SA_OK:
        raise SparseAttnError(rc, where)


def sparse_attn_set_checks(enable: bool) -> None:
    """Far-list checks on every later call of this host thread (see the C
    header): the calls then synchronise their stream."""
    _check(load_library().sparse_attn_set_checks(int(bool(enable))), "sparse_attn_set_checks")


def sparse_attn_check_far_lists(*, batch, n_q_heads, n_kv_heads, seq_len, block_size, top_k,
                                span, kslots, rows_per_chunk, ordered, sel, list_off, list_ch,
                                chunk_list, chunk_start, entries, max_entries, max_chunks):
    """Check host copies of far-block lists against a selection (int32 numpy
    arrays); returns (status, message)."""
    import numpy as np
    arrs = [np.ascontiguousarray(a, dtype=np.int32) for a in
            (sel, list_off, list_ch, chunk_list, chunk_start, entries)]
    n_blocks = seq_len // block_size
    lists = batch * n_kv_heads * n_blocks
    _need(arrs[0].size == batch * n_q_heads * seq_len * top_k, "sel size")
    _need(arrs[1].size == lists + 1 and arrs[2].size == lists + 1, "list_off / list_ch size")
    _need(arrs[3].size == arrs[4].size, "chunk_list / chunk_start size")
    _need(int(arrs[1][-1]) <= arrs[5].size or int(arrs[1][-1]) < 0, "entries shorter than list_off says")
    msg = ctypes.create_string_buffer(400)
    f = SparseAttnFarLists(batch, n_q_heads, n_kv_heads, seq_len, block_size, n_blocks, top_k,
                           span, kslots, rows_per_chunk, int(bool(ordered)), arrs[3].size,
                           int(max_entries), int(max_chunks),
                           *[a.ctypes.data if a.size else None for a in arrs],
                           ctypes.cast(msg, ctypes.c_char_p), 400)
    rc = load_library().sparse_attn_check_far_lists(ctypes.byref(f))
    return rc, msg.value.decode()


def sparse_attn_workspace_bytes(cfg: SparseAttnCfg) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().sparse_attn_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)),
           "sparse_attn_workspace_bytes")
    return n.value


def sparse_attn_bwd_workspace_bytes(cfg: SparseAttnCfg) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().sparse_attn_bwd_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)),
           "sparse_attn_bwd_workspace_bytes")
    return n.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def sparse_attn_fwd(q, k, v, cfg: SparseAttnCfg, out, lse) -> None:
    _check(load_library().sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(cfg),
                                          _ptr(out), _ptr(lse)), "sparse_attn_fwd")


def sparse_attn_fwd_noalloc(q, k, v, cfg: SparseAttnCfg, out, lse) -> None:
    _check(load_library().sparse_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(cfg),
                                                  _ptr(out), _ptr(lse)), "sparse_attn_fwd_noalloc")


def sparse_attn_block_pool(k, cfg: SparseAttnCfg, kbar) -> None:
    _check(load_library().sparse_attn_block_pool(_ptr(k), ctypes.byref(cfg), _ptr(kbar)),
           "sparse_attn_block_pool")


def sparse_attn_set_timing(enable: bool) -> None:
    _check(load_library().sparse_attn_set_timing(1 if enable else 0), "sparse_attn_set_timing")


def sparse_attn_stage_times(capacity: int = 16) -> list[tuple[str, float]]:
    n = ctypes.c_int32(0)
    names = (ctypes.c_char_p * capacity)()
    ms = (ctypes.c_float * capacity)()
    _check(load_library().sparse_attn_stage_times(ctypes.byref(n), names, ms, capacity),
           "sparse_attn_stage_times")
    return [(names[i].decode(), float(ms[i])) for i in range(min(n.value, capacity))]


# ---------------------------------------------------------------------------
# torch-facing convenience wrapper
# ---------------------------------------------------------------------------
GATE_REPR = {"mean": SA_GATE_MEAN, "minmax": SA_GATE_MINMAX}


def params_for(q, k, *, block_size=0, top_k=0, window=0, token_top_k=0, index_dim=0,
               scale=None, gate_repr="mean", gate_shared=False, gate_first=False,
               cmp_block=0) -> Params:
    import torch
    Bt, Hq, N, d = q.shape
    dt = {torch.bfloat16: SA_BF16, torch.float32: SA_F32,
          torch.float8_e4m3fn: SA_FP8}.get(q.dtype)
    if dt is None:
        raise TypeError(f"q dtype {q.dtype} not supported (bfloat16, float32 or float8_e4m3fn)")
    if gate_repr not in GATE_REPR:
        raise ValueError("gate_repr is 'mean' or 'minmax'")
    Nk = k.shape[2]
    return Params(Bt, Hq, k.shape[1], N, d, dt, block_size, top_k, window, token_top_k,
                  index_dim, 0.0 if scale is None else float(scale), Nk if Nk != N else 0,
                  GATE_REPR[gate_repr], int(bool(gate_shared)), int(bool(gate_first)),
                  int(cmp_block))


class Workspace:
    """A reusable device workspace (grown on demand, never shrunk), used on
    torch's current stream of the call.  A buffer reused on a stream other
    than the one it was allocated on is recorded on that stream, so the
    caching allocator does not hand its memory out again (when the buffer
    grows) before the work queued there is done."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes: int, device):
        import torch
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        else:
            self.buf.record_stream(torch.cuda.current_stream(device))
        return self.buf


# Default workspaces, one per (device, stream).
_default_ws: dict = {}


def _workspace_for(workspace, device):
    import torch
    if workspace is not None:
        return workspace
    key = (str(device), torch.cuda.current_stream(device).cuda_stream)
    return _default_ws.setdefault(key, Workspace())


def _need(cond: bool, msg: str, exc=ValueError):
    if not cond:
        raise exc(msg)


def _check_fwd_tensors(q, k, v, idx_q, idx_k, sink, out, lse, token_top_k):
    """Shapes, dtypes, contiguity and device of every tensor the call hands
    to the library, against q (checked before any launch: a mismatch would
    make the kernels read or write past an allocation)."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t.dim() == 4, f"{name} must be 4-D [batch, heads, positions, head_dim]")
        _need(t.dtype == q.dtype, "q, k, v must share one dtype", TypeError)
        _need(t.is_contiguous(), f"{name} must be contiguous")
    Bt, Hq, N, d = q.shape
    _need(tuple(v.shape) == tuple(k.shape), "v must have k's shape")
    _need(k.shape[0] == Bt and k.shape[3] == d, "k, v must match q's batch and head_dim")
    Nk = k.shape[2]
    _need((idx_q is None) == (idx_k is None), "idx_q and idx_k go together")
    _need(token_top_k == 0 or idx_q is not None, "token_top_k needs idx_q and idx_k")
    if idx_q is not None:
        for name, t, n in (("idx_q", idx_q, N), ("idx_k", idx_k, Nk)):
            _need(t.dim() == 3 and t.shape[0] == Bt and t.shape[1] == n,
                  f"{name} must be [batch, {n}, index_dim]")
            _need(t.dtype == q.dtype, f"{name} must have q's dtype", TypeError)
            _need(t.is_contiguous(), f"{name} must be contiguous")
        _need(idx_q.shape[2] == idx_k.shape[2], "idx_q and idx_k index dims differ")
    if sink is not None:
        _need(sink.dtype == torch.float32, "sink must be float32", TypeError)
        _need(tuple(sink.shape) == (Hq,) and sink.is_contiguous(),
              "sink must be a contiguous [n_q_heads] tensor")
    out_dt = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    if out is not None:
        _need(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
        _need(out.dtype == out_dt, f"out must be {out_dt}", TypeError)
        _need(out.is_contiguous(), "out must be contiguous")
    if lse is not None:
        _need(tuple(lse.shape) == (Bt, Hq, N), "lse must be [batch, n_q_heads, positions]")
        _need(lse.dtype == torch.float32, "lse must be float32", TypeError)
        _need(lse.is_contiguous(), "lse must be contiguous")
    for name, t in (("q", q), ("k", k), ("v", v), ("idx_q", idx_q), ("idx_k", idx_k),
                    ("sink", sink), ("out", out), ("lse", lse)):
        if t is not None:
            _need(t.is_cuda and t.device == q.device, f"{name} must be on q's device ({q.device})")


def forward(q, k, v, *, block_size=0, top_k=0, window=0, idx_q=None, idx_k=None,
            token_top_k=0, sink=None, scale=None, return_selection=False,
            workspace: Workspace | None = None, out=None, lse=None, gate_repr="mean",
            gate_shared=False, gate_first=False, cmp_block=0, noalloc=False, block_means=None):
    """Causal sparse-attention prefill on q's device and torch's current
    stream.  Returns (out, lse) or, with return_selection,
    (out, lse, block_sel, token_sel).  When k, v (and idx_k) hold more
    positions than q (and idx_q), the call is a decode/append step: the
    queries are the newest positions of that history.  gate_repr ("mean" or
    "minmax"), gate_shared and gate_first select the block gate's variant;
    cmp_block > 0 adds the compressed branch (see the C header).  noalloc:
    call sparse_attn_fwd_noalloc (the library's static scratch instead of a
    workspace; out and lse are still allocated here unless given).
    block_means: for a decode step under the block gate, the fp32 means of the
    history's complete blocks [batch, n_kv_heads, kv_len // block_size, d]
    (see block_pool), used instead of pooling the cache."""
    import torch
    _check_fwd_tensors(q, k, v, idx_q, idx_k, sink, out, lse, token_top_k)
    index_dim = idx_q.shape[-1] if idx_q is not None else 0
    p = params_for(q, k, block_size=block_size, top_k=top_k, window=window,
                   token_top_k=token_top_k, index_dim=index_dim, scale=scale,
                   gate_repr=gate_repr, gate_shared=gate_shared, gate_first=gate_first,
                   cmp_block=cmp_block)
    cfg = p.cfg()
    dev = q.device
    if out is None:   # FP8 inputs give a bf16 out
        out = torch.empty(q.shape, dtype=torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype,
                          device=q.device)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    bsel = tsel = None
    if return_selection and top_k > 0:
        bsel = torch.empty(q.shape[:3] + (top_k,), dtype=torch.int32, device=dev)
        cfg.block_sel_out = bsel.data_ptr()
    if return_selection and token_top_k > 0:
        tsel = torch.empty((q.shape[0], q.shape[2], token_top_k), dtype=torch.int32, device=dev)
        cfg.token_sel_out = tsel.data_ptr()
    if idx_q is not None:
        cfg.idx_q, cfg.idx_k = idx_q.data_ptr(), idx_k.data_ptr()
    if sink is not None:
        cfg.sink = sink.data_ptr()
    if block_means is not None:
        Nk = k.shape[2]
        _need(q.shape[2] < Nk and top_k > 0, "block_means serve a decode step under the block gate")
        _need(tuple(block_means.shape) == (q.shape[0], k.shape[1], Nk // block_size, q.shape[3]),
              "block_means must be [batch, n_kv_heads, kv_len // block_size, head_dim]")
        _need(block_means.dtype == torch.float32, "block_means must be float32", TypeError)
        _need(block_means.is_contiguous() and block_means.device == q.device,
              "block_means must be contiguous on q's device")
        cfg.block_means = block_means.data_ptr()
    cfg.stream = torch.cuda.current_stream(dev).cuda_stream
    if noalloc:
        sparse_attn_fwd_noalloc(q, k, v, cfg, out, lse)
    else:
        nbytes = sparse_attn_workspace_bytes(cfg)
        ws = _workspace_for(workspace, dev).get(nbytes, dev)
        cfg.workspace = None if ws is None else ws.data_ptr()
        cfg.workspace_bytes = nbytes
        sparse_attn_fwd(q, k, v, cfg, out, lse)
    if return_selection:
        return out, lse, bsel, tsel
    return out, lse


def block_pool(k, block_size: int, gate_repr: str = "mean"):
    """The pooling stage alone, fp32: mean keys [Bt, Hkv, N/B, d], or for
    gate_repr="minmax" the per-dimension (min, max) [Bt, Hkv, N/B, 2, d]."""
    import torch
    _need(k.dim() == 4 and k.is_contiguous(), "k must be a contiguous 4-D tensor")
    _need(k.is_cuda, "k must be a device tensor")
    Bt, Hkv, N, d = k.shape
    p = params_for(k, k, block_size=block_size, top_k=1, gate_repr=gate_repr)
    cfg = p.cfg()
    cfg.stream = torch.cuda.current_stream(k.device).cuda_stream
    shape = (Bt, Hkv, N // max(block_size, 1)) + ((2, d) if gate_repr == "minmax" else (d,))
    kbar = torch.empty(shape, dtype=torch.float32, device=k.device)
    sparse_attn_block_pool(k, cfg, kbar)
    return kbar


def backward(q, k, v, out, lse, dout, *, block_size=0, top_k=0, window=0, idx_q=None,
             idx_k=None, token_top_k=0, sink=None, scale=None, gate_repr="mean",
             gate_shared=False, gate_first=False, cmp_block=0,
             workspace: Workspace | None = None):
    """Gradients of the prefill for the selection the forward makes (same
    arguments as forward, the compressed branch included; out and lse are
    its results, dout the gradient of out).  bf16 tensors on one device;
    returns (dq, dk, dv, dsink), dsink None without a sink."""
    import torch
    _need(q.dtype == torch.bfloat16, "the backward takes bfloat16 tensors", TypeError)
    _need(q.dim() == 4 and k.dim() == 4 and k.shape[2] == q.shape[2],
          "the backward is a prefill: k, v over q's positions")
    _need(tuple(dout.shape) == tuple(q.shape) and dout.dtype == q.dtype and dout.is_contiguous(),
          "dout must be a contiguous tensor of q's shape and dtype")
    _check_fwd_tensors(q, k, v, idx_q, idx_k, sink, out, lse, token_top_k)
    _need(dout.is_cuda and dout.device == q.device, "dout must be on q's device")
    index_dim = idx_q.shape[-1] if idx_q is not None else 0
    p = params_for(q, k, block_size=block_size, top_k=top_k, window=window,
                   token_top_k=token_top_k, index_dim=index_dim, scale=scale,
                   gate_repr=gate_repr, gate_shared=gate_shared, gate_first=gate_first,
                   cmp_block=cmp_block)
    cfg = p.cfg()
    dev = q.device
    if sink is not None:
        cfg.sink = sink.data_ptr()
    if idx_q is not None:
        cfg.idx_q, cfg.idx_k = idx_q.data_ptr(), idx_k.data_ptr()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dsink = None if sink is None else torch.empty_like(sink)
    nbytes = sparse_attn_bwd_workspace_bytes(cfg)
    ws = _workspace_for(workspace, dev).get(nbytes, dev)
    cfg.workspace = None if ws is None else ws.data_ptr()
    cfg.workspace_bytes = nbytes
    cfg.stream = torch.cuda.current_stream(dev).cuda_stream
    _check(load_library().sparse_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                          _ptr(dout), ctypes.byref(cfg), _ptr(dq), _ptr(dk),
                                          _ptr(dv), _ptr(dsink)), "sparse_attn_bwd")
    return dq, dk, dv, dsink
