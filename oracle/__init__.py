"""fp64 CPU oracle for the causal sparse-attention prefill.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and never calls it.

``oracle.c`` holds the definitions (pooled keys, block and token selection,
attention over the union with a sink); this module builds it with gcc,
loads it with ctypes and wraps it for numpy arrays.  ``brute.py`` is a
second, exact pure-Python version for tiny inputs used to pin this one.

Every function takes the exact input values as float32 numpy arrays in the
layouts q [Bt,Hq,N,d], k/v [Bt,Hkv,N,d], idx_q/idx_k [Bt,N,dI].  For a
decode/append step q and idx_q hold only the Nq newest positions of a
history of Nk keys (query row rq at position rq + Nk - Nq).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load(path=None):
    global _lib
    if _lib is not None and path is None:
        return _lib
    # SA_ORACLE_LIB: another build of oracle.c (the sanitizer run uses one)
    path = path or os.environ.get("SA_ORACLE_LIB") or None
    if path is None and not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(path or _LIB)
    lib.orc_block_pool.argtypes = [_f32p, _i64, _i64, _i64, _i64, _f64p]
    lib.orc_block_pool.restype = None
    lib.orc_block_minmax.argtypes = [_f32p, _i64, _i64, _i64, _i64, _f64p]
    lib.orc_block_minmax.restype = None
    lib.orc_block_scores.argtypes = [_f32p, _f64p, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                     _i64, _i64p, _i64, _f64p]
    lib.orc_block_scores.restype = None
    lib.orc_block_select.argtypes = [_f32p, _f64p, _i64, _i64, _i64, _i64, _i64, _i64,
                                     _i64, _i64, _i64, _i64p, _i64, _i32p, _f64p, _f64p]
    lib.orc_block_select.restype = None
    lib.orc_block_select_at.argtypes = [_f32p, _f64p, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                        _i64, _i64, _i64, _i64, _i64p, _i64, _i32p, _f64p, _f64p]
    lib.orc_block_select_at.restype = None
    lib.orc_token_scores.argtypes = [_f32p, _f32p, _i64, _i64, _i64p, _i64, _f64p]
    lib.orc_token_scores.restype = None
    lib.orc_token_select.argtypes = [_f32p, _f32p, _i64, _i64, _i64, _i64p, _i64,
                                     _i32p, _f64p, _f64p]
    lib.orc_token_select.restype = None
    lib.orc_attend.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, _i64, _i64,
                               ctypes.c_double, _i64, _i64,
                               ctypes.c_void_p, _i64, ctypes.c_void_p, _i64,
                               ctypes.c_void_p, _i64p, _i64, _f64p, _f64p, _i64p]
    lib.orc_attend.restype = ctypes.c_int
    lib.orc_token_scores_at.argtypes = [_f32p, _f32p, _i64, _i64, _i64, _i64, _i64p, _i64, _f64p]
    lib.orc_token_scores_at.restype = None
    lib.orc_token_select_at.argtypes = [_f32p, _f32p, _i64, _i64, _i64, _i64, _i64, _i64p, _i64,
                                        _i32p, _f64p, _f64p]
    lib.orc_token_select_at.restype = None
    lib.orc_attend_at.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, _i64, _i64, _i64, _i64,
                                  ctypes.c_double, _i64, _i64,
                                  ctypes.c_void_p, _i64, ctypes.c_void_p, _i64,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, _i64,
                                  _i64p, _i64, _f64p, _f64p, _i64p]
    lib.orc_attend_at.restype = ctypes.c_int
    lib.orc_attend_bwd.argtypes = [_f32p, _f32p, _f32p, _f32p, _i64, _i64, _i64, _i64, _i64,
                                   ctypes.c_double, _i64, _i64, ctypes.c_void_p, _i64,
                                   ctypes.c_void_p, _i64,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, _i64,
                                   _f64p, _f64p, _f64p, _f64p]
    lib.orc_attend_bwd.restype = ctypes.c_int
    lib.orc_attend_bwd_at.argtypes = [_f32p, _f32p, _f32p, _f32p, _i64, _i64, _i64, _i64, _i64,
                                      ctypes.c_double, _i64, _i64, ctypes.c_void_p, _i64,
                                      ctypes.c_void_p, _i64, ctypes.c_void_p,
                                      _i64p, _i64, _i64p, _i64, _f64p, _f64p, _f64p]
    lib.orc_attend_bwd_at.restype = ctypes.c_int
    _lib = lib
    return lib


class use_library:
    """Context manager running the wrappers on another build of oracle.c
    (the mutation tests use it to check that the pins catch planted bugs)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = None
        _load(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _rows(rows, total):
    if rows is None:
        return np.arange(total, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if len(rows) and (rows.min() < 0 or rows.max() >= total):
        raise IndexError("row id out of range")
    return rows


_REPR = {"mean": 0, "minmax": 1}


def _repr(gate_repr):
    if gate_repr not in _REPR:
        raise ValueError("gate_repr is 'mean' or 'minmax'")
    return _REPR[gate_repr]


def block_pool(k, B, gate_repr="mean"):
    """Pooled block keys, fp64: mean keys [Bt, Hkv, N/B, d], or for
    gate_repr="minmax" the per-dimension (min, max) [Bt, Hkv, N/B, 2, d]."""
    k = _f32(k)
    Bt, Hkv, N, d = k.shape
    if B <= 0 or N % B:
        raise ValueError("block size must divide N")
    if _repr(gate_repr) == 1:
        kmm = np.empty((Bt, Hkv, N // B, 2, d), dtype=np.float64)
        _load().orc_block_minmax(k, Bt * Hkv, N, d, B, kmm)
        return kmm
    kbar = np.empty((Bt, Hkv, N // B, d), dtype=np.float64)
    _load().orc_block_pool(k, Bt * Hkv, N, d, B, kbar)
    return kbar


def _gate_args(kb, gate_repr, d):
    rep = _repr(gate_repr)
    want = (2, d) if rep else (d,)
    if tuple(kb.shape[3:]) != want:
        raise ValueError("pooled keys do not match gate_repr")
    return rep


def compress(x, C):
    """Compressed keys or values: the mean of each complete group of C
    consecutive tokens, [Bt, Hkv, N // C, d] fp64 (the NSA branch's 8:1
    compression under the mean reading; the same pooling as block_pool)."""
    x = _f32(x)
    Bt, Hkv, N, d = x.shape
    if C <= 0:
        raise ValueError("group size must be positive")
    xc = np.empty((Bt, Hkv, N // C, d), dtype=np.float64)
    if N // C:
        _load().orc_block_pool(x, Bt * Hkv, N, d, C, xc)
    return xc


def block_scores(q, kb, B, rows, gate_repr="mean", shared=False, first=False):
    """Gate scores [len(rows), n]; -inf for blocks that are not candidates
    (later blocks, the own block, and block 0 when it is forced)."""
    q = _f32(q)
    Bt, Hq, N, d = q.shape
    Hkv, n = kb.shape[1], kb.shape[2]
    rep = _gate_args(kb, gate_repr, d)
    rows = _rows(rows, Bt * Hq * N)
    out = np.empty((len(rows), n), dtype=np.float64)
    _load().orc_block_scores(q, np.ascontiguousarray(kb), Hq, Hkv, N, d, B, rep, int(shared),
                             int(first), rows, len(rows), out)
    return out


def block_select(q, kb, B, top_k, rows=None, gate_repr="mean", shared=False, first=False,
                 nk=None):
    """Selected blocks per row [len(rows), top_k] (ascending, -1 padded) and the
    scores of the last kept / first dropped candidate (NaN when absent).
    shared: one selection per kv group (scores summed over its heads);
    first: block 0 always kept, taking a slot (needs top_k >= 2).
    nk: length of the history when the queries continue it (a decode step:
    row rq at position rq + nk - Nq; kb then holds its nk // B complete
    blocks); None for a prefill."""
    q = _f32(q)
    Bt, Hq, Nq, d = q.shape
    Hkv = kb.shape[1]
    rep = _gate_args(kb, gate_repr, d)
    if first and top_k < 2:
        raise ValueError("keeping the first block needs top_k >= 2")
    nk = Nq if nk is None else nk
    off = _offset(Nq, nk)
    if kb.shape[2] != nk // B:
        raise ValueError("kb must hold the history's complete blocks")
    rows = _rows(rows, Bt * Hq * Nq)
    sel = np.empty((len(rows), top_k), dtype=np.int32)
    s_last = np.empty(len(rows), dtype=np.float64)
    s_next = np.empty(len(rows), dtype=np.float64)
    _load().orc_block_select_at(q, np.ascontiguousarray(kb), Hq, Hkv, Nq, nk, d, off, B, top_k,
                                rep, int(shared), int(first), rows, len(rows), sel, s_last,
                                s_next)
    return sel, s_last, s_next


def token_scores(idx_q, idx_k, rows):
    """Indexer scores [len(rows), Nk] of token rows r = b*Nq + rq; -inf for
    keys that are not candidates (j >= position)."""
    iq, ik = _f32(idx_q), _f32(idx_k)
    Bt, Nq, dI = iq.shape
    Nk = ik.shape[1]
    rows = _rows(rows, Bt * Nq)
    out = np.empty((len(rows), Nk), dtype=np.float64)
    _load().orc_token_scores_at(iq, ik, Nq, Nk, dI, _offset(Nq, Nk), rows, len(rows), out)
    return out


def _offset(nq, nk):
    """Position of query row 0: the queries continue a history of nk keys
    (nk - nq; 0 for a prefill)."""
    if nk < nq:
        raise ValueError("fewer keys than queries")
    return nk - nq


def token_select(idx_q, idx_k, top_t, rows=None):
    """Selected tokens per token row r = b*Nq + rq: [len(rows), top_t].
    idx_q [Bt, Nq, dI], idx_k [Bt, Nk, dI]; row rq sits at position
    rq + Nk - Nq (a prefill when Nq = Nk)."""
    iq, ik = _f32(idx_q), _f32(idx_k)
    Bt, Nq, dI = iq.shape
    Nk = ik.shape[1]
    off = _offset(Nq, Nk)
    rows = _rows(rows, Bt * Nq)
    tsel = np.empty((len(rows), top_t), dtype=np.int32)
    s_last = np.empty(len(rows), dtype=np.float64)
    s_next = np.empty(len(rows), dtype=np.float64)
    _load().orc_token_select_at(iq, ik, Nq, Nk, dI, top_t, off, rows, len(rows), tsel, s_last,
                                s_next)
    return tsel, s_last, s_next


def attend(q, k, v, *, scale=None, window=0, block_size=0, sel=None, tsel=None,
           sink=None, rows=None, cmp_block=0):
    """Attention of the listed rows under a given selection.
    sel [len(rows), w] block ids and tsel [len(rows), w'] token ids are per
    listed row.  cmp_block > 0 adds the compressed columns (groups of
    cmp_block tokens, see compress) to the same softmax.  Returns out
    [len(rows), d] fp64, lse fp64, |A(i)| int64 (compressed columns
    included)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    Bt, Hq, Nq, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    off = _offset(Nq, N)
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    rows = _rows(rows, Bt * Hq * Nq)
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.empty((len(rows), d), dtype=np.float64)
    lse = np.empty(len(rows), dtype=np.float64)
    cnt = np.empty(len(rows), dtype=np.int64)
    sel_a = None if sel is None else np.ascontiguousarray(sel, dtype=np.int32)
    tsel_a = None if tsel is None else np.ascontiguousarray(tsel, dtype=np.int32)
    sink_a = None if sink is None else _f32(sink)
    for a in (sel_a, tsel_a):
        if a is not None and a.shape[0] != len(rows):
            raise ValueError("selections are per listed row")
    kc = vc = None
    if cmp_block:
        kc, vc = compress(k, cmp_block), compress(v, cmp_block)
    rc = _load().orc_attend_at(
        q, k, v, Hq, Hkv, Nq, N, d, off, scale, int(window), int(block_size),
        None if sel_a is None else sel_a.ctypes.data, 0 if sel_a is None else sel_a.shape[1],
        None if tsel_a is None else tsel_a.ctypes.data, 0 if tsel_a is None else tsel_a.shape[1],
        None if sink_a is None else sink_a.ctypes.data,
        None if kc is None else kc.ctypes.data, None if vc is None else vc.ctypes.data,
        int(cmp_block), rows, len(rows), out, lse, cnt)
    if rc != 0:
        raise ValueError("selection id out of range")
    return out, lse, cnt


def forward(q, k, v, *, block_size=0, top_k=0, window=0, idx_q=None, idx_k=None,
            token_top_k=0, sink=None, scale=None, rows=None, gate_repr="mean",
            gate_shared=False, gate_first=False, cmp_block=0):
    """The whole path for the listed rows: pool, gate, token select, attend.
    Returns a dict with out, lse, count, sel, s_last, s_next, tsel, t_last,
    t_next (selection entries are None when that gate is off).

    q [Bt, Hq, Nq, d] may be shorter than k, v [Bt, Hkv, Nk, d] (and idx_q
    than idx_k): the queries then continue the cached history, row rq at
    position rq + Nk - Nq.  Under block gating such a query is gated as the
    same position of a prefill over the history: its candidates are the
    complete blocks before its own, pooled from the cache (Nk need not be a
    multiple of the block size; the own block may be incomplete).
    gate_repr / gate_shared / gate_first pick the block gate's variant
    (see block_pool and block_select); cmp_block > 0 adds the compressed
    branch (see attend)."""
    Bt, Hq, N, d = np.shape(q)
    Nk = np.shape(k)[2]
    rows = _rows(rows, Bt * Hq * N)
    res = dict(sel=None, s_last=None, s_next=None, tsel=None, t_last=None, t_next=None)
    if top_k > 0:
        nfull = Nk // block_size * block_size
        kb = block_pool(np.asarray(k)[:, :, :nfull], block_size, gate_repr)
        res["sel"], res["s_last"], res["s_next"] = block_select(
            q, kb, block_size, top_k, rows, gate_repr, gate_shared, gate_first, nk=Nk)
    if token_top_k > 0:
        trow = (rows // (Hq * N)) * N + rows % N
        uniq, inv = np.unique(trow, return_inverse=True)
        ts, tl, tn = token_select(idx_q, idx_k, token_top_k, uniq)
        res["tsel"], res["t_last"], res["t_next"] = ts[inv], tl[inv], tn[inv]
    out, lse, cnt = attend(q, k, v, scale=scale, window=window, block_size=block_size,
                           sel=res["sel"], tsel=res["tsel"], sink=sink, rows=rows,
                           cmp_block=cmp_block)
    res.update(out=out, lse=lse, count=cnt)
    return res


def attend_bwd(q, k, v, dout, *, scale=None, window=0, block_size=0, sel=None, tsel=None,
               sink=None, cmp_block=0):
    """Gradients of sum(dout * out) for a fixed selection: window, kept
    blocks (sel [Bt*Hq*N, w] per row, or None), kept tokens (tsel [Bt*N, w']
    per position, shared by the heads, or None), sink, and with cmp_block > 0
    the compressed columns (see compress; their gradient reaches k and v
    through the group means).  Returns dq [Bt,Hq,N,d], dk, dv [Bt,Hkv,N,d]
    and dsink [Hq] (None without a sink), all fp64."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    Bt, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape[2] != N or dout.shape != q.shape:
        raise ValueError("the backward is a prefill: q, k, v, dout over the same positions")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    sel_a = None if sel is None else np.ascontiguousarray(sel, dtype=np.int32)
    if sel_a is not None and sel_a.shape[0] != Bt * Hq * N:
        raise ValueError("sel holds one row per query row")
    tsel_a = None if tsel is None else np.ascontiguousarray(tsel, dtype=np.int32)
    if tsel_a is not None and tsel_a.shape[0] != Bt * N:
        raise ValueError("tsel holds one row per position")
    sink_a = None if sink is None else _f32(sink)
    kc = vc = None
    if cmp_block:
        kc, vc = compress(k, cmp_block), compress(v, cmp_block)
    dq = np.empty((Bt, Hq, N, d), dtype=np.float64)
    dk = np.empty((Bt, Hkv, N, d), dtype=np.float64)
    dv = np.empty((Bt, Hkv, N, d), dtype=np.float64)
    dsink = np.empty(Hq, dtype=np.float64)
    rc = _load().orc_attend_bwd(
        q, k, v, dout, Bt, Hq, Hkv, N, d, scale, int(window), int(block_size),
        None if sel_a is None else sel_a.ctypes.data, 0 if sel_a is None else sel_a.shape[1],
        None if tsel_a is None else tsel_a.ctypes.data, 0 if tsel_a is None else tsel_a.shape[1],
        None if sink_a is None else sink_a.ctypes.data,
        None if kc is None else kc.ctypes.data, None if vc is None else vc.ctypes.data,
        int(cmp_block), dq, dk, dv, dsink)
    if rc != 0:
        raise ValueError("selection id out of range")
    return dq, dk, dv, (dsink if sink is not None else None)


def attend_bwd_at(q, k, v, dout, *, rows, keys, scale=None, window=0, block_size=0, sel=None,
                  tsel=None, sink=None):
    """attend_bwd at listed outputs (no compressed columns): dq of the q
    rows `rows` (flat ids (b*Hq + h)*N + i) and dk, dv of the keys `keys`
    (flat ids (b*Hkv + g)*N + j), for a fixed selection of every row (sel
    [Bt*Hq*N, w] or None, tsel [Bt*N, w'] or None).  Returns (dq
    [len(rows), d], dk [len(keys), d], dv [len(keys), d]) fp64."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    Bt, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape[2] != N or dout.shape != q.shape:
        raise ValueError("the backward is a prefill: q, k, v, dout over the same positions")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    sel_a = None if sel is None else np.ascontiguousarray(sel, dtype=np.int32)
    if sel_a is not None and sel_a.shape[0] != Bt * Hq * N:
        raise ValueError("sel holds one row per query row")
    tsel_a = None if tsel is None else np.ascontiguousarray(tsel, dtype=np.int32)
    if tsel_a is not None and tsel_a.shape[0] != Bt * N:
        raise ValueError("tsel holds one row per position")
    sink_a = None if sink is None else _f32(sink)
    rows_a = np.ascontiguousarray(rows, dtype=np.int64)
    keys_a = np.ascontiguousarray(keys, dtype=np.int64)
    dq = np.empty((len(rows_a), d), dtype=np.float64)
    dk = np.empty((len(keys_a), d), dtype=np.float64)
    dv = np.empty((len(keys_a), d), dtype=np.float64)
    rc = _load().orc_attend_bwd_at(
        q, k, v, dout, Bt, Hq, Hkv, N, d, scale, int(window), int(block_size),
        None if sel_a is None else sel_a.ctypes.data, 0 if sel_a is None else sel_a.shape[1],
        None if tsel_a is None else tsel_a.ctypes.data, 0 if tsel_a is None else tsel_a.shape[1],
        None if sink_a is None else sink_a.ctypes.data, rows_a, len(rows_a), keys_a, len(keys_a),
        dq, dk, dv)
    if rc != 0:
        raise ValueError("row, key or selection id out of range")
    return dq, dk, dv


def backward(q, k, v, dout, *, block_size=0, top_k=0, window=0, sink=None, scale=None,
             gate_repr="mean", gate_shared=False, gate_first=False, idx_q=None, idx_k=None,
             token_top_k=0, cmp_block=0):
    """Gradients of sum(dout * out) of the prefill with block gating or the
    token gate and a window, and the compressed columns when cmp_block > 0
    (the selection the forward makes, held fixed).  Returns (dq, dk, dv,
    dsink, sel), sel the block selection, or the token selection
    [Bt*N, token_top_k] under the token gate."""
    Bt, Hq, N, d = np.shape(q)
    sel = tsel = None
    if top_k > 0:
        kb = block_pool(k, block_size, gate_repr)
        sel, _, _ = block_select(q, kb, block_size, top_k, None, gate_repr, gate_shared,
                                 gate_first)
    if token_top_k > 0:
        tsel, _, _ = token_select(idx_q, idx_k, token_top_k)
    dq, dk, dv, dsink = attend_bwd(q, k, v, dout, scale=scale, window=window,
                                   block_size=block_size, sel=sel, tsel=tsel, sink=sink,
                                   cmp_block=cmp_block)
    return dq, dk, dv, dsink, (tsel if token_top_k > 0 else sel)
