"""Parity checker: the HIP path against the fp64 oracle.

Selections
    A row's kept set is decided by the gap between the last kept candidate
    score s_last and the best dropped one s_next (oracle, fp64):
    gap_rel = (s_last - s_next) / max(|s_last|, |s_next|).
    * decisive rows (gap_rel > 1e-3, or no competition at all): the device
      set must equal the oracle set exactly;
    * other rows: the device set must be a valid tolerant top-m -- every
      kept candidate scores >= s_last - delta, every dropped one
      <= s_next + delta, delta = 1e-3 * max(|s_last|, |s_next|) -- and the
      outputs are then compared with the oracle evaluated under the device's
      own selection.
Outputs (bf16 inputs, fp32 accumulation)
    max |out - out*| <= 1e-2, mean |out - out*| <= 1e-3, max |lse - lse*| <= 1e-3.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import oracle

GAP_REL = 1e-3
OUT_MAX, OUT_MEAN, LSE_MAX = 1e-2, 1e-3, 1e-3


@dataclass
class Report:
    rows: int = 0
    decisive: int = 0
    mismatched: int = 0
    non_decisive: int = 0
    invalid: int = 0
    out_max: float = 0.0
    out_mean: float = 0.0
    lse_max: float = 0.0
    ref_out_absmax: float = 0.0
    attended_pairs: int = 0
    notes: list = field(default_factory=list)

    def ok(self) -> bool:
        return (self.mismatched == 0 and self.invalid == 0 and self.out_max <= OUT_MAX
                and self.out_mean <= OUT_MEAN and self.lse_max <= LSE_MAX)

    def __str__(self):
        return (f"rows={self.rows} decisive={self.decisive} mismatched={self.mismatched} "
                f"non_decisive={self.non_decisive} invalid={self.invalid} "
                f"out_max={self.out_max:.3e} out_mean={self.out_mean:.3e} "
                f"lse_max={self.lse_max:.3e} |out*|max={self.ref_out_absmax:.3f}")


def _gap_rel(s_last, s_next):
    with np.errstate(invalid="ignore", divide="ignore"):
        den = np.maximum(np.abs(s_last), np.abs(s_next))
        g = (s_last - s_next) / den
    # No competition (nothing kept or nothing dropped) -> decided.
    g = np.where(np.isnan(s_last) | np.isnan(s_next), np.inf, g)
    return np.where(den == 0, np.where(s_last == s_next, 0.0, np.inf), g)


def _valid_tolerant(chosen: set, scores: np.ndarray, s_last, s_next) -> bool:
    delta = GAP_REL * max(abs(s_last), abs(s_next))
    cand = np.flatnonzero(np.isfinite(scores))
    for c in cand:
        if c in chosen and scores[c] < s_last - delta:
            return False
        if c not in chosen and scores[c] > s_next + delta:
            return False
    return all(np.isfinite(scores[c]) for c in chosen)


def check(inp, dev_out, dev_lse, rows, dev_bsel=None, dev_tsel=None, *, kbar=None) -> Report:
    """Compare device outputs (numpy, full tensors) with the oracle on `rows`
    (flat ids (b*Hq + h)*N + i)."""
    wl = inp.wl
    Bt, Hq, N, d = inp.q.shape
    rows = np.asarray(rows, dtype=np.int64)
    rep = Report(rows=len(rows))
    gv = dict(gate_repr=wl.gate_repr, gate_shared=wl.gate_shared, gate_first=wl.gate_first,
              cmp_block=wl.cmp_block)
    res = oracle.forward(inp.q, inp.k, inp.v, block_size=wl.block_size, top_k=wl.top_k,
                         window=wl.window, idx_q=inp.idx_q, idx_k=inp.idx_k,
                         token_top_k=wl.token_top_k, sink=inp.sink, rows=rows, **gv)
    ref_out, ref_lse = res["out"].copy(), res["lse"].copy()
    redo = np.zeros(len(rows), dtype=bool)
    use_bsel = res["sel"]
    use_tsel = res["tsel"]

    if wl.top_k:
        gsel = dev_bsel.reshape(-1, wl.top_k)[rows]
        gap = _gap_rel(res["s_last"], res["s_next"])
        same = np.array([set(a[a >= 0]) == set(b[b >= 0]) for a, b in zip(gsel, res["sel"])])
        dec = gap > GAP_REL
        rep.decisive += int(dec.sum())
        rep.mismatched += int((dec & ~same).sum())
        nd = np.flatnonzero(~dec & ~same)
        rep.non_decisive += int((~dec).sum())
        if len(nd):
            kb = kbar if kbar is not None else oracle.block_pool(inp.k, wl.block_size,
                                                                 wl.gate_repr)
            sc = oracle.block_scores(inp.q, kb, wl.block_size, rows[nd], wl.gate_repr,
                                     wl.gate_shared, wl.gate_first)
            for t, r in enumerate(nd):
                own = (rows[r] % N) // wl.block_size
                forced = {own} | ({0} if wl.gate_first and own > 0 else set())
                got = set(gsel[r].tolist())
                chosen = {int(c) for c in got if c >= 0 and c not in forced}
                if not forced <= got or len(chosen) != len(
                        [c for c in res["sel"][r] if c >= 0]) - len(forced) or not _valid_tolerant(
                        chosen, sc[t], res["s_last"][r], res["s_next"][r]):
                    rep.invalid += 1
        redo |= ~same
        use_bsel = np.where(redo[:, None], gsel, res["sel"])
    if wl.token_top_k:
        trow = (rows // (Hq * N)) * N + rows % N
        gts = dev_tsel.reshape(-1, wl.token_top_k)[trow]
        gap = _gap_rel(res["t_last"], res["t_next"])
        same = np.array([set(a[a >= 0]) == set(b[b >= 0]) for a, b in zip(gts, res["tsel"])])
        dec = gap > GAP_REL
        rep.decisive += int(dec.sum())
        rep.mismatched += int((dec & ~same).sum())
        rep.non_decisive += int((~dec).sum())
        nd = np.flatnonzero(~dec & ~same)
        if len(nd):
            uniq = np.unique(trow[nd])
            sc = dict(zip(uniq.tolist(), oracle.token_scores(inp.idx_q, inp.idx_k, uniq)))
            for r in nd:
                chosen = {int(j) for j in gts[r] if j >= 0}
                want = len([j for j in res["tsel"][r] if j >= 0])
                if len(chosen) != want or not _valid_tolerant(
                        chosen, sc[int(trow[r])], res["t_last"][r], res["t_next"][r]):
                    rep.invalid += 1
        redo |= ~same
        use_tsel = np.where((~same)[:, None], gts, res["tsel"])
    if redo.any():
        idx = np.flatnonzero(redo)
        o2, l2, c2 = oracle.attend(
            inp.q, inp.k, inp.v, window=wl.window, block_size=wl.block_size,
            sel=None if use_bsel is None else use_bsel[idx],
            tsel=None if use_tsel is None else use_tsel[idx], sink=inp.sink, rows=rows[idx],
            cmp_block=wl.cmp_block)
        ref_out[idx], ref_lse[idx] = o2, l2
        res["count"][idx] = c2
        rep.notes.append(f"{len(idx)} rows re-evaluated under the device selection")

    got_out = dev_out.reshape(-1, d)[rows].astype(np.float64)
    got_lse = dev_lse.reshape(-1)[rows].astype(np.float64)
    err = np.abs(got_out - ref_out)
    rep.out_max = float(err.max()) if err.size else 0.0
    rep.out_mean = float(err.mean()) if err.size else 0.0
    rep.lse_max = float(np.abs(got_lse - ref_lse).max()) if len(rows) else 0.0
    rep.ref_out_absmax = float(np.abs(ref_out).max()) if err.size else 0.0
    rep.attended_pairs = int(res["count"].sum())
    return rep


def check_token_selection(inp, dev_tsel, trows) -> Report:
    """The token selection alone on token rows r = b*N + i (the selection is
    shared by every head): exact on decisive rows, a valid tolerant top-m
    elsewhere (the rule of `check`).  No outputs are compared, so rows cost
    only the oracle's indexer scores and sort (i x index_dim MACs each)."""
    wl = inp.wl
    trows = np.asarray(trows, dtype=np.int64)
    rep = Report(rows=len(trows))
    ts, t_last, t_next = oracle.token_select(inp.idx_q, inp.idx_k, wl.token_top_k, trows)
    gts = dev_tsel.reshape(-1, wl.token_top_k)[trows]
    gap = _gap_rel(t_last, t_next)
    same = np.array([set(a[a >= 0]) == set(b[b >= 0]) for a, b in zip(gts, ts)])
    dec = gap > GAP_REL
    rep.decisive = int(dec.sum())
    rep.mismatched = int((dec & ~same).sum())
    rep.non_decisive = int((~dec).sum())
    nd = np.flatnonzero(~dec & ~same)
    if len(nd):
        sc = oracle.token_scores(inp.idx_q, inp.idx_k, trows[nd])
        for t, r in enumerate(nd):
            chosen = {int(j) for j in gts[r] if j >= 0}
            want = len([j for j in ts[r] if j >= 0])
            if len(chosen) != want or not _valid_tolerant(chosen, sc[t], t_last[r], t_next[r]):
                rep.invalid += 1
    return rep


# Gradients (bf16 outputs; fp16 P and dS operands; D_i from the bf16 forward
# output): per tensor, max |g - g*| <= 2e-2 S_max and mean |g - g*| <=
# 1e-2 S_mean, S = the tensor's own max |g*| (mean |g*|), floored at 1e-2 of
# the largest of dq, dk, dv: where the softmax Jacobian cancels (a row with
# one key has dq = dk = 0 exactly) the error is judged against the call's
# gradient scale, not against zero.
GRAD_MAX, GRAD_MEAN = 2e-2, 1e-2


def check_grads(inp, dout, dev_sel, dev_grads, *, sink=None, joint_floor=True, dev_tsel=None):
    """Compare device (dq, dk, dv, dsink) with the oracle's backward under the
    device's own block selection.  Returns {name: (max_rel, mean_rel)}.
    joint_floor=False floors each tensor at 1e-2 of its own largest |g*|
    instead (inputs whose gradients differ by orders of magnitude between
    tensors, where the joint floor would leave the small ones unchecked).
    dev_tsel: the device's token selection ([Bt, N, top_t]) under the token
    gate, held fixed like the block selection."""
    wl = inp.wl
    sel = None if dev_sel is None else dev_sel.reshape(-1, wl.top_k)
    tsel = None if dev_tsel is None else dev_tsel.reshape(-1, wl.token_top_k)
    ref = oracle.attend_bwd(inp.q, inp.k, inp.v, dout, window=wl.window,
                            block_size=wl.block_size, sel=sel, tsel=tsel, sink=sink,
                            cmp_block=wl.cmp_block)
    joint_max = max(float(np.abs(r).max()) for r in ref[:3])
    joint_mean = max(float(np.abs(r).mean()) for r in ref[:3])
    res = {}
    for name, g, r in zip(("dq", "dk", "dv", "dsink"), dev_grads, ref):
        if r is None:
            continue
        g = np.asarray(g, dtype=np.float64)
        err = np.abs(g - r)
        own_max = float(np.abs(r).max())
        floor_max = 1e-2 * (joint_max if joint_floor else own_max) if name != "dsink" else 1e-30
        floor_mean = 1e-2 * (joint_mean if joint_floor else own_max) if name != "dsink" else 1e-30
        res[name] = (float(err.max() / max(np.abs(r).max(), floor_max)),
                     float(err.mean() / max(np.abs(r).mean(), floor_mean)))
    return res


def check_grads_at(dev, ref):
    """check_grads at listed outputs: dev and ref are (dq of listed rows, dk
    and dv of listed keys) as [n, d] arrays; the same relative measures, with
    the floor at 1e-2 of the largest |g*| (and of the largest mean |g*|) over
    the three.  Returns {name: (max_rel, mean_rel)}."""
    ref = [np.asarray(r, dtype=np.float64) for r in ref]
    joint_max = max(float(np.abs(r).max()) for r in ref)
    joint_mean = max(float(np.abs(r).mean()) for r in ref)
    res = {}
    for name, g, r in zip(("dq", "dk", "dv"), dev, ref):
        err = np.abs(np.asarray(g, dtype=np.float64) - r)
        res[name] = (float(err.max() / max(np.abs(r).max(), 1e-2 * joint_max)),
                     float(err.mean() / max(np.abs(r).mean(), 1e-2 * joint_mean)))
    return res


def grads_ok(res) -> bool:
    return all(m <= GRAD_MAX and a <= GRAD_MEAN for m, a in res.values())
