"""The parity checker itself, pinned on the CPU.

Every GPU verdict goes through ``parity.check`` and ``parity.check_grads``.
Here they are fed the oracle's own results as the "device" results (which
must pass), then the same results with one planted fault each -- a swapped
block or token on a row the gap rule decides, a swap inside and one outside
the tolerance band on a near-tie row, a missing own block, a wrong count,
an output element, the output mean, an lse value, a NaN, a gradient off by
a few percent -- each of which must fail.  The near-tie rows are built by
copying one candidate's keys onto its rival's, which makes the two scores
equal exactly (gap 0) while every other score stays where it was.

The selection rule follows the benchmark statement (sets equal wherever the
k-th vs (k+1)-th gap exceeds 1e-3 relative) and the outputs its bounds
(max 1e-2, mean 1e-3, lse 1e-3); the block gate follows the MoBA page's
"블록 분할과 top-k 게이팅", the token gate the Naive page's "SWA와 DSA를
결합한 어텐션".
"""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import GAP_REL, check, check_grads, check_grads_at, grads_ok

GATE_WL = W.Workload("pc_gate", 1, 2, 1, 768, 64, "bf16", block_size=64, top_k=4, window=0,
                     block_offsets=True)
TOK_WL = W.Workload("pc_tok", 1, 2, 1, 400, 64, "bf16", window=4, token_top_k=24,
                    index_dim=64, sink=True)


def oracle_as_device(inp):
    """The oracle's whole-path results shaped like the device's."""
    wl = inp.wl
    Bt, Hq, N, d = inp.q.shape
    res = oracle.forward(inp.q, inp.k, inp.v, block_size=wl.block_size, top_k=wl.top_k,
                         window=wl.window, idx_q=inp.idx_q, idx_k=inp.idx_k,
                         token_top_k=wl.token_top_k, sink=inp.sink)
    out = res["out"].astype(np.float32).reshape(Bt, Hq, N, d)
    lse = res["lse"].astype(np.float32).reshape(Bt, Hq, N)
    bsel = None if res["sel"] is None else res["sel"].reshape(Bt, Hq, N, wl.top_k).copy()
    tsel = None
    if wl.token_top_k:
        # token selections are per (batch, position): take head 0's rows
        tsel = res["tsel"].reshape(Bt, Hq, N, wl.token_top_k)[:, 0].copy()
    return res, out, lse, bsel, tsel


def all_rows(inp):
    return np.arange(int(np.prod(inp.q.shape[:3])))


def gap(res, prefix):
    s_last, s_next = res[prefix + "_last"], res[prefix + "_next"]
    with np.errstate(invalid="ignore", divide="ignore"):
        return (s_last - s_next) / np.maximum(np.abs(s_last), np.abs(s_next))


def reevaluate(inp, out, lse, row, *, sel=None, tsel=None):
    """Write the oracle's result for one row under a given selection into the
    device-shaped out / lse (what a correct device would return for it)."""
    wl = inp.wl
    o, l_, _ = oracle.attend(inp.q, inp.k, inp.v, window=wl.window, block_size=wl.block_size,
                             sel=None if sel is None else np.asarray([sel], np.int32),
                             tsel=None if tsel is None else np.asarray([tsel], np.int32),
                             sink=inp.sink, rows=[row])
    out.reshape(-1, out.shape[-1])[row] = o[0]
    lse.reshape(-1)[row] = l_[0]


# --- block selections ---------------------------------------------------------

@pytest.fixture(scope="module")
def gate_case():
    inp = W.make_inputs(GATE_WL, 201)
    return inp, oracle_as_device(inp)


def test_clean_gate_passes(gate_case):
    inp, (res, out, lse, bsel, _) = gate_case
    rep = check(inp, out, lse, all_rows(inp), bsel)
    assert rep.ok(), str(rep)
    assert rep.mismatched == 0 and rep.invalid == 0
    assert rep.decisive > 0.9 * rep.rows
    # the sampled-row path as well
    rows = np.arange(0, rep.rows, 7)
    assert check(inp, out, lse, rows, bsel).ok()


def decisive_swap_row(res, wl):
    """A row decided by the gap rule with a kept past block and a dropped
    candidate."""
    N = wl.seq_len
    g = gap(res, "s")
    for r in np.flatnonzero(g > 10 * GAP_REL):
        own = (r % N) // wl.block_size
        kept = [c for c in res["sel"][r] if 0 <= c < own]
        dropped = [c for c in range(own) if c not in res["sel"][r]]
        if kept and dropped:
            return int(r), kept[0], dropped[0]
    raise AssertionError("no decisive row with a free slot")


def test_gate_decisive_swap_fails(gate_case):
    inp, (res, out, lse, bsel, _) = gate_case
    wl = inp.wl
    r, keep, drop = decisive_swap_row(res, wl)
    b2, o2, l2 = bsel.copy(), out.copy(), lse.copy()
    row_sel = b2.reshape(-1, wl.top_k)[r]
    row_sel[row_sel == keep] = drop
    row_sel.sort()
    # even with outputs that match the wrong selection exactly
    reevaluate(inp, o2, l2, r, sel=row_sel)
    rep = check(inp, o2, l2, all_rows(inp), b2)
    assert rep.mismatched == 1 and not rep.ok(), str(rep)


def test_gate_missing_own_block_fails(gate_case):
    inp, (res, out, lse, bsel, _) = gate_case
    wl = inp.wl
    r, _, drop = decisive_swap_row(res, wl)
    own = (r % wl.seq_len) // wl.block_size
    b2 = bsel.copy()
    row_sel = b2.reshape(-1, wl.top_k)[r]
    row_sel[row_sel == own] = drop
    row_sel.sort()
    rep = check(inp, out, lse, all_rows(inp), b2)
    assert rep.mismatched == 1 and not rep.ok(), str(rep)


@pytest.fixture(scope="module")
def gate_tie_case():
    """A row whose m-th and (m+1)-th candidate blocks score equal exactly."""
    wl = GATE_WL
    inp = W.make_inputs(wl, 202)
    N, B, m = wl.seq_len, wl.block_size, wl.top_k - 1
    kb = oracle.block_pool(inp.k, B)
    row = N - 1             # head 0, last position: 11 candidates for 3 slots
    sc = oracle.block_scores(inp.q, kb, B, [row])[0]
    order = [int(c) for c in np.argsort(-sc, kind="stable") if np.isfinite(sc[c])]
    a, b = order[m - 1], order[m]          # last kept, first dropped
    k = inp.k.copy()
    k[0, 0, b * B:(b + 1) * B] = k[0, 0, a * B:(a + 1) * B]
    tied = W.Inputs(wl, inp.q, k, inp.v, inp.sink, inp.idx_q, inp.idx_k)
    res, out, lse, bsel, _ = oracle_as_device(tied)
    assert res["s_last"][row] == res["s_next"][row]          # an exact tie at the boundary
    far = [c for c in order[m + 3:]]                           # clearly below the band
    s_far = sc[far[0]]
    delta = GAP_REL * max(abs(res["s_last"][row]), abs(res["s_next"][row]))
    assert s_far < res["s_next"][row] - delta
    return tied, res, out, lse, bsel, row, (a, b), far[0]


def test_gate_tie_swap_inside_band_passes(gate_tie_case):
    inp, res, out, lse, bsel, row, (a, b), _ = gate_tie_case
    wl = inp.wl
    sel = bsel.reshape(-1, wl.top_k)[row]
    lo, hi = min(a, b), max(a, b)
    assert lo in sel and hi not in sel                       # the oracle takes the lower id
    b2, o2, l2 = bsel.copy(), out.copy(), lse.copy()
    rs = b2.reshape(-1, wl.top_k)[row]
    rs[rs == lo] = hi
    rs.sort()
    reevaluate(inp, o2, l2, row, sel=rs)
    rep = check(inp, o2, l2, all_rows(inp), b2)
    assert rep.ok(), str(rep)
    assert rep.invalid == 0 and rep.mismatched == 0
    assert any("re-evaluated" in n for n in rep.notes)


def test_gate_tie_swap_needs_matching_outputs(gate_tie_case):
    # The swapped (valid) selection with the outputs of the oracle's own
    # selection: the re-evaluation under the device selection must see it.
    inp, res, out, lse, bsel, row, (a, b), _ = gate_tie_case
    wl = inp.wl
    lo, hi = min(a, b), max(a, b)
    b2 = bsel.copy()
    rs = b2.reshape(-1, wl.top_k)[row]
    rs[rs == lo] = hi
    rs.sort()
    # block hi holds block lo's keys but its own values: the outputs differ
    rep = check(inp, out, lse, all_rows(inp), b2)
    assert not rep.ok(), str(rep)


def test_gate_tie_swap_outside_band_fails(gate_tie_case):
    inp, res, out, lse, bsel, row, (a, b), far = gate_tie_case
    wl = inp.wl
    lo = min(a, b)
    b2, o2, l2 = bsel.copy(), out.copy(), lse.copy()
    rs = b2.reshape(-1, wl.top_k)[row]
    rs[rs == lo] = far
    rs.sort()
    reevaluate(inp, o2, l2, row, sel=rs)
    rep = check(inp, o2, l2, all_rows(inp), b2)
    assert rep.invalid == 1 and not rep.ok(), str(rep)


def test_gate_tie_missing_own_block_fails(gate_tie_case):
    inp, res, out, lse, bsel, row, (a, b), _ = gate_tie_case
    wl = inp.wl
    own = (row % wl.seq_len) // wl.block_size
    hi = max(a, b)
    b2, o2, l2 = bsel.copy(), out.copy(), lse.copy()
    rs = b2.reshape(-1, wl.top_k)[row]
    rs[rs == own] = hi
    rs.sort()
    reevaluate(inp, o2, l2, row, sel=rs)
    rep = check(inp, o2, l2, all_rows(inp), b2)
    assert rep.invalid == 1 and not rep.ok(), str(rep)


def test_gate_tie_wrong_count_fails(gate_tie_case):
    inp, res, out, lse, bsel, row, (a, b), _ = gate_tie_case
    wl = inp.wl
    lo = min(a, b)
    b2, o2, l2 = bsel.copy(), out.copy(), lse.copy()
    rs = b2.reshape(-1, wl.top_k)[row]
    rs[rs == lo] = -1
    rs[:] = np.concatenate([rs[rs >= 0], rs[rs < 0]])
    reevaluate(inp, o2, l2, row, sel=rs)
    rep = check(inp, o2, l2, all_rows(inp), b2)
    assert rep.invalid == 1 and not rep.ok(), str(rep)


# --- outputs and lse ------------------------------------------------------------

@pytest.mark.parametrize("fault", ["out_max", "out_mean", "lse", "out_nan", "lse_nan"])
def test_output_faults_fail(gate_case, fault):
    inp, (res, out, lse, bsel, _) = gate_case
    o2, l2 = out.copy(), lse.copy()
    flat = o2.reshape(-1)
    if fault == "out_max":
        flat[12345] += 1.1e-2
    elif fault == "out_mean":
        flat += np.float32(1.1e-3)
    elif fault == "lse":
        l2.reshape(-1)[777] += 1.1e-3
    elif fault == "out_nan":
        flat[4321] = np.nan
    else:
        l2.reshape(-1)[99] = np.nan
    rep = check(inp, o2, l2, all_rows(inp), bsel)
    assert not rep.ok(), f"{fault}: {rep}"


def test_output_errors_inside_bounds_pass(gate_case):
    inp, (res, out, lse, bsel, _) = gate_case
    o2, l2 = out.copy(), lse.copy()
    o2.reshape(-1)[12345] += 0.9e-2
    o2 += np.float32(0.8e-3)
    l2.reshape(-1)[777] += 0.9e-3
    rep = check(inp, o2, l2, all_rows(inp), bsel)
    assert rep.ok(), str(rep)


# --- token selections -------------------------------------------------------------

@pytest.fixture(scope="module")
def tok_case():
    inp = W.make_inputs(TOK_WL, 203)
    return inp, oracle_as_device(inp)


def test_clean_token_passes(tok_case):
    inp, (res, out, lse, _, tsel) = tok_case
    rep = check(inp, out, lse, all_rows(inp), None, tsel)
    assert rep.ok(), str(rep)
    assert rep.decisive > 0.9 * rep.rows


def test_token_decisive_swap_fails(tok_case):
    inp, (res, out, lse, _, tsel) = tok_case
    wl = inp.wl
    N = wl.seq_len
    g = gap(res, "t")
    r = next(int(r) for r in np.flatnonzero(g > 10 * GAP_REL)
             if r < N and (r % N) > wl.token_top_k + 2)
    i = r % N
    kept = [int(j) for j in res["tsel"][r] if j >= 0]
    drop = next(j for j in range(i) if j not in kept)
    t2 = tsel.copy()
    ts = t2[0, i]
    ts[ts == kept[0]] = drop
    ts.sort()
    rep = check(inp, out, lse, all_rows(inp), None, t2)
    # both heads of the position read the one token selection
    assert rep.mismatched == 2 and not rep.ok(), str(rep)


@pytest.fixture(scope="module")
def tok_tie_case():
    wl = TOK_WL
    inp = W.make_inputs(wl, 204)
    N, m = wl.seq_len, wl.token_top_k
    i = N - 1
    sc = oracle.token_scores(inp.idx_q, inp.idx_k, [i])[0]
    order = [int(j) for j in np.argsort(-sc, kind="stable") if np.isfinite(sc[j])]
    a, b = order[m - 1], order[m]
    ik = inp.idx_k.copy()
    ik[0, b] = ik[0, a]
    tied = W.Inputs(wl, inp.q, inp.k, inp.v, inp.sink, inp.idx_q, ik)
    res, out, lse, _, tsel = oracle_as_device(tied)
    assert res["t_last"][i] == res["t_next"][i]
    far = order[m + 5]
    delta = GAP_REL * max(abs(res["t_last"][i]), abs(res["t_next"][i]))
    assert sc[far] < res["t_next"][i] - delta
    return tied, res, out, lse, tsel, i, (a, b), far


def test_token_tie_swap_inside_band_passes(tok_tie_case):
    inp, res, out, lse, tsel, i, (a, b), _ = tok_tie_case
    lo, hi = min(a, b), max(a, b)
    assert lo in tsel[0, i] and hi not in tsel[0, i]
    t2, o2, l2 = tsel.copy(), out.copy(), lse.copy()
    ts = t2[0, i]
    ts[ts == lo] = hi
    ts.sort()
    for h in range(inp.wl.n_q_heads):
        reevaluate(inp, o2, l2, h * inp.wl.seq_len + i, tsel=ts)
    rep = check(inp, o2, l2, all_rows(inp), None, t2)
    assert rep.ok(), str(rep)


@pytest.mark.parametrize("fault", ["outside_band", "wrong_count"])
def test_token_tie_faults_fail(tok_tie_case, fault):
    inp, res, out, lse, tsel, i, (a, b), far = tok_tie_case
    lo = min(a, b)
    t2, o2, l2 = tsel.copy(), out.copy(), lse.copy()
    ts = t2[0, i]
    if fault == "outside_band":
        ts[ts == lo] = far
        ts.sort()
    else:
        ts[ts == lo] = -1
        ts[:] = np.concatenate([np.sort(ts[ts >= 0]), ts[ts < 0]])
    for h in range(inp.wl.n_q_heads):
        reevaluate(inp, o2, l2, h * inp.wl.seq_len + i, tsel=ts)
    rep = check(inp, o2, l2, all_rows(inp), None, t2)
    assert rep.invalid == inp.wl.n_q_heads and not rep.ok(), str(rep)


# --- gradients --------------------------------------------------------------------

@pytest.fixture(scope="module")
def grad_case():
    wl = W.Workload("pc_bwd", 1, 2, 1, 192, 64, "bf16", block_size=64, top_k=2, window=20,
                    sink=True, block_offsets=True)
    inp = W.make_inputs(wl, 205)
    dout = W._round(np.random.default_rng(206).standard_normal(inp.q.shape, dtype=np.float32),
                    "bf16")
    dq, dk, dv, ds, sel = oracle.backward(inp.q, inp.k, inp.v, dout, block_size=wl.block_size,
                                          top_k=wl.top_k, window=wl.window, sink=inp.sink)
    return inp, dout, sel, (dq, dk, dv, ds)


def test_clean_grads_pass(grad_case):
    inp, dout, sel, ref = grad_case
    res = check_grads(inp, dout, sel, [g.astype(np.float32) for g in ref], sink=inp.sink)
    assert grads_ok(res), res


@pytest.mark.parametrize("name,kind", [("dq", "max"), ("dk", "max"), ("dv", "max"),
                                       ("dsink", "max"), ("dk", "mean"), ("dv", "mean")])
def test_grad_faults_fail(grad_case, name, kind):
    inp, dout, sel, ref = grad_case
    g = [x.copy() for x in ref]
    t = ("dq", "dk", "dv", "dsink").index(name)
    x = g[t].reshape(-1)
    if kind == "max":
        j = int(np.argmax(np.abs(x)))
        x[j] += 3e-2 * np.abs(x).max()
    else:
        x *= 1 + 1.1e-2
    res = check_grads(inp, dout, sel, g, sink=inp.sink)
    assert not grads_ok(res), (name, kind, res)


@pytest.mark.parametrize("name,kind", [(None, None), ("dq", "max"), ("dk", "max"), ("dv", "max"),
                                       ("dk", "mean"), ("dv", "mean")])
def test_grad_at_listed_outputs(grad_case, name, kind):
    # the checker of sampled gradients: the oracle's own values pass, a 3e-2
    # error at the largest entry or a 1.1e-2 mean shift of one tensor fails
    inp, dout, sel, ref = grad_case
    d = inp.q.shape[-1]
    rows, keys = np.array([0, 40, 191, 250, 383]), np.array([3, 64, 100, 191])
    want = [ref[0].reshape(-1, d)[rows], ref[1].reshape(-1, d)[keys], ref[2].reshape(-1, d)[keys]]
    got = [w.astype(np.float32).astype(np.float64) for w in want]
    if name is None:
        assert grads_ok(check_grads_at(got, want))
        return
    x = got[("dq", "dk", "dv").index(name)].reshape(-1)
    if kind == "max":
        j = int(np.argmax(np.abs(x)))
        x[j] += 3e-2 * np.abs(x).max()
    else:
        x *= 1 + 1.1e-2
    assert not grads_ok(check_grads_at(got, want)), (name, kind)


def test_grad_per_tensor_floor(grad_case):
    # A tensor 1e4 times smaller than the others: under the joint floor its
    # 30% error hides below 1e-2 of the largest gradient; with its own floor
    # the same error fails, and the clean gradients still pass.
    inp, dout, sel, ref = grad_case
    g = [x.astype(np.float64).copy() for x in ref]
    r = [x.astype(np.float64).copy() for x in ref]
    for t in (0,):
        g[t] *= 1e-4
        r[t] *= 1e-4
    import parity

    def check_scaled(grads, joint):
        orig = parity.oracle.attend_bwd
        parity.oracle.attend_bwd = lambda *a, **k: tuple(r)
        try:
            return check_grads(inp, dout, sel, grads, sink=inp.sink, joint_floor=joint)
        finally:
            parity.oracle.attend_bwd = orig
    assert grads_ok(check_scaled(g, False))
    bad = [x.copy() for x in g]
    bad[0] *= 1.3
    assert grads_ok(check_scaled(bad, True))
    assert not grads_ok(check_scaled(bad, False))


def test_token_selection_only_checker(tok_case, tok_tie_case):
    from parity import check_token_selection
    inp, (res, out, lse, _, tsel) = tok_case
    N = inp.wl.seq_len
    rows = np.arange(N)
    assert check_token_selection(inp, tsel, rows).ok()
    r = next(int(r) for r in np.flatnonzero(gap(res, "t") > 10 * GAP_REL)
             if r < N and r > inp.wl.token_top_k + 2)
    kept = [int(j) for j in tsel[0, r] if j >= 0]
    t2 = tsel.copy()
    t2[0, r][t2[0, r] == kept[3]] = next(j for j in range(r) if j not in kept)
    rep = check_token_selection(inp, t2, rows)
    assert rep.mismatched == 1 and not rep.ok(), str(rep)
    # near tie: a swap inside the band passes, one outside fails
    inp, res, out, lse, tsel, i, (a, b), far = tok_tie_case
    lo, hi = min(a, b), max(a, b)
    for repl, ok in ((hi, True), (far, False)):
        t2 = tsel.copy()
        t2[0, i][t2[0, i] == lo] = repl
        rep = check_token_selection(inp, t2, rows)
        assert rep.ok() == ok and rep.invalid == (0 if ok else 1), str(rep)
