"""Pins of the fp64 oracle against things other than itself: textbook
attention (torch SDPA in fp64), closed forms, invariants, the sparsity values
printed on the MoBA page, and an exact brute-force enumeration.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute

HERE = os.path.dirname(os.path.abspath(__file__))


def rnd(shape, seed, scale=1.0):
    return (scale * np.random.default_rng(seed).standard_normal(shape)).astype(np.float32)


def sdpa(q, k, v, mask=None, causal=False, scale=None):
    """torch SDPA in fp64 on the CPU; returns (out, lse) with lse from
    torch.logsumexp of the masked, scaled logits."""
    qt, kt, vt = (torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (q, k, v))
    d = qt.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    N = qt.shape[-2]
    if causal:
        mask = np.tril(np.ones((N, N), dtype=bool))
    m = torch.from_numpy(mask)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    logits = torch.matmul(qt, kt.transpose(-1, -2)) * scale
    logits = logits.masked_fill(~m, -math.inf)
    lse = torch.logsumexp(logits, dim=-1)
    return out.numpy(), lse.numpy()


def run(q, k, v, **kw):
    Bt, Hq, N, d = q.shape
    r = oracle.forward(q, k, v, **kw)
    return r, r["out"].reshape(Bt, Hq, N, d), r["lse"].reshape(Bt, Hq, N)


# P1: with k = n blocks kept, block gating is full causal attention (MoBA page,
# "세밀한 블록 분할과 유연한 하이브리드": MoBA is a drop-in replacement of
# full attention), for any window.
@pytest.mark.parametrize("window", [0, 1, 7, 1000])
def test_p1_all_blocks_is_dense_causal(window):
    q, k, v = rnd((1, 2, 64, 16), 1), rnd((1, 2, 64, 16), 2), rnd((1, 2, 64, 16), 3)
    _, out, lse = run(q, k, v, block_size=8, top_k=8, window=window)
    ro, rl = sdpa(q, k, v, causal=True)
    np.testing.assert_allclose(out, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)


# P2: the window alone (Bit-Axon "SWA + MoE", sliding-window mask): w >= N is
# causal; 1 <= w < N is SDPA with the mask of that page's three-line code.
@pytest.mark.parametrize("window", [1, 2, 5, 16, 63, 64, 500])
def test_p2_window_matches_sdpa_mask(window):
    N = 64
    q, k, v = rnd((2, 3, N, 8), 4), rnd((2, 3, N, 8), 5), rnd((2, 3, N, 8), 6)
    _, out, lse = run(q, k, v, window=window)
    q_pos, k_pos = np.arange(N), np.arange(N)
    causal_mask = k_pos[None, :] <= q_pos[:, None]
    window_mask = q_pos[:, None] - k_pos[None, :] < window
    ro, rl = sdpa(q, k, v, mask=causal_mask & window_mask)
    np.testing.assert_allclose(out, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)
    if window >= N:
        ro2, rl2 = sdpa(q, k, v, causal=True)
        np.testing.assert_allclose(out, ro2, atol=1e-12)


# P3: w = 1 attends to the query's own key only.
def test_p3_window_one_is_identity():
    q, k, v = rnd((1, 2, 40, 8), 7), rnd((1, 2, 40, 8), 8), rnd((1, 2, 40, 8), 9)
    r, out, lse = run(q, k, v, window=1)
    np.testing.assert_array_equal(out, v.astype(np.float64))
    x = (q.astype(np.float64) * k.astype(np.float64)).sum(-1) / math.sqrt(8)
    np.testing.assert_allclose(lse, x, atol=1e-13)
    assert (r["count"] == 1).all()


# P4: top_k = 1 keeps only the own block under a causal mask (MoBA page,
# "인과성 보존"): per-block causal attention.  With B = 1 that is out = v.
def test_p4_topk_one_is_blockwise_causal():
    B, N = 8, 48
    q, k, v = rnd((1, 2, N, 8), 10), rnd((1, 2, N, 8), 11), rnd((1, 2, N, 8), 12)
    r, out, lse = run(q, k, v, block_size=B, top_k=1)
    for c in range(N // B):
        s = slice(c * B, (c + 1) * B)
        ro, rl = sdpa(q[:, :, s], k[:, :, s], v[:, :, s], causal=True)
        np.testing.assert_allclose(out[:, :, s], ro, atol=1e-12)
        np.testing.assert_allclose(lse[:, :, s], rl, atol=1e-12)
    _, out1, _ = run(q, k, v, block_size=1, top_k=1)
    np.testing.assert_array_equal(out1, v.astype(np.float64))


# P5a: all keys equal -> all gate scores tie -> the lowest past blocks win.
def test_p5_ties_go_to_lower_block():
    B, N, top_k = 4, 40, 4
    q = rnd((1, 1, N, 8), 13)
    k = np.broadcast_to(rnd((1, 1, 1, 8), 14), (1, 1, N, 8)).copy()
    v = rnd((1, 1, N, 8), 15)
    r, _, _ = run(q, k, v, block_size=B, top_k=top_k)
    for i in range(N):
        b = i // B
        m = min(top_k - 1, b)
        want = list(range(m)) + [b] + [-1] * (top_k - 1 - m)
        assert r["sel"][i].tolist() == want, i


# P5b: block offsets growing along a direction u with <q, u> > 0 make the
# most recent blocks score highest: block gating becomes block-level SWA
# (MoBA page: sliding-window attention is MoBA whose gate keeps the latest
# blocks).
def test_p5_monotone_offsets_give_recent_blocks():
    B, N, top_k, d = 4, 64, 3, 8
    rng = np.random.default_rng(16)
    u = np.zeros(d, np.float32); u[0] = 1.0
    k = (0.01 * rng.standard_normal((1, 1, N, d))).astype(np.float32)
    for c in range(N // B):
        k[0, 0, c * B:(c + 1) * B] += c * u
    q = (0.01 * rng.standard_normal((1, 1, N, d))).astype(np.float32)
    q[..., 0] = 1.0
    v = rnd((1, 1, N, d), 17)
    r, _, _ = run(q, k, v, block_size=B, top_k=top_k)
    for i in range(N):
        b = i // B
        want = list(range(max(0, b - top_k + 1), b + 1))
        want += [-1] * (top_k - len(want))
        assert r["sel"][i].tolist() == want, i


# P6: the sparsity values printed on the MoBA page (and BORA's 16 of 32
# blocks) fix that the own block takes one of the k slots: the last query of
# a sequence attends exactly k*B keys.
def test_p6_printed_sparsity():
    cases = json.load(open(os.path.join(HERE, "golden", "moba_sparsity.json")))["cases"]
    for c in cases:
        N, B, top_k = c["N"], c["B"], c["top_k"]
        d = 2
        rng = np.random.default_rng(N + B)
        q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
        k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
        r = oracle.forward(q, k, k, block_size=B, top_k=top_k, rows=np.array([N - 1]))
        attended = int(r["count"][0])
        assert attended == top_k * B
        assert round(100.0 * (1.0 - attended / N), 2) == c["percent"], c["cite"]


# P7: exact brute force (rational gate scores, subset enumeration, pairwise
# mask clauses) on tiny inputs, over every feature combination; inputs drawn
# from a small integer set so that exact ties occur.
BRUTE_CASES = [
    dict(block_size=2, top_k=3),
    dict(block_size=4, top_k=2, window=3),
    dict(block_size=2, top_k=4, window=5, sink=True),
    dict(window=4, token_top_k=3, sink=True),
    dict(block_size=4, top_k=2, window=2, token_top_k=2),
    dict(block_size=1, top_k=5),
]


@pytest.mark.parametrize("case", range(len(BRUTE_CASES)))
@pytest.mark.parametrize("ties", [False, True])
def test_p7_brute_force(case, ties):
    kw = dict(BRUTE_CASES[case])
    use_sink = kw.pop("sink", False)
    Bt, Hq, Hkv, N, d, dI = 1, 2, 1, 16, 4, 3
    rng = np.random.default_rng(100 + case + 50 * ties)
    draw = (lambda s: rng.integers(-1, 2, size=s).astype(np.float32)) if ties else \
           (lambda s: rng.standard_normal(s).astype(np.float32))
    q, k, v = draw((Bt, Hq, N, d)), draw((Bt, Hkv, N, d)), draw((Bt, Hkv, N, d))
    iq = ik = None
    if kw.get("token_top_k"):
        iq, ik = draw((Bt, N, dI)), draw((Bt, N, dI))
    sink = rng.standard_normal(Hq).astype(np.float32) if use_sink else None
    r, out, lse = run(q, k, v, idx_q=iq, idx_k=ik, sink=sink, **kw)
    bo, bl, bsel, btsel, bcnt = brute.forward(q, k, v, idx_q=iq, idx_k=ik, sink=sink, **kw)
    np.testing.assert_allclose(out, bo, atol=1e-12)
    np.testing.assert_allclose(lse, bl, atol=1e-12)
    np.testing.assert_array_equal(r["count"].reshape(Bt, Hq, N), bcnt)
    for t, (b, h, i) in enumerate((b, h, i) for b in range(Bt) for h in range(Hq) for i in range(N)):
        if kw.get("top_k"):
            got = {c for c in r["sel"][t].tolist() if c >= 0}
            assert got == bsel[(b, h, i)], (b, h, i)
        if kw.get("token_top_k"):
            got = {j for j in r["tsel"][t].tolist() if j >= 0}
            assert got == btsel[(b, i)], (b, i)


# P8: GQA equals MHA with every kv head repeated for its query group, with
# per-head block selection.
def test_p8_gqa_is_repeated_mha():
    Bt, Hq, Hkv, N, d = 2, 6, 2, 32, 8
    q, k, v = rnd((Bt, Hq, N, d), 20), rnd((Bt, Hkv, N, d), 21), rnd((Bt, Hkv, N, d), 22)
    kw = dict(block_size=4, top_k=3, window=5)
    r1, o1, l1 = run(q, k, v, **kw)
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    r2, o2, l2 = run(q, kr, vr, **kw)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    np.testing.assert_array_equal(r1["sel"], r2["sel"])


# P9: a sink logit z with a zero value rescales the sink-free result:
# out_s = out * e^lse / (e^lse + e^z), lse_s = logaddexp(lse, z); z -> -inf
# gives the sink-free result back.
def test_p9_sink_closed_form():
    Bt, Hq, N, d = 1, 3, 48, 8
    q, k, v = rnd((Bt, Hq, N, d), 23), rnd((Bt, Hq, N, d), 24), rnd((Bt, Hq, N, d), 25)
    z = np.array([0.5, -2.0, 3.0], np.float32)
    kw = dict(block_size=8, top_k=2, window=6)
    _, o, l = run(q, k, v, **kw)
    _, os_, ls = run(q, k, v, sink=z, **kw)
    zz = z.astype(np.float64)[None, :, None]
    np.testing.assert_allclose(ls, np.logaddexp(l, zz), atol=1e-12)
    np.testing.assert_allclose(os_, o * (np.exp(l) / (np.exp(l) + np.exp(zz)))[..., None], atol=1e-12)
    _, o3, l3 = run(q, k, v, sink=np.full(Hq, -1e30, np.float32), **kw)
    np.testing.assert_allclose(o3, o, atol=1e-14)
    np.testing.assert_allclose(l3, l, atol=1e-14)


# P10: token selection (Naive-N0.5-Flash page, SWA combined with DSA):
# keeping at least i earlier tokens is dense causal; equal indexer keys keep
# the lowest token ids.
def test_p10_token_selection_cases():
    Bt, Hq, N, d, dI = 1, 2, 40, 8, 4
    q, k, v = rnd((Bt, Hq, N, d), 26), rnd((Bt, Hq, N, d), 27), rnd((Bt, Hq, N, d), 28)
    iq, ik = rnd((Bt, N, dI), 29), rnd((Bt, N, dI), 30)
    _, o, l = run(q, k, v, window=2, idx_q=iq, idx_k=ik, token_top_k=N - 1)
    ro, rl = sdpa(q, k, v, causal=True)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(l, rl, atol=1e-12)
    ik_eq = np.broadcast_to(ik[:, :1], ik.shape).copy()
    r, _, _ = run(q, k, v, window=1, idx_q=iq, idx_k=ik_eq, token_top_k=5)
    for t in range(Hq * N):
        i = t % N
        m = min(5, i)
        assert r["tsel"][t].tolist() == list(range(m)) + [-1] * (5 - m)


# P11: union idempotence.  top_k = 1 with w >= B: the own block's causal part
# is inside the window, so the union is the window alone; w = 1 lies inside
# the own block, so the union is block gating alone; w >= N is causal.
def test_p11_union_idempotence():
    Bt, Hq, N, d = 1, 2, 64, 8
    q, k, v = rnd((Bt, Hq, N, d), 31), rnd((Bt, Hq, N, d), 32), rnd((Bt, Hq, N, d), 33)
    _, o1, l1 = run(q, k, v, block_size=8, top_k=1, window=8)
    _, o2, l2 = run(q, k, v, window=8)
    np.testing.assert_array_equal(o1, o2); np.testing.assert_array_equal(l1, l2)
    _, o3, l3 = run(q, k, v, block_size=8, top_k=3, window=1)
    _, o4, l4 = run(q, k, v, block_size=8, top_k=3)
    np.testing.assert_array_equal(o3, o4); np.testing.assert_array_equal(l3, l4)
    _, o5, l5 = run(q, k, v, block_size=8, top_k=3, window=N)
    ro, rl = sdpa(q, k, v, causal=True)
    np.testing.assert_allclose(o5, ro, atol=1e-12); np.testing.assert_allclose(l5, rl, atol=1e-12)


# P12: softmax over a disjoint union equals the online-softmax merge of the
# parts (MoBA page, implementation step 5: partial results are combined with
# online softmax): window part and far-block part merged by their lse.
def test_p12_merge_of_disjoint_parts():
    Bt, Hq, N, d, B, w = 1, 2, 64, 8, 8, 6
    q, k, v = rnd((Bt, Hq, N, d), 34), rnd((Bt, Hq, N, d), 35), rnd((Bt, Hq, N, d), 36)
    rows = np.array([r for r in range(Bt * Hq * N) if (r % N) // B >= 3], dtype=np.int64)
    far = np.full((len(rows), 2), -1, np.int32)
    for t, r in enumerate(rows):
        b = (r % N) // B
        far[t] = [0, b - 2]          # both end before the window starts
    ow, lw, cw = oracle.attend(q, k, v, window=w, rows=rows)
    of, lf, cf = oracle.attend(q, k, v, block_size=B, sel=far, rows=rows)
    ou, lu, cu = oracle.attend(q, k, v, window=w, block_size=B, sel=far, rows=rows)
    assert (cu == cw + cf).all()
    lm = np.logaddexp(lw, lf)
    om = ow * np.exp(lw - lm)[:, None] + of * np.exp(lf - lm)[:, None]
    np.testing.assert_allclose(lu, lm, atol=1e-12)
    np.testing.assert_allclose(ou, om, atol=1e-12)


# P13: adding a constant to every logit of a row leaves out unchanged and
# shifts lse by that constant (done through a key component that is 1 for
# every key, which also shifts every gate score equally).
def test_p13_shift_invariance():
    Bt, Hq, N, d = 1, 2, 48, 8
    q, k, v = rnd((Bt, Hq, N, d), 37), rnd((Bt, Hq, N, d), 38), rnd((Bt, Hq, N, d), 39)
    k[..., 0] = 1.0
    q[..., 0] = 0.0
    kw = dict(block_size=8, top_k=3, window=5)
    r0, o0, l0 = run(q, k, v, **kw)
    q2 = q.copy(); q2[..., 0] = 2.0
    r1, o1, l1 = run(q2, k, v, **kw)
    np.testing.assert_array_equal(r0["sel"], r1["sel"])
    np.testing.assert_allclose(o1, o0, atol=1e-12)
    np.testing.assert_allclose(l1, l0 + 2.0 / math.sqrt(d), atol=1e-12)


# P14: permuting batches, or kv heads together with their query groups,
# permutes the outputs the same way.
def test_p14_permutation_equivariance():
    Bt, Hq, Hkv, N, d = 2, 4, 2, 32, 8
    q, k, v = rnd((Bt, Hq, N, d), 40), rnd((Bt, Hkv, N, d), 41), rnd((Bt, Hkv, N, d), 42)
    kw = dict(block_size=4, top_k=3, window=3)
    _, o, l = run(q, k, v, **kw)
    pb, pg = [1, 0], [1, 0]
    pq = [2, 3, 0, 1]
    _, o2, l2 = run(q[pb][:, pq], k[pb][:, pg], v[pb][:, pg], **kw)
    np.testing.assert_array_equal(o2, o[pb][:, pq])
    np.testing.assert_array_equal(l2, l[pb][:, pq])


# P15: a decode/append step -- Nq new queries continuing a history of Nk
# keys, query row rq at position rq + Nk - Nq (the causal offset of the
# Bit-Axon page, "슬라이딩 윈도우 마스크") -- gives exactly the last Nq rows
# of the prefill over the whole sequence (window, token gate, sink, GQA,
# full attention as a window past the sequence).
DECODE_CASES = [
    dict(window=7),
    dict(window=1000),
    dict(window=5, token_top_k=6, sink=True),
    dict(window=1, token_top_k=40),
    # block gating during decode: each new query gated as that position of
    # a prefill over the same history
    dict(block_size=4, top_k=3, window=3, sink=True),
    dict(block_size=4, top_k=2),
    dict(block_size=4, top_k=4, window=1),
    # the gate variants during decode
    dict(block_size=4, top_k=3, window=2, gate_repr="minmax"),
    dict(block_size=4, top_k=3, gate_shared=True, gate_first=True, sink=True),
]


@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
@pytest.mark.parametrize("nq", [1, 5, 64])
def test_p15_decode_is_last_prefill_rows(case, nq):
    kw = dict(DECODE_CASES[case])
    use_sink = kw.pop("sink", False)
    Bt, Hq, Hkv, Nk, d, dI = 2, 4, 2, 64, 8, 6
    q, k, v = rnd((Bt, Hq, Nk, d), 60 + case), rnd((Bt, Hkv, Nk, d), 61), rnd((Bt, Hkv, Nk, d), 62)
    iq = ik = None
    if kw.get("token_top_k"):
        iq, ik = rnd((Bt, Nk, dI), 63), rnd((Bt, Nk, dI), 64)
    sink = rnd(Hq, 65) if use_sink else None
    full = oracle.forward(q, k, v, idx_q=iq, idx_k=ik, sink=sink, **kw)
    off = Nk - nq
    dec = oracle.forward(np.ascontiguousarray(q[:, :, off:]), k, v,
                         idx_q=None if iq is None else np.ascontiguousarray(iq[:, off:]),
                         idx_k=ik, sink=sink, **kw)
    last = np.array([(bh * Nk + off + r) for bh in range(Bt * Hq) for r in range(nq)])
    np.testing.assert_array_equal(dec["out"], full["out"][last])
    np.testing.assert_array_equal(dec["lse"], full["lse"][last])
    np.testing.assert_array_equal(dec["count"], full["count"][last])
    if kw.get("token_top_k"):
        np.testing.assert_array_equal(dec["tsel"], full["tsel"][last])
    if kw.get("top_k"):
        np.testing.assert_array_equal(dec["sel"], full["sel"][last])


# P16: the decode step against the exact brute force, which places the
# queries by its own reading of the offset.
@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
@pytest.mark.parametrize("ties", [False, True])
def test_p16_decode_brute_force(case, ties):
    kw = dict(DECODE_CASES[case])
    use_sink = kw.pop("sink", False)
    Bt, Hq, Hkv, Nq, Nk, d, dI = 1, 2, 1, 3, 16, 4, 3
    kw["window"] = min(kw.get("window", 0), 20)
    kw["token_top_k"] = min(kw.get("token_top_k", 0), 9)
    rng = np.random.default_rng(200 + case + 50 * ties)
    draw = (lambda s: rng.integers(-1, 2, size=s).astype(np.float32)) if ties else \
           (lambda s: rng.standard_normal(s).astype(np.float32))
    q, k, v = draw((Bt, Hq, Nq, d)), draw((Bt, Hkv, Nk, d)), draw((Bt, Hkv, Nk, d))
    iq = ik = None
    if kw["token_top_k"]:
        iq, ik = draw((Bt, Nq, dI)), draw((Bt, Nk, dI))
    sink = rng.standard_normal(Hq).astype(np.float32) if use_sink else None
    r = oracle.forward(q, k, v, idx_q=iq, idx_k=ik, sink=sink, **kw)
    bo, bl, _, btsel, bcnt = brute.forward(q, k, v, idx_q=iq, idx_k=ik, sink=sink, **kw)
    np.testing.assert_allclose(r["out"].reshape(bo.shape), bo, atol=1e-12)
    np.testing.assert_allclose(r["lse"].reshape(bl.shape), bl, atol=1e-12)
    np.testing.assert_array_equal(r["count"].reshape(bcnt.shape), bcnt)
    if kw["token_top_k"]:
        for t, (b, h, iqr) in enumerate((b, h, i) for b in range(Bt) for h in range(Hq)
                                        for i in range(Nq)):
            assert {j for j in r["tsel"][t].tolist() if j >= 0} == btsel[(b, iqr)]


# ---------------------------------------------------------------------------
# Gate variants (MoBA summary page: the related-work remark casting attention
# sinks, Quest and LongHeads as MoBA with other gates; BORA page: block
# selection in GQA layers).
# ---------------------------------------------------------------------------

# P17: min/max blocks of one key are that key: the min/max score is then the
# plain dot product q . k_c, and the selection is the mean gate's (B = 1).
def test_p17_minmax_block_of_one_is_dot_product():
    Bt, Hq, Hkv, N, d = 1, 4, 2, 24, 8
    q, k = rnd((Bt, Hq, N, d), 300), rnd((Bt, Hkv, N, d), 301)
    kmm = oracle.block_pool(k, 1, "minmax")
    np.testing.assert_array_equal(kmm[:, :, :, 0], k.astype(np.float64))
    np.testing.assert_array_equal(kmm[:, :, :, 1], k.astype(np.float64))
    rows = np.arange(Bt * Hq * N)
    sc = oracle.block_scores(q, kmm, 1, rows, "minmax")
    kv = np.repeat(k.astype(np.float64), Hq // Hkv, axis=1)          # [Bt, Hq, N, d]
    dots = np.einsum("bhid,bhjd->bhij", q.astype(np.float64), kv).reshape(-1, N)
    i = rows % N
    for t in range(len(rows)):
        np.testing.assert_allclose(sc[t, :i[t]], dots[t, :i[t]], rtol=1e-13, atol=1e-13)
        assert np.isneginf(sc[t, i[t]:]).all()
    s_mm, _, _ = oracle.block_select(q, kmm, 1, 5, None, "minmax")
    s_mean, _, _ = oracle.block_select(q, oracle.block_pool(k, 1), 1, 5)
    np.testing.assert_array_equal(s_mm, s_mean)


# P18: the min/max score bounds every key of the block from above, is the
# maximum over the corners of the block's box (enumerated), is at least the
# mean key's score, and equals the key score when the block's keys agree.
def test_p18_minmax_bounds_and_box_corners():
    Bt, Hq, Hkv, N, d, B = 1, 2, 1, 32, 5, 4
    q, k = rnd((Bt, Hq, N, d), 302), rnd((Bt, Hkv, N, d), 303)
    k[:, :, 8:12] = k[:, :, 8:9]                # block 2: four equal keys
    kmm = oracle.block_pool(k, B, "minmax")
    kbar = oracle.block_pool(k, B)
    rows = np.arange(Bt * Hq * N)
    sc = oracle.block_scores(q, kmm, B, rows, "minmax")
    sm = oracle.block_scores(q, kbar, B, rows)
    q64, k64 = q.astype(np.float64), k.astype(np.float64)
    blocks = k64.reshape(Bt, Hkv, N // B, B, d)
    lo, hi = kmm[:, :, :, 0][:, :, :, None], kmm[:, :, :, 1][:, :, :, None]
    assert ((lo <= blocks) & (blocks <= hi)).all()             # the box holds every key
    assert ((blocks == lo).any(axis=3) & (blocks == hi).any(axis=3)).all()   # and is tight
    corners = np.array(list(__import__("itertools").product((0, 1), repeat=d)))
    for t, r in enumerate(rows):
        h, i = r // N, r % N
        for c in range(i // B):
            keys = k64[0, 0, c * B:(c + 1) * B]
            qv = q64[0, h, i]
            assert sc[t, c] >= (keys @ qv).max() - 1e-12
            assert sc[t, c] >= sm[t, c] - 1e-12
            box = np.where(corners == 1, kmm[0, 0, c, 1], kmm[0, 0, c, 0])  # [2^d, d]
            np.testing.assert_allclose(sc[t, c], (box @ qv).max(), rtol=1e-13, atol=1e-13)
            if c == 2:
                np.testing.assert_allclose(sc[t, c], keys[0] @ qv, rtol=1e-13, atol=1e-13)


# P19: with one query head per kv head, sharing the selection across the
# group changes nothing.
@pytest.mark.parametrize("gate_repr", ["mean", "minmax"])
def test_p19_shared_with_one_head_per_group(gate_repr):
    q, k = rnd((2, 3, 48, 8), 304), rnd((2, 3, 48, 8), 305)
    kb = oracle.block_pool(k, 4, gate_repr)
    a, _, _ = oracle.block_select(q, kb, 4, 4, None, gate_repr, False)
    b, _, _ = oracle.block_select(q, kb, 4, 4, None, gate_repr, True)
    np.testing.assert_array_equal(a, b)


# P20: for mean blocks, the group's shared selection is the per-head
# selection of the group's summed query (sum_h <q_h, kbar> = <sum_h q_h,
# kbar>); inputs on a coarse grid so the fp32 sums are exact.  Every head of
# a group keeps the same blocks.
def test_p20_shared_is_summed_query():
    Bt, Hq, Hkv, N, d, B = 2, 8, 2, 64, 8, 4
    rng = np.random.default_rng(306)
    q = (rng.integers(-8, 9, size=(Bt, Hq, N, d)) / 4).astype(np.float32)
    k = rnd((Bt, Hkv, N, d), 307)
    G = Hq // Hkv
    qs = q.reshape(Bt, Hkv, G, N, d).sum(axis=2, dtype=np.float32)
    q2 = np.repeat(qs, G, axis=1)                                     # [Bt, Hq, N, d]
    kb = oracle.block_pool(k, B)
    shared, _, _ = oracle.block_select(q, kb, B, 5, None, "mean", True)
    per_head, _, _ = oracle.block_select(q2, kb, B, 5)
    np.testing.assert_array_equal(shared, per_head)
    sel = shared.reshape(Bt, Hkv, G, N, 5)
    assert (sel == sel[:, :, :1]).all()


# P21: always keeping the first block with top_k = 2 is the static
# attention-sink pattern the MoBA page describes: every query attends to
# block 0 and to its own block (causally), nothing else.
@pytest.mark.parametrize("gate_repr", ["mean", "minmax"])
def test_p21_first_block_top2_is_sink_pattern(gate_repr):
    B, N = 4, 40
    q, k, v = rnd((1, 2, N, 8), 308), rnd((1, 2, N, 8), 309), rnd((1, 2, N, 8), 310)
    r, out, lse = run(q, k, v, block_size=B, top_k=2, gate_repr=gate_repr, gate_first=True)
    pos = np.arange(N)
    mask = (pos[None, :] <= pos[:, None]) & ((pos[None, :] < B) |
                                              (pos[None, :] // B == pos[:, None] // B))
    ro, rl = sdpa(q, k, v, mask=mask)
    np.testing.assert_allclose(out, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)


# P22: for queries past block 0, keeping block 0 leaves the ordinary gate,
# with one slot less, on the history without block 0 (the other blocks'
# pooled keys and scores do not depend on it; block ids shift by one).
@pytest.mark.parametrize("gate_repr", ["mean", "minmax"])
def test_p22_first_block_is_gate_on_shifted_history(gate_repr):
    Bt, Hq, Hkv, N, d, B, K = 1, 4, 2, 64, 8, 4, 5
    q, k = rnd((Bt, Hq, N, d), 311), rnd((Bt, Hkv, N, d), 312)
    rows = np.array([(h * N + i) for h in range(Hq) for i in range(B, N)])
    first, _, _ = oracle.block_select(q, oracle.block_pool(k, B, gate_repr), B, K, rows,
                                      gate_repr, False, True)
    qs, ks = np.ascontiguousarray(q[:, :, B:]), np.ascontiguousarray(k[:, :, B:])
    rows_s = np.array([(h * (N - B) + i - B) for h in range(Hq) for i in range(B, N)])
    plain, _, _ = oracle.block_select(qs, oracle.block_pool(ks, B, gate_repr), B, K - 1,
                                      rows_s, gate_repr)
    for a, b in zip(first, plain):
        got = sorted(c for c in a.tolist() if c >= 0)
        want = [0] + sorted(c + 1 for c in b.tolist() if c >= 0)
        assert got == want


# P23: exact brute force (rational scores, box corners, subset enumeration)
# over the gate variants and their combinations, with and without ties.
VARIANT_CASES = [
    dict(block_size=2, top_k=3, gate_repr="minmax"),
    dict(block_size=4, top_k=2, window=3, gate_shared=True),
    dict(block_size=2, top_k=3, gate_first=True, sink=True),
    dict(block_size=2, top_k=4, window=2, gate_repr="minmax", gate_shared=True, gate_first=True),
    dict(block_size=1, top_k=3, gate_repr="minmax", gate_shared=True),
]


@pytest.mark.parametrize("case", range(len(VARIANT_CASES)))
@pytest.mark.parametrize("ties", [False, True])
def test_p23_variants_brute_force(case, ties):
    kw = dict(VARIANT_CASES[case])
    use_sink = kw.pop("sink", False)
    Bt, Hq, Hkv, N, d = 1, 4, 2, 12, 3
    rng = np.random.default_rng(400 + case + 50 * ties)
    draw = (lambda s: rng.integers(-1, 2, size=s).astype(np.float32)) if ties else \
           (lambda s: rng.standard_normal(s).astype(np.float32))
    q, k, v = draw((Bt, Hq, N, d)), draw((Bt, Hkv, N, d)), draw((Bt, Hkv, N, d))
    sink = rng.standard_normal(Hq).astype(np.float32) if use_sink else None
    r, out, lse = run(q, k, v, sink=sink, **kw)
    bo, bl, bsel, _, bcnt = brute.forward(q, k, v, sink=sink, **kw)
    np.testing.assert_allclose(out, bo, atol=1e-12)
    np.testing.assert_allclose(lse, bl, atol=1e-12)
    np.testing.assert_array_equal(r["count"].reshape(Bt, Hq, N), bcnt)
    for t, (h, i) in enumerate((h, i) for h in range(Hq) for i in range(N)):
        assert {c for c in r["sel"][t].tolist() if c >= 0} == bsel[(0, h, i)], (h, i)


# ---------------------------------------------------------------------------
# Compressed branch (BORA model card, NSA: 8 tokens -> one compressed key and
# value, next to block selection and the sliding window).
# ---------------------------------------------------------------------------

# P24: groups of one token are the tokens themselves: every causal key then
# appears once more as a compressed column, so window keys count twice --
# SDPA with an additive log 2 on the window and 0 on the other causal keys.
def test_p24_groups_of_one_double_the_causal_keys():
    N, w = 48, 5
    q, k, v = rnd((1, 3, N, 8), 320), rnd((1, 3, N, 8), 321), rnd((1, 3, N, 8), 322)
    r, out, lse = run(q, k, v, window=w, cmp_block=1)
    pos = np.arange(N)
    causal = pos[None, :] <= pos[:, None]
    bias = np.where(causal, np.where(pos[:, None] - pos[None, :] < w, math.log(2.0), 0.0), -np.inf)
    qt, kt, vt = (torch.from_numpy(a.astype(np.float64)) for a in (q, k, v))
    bt = torch.from_numpy(bias)
    ro = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=bt,
                                                          scale=1 / math.sqrt(8))
    logits = torch.matmul(qt, kt.transpose(-1, -2)) / math.sqrt(8) + bt
    np.testing.assert_allclose(out, ro.numpy(), atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, -1).numpy(), atol=1e-12)
    assert (r["count"].reshape(3, N) == np.minimum(pos + 1, w) + pos + 1).all()


# P25: the compressed columns alone are SDPA over the group means (torch
# reductions) with the group-causal mask (c+1)C - 1 <= i; group size 8 as
# on the BORA card, N not a multiple of it (the last partial group is never
# seen).
def test_p25_compressed_columns_are_group_mean_attention():
    N, C = 70, 8
    q, k, v = rnd((2, 4, N, 8), 323), rnd((2, 2, N, 8), 324), rnd((2, 2, N, 8), 325)
    kc = torch.from_numpy(k[:, :, :N // C * C].astype(np.float64)).reshape(2, 2, N // C, C, 8).mean(3)
    vc = torch.from_numpy(v[:, :, :N // C * C].astype(np.float64)).reshape(2, 2, N // C, C, 8).mean(3)
    np.testing.assert_allclose(oracle.compress(k, C), kc.numpy(), atol=1e-15)
    kcr, vcr = kc.repeat_interleave(2, dim=1), vc.repeat_interleave(2, dim=1)   # GQA 4/2
    pos, grp = np.arange(N), np.arange(N // C)
    mask = (grp[None, :] + 1) * C - 1 <= pos[:, None]
    rows = np.array([(b * 4 + h) * N + i for b in range(2) for h in range(4) for i in range(C - 1, N)])
    o, l, cnt = oracle.attend(q, k, v, cmp_block=C, rows=rows)
    qt = torch.from_numpy(q.astype(np.float64))
    ro = torch.nn.functional.scaled_dot_product_attention(qt, kcr, vcr, attn_mask=torch.from_numpy(mask))
    i = rows % N
    np.testing.assert_allclose(o, ro.numpy().reshape(-1, N, 8)[np.arange(len(rows)) // (N - C + 1), i],
                               atol=1e-12)
    np.testing.assert_array_equal(cnt, (i + 1) // C)


# P26: one softmax over the union: merging the window-only and the
# compressed-only results by their lse gives the joint result (the rule the
# GPU uses to combine the two kernels' outputs).
def test_p26_union_merges_by_lse():
    N, C, w = 64, 8, 6
    q, k, v = rnd((1, 2, N, 16), 326), rnd((1, 2, N, 16), 327), rnd((1, 2, N, 16), 328)
    sink = rnd((2,), 329)
    rows = np.arange(2 * N)
    o, l, _ = oracle.attend(q, k, v, window=w, cmp_block=C, sink=sink, rows=rows)
    ow, lw, _ = oracle.attend(q, k, v, window=w, sink=sink, rows=rows)
    oc, lc, _ = oracle.attend(q, k, v, cmp_block=C, rows=rows)
    lm = np.logaddexp(lw, lc)
    np.testing.assert_allclose(l, lm, atol=1e-12)
    wc = np.where(np.isneginf(lc), 0.0, np.exp(lc - lm))
    np.testing.assert_allclose(o, ow * np.exp(lw - lm)[:, None] + np.nan_to_num(oc) * wc[:, None],
                               atol=1e-12)


# P27: exact brute force with the compressed branch, alone with a window and
# together with block gating and its variants, with and without ties.
CMP_CASES = [
    dict(window=3, cmp_block=4),
    dict(window=1, cmp_block=5, sink=True),
    dict(block_size=4, top_k=2, cmp_block=2),
    dict(block_size=2, top_k=3, window=2, cmp_block=3, gate_first=True, gate_repr="minmax"),
]


@pytest.mark.parametrize("case", range(len(CMP_CASES)))
@pytest.mark.parametrize("ties", [False, True])
def test_p27_compressed_brute_force(case, ties):
    kw = dict(CMP_CASES[case])
    use_sink = kw.pop("sink", False)
    Bt, Hq, Hkv, N, d = 1, 4, 2, 13, 3
    rng = np.random.default_rng(500 + case + 50 * ties)
    draw = (lambda s: rng.integers(-1, 2, size=s).astype(np.float32)) if ties else \
           (lambda s: rng.standard_normal(s).astype(np.float32))
    q, k, v = draw((Bt, Hq, N, d)), draw((Bt, Hkv, N, d)), draw((Bt, Hkv, N, d))
    if "block_size" in kw:   # block gating needs whole blocks
        N2 = N // kw["block_size"] * kw["block_size"]
        q, k, v = (np.ascontiguousarray(a[:, :, :N2]) for a in (q, k, v))
        N = N2
    sink = rng.standard_normal(Hq).astype(np.float32) if use_sink else None
    r, out, lse = run(q, k, v, sink=sink, **kw)
    bo, bl, bsel, _, bcnt = brute.forward(q, k, v, sink=sink, **kw)
    np.testing.assert_allclose(out, bo, atol=1e-12)
    np.testing.assert_allclose(lse, bl, atol=1e-12)
    np.testing.assert_array_equal(r["count"].reshape(Bt, Hq, N), bcnt)


# ---------------------------------------------------------------------------
# Backward for a fixed selection (MoBA trains through the attention of the
# chosen blocks; the top-k choice itself has no gradient).
# ---------------------------------------------------------------------------
def torch_dense_grads(q, k, v, dout, sel, B, window, sink, tsel=None, cmp_block=0):
    """Autograd (fp64, CPU) of sum(dout * out) for the dense attention with
    the boolean mask of window | kept blocks | kept tokens (tsel per
    position, shared by the heads) and the sink as an extra column of zero
    value.  cmp_block = C > 0 adds the compressed columns: torch means of
    each complete group of C keys and values (taken from the leaf tensors,
    so autograd carries their gradient back through the mean), group c
    visible to row i iff (c+1)C - 1 <= i."""
    Bt, Hq, N, d = q.shape
    Hkv = k.shape[1]
    pos = np.arange(N)
    causal = pos[None, :] <= pos[:, None]
    mask = np.zeros((Bt, Hq, N, N), dtype=bool)
    if window:
        mask |= (causal & (pos[:, None] - pos[None, :] < window))[None, None]
    if sel is not None:
        s3 = sel.reshape(Bt, Hq, N, -1)
        blk = pos // B
        for b in range(Bt):
            for h in range(Hq):
                for i in range(N):
                    kept = set(int(c) for c in s3[b, h, i] if c >= 0)
                    mask[b, h, i] |= np.isin(blk, list(kept)) & (pos <= i)
    if tsel is not None:
        t3 = tsel.reshape(Bt, N, -1)
        for b in range(Bt):
            for i in range(N):
                for j in t3[b, i]:
                    if 0 <= j <= i:
                        mask[b, :, i, j] = True
    qt, kt, vt = (torch.tensor(a.astype(np.float64), requires_grad=True) for a in (q, k, v))
    zt = torch.tensor(sink.astype(np.float64), requires_grad=True) if sink is not None else None
    G = Hq // Hkv
    kr, vr = kt.repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1)
    logits = torch.matmul(qt, kr.transpose(-1, -2)) / math.sqrt(d)
    logits = logits.masked_fill(~torch.from_numpy(mask), -math.inf)
    cols, vals = [logits], [vr]
    if cmp_block:
        C = cmp_block
        Nc = N // C
        kc = kt[:, :, :Nc * C].reshape(Bt, Hkv, Nc, C, d).mean(dim=3)
        vc = vt[:, :, :Nc * C].reshape(Bt, Hkv, Nc, C, d).mean(dim=3)
        lc = torch.matmul(qt, kc.repeat_interleave(G, dim=1).transpose(-1, -2)) / math.sqrt(d)
        vis = (np.arange(Nc)[None, :] + 1) * C - 1 <= pos[:, None]
        cols.append(lc.masked_fill(~torch.from_numpy(vis), -math.inf))
        vals.append(vc.repeat_interleave(G, dim=1))
    if zt is not None:
        cols.append(zt.view(1, Hq, 1, 1).expand(Bt, Hq, N, 1))
    p = torch.softmax(torch.cat(cols, dim=-1), dim=-1)
    out, at = 0, 0
    for val in vals:
        out = out + torch.matmul(p[..., at:at + val.shape[2]], val)
        at += val.shape[2]
    (out * torch.from_numpy(dout.astype(np.float64))).sum().backward()
    return (qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(),
            None if zt is None else zt.grad.numpy())


BWD_CASES = [
    dict(window=5),
    dict(block_size=4, top_k=3, sink=True),
    dict(block_size=4, top_k=2, window=3, sink=True),
    dict(block_size=2, top_k=4, window=2, gate_repr="minmax", gate_first=True),
]


# P28: the backward equals autograd of the dense masked attention (window |
# kept blocks, sink column), GQA 4/2.
@pytest.mark.parametrize("case", range(len(BWD_CASES)))
def test_p28_backward_is_autograd(case):
    kw = dict(BWD_CASES[case])
    use_sink = kw.pop("sink", False)
    Bt, Hq, Hkv, N, d = 2, 4, 2, 24, 8
    q, k, v = rnd((Bt, Hq, N, d), 330 + case), rnd((Bt, Hkv, N, d), 340 + case), rnd((Bt, Hkv, N, d), 350)
    dout = rnd((Bt, Hq, N, d), 360 + case)
    sink = rnd((Hq,), 370) if use_sink else None
    dq, dk, dv, dsink, sel = oracle.backward(q, k, v, dout, sink=sink, **kw)
    tq, tk, tv, tz = torch_dense_grads(q, k, v, dout, sel, kw.get("block_size", 0),
                                       kw.get("window", 0), sink)
    for a, b_ in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, b_, atol=1e-12)
    if use_sink:
        np.testing.assert_allclose(dsink, tz, atol=1e-12)


# P29: central finite differences of the oracle's own forward (selection
# held fixed) agree with its backward on sampled coordinates.
def test_p29_backward_matches_finite_differences():
    Bt, Hq, Hkv, N, d, B = 1, 2, 1, 12, 3, 3
    q, k, v = rnd((Bt, Hq, N, d), 380), rnd((Bt, Hkv, N, d), 381), rnd((Bt, Hkv, N, d), 382)
    dout, sink = rnd((Bt, Hq, N, d), 383), rnd((Hq,), 384)
    dq, dk, dv, dsink, sel = oracle.backward(q, k, v, dout, block_size=B, top_k=2, window=2,
                                             sink=sink)

    def loss(q_, k_, v_, z_):
        o, _, _ = oracle.attend(q_, k_, v_, window=2, block_size=B, sel=sel, sink=z_)
        return float((o.reshape(dout.shape) * dout.astype(np.float64)).sum())

    rng = np.random.default_rng(385)
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("sink", sink, dsink)):
        for _ in range(6):
            idx = tuple(rng.integers(0, s_) for s_ in arr.shape)
            a_p, a_m = arr.copy(), arr.copy()
            a_p[idx] += np.float32(1e-3)
            a_m[idx] -= np.float32(1e-3)
            args_p = dict(q=q, k=k, v=v, z=sink); args_m = dict(args_p)
            key = {"q": "q", "k": "k", "v": "v", "sink": "z"}[name]
            args_p[key], args_m[key] = a_p, a_m
            fd = (loss(args_p["q"], args_p["k"], args_p["v"], args_p["z"]) -
                  loss(args_m["q"], args_m["k"], args_m["v"], args_m["z"])) / \
                 (float(a_p[idx]) - float(a_m[idx]))
            assert abs(fd - grad[idx]) <= 1e-5 * max(1.0, abs(grad[idx])), (name, idx, fd, grad[idx])


# P28 with the token gate: the backward under a token selection (window 3,
# top 5 of an indexer over 8 dims, sink) equals autograd of the dense
# attention masked to window | kept tokens.
def test_p28_token_backward_is_autograd():
    Bt, Hq, Hkv, N, d = 2, 4, 2, 24, 8
    q, k, v = rnd((Bt, Hq, N, d), 430), rnd((Bt, Hkv, N, d), 431), rnd((Bt, Hkv, N, d), 432)
    dout, sink = rnd((Bt, Hq, N, d), 433), rnd((Hq,), 434)
    iq, ik = rnd((Bt, N, 8), 435), rnd((Bt, N, 8), 436)
    dq, dk, dv, dsink, tsel = oracle.backward(q, k, v, dout, window=3, sink=sink, idx_q=iq,
                                              idx_k=ik, token_top_k=5)
    assert tsel.shape == (Bt * N, 5)
    tq, tk, tv, tz = torch_dense_grads(q, k, v, dout, None, 0, 3, sink, tsel=tsel)
    for a, b_ in ((dq, tq), (dk, tk), (dv, tv), (dsink, tz)):
        np.testing.assert_allclose(a, b_, atol=1e-12)


# P29 with the token gate: finite differences of the forward under the
# selection (held fixed) agree with the backward.
def test_p29_token_backward_matches_finite_differences():
    Bt, Hq, Hkv, N, d = 1, 2, 1, 14, 3
    q, k, v = rnd((Bt, Hq, N, d), 440), rnd((Bt, Hkv, N, d), 441), rnd((Bt, Hkv, N, d), 442)
    dout = rnd((Bt, Hq, N, d), 443)
    iq, ik = rnd((Bt, N, 4), 444), rnd((Bt, N, 4), 445)
    dq, dk, dv, _, tsel = oracle.backward(q, k, v, dout, window=2, idx_q=iq, idx_k=ik,
                                          token_top_k=3)
    rows_t = np.repeat(tsel.reshape(Bt, 1, N, -1), Hq, axis=1).reshape(Bt * Hq * N, -1)

    def loss(q, k, v):
        o, _, _ = oracle.attend(q, k, v, window=2, tsel=rows_t)
        return float((o.reshape(dout.shape) * dout.astype(np.float64)).sum())

    rng = np.random.default_rng(446)
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(rng.integers(0, s_) for s_ in arr.shape)
            a_p, a_m = arr.copy(), arr.copy()
            a_p[idx] += np.float32(1e-3)
            a_m[idx] -= np.float32(1e-3)
            args_p = dict(q=q, k=k, v=v); args_m = dict(args_p)
            args_p[name], args_m[name] = a_p, a_m
            fd = (loss(**{kk: args_p[kk] for kk in ("q", "k", "v")}) -
                  loss(**{kk: args_m[kk] for kk in ("q", "k", "v")})) / \
                 (float(a_p[idx]) - float(a_m[idx]))
            assert abs(fd - grad[idx]) <= 1e-5 * max(1.0, abs(grad[idx])), (name, idx, fd, grad[idx])


# P28 with the compressed columns: the backward with groups of C tokens
# (C = 1: every token is also its own group; C = 5 and 4 leave a ragged
# tail that no group covers) next to a window, block gating and a sink
# equals autograd through torch's group means.
CMP_BWD_CASES = [
    dict(window=3, cmp_block=4, sink=True),
    dict(window=1, cmp_block=1),
    dict(window=2, block_size=4, top_k=2, cmp_block=5, sink=True),
    dict(window=4, block_size=4, top_k=3, cmp_block=4, gate_shared=True),
]


@pytest.mark.parametrize("case", range(len(CMP_BWD_CASES)))
def test_p28_compressed_backward_is_autograd(case):
    kw = dict(CMP_BWD_CASES[case])
    use_sink = kw.pop("sink", False)
    Bt, Hq, Hkv, N, d = 2, 4, 2, 24, 8
    if case == 0:
        N = 26   # two tokens past the last group of 4
    q, k, v = rnd((Bt, Hq, N, d), 450 + case), rnd((Bt, Hkv, N, d), 455 + case), rnd((Bt, Hkv, N, d), 460)
    dout = rnd((Bt, Hq, N, d), 465 + case)
    sink = rnd((Hq,), 470) if use_sink else None
    dq, dk, dv, dsink, sel = oracle.backward(q, k, v, dout, sink=sink, **kw)
    tq, tk, tv, tz = torch_dense_grads(q, k, v, dout, sel, kw.get("block_size", 0),
                                       kw.get("window", 0), sink, cmp_block=kw["cmp_block"])
    for a, b_ in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, b_, atol=1e-12)
    if use_sink:
        np.testing.assert_allclose(dsink, tz, atol=1e-12)


# P29 with the compressed columns: finite differences of the oracle's
# forward (groups of 5 over 12 tokens, window 2, kept blocks held fixed).
def test_p29_compressed_backward_matches_finite_differences():
    Bt, Hq, Hkv, N, d, B, C = 1, 2, 1, 12, 3, 3, 5
    q, k, v = rnd((Bt, Hq, N, d), 475), rnd((Bt, Hkv, N, d), 476), rnd((Bt, Hkv, N, d), 477)
    dout, sink = rnd((Bt, Hq, N, d), 478), rnd((Hq,), 479)
    dq, dk, dv, dsink, sel = oracle.backward(q, k, v, dout, block_size=B, top_k=2, window=2,
                                             sink=sink, cmp_block=C)

    def loss(q_, k_, v_, z_):
        o, _, _ = oracle.attend(q_, k_, v_, window=2, block_size=B, sel=sel, sink=z_, cmp_block=C)
        return float((o.reshape(dout.shape) * dout.astype(np.float64)).sum())

    rng = np.random.default_rng(480)
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("sink", sink, dsink)):
        for _ in range(8):
            idx = tuple(rng.integers(0, s_) for s_ in arr.shape)
            a_p, a_m = arr.copy(), arr.copy()
            a_p[idx] += np.float32(1e-3)
            a_m[idx] -= np.float32(1e-3)
            args_p = dict(q=q, k=k, v=v, z=sink); args_m = dict(args_p)
            key = {"q": "q", "k": "k", "v": "v", "sink": "z"}[name]
            args_p[key], args_m[key] = a_p, a_m
            fd = (loss(args_p["q"], args_p["k"], args_p["v"], args_p["z"]) -
                  loss(args_m["q"], args_m["k"], args_m["v"], args_m["z"])) / \
                 (float(a_p[idx]) - float(a_m[idx]))
            assert abs(fd - grad[idx]) <= 1e-5 * max(1.0, abs(grad[idx])), (name, idx, fd, grad[idx])


# P31: the backward at listed outputs (dq of some rows, dk and dv of some
# keys) equals the full backward there (window, kept blocks or kept tokens,
# sink, GQA 4/2; every key of one kv group and rows of every head).
@pytest.mark.parametrize("kw", [
    dict(window=5, sink=True),
    dict(block_size=4, top_k=3, window=3),
    dict(window=2, token_top_k=5, sink=True),
])
def test_p31_backward_at_listed_outputs(kw):
    kw = dict(kw)
    use_sink = kw.pop("sink", False)
    Bt, Hq, Hkv, N, d = 2, 4, 2, 24, 8
    q, k, v = rnd((Bt, Hq, N, d), 490), rnd((Bt, Hkv, N, d), 491), rnd((Bt, Hkv, N, d), 492)
    dout, sink = rnd((Bt, Hq, N, d), 493), (rnd((Hq,), 494) if use_sink else None)
    iq = ik = None
    if kw.get("token_top_k"):
        iq, ik = rnd((Bt, N, 8), 495), rnd((Bt, N, 8), 496)
    dq, dk, dv, _, sel = oracle.backward(q, k, v, dout, sink=sink, idx_q=iq, idx_k=ik, **kw)
    tok = kw.get("token_top_k", 0) > 0
    rows = np.array([0, 5, 23, 24 * 3 + 11, 24 * 6 + 23, 24 * 7 + 1])
    keys = np.arange(Bt * Hkv * N)[N: 2 * N]          # every key of (b 0, g 1)
    keys = np.concatenate([keys, [2 * N + 3, 3 * N + 23]])
    gq, gk, gv = oracle.attend_bwd_at(q, k, v, dout, rows=rows, keys=keys,
                                      window=kw.get("window", 0),
                                      block_size=kw.get("block_size", 0),
                                      sel=None if tok else sel, tsel=sel if tok else None,
                                      sink=sink)
    np.testing.assert_allclose(gq, dq.reshape(-1, d)[rows], atol=1e-12)
    np.testing.assert_allclose(gk, dk.reshape(-1, d)[keys], atol=1e-12)
    np.testing.assert_allclose(gv, dv.reshape(-1, d)[keys], atol=1e-12)


# P30: shifting all logits of a row leaves its output unchanged, so the
# score gradients of a row sum to minus that of its sink column: summed over
# the keys of a kv group, dk = scale * sum_i q_i P_i,sink D_i (zero without a
# sink).
# With the compressed columns (C = 8) the identity holds unchanged: a
# group's key gradient reaches its C tokens in equal parts.
@pytest.mark.parametrize("use_sink,cmp_block", [(False, 0), (True, 0), (True, 8)])
def test_p30_key_gradients_sum_to_sink_term(use_sink, cmp_block):
    Bt, Hq, Hkv, N, d = 2, 4, 2, 32, 8
    q, k, v = rnd((Bt, Hq, N, d), 390), rnd((Bt, Hkv, N, d), 391), rnd((Bt, Hkv, N, d), 392)
    dout = rnd((Bt, Hq, N, d), 393)
    sink = rnd((Hq,), 394) if use_sink else None
    dq, dk, dv, dsink, sel = oracle.backward(q, k, v, dout, block_size=4, top_k=3, window=4,
                                             sink=sink, cmp_block=cmp_block)
    want = np.zeros((Bt, Hkv, d))
    if use_sink:
        o, lse, _ = oracle.attend(q, k, v, window=4, block_size=4, sel=sel, sink=sink,
                                  cmp_block=cmp_block)
        o, lse = o.reshape(Bt, Hq, N, d), lse.reshape(Bt, Hq, N)
        D = (o * dout).sum(-1)
        p0 = np.exp(sink[None, :, None] - lse)
        w = (p0 * D)[..., None] * q.astype(np.float64) / math.sqrt(d)   # [Bt, Hq, N, d]
        want = w.reshape(Bt, Hkv, Hq // Hkv, N, d).sum(axis=(2, 3))
    np.testing.assert_allclose(dk.sum(axis=2), want, atol=1e-12)


def test_gate_variant_arguments_checked():
    q, k = rnd((1, 2, 16, 4), 313), rnd((1, 2, 16, 4), 314)
    with pytest.raises(ValueError):
        oracle.block_pool(k, 4, "max")
    with pytest.raises(ValueError):   # pooled keys of the other representation
        oracle.block_select(q, oracle.block_pool(k, 4), 4, 2, None, "minmax")
    with pytest.raises(ValueError):   # the forced first block needs a slot of its own
        oracle.block_select(q, oracle.block_pool(k, 4), 4, 1, None, "mean", False, True)


# A block-gated decode step over a history whose length is not a multiple of
# the block size (the own block of the newest queries is incomplete) equals
# a prefill over that history padded with arbitrary keys to whole blocks, at
# the same positions: the padding sits after every query, so it is never
# attended, and its block is never a candidate for them.
@pytest.mark.parametrize("nq", [1, 3])
def test_p15_block_decode_over_incomplete_last_block(nq):
    Bt, Hq, Hkv, Nk, B, d = 1, 4, 2, 61, 8, 8
    q = rnd((Bt, Hq, 64, d), 72)
    k, v = rnd((Bt, Hkv, 64, d), 73), rnd((Bt, Hkv, 64, d), 74)
    kw = dict(block_size=B, top_k=3, window=5)
    full = oracle.forward(q, k, v, **kw)
    off = Nk - nq
    dec = oracle.forward(np.ascontiguousarray(q[:, :, off:Nk]), np.ascontiguousarray(k[:, :, :Nk]),
                         np.ascontiguousarray(v[:, :, :Nk]), **kw)
    last = np.array([(bh * 64 + off + r) for bh in range(Bt * Hq) for r in range(nq)])
    np.testing.assert_array_equal(dec["sel"], full["sel"][last])
    np.testing.assert_array_equal(dec["out"], full["out"][last])
    np.testing.assert_array_equal(dec["lse"], full["lse"][last])


# The pooled keys are block means (checked with numpy's mean, a different
# summation routine than the oracle's loop).
def test_pool_is_block_mean():
    k = rnd((2, 3, 64, 5), 43)
    kb = oracle.block_pool(k, 16)
    np.testing.assert_allclose(kb, k.astype(np.float64).reshape(2, 3, 4, 16, 5).mean(3), atol=1e-14)


def test_gaps_reported():
    q, k = rnd((1, 1, 64, 8), 44), rnd((1, 1, 64, 8), 45)
    kbar = oracle.block_pool(k, 8)
    sel, s_last, s_next = oracle.block_select(q, kbar, 8, 3)
    sc = oracle.block_scores(q, kbar, 8, np.arange(64))
    for i in range(64):
        b = i // 8
        cand = sorted(sc[i, :b], reverse=True)
        m = min(2, b)
        if m:
            assert s_last[i] == cand[m - 1]
        else:
            assert np.isnan(s_last[i])
        if m < b:
            assert s_next[i] == cand[m]
        else:
            assert np.isnan(s_next[i])


# The score helpers the parity checker uses are plain dot products: compare
# them with numpy's matmul of the same operands (future candidates -inf).
def test_score_helpers_are_dot_products():
    q, k = rnd((1, 2, 64, 8), 46), rnd((1, 1, 64, 8), 47)
    kbar = oracle.block_pool(k, 8)
    rows = np.arange(2 * 64)
    sc = oracle.block_scores(q, kbar, 8, rows)
    ref = np.einsum("hid,cd->hic", q[0].astype(np.float64), kbar[0, 0]).reshape(128, 8)
    own = (rows % 64) // 8
    for t in range(128):
        np.testing.assert_allclose(sc[t, :own[t]], ref[t, :own[t]], atol=1e-12)
        assert np.all(np.isneginf(sc[t, own[t]:]))
    iq, ik = rnd((2, 40, 5), 48), rnd((2, 40, 5), 49)
    trows = np.arange(80)
    ts = oracle.token_scores(iq, ik, trows)
    for r in trows:
        b, i = divmod(int(r), 40)
        ref = ik[b].astype(np.float64) @ iq[b, i].astype(np.float64)
        np.testing.assert_allclose(ts[r, :i], ref[:i], atol=1e-12)
        assert np.all(np.isneginf(ts[r, i:]))
    # decode form: 7 queries at positions 33..39 of a 40-token history
    ts = oracle.token_scores(iq[:, 33:], ik, np.arange(14))
    for r in range(14):
        b, i = divmod(r, 7)
        ref = ik[b].astype(np.float64) @ iq[b, 33 + i].astype(np.float64)
        np.testing.assert_allclose(ts[r, :33 + i], ref[:33 + i], atol=1e-12)
        assert np.all(np.isneginf(ts[r, 33 + i:]))
