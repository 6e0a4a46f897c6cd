"""Parity of the HIP path with the fp64 oracle, through the C ABI.

Small shapes compare every row; the full-size workloads compare sampled rows
(first/last rows of every head, rows at block and window edges, random rows)
in the launch configuration the benchmark times.  Tolerances and the
selection rule are in parity.py."""
import sys

import numpy as np
import pytest

import oracle
import workloads as W
from parity import check, check_grads, grads_ok

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import sliding_window_long_amd as sa
    sa.load_library()
    return torch.device("cuda:0")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_device(inp, dev):
    import torch
    import sliding_window_long_amd as sa
    wl = inp.wl
    t = inp.tensors()
    g = {k_: (None if v_ is None else v_.to(dev)) for k_, v_ in t.items()}
    out, lse, bsel, tsel = sa.forward(
        g["q"], g["k"], g["v"], block_size=wl.block_size, top_k=wl.top_k, window=wl.window,
        idx_q=g["idx_q"], idx_k=g["idx_k"], token_top_k=wl.token_top_k, sink=g["sink"],
        return_selection=True, gate_repr=wl.gate_repr, gate_shared=wl.gate_shared,
        gate_first=wl.gate_first, cmp_block=wl.cmp_block)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy(), lse.cpu().numpy(),
            None if bsel is None else bsel.cpu().numpy(),
            None if tsel is None else tsel.cpu().numpy())


def run_and_check(inp, dev, rows=None, label=""):
    wl = inp.wl
    log(f"[gpu] {label} {wl}")
    out, lse, bsel, tsel = run_device(inp, dev)
    if rows is None:
        rows = np.arange(inp.q.shape[0] * inp.q.shape[1] * inp.q.shape[2])   # every query row
    rep = check(inp, out, lse, rows, bsel, tsel)
    log(f"[gpu] {label} {rep}")
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert rep.ok(), str(rep)
    return rep


# --- window only (the Bit-Axon SWA shape family) ---------------------------
@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("N,window", [(1, 4), (63, 1), (300, 17), (300, 64), (513, 1000)])
def test_window_small(dev, d, N, window):
    wl = W.Workload(f"swa_small", 2, 4, 2, N, d, "bf16", window=window)
    run_and_check(W.make_inputs(wl, 7 + d + N), dev, label="window_small")


def test_window_one_is_v(dev):
    wl = W.Workload("swa_w1", 1, 2, 2, 200, 80, "bf16", window=1)
    inp = W.make_inputs(wl, 3)
    out, lse, _, _ = run_device(inp, dev)
    # exact wherever V is an fp16 normal number (P V runs in fp16)
    normal = np.abs(inp.v) >= 2.0 ** -14
    np.testing.assert_array_equal(out[normal], inp.v[normal])
    np.testing.assert_allclose(out, inp.v, atol=2e-7, rtol=0)


def test_bitaxon_reduced_all_rows(dev):
    wl = W.BITAXON_SWA.replace(n_q_heads=4, n_kv_heads=4, seq_len=2048 + 37, window=512)
    run_and_check(W.make_inputs(wl, 103), dev, label="bitaxon_reduced")


def test_bitaxon_full_sampled(dev):
    wl = W.BITAXON_SWA
    run_and_check(W.make_inputs(wl, 103), dev, W.sample_rows(wl, 3000, 1), label="bitaxon_full")


# --- block gating -----------------------------------------------------------
def test_tiny_moba_fp32_all_rows(dev):
    run_and_check(W.make_inputs(W.TINY_MOBA, 101), dev, label="tiny_moba")


def test_bora_hybrid_all_rows(dev):
    run_and_check(W.make_inputs(W.BORA_HYBRID, 102), dev, label="bora_hybrid")


def test_long_moba_reduced_sampled(dev):
    wl = W.LONG_MOBA.replace(seq_len=W.LONG_MOBA.seq_len // 8)
    run_and_check(W.make_inputs(wl, 104), dev, W.sample_rows(wl, 4096, 2), label="long_moba_n/8")


def test_long_moba_full_sampled(dev):
    wl = W.LONG_MOBA
    run_and_check(W.make_inputs(wl, 104), dev, W.sample_rows(wl, 2048, 3), label="long_moba_full")


@pytest.mark.parametrize("kw", [
    dict(block_size=64, top_k=8),                 # k = n: dense causal
    dict(block_size=64, top_k=1),                 # own block only
    dict(block_size=64, top_k=3, window=1),       # window inside own block
    dict(block_size=64, top_k=3, window=100000),  # window covers everything
    dict(block_size=128, top_k=2, window=200),    # near block partly in window
    dict(block_size=64, top_k=5, window=70),
])
@pytest.mark.parametrize("d", [64, 128])
def test_gate_edges(dev, kw, d):
    wl = W.Workload("gate_edge", 2, 4, 2, 512, d, "bf16", block_offsets=True, **kw)
    run_and_check(W.make_inputs(wl, 11 + d), dev, label=f"gate_edge {kw}")


def test_gate_wide_group(dev):
    wl = W.Workload("gqa16", 1, 16, 1, 1024, 80, "bf16", block_size=128, top_k=4, window=64,
                    block_offsets=True)
    run_and_check(W.make_inputs(wl, 12), dev, label="gqa16")


def test_fp32_window_and_gate(dev):
    wl = W.Workload("f32_mix", 1, 2, 1, 384, 128, "f32", block_size=64, top_k=3, window=40,
                    block_offsets=True)
    run_and_check(W.make_inputs(wl, 13), dev, label="f32_mix")


def test_block_pool_stage(dev):
    import torch
    import sliding_window_long_amd as sa
    for wl, seed in ((W.BORA_HYBRID, 1), (W.TINY_MOBA, 2)):
        inp = W.make_inputs(wl, seed)
        kd = inp.tensors()["k"].to(dev)
        got = sa.block_pool(kd, wl.block_size).cpu().numpy()
        torch.cuda.synchronize()
        ref = oracle.block_pool(inp.k, wl.block_size)
        np.testing.assert_allclose(got, ref, atol=2e-6, rtol=1e-5)


def test_deterministic(dev):
    inp = W.make_inputs(W.BORA_HYBRID, 5)
    a = run_device(inp, dev)
    b = run_device(inp, dev)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# --- gate variants: min/max summary, selection shared per kv group, first
# block always kept ------------------------------------------------------------
VARIANTS = [
    dict(gate_repr="minmax"),
    dict(gate_shared=True),
    dict(gate_first=True),
    dict(gate_repr="minmax", gate_shared=True),
    dict(gate_repr="minmax", gate_shared=True, gate_first=True),
]
VARIANT_IDS = ["minmax", "shared", "first", "minmax_shared", "all"]


@pytest.mark.parametrize("var", VARIANTS, ids=VARIANT_IDS)
@pytest.mark.parametrize("d", [64, 80, 128])
def test_gate_variants_small(dev, var, d):
    wl = W.Workload("gate_var", 2, 8, 2, 1024 + 64, d, "bf16", block_size=64, top_k=5,
                    window=100, block_offsets=True, **var)
    run_and_check(W.make_inputs(wl, 31 + d), dev, label=f"gate_var {var}")


@pytest.mark.parametrize("var", VARIANTS, ids=VARIANT_IDS)
def test_gate_variants_fp32(dev, var):
    wl = W.Workload("gate_var_f32", 1, 4, 2, 384, 64, "f32", block_size=64, top_k=3, window=40,
                    block_offsets=True, **var)
    run_and_check(W.make_inputs(wl, 41), dev, label=f"gate_var_f32 {var}")


@pytest.mark.parametrize("kw", [
    dict(top_k=2, gate_first=True),                            # block 0 and own: sink pattern
    dict(top_k=8, gate_first=True),                            # k = n: dense causal
    dict(top_k=3, gate_first=True, window=100000),
    dict(top_k=8, gate_repr="minmax"),
    dict(top_k=2, gate_repr="minmax", gate_shared=True, window=1),
])
def test_gate_variant_edges(dev, kw):
    wl = W.Workload("gate_var_edge", 1, 4, 2, 512, 128, "bf16", block_size=64,
                    block_offsets=True, **kw)
    run_and_check(W.make_inputs(wl, 51), dev, label=f"gate_var_edge {kw}")


def test_first_block_top2_selects_block0_and_own(dev):
    wl = W.Workload("first_top2", 1, 4, 2, 640, 64, "bf16", block_size=64, top_k=2,
                    gate_first=True, block_offsets=True)
    out, lse, bsel, _ = run_device(W.make_inputs(wl, 52), dev)
    own = np.arange(wl.seq_len) // wl.block_size
    want = np.stack([np.where(own > 0, 0, own), np.where(own > 0, own, -1)], axis=1)
    for h in range(wl.n_q_heads):
        np.testing.assert_array_equal(bsel[0, h], want)


def test_shared_selection_same_for_the_group(dev):
    for repr_ in ("mean", "minmax"):
        wl = W.Workload("shared_grp", 2, 12, 3, 1024, 80, "bf16", block_size=64, top_k=6,
                        window=64, gate_repr=repr_, gate_shared=True, block_offsets=True)
        _, _, bsel, _ = run_device(W.make_inputs(wl, 53), dev)
        g = bsel.reshape(2, 3, 4, 1024, 6)
        assert (g == g[:, :, :1]).all(), repr_


def test_block_pool_minmax_stage(dev):
    import torch
    import sliding_window_long_amd as sa
    for wl, seed in ((W.BORA_HYBRID, 1), (W.TINY_MOBA, 2)):
        inp = W.make_inputs(wl, seed)
        kd = inp.tensors()["k"].to(dev)
        got = sa.block_pool(kd, wl.block_size, "minmax").cpu().numpy()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got, oracle.block_pool(inp.k, wl.block_size, "minmax"))


def test_bora_hybrid_shared_first_all_rows(dev):
    # The BORA shape (GQA 8/4) with one selection per kv group, block 0 kept.
    wl = W.BORA_HYBRID.replace(name="bora_hybrid_shared_first", gate_shared=True,
                               gate_first=True)
    run_and_check(W.make_inputs(wl, 102), dev, label="bora_shared_first")


def test_long_moba_minmax_reduced_sampled(dev):
    wl = W.LONG_MOBA.replace(name="long_moba_minmax", seq_len=W.LONG_MOBA.seq_len // 8,
                             gate_repr="minmax")
    run_and_check(W.make_inputs(wl, 104), dev, W.sample_rows(wl, 4096, 2),
                  label="long_moba_minmax_n/8")


def test_long_moba_minmax_full_sampled(dev):
    wl = W.LONG_MOBA.replace(name="long_moba_minmax", gate_repr="minmax")
    run_and_check(W.make_inputs(wl, 104), dev, W.sample_rows(wl, 2048, 3),
                  label="long_moba_minmax_full")


# --- compressed branch (NSA: 8 tokens -> one compressed key and value) --------
@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("N,C,window", [(1, 8, 4), (7, 8, 3), (300, 8, 17), (1000, 8, 64),
                                        (513, 1, 1), (700, 64, 100), (200, 300, 8)])
def test_compressed_window(dev, d, N, C, window):
    wl = W.Workload("cmp_swa", 2, 4, 2, N, d, "bf16", window=window, cmp_block=C, sink=True)
    run_and_check(W.make_inputs(wl, 61 + d + N + C), dev, label=f"cmp_window N={N} C={C}")


@pytest.mark.parametrize("var", [dict(), dict(gate_shared=True, gate_first=True),
                                 dict(gate_repr="minmax")], ids=["mean", "shared_first", "minmax"])
def test_compressed_with_block_gate(dev, var):
    wl = W.Workload("cmp_gate", 2, 8, 4, 1024, 128, "bf16", block_size=128, top_k=4, window=128,
                    cmp_block=8, block_offsets=True, **var)
    run_and_check(W.make_inputs(wl, 62), dev, label=f"cmp_gate {var}")


def test_compressed_fp32(dev):
    wl = W.Workload("cmp_f32", 1, 2, 1, 384, 64, "f32", block_size=64, top_k=3, window=40,
                    cmp_block=8, sink=True, block_offsets=True)
    run_and_check(W.make_inputs(wl, 63), dev, label="cmp_f32")


def test_bora_nsa_all_rows(dev):
    # The BORA NSA layout: GQA 8/4, 8:1 compression, top 16 of 32 blocks,
    # window 512, one selection per kv group.
    wl = W.BORA_HYBRID.replace(name="bora_nsa_n4096", cmp_block=8, gate_shared=True)
    run_and_check(W.make_inputs(wl, 102), dev, label="bora_nsa")


# --- FP8 (E4M3) inputs: decoded exactly, computed as bf16, out bf16 ---------
@pytest.mark.parametrize("kw", [
    dict(window=100, sink=True),
    dict(block_size=64, top_k=4, window=70, block_offsets=True),
    dict(block_size=128, top_k=3, gate_shared=True, gate_repr="minmax", cmp_block=8,
         block_offsets=True),
    dict(window=16, token_top_k=40, index_dim=64, sink=True),
])
def test_fp8_inputs(dev, kw):
    wl = W.Workload("fp8", 2, 8, 4, 1024, 128, "fp8", **kw)
    inp = W.make_inputs(wl, 91)
    assert np.abs(inp.q).max() <= 448
    run_and_check(inp, dev, label=f"fp8 {kw}")


def test_fp8_decode(dev):
    wl = W.Workload("fp8_dec", 2, 4, 2, 3000, 128, "fp8", window=64, token_top_k=200,
                    index_dim=64, sink=True)
    run_and_check(decode_inputs(wl, 5, 92), dev, label="fp8_decode")


def test_fp8_bitaxon_full_sampled(dev):
    wl = W.BITAXON_SWA.replace(name="bitaxon_swa_n16384_fp8", dtype="fp8")
    run_and_check(W.make_inputs(wl, 103), dev, W.sample_rows(wl, 3000, 1), label="fp8_bitaxon")


# --- backward (window and block gating, bf16) -------------------------------
def run_backward(inp, dev, seed):
    import torch
    import sliding_window_long_amd as sa
    wl = inp.wl
    t = inp.tensors()
    g = {k_: (None if v_ is None else v_.to(dev)) for k_, v_ in t.items()}
    kw = dict(block_size=wl.block_size, top_k=wl.top_k, window=wl.window, sink=g["sink"],
              gate_repr=wl.gate_repr, gate_shared=wl.gate_shared, gate_first=wl.gate_first)
    out, lse, bsel, _ = sa.forward(g["q"], g["k"], g["v"], return_selection=True, **kw)
    dout = W._round(np.random.default_rng(seed).standard_normal(inp.q.shape, dtype=np.float32),
                    "bf16")
    dq, dk, dv, ds = sa.backward(g["q"], g["k"], g["v"], out, lse,
                                 torch.from_numpy(dout).to(torch.bfloat16).to(dev), **kw)
    torch.cuda.synchronize()
    grads = tuple(None if x is None else x.float().cpu().numpy() for x in (dq, dk, dv, ds))
    return dout, (None if bsel is None else bsel.cpu().numpy()), grads


def bwd_and_check(inp, dev, seed, label):
    log(f"[gpu] {label} {inp.wl}")
    dout, bsel, grads = run_backward(inp, dev, seed)
    for x in grads:
        assert x is None or np.isfinite(x).all()
    res = check_grads(inp, dout, bsel, grads, sink=inp.sink)
    log(f"[gpu] {label} " + " ".join(f"{k}: max {m:.2e} mean {a:.2e}" for k, (m, a) in res.items()))
    assert grads_ok(res), str(res)
    return grads


BWD_SHAPES = [
    dict(window=64),
    dict(window=1),
    dict(block_size=64, top_k=3),                       # own + far blocks, no window
    dict(block_size=64, top_k=4, window=100),           # near and far blocks
    dict(block_size=128, top_k=3, window=200, sink=True),
    dict(block_size=64, top_k=8),                       # k = n: dense causal
    dict(block_size=64, top_k=3, window=70, gate_shared=True, gate_first=True),
    dict(block_size=64, top_k=4, gate_repr="minmax", sink=True),
]


@pytest.mark.parametrize("case", range(len(BWD_SHAPES)))
@pytest.mark.parametrize("d", [64, 80, 128])
def test_backward_small(dev, case, d):
    kw = dict(BWD_SHAPES[case])
    wl = W.Workload("bwd_small", 2, 4, 2, 512, d, "bf16", block_offsets="block_size" in kw, **kw)
    bwd_and_check(W.make_inputs(wl, 71 + case + d), dev, 81 + case, label=f"bwd {kw}")


def test_backward_ragged(dev):
    wl = W.Workload("bwd_ragged", 1, 3, 1, 300, 80, "bf16", window=37, sink=True)
    bwd_and_check(W.make_inputs(wl, 72), dev, 82, label="bwd_ragged")


def test_backward_bora_all_rows(dev):
    bwd_and_check(W.make_inputs(W.BORA_HYBRID, 102), dev, 83, label="bwd_bora")


def test_backward_deterministic(dev):
    # dq and (without far blocks) dk, dv are bitwise reproducible.  With far
    # blocks, dk and dv sum the far rows in the order of the compaction's
    # lists, which its atomics fill in no fixed order: two runs may then
    # differ by fp32 rounding (a bf16 step where it crosses a rounding
    # boundary), far below the gradients' scale.
    for kw, far in ((dict(window=50), False), (dict(block_size=64, top_k=3, window=50), True)):
        wl = W.Workload("bwd_det", 1, 4, 2, 640, 64, "bf16", block_offsets=far, **kw)
        inp = W.make_inputs(wl, 73)
        a = run_backward(inp, dev, 84)[2]
        b = run_backward(inp, dev, 84)[2]
        np.testing.assert_array_equal(a[0], b[0])
        for x, y in zip(a[1:3], b[1:3]):
            if far:
                log(f"[gpu] bwd_det far: max |run1 - run2| = {np.abs(x - y).max():.3e}, "
                    f"max |g| = {np.abs(x).max():.3e}")
                assert np.abs(x - y).max() <= 1e-3 * np.abs(x).max()
            else:
                np.testing.assert_array_equal(x, y)


# --- token top-k (Naive SWA + DSA shape) -------------------------------------
@pytest.mark.parametrize("N,top_t,window,sink", [
    (1, 4, 1, False), (33, 5, 2, True), (64, 8, 1, False), (300, 16, 8, True),
    (1024, 100, 128, True), (1000, 1, 4, False), (256, 300, 2, True), (8400, 700, 16, False)])
@pytest.mark.parametrize("d", [64, 128])
def test_token_small_all_rows(dev, N, top_t, window, sink, d):
    wl = W.Workload("tok_small", 1, 4, 1, N, d, "bf16", window=window, token_top_k=top_t,
                    index_dim=64, sink=sink)
    run_and_check(W.make_inputs(wl, 21 + N + d), dev, label=f"tok_small N={N} k={top_t}")


@pytest.mark.parametrize("N", [512, 1500])
def test_token_ties_go_to_lower_index(dev, N):
    # Equal indexer keys: every candidate of a row ties, the lowest token ids
    # must win.  Rows with up to 512 candidates are settled by the binned
    # path's candidate select (index bytes), longer rows by the radix
    # fallback; row tile 16 mixes both.
    wl = W.Workload("tok_ties", 1, 2, 1, N, 64, "bf16", window=2, token_top_k=37, index_dim=64)
    inp = W.make_inputs(wl, 5)
    inp.idx_k[:] = inp.idx_k[:, :1]
    out, lse, _, tsel = run_device(inp, dev)
    for i in range(wl.seq_len):
        m = min(37, i)
        assert tsel[0, i].tolist() == list(range(m)) + [-1] * (37 - m), i
    rep = check(inp, out, lse, np.arange(2 * N), None, tsel)
    log(f"[gpu] tok_ties {rep}")
    assert rep.ok(), str(rep)


def test_token_fp32(dev):
    wl = W.Workload("tok_f32", 1, 2, 2, 320, 64, "f32", window=16, token_top_k=24, index_dim=64,
                    sink=True)
    run_and_check(W.make_inputs(wl, 6), dev, label="tok_f32")


def test_swa_token_reduced_sampled(dev):
    wl = W.SWA_TOKEN_TOPK.replace(seq_len=W.SWA_TOKEN_TOPK.seq_len // 8)
    run_and_check(W.make_inputs(wl, 105), dev, W.sample_rows(wl, 768, 4), label="swa_token_n/8")


def test_swa_token_full_sampled(dev):
    wl = W.SWA_TOKEN_TOPK
    run_and_check(W.make_inputs(wl, 105), dev, W.sample_rows(wl, 160, 5), label="swa_token_full")


# --- decode/append step (queries continuing a cached history) ---------------
def decode_inputs(wl, nq, seed):
    """The last nq positions of a seeded full-length input as the queries;
    k, v, idx_k keep the whole history."""
    inp = W.make_inputs(wl, seed)
    off = wl.seq_len - nq
    iq = None if inp.idx_q is None else np.ascontiguousarray(inp.idx_q[:, off:])
    return W.Inputs(wl, np.ascontiguousarray(inp.q[:, :, off:]), inp.k, inp.v, inp.sink, iq,
                    inp.idx_k)


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("Nk,nq,window", [(300, 1, 17), (300, 7, 1), (1000, 64, 300),
                                          (1000, 3, 5000), (513, 64, 64)])
def test_decode_window(dev, d, Nk, nq, window):
    wl = W.Workload("dec_swa", 2, 4, 2, Nk, d, "bf16", window=window)
    run_and_check(decode_inputs(wl, nq, 11 + d + Nk + nq), dev, label=f"decode_window nq={nq}")


def test_decode_fp32_sink(dev):
    wl = W.Workload("dec_f32", 1, 6, 3, 700, 64, "f32", window=200, sink=True)
    run_and_check(decode_inputs(wl, 9, 4), dev, label="decode_f32")


@pytest.mark.parametrize("Nk,nq,top_t,window", [(3000, 1, 100, 16), (3000, 5, 100, 1),
                                                (3000, 64, 700, 64), (200, 8, 300, 4),
                                                (2100, 3, 2048, 128)])
def test_decode_token(dev, Nk, nq, top_t, window):
    wl = W.Workload("dec_tok", 1, 4, 1, Nk, 128, "bf16", window=window, token_top_k=top_t,
                    index_dim=64, sink=True)
    run_and_check(decode_inputs(wl, nq, 31 + nq + top_t), dev, label=f"decode_token nq={nq}")


@pytest.mark.parametrize("Nk,nq,top_t,window", [(17000, 3, 2048, 16), (40000, 2, 5, 64),
                                                (40000, 2, 3000, 8), (65536, 1, 1, 1),
                                                (20000, 40, 100, 16)])
def test_decode_token_long_history(dev, Nk, nq, top_t, window):
    # Histories over 16384 keys: with top_t <= 2048 the selection runs per
    # slice of 8192 ids and merges (17000: the slices pass on 576, 576 and
    # 616 ids, fewer than top_t, so the query is selected again whole;
    # 65536: every slice full); top_t 3000, and 40 queries (enough
    # workgroups to spread), take the one-workgroup-per-query selection.
    wl = W.Workload("dec_long", 1, 2, 1, Nk, 64, "bf16", window=window, token_top_k=top_t,
                    index_dim=64, sink=True)
    run_and_check(decode_inputs(wl, nq, 7 + nq + top_t), dev, label=f"decode_long Nk={Nk} k={top_t}")


def test_decode_token_long_history_batch(dev):
    # Two sequences: the slice lists, counts and redo flags of each
    # (sequence, query) are kept apart.
    wl = W.Workload("dec_long_b2", 2, 2, 1, 20000, 64, "bf16", window=16, token_top_k=300,
                    index_dim=64, sink=True)
    run_and_check(decode_inputs(wl, 3, 77), dev, label="decode_long batch 2")


@pytest.mark.parametrize("Nk,top_t", [(1500, 37), (20000, 37), (20000, 300)])
def test_decode_token_ties(dev, Nk, top_t):
    # Equal indexer keys: the lowest token ids win in the decode step too.
    # (20000 keys: per-slice selections and their merge; with top 300 the
    # first slice passes on only its best 139, all of them kept, so the
    # query is selected again whole.)
    wl = W.Workload("dec_ties", 1, 2, 1, Nk, 64, "bf16", window=2, token_top_k=top_t, index_dim=64)
    inp = decode_inputs(wl, 4, 5)
    inp.idx_k[:] = inp.idx_k[:, :1]
    out, lse, _, tsel = run_device(inp, dev)
    for r in range(4):
        assert tsel[0, r].tolist() == list(range(top_t)), r
    rep = check(inp, out, lse, np.arange(2 * 4), None, tsel)
    log(f"[gpu] decode_ties {rep}")
    assert rep.ok(), str(rep)


def test_decode_token_crowded_bins(dev):
    # Seven distinct indexer keys repeated over a 20000-token history, and
    # one key of 32x the norm: the outlier stretches the score range and the
    # repeats tie, so the threshold falls in a bin of ~2900 keys (the radix
    # resolution of the decode select; ties go to the lower token id).
    wl = W.Workload("dec_crowd", 1, 2, 1, 20000, 64, "bf16", window=8, token_top_k=1000, index_dim=64)
    inp = decode_inputs(wl, 6, 17)
    base = inp.idx_k[:, :7].copy()
    inp.idx_k[:] = base[:, np.arange(wl.seq_len) % 7]
    inp.idx_k[:, 123] = 32 * base[:, 0]   # exact in bf16
    run_and_check(inp, dev, label="decode_token_crowded")


def test_decode_bitaxon_full_size(dev):
    # One new token (and a 16-token append) after a 16384-token cache, 32
    # heads, d = 80, window 4096.
    for nq in (1, 16):
        run_and_check(decode_inputs(W.BITAXON_SWA, nq, 105), dev, label=f"decode_bitaxon nq={nq}")


def test_decode_token_full_size(dev):
    # Four new tokens after a 65536-token cache: window 128 plus the top 2048
    # of the whole history, sink, GQA 16/4.
    run_and_check(decode_inputs(W.SWA_TOKEN_TOPK, 4, 105), dev, label="decode_token_full")
