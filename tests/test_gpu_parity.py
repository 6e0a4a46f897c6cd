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


@pytest.mark.parametrize("wl", [
    # window of 41 blocks of 64 under the block gate (near blocks past 32)
    W.Workload("gate_span41_d64", 1, 4, 2, 64 * 72, 64, "bf16", block_size=64, top_k=6,
               window=64 * 40 + 10, block_offsets=True),
    W.Workload("gate_span41_d128", 1, 4, 2, 64 * 72, 128, "bf16", block_size=64, top_k=6,
               window=64 * 40 + 10, block_offsets=True, sink=True),
    # the Bit-Axon window (4096) with blocks of 64: 64 near blocks
    W.Workload("gate_span64", 1, 2, 2, 8192, 80, "bf16", block_size=64, top_k=8, window=4096,
               block_offsets=True),
], ids=lambda w: w.name)
def test_gate_long_window(dev, wl):
    run_and_check(W.make_inputs(wl, 14), dev, W.sample_rows(wl, 1024, 6), label=wl.name)


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


# Blocks smaller than the 64-key tile (Quest-style pages of 8, 16 or 32
# keys): a tile holds several blocks, near tiles get per-key block bits and
# a far block attends one masked tile.  N = 992 leaves a ragged 64-key tile.
SMALL_BLOCK_CASES = [
    dict(block_size=32, top_k=4),                                  # own + far blocks
    dict(block_size=16, top_k=6, window=40),                       # near and far blocks
    dict(block_size=8, top_k=8, window=100, sink=True),            # 13 near blocks
    dict(block_size=16, top_k=5, gate_repr="minmax", sink=True),   # Quest's min/max pages
    dict(block_size=32, top_k=3, window=70, gate_shared=True, gate_first=True),
    dict(block_size=16, top_k=4, window=700),                      # window of 44 blocks
]


@pytest.mark.parametrize("case", range(len(SMALL_BLOCK_CASES)))
@pytest.mark.parametrize("d", [64, 80, 128])
def test_small_blocks(dev, case, d):
    kw = SMALL_BLOCK_CASES[case]
    wl = W.Workload("small_blk", 2, 8, 2, 992, d, "bf16", block_offsets=True, **kw)
    run_and_check(W.make_inputs(wl, 141 + case + d), dev, label=f"small_blk {kw}")


@pytest.mark.parametrize("B", [8, 16, 32])
def test_small_blocks_dense(dev, B):
    # k = n: every earlier block kept, dense causal attention
    wl = W.Workload("small_blk_dense", 1, 4, 2, 32 * B, 64, "bf16", block_size=B, top_k=32,
                    block_offsets=True)
    run_and_check(W.make_inputs(wl, 150 + B), dev, label=f"small_blk_dense B={B}")


def test_small_blocks_fp32(dev):
    wl = W.Workload("small_blk_f32", 1, 4, 2, 384, 64, "f32", block_size=16, top_k=5, window=24,
                    block_offsets=True, sink=True)
    run_and_check(W.make_inputs(wl, 155), dev, label="small_blk_f32")


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


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("N,window", [(300, 17), (1000, 256)])
def test_fp8_window_qk8(dev, d, N, window):
    # FP8 prefill without block gating: K Q^T on the FP8 matrix cores from
    # the E4M3 inputs, V straight from E4M3 to its fp16 copy.
    wl = W.Workload("fp8_win", 2, 4, 2, N, d, "fp8", window=window, sink=True)
    run_and_check(W.make_inputs(wl, 93 + d + N), dev, label=f"fp8_qk8 d={d} N={N}")


def test_fp8_decode(dev):
    wl = W.Workload("fp8_dec", 2, 4, 2, 3000, 128, "fp8", window=64, token_top_k=200,
                    index_dim=64, sink=True)
    run_and_check(decode_inputs(wl, 5, 92), dev, label="fp8_decode")


def test_fp8_bitaxon_full_sampled(dev):
    wl = W.BITAXON_SWA.replace(name="bitaxon_swa_n16384_fp8", dtype="fp8")
    run_and_check(W.make_inputs(wl, 103), dev, W.sample_rows(wl, 3000, 1), label="fp8_bitaxon")


# --- backward (window and block gating, bf16) -------------------------------
def run_backward(inp, dev, seed, do_scale=1.0):
    import torch
    import sliding_window_long_amd as sa
    wl = inp.wl
    t = inp.tensors()
    g = {k_: (None if v_ is None else v_.to(dev)) for k_, v_ in t.items()}
    kw = dict(block_size=wl.block_size, top_k=wl.top_k, window=wl.window, sink=g["sink"],
              gate_repr=wl.gate_repr, gate_shared=wl.gate_shared, gate_first=wl.gate_first,
              idx_q=g["idx_q"], idx_k=g["idx_k"], token_top_k=wl.token_top_k,
              cmp_block=wl.cmp_block)
    out, lse, bsel, tsel = sa.forward(g["q"], g["k"], g["v"], return_selection=True, **kw)
    dout = W._round(np.random.default_rng(seed).standard_normal(inp.q.shape, dtype=np.float32)
                    * np.float32(do_scale), "bf16")
    dq, dk, dv, ds = sa.backward(g["q"], g["k"], g["v"], out, lse,
                                 torch.from_numpy(dout).to(torch.bfloat16).to(dev), **kw)
    torch.cuda.synchronize()
    grads = tuple(None if x is None else x.float().cpu().numpy() for x in (dq, dk, dv, ds))
    sel = tsel if wl.token_top_k else bsel
    return dout, (None if sel is None else sel.cpu().numpy()), grads


def bwd_and_check(inp, dev, seed, label):
    log(f"[gpu] {label} {inp.wl}")
    dout, sel, grads = run_backward(inp, dev, seed)
    for x in grads:
        assert x is None or np.isfinite(x).all()
    if inp.wl.token_top_k:
        res = check_grads(inp, dout, None, grads, sink=inp.sink, dev_tsel=sel)
    else:
        res = check_grads(inp, dout, sel, grads, sink=inp.sink)
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


def test_backward_long_window(dev):
    # window of 36 blocks of 64 under the block gate (near blocks past 32)
    wl = W.Workload("bwd_span36", 1, 4, 2, 64 * 48, 64, "bf16", block_size=64, top_k=5,
                    window=64 * 36, block_offsets=True, sink=True)
    bwd_and_check(W.make_inputs(wl, 74), dev, 86, label="bwd_span36")


@pytest.mark.parametrize("N,top_t,window,sink", [
    (1, 4, 1, False), (300, 16, 8, True), (1000, 100, 128, True), (1500, 40, 1, False),
    (2048, 300, 64, True)])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_token_gate(dev, N, top_t, window, sink, d):
    # the token gate's selection (shared by the heads, GQA 4/1), held fixed
    wl = W.Workload("bwd_tok", 1, 4, 1, N, d, "bf16", window=window, token_top_k=top_t,
                    index_dim=64, sink=sink)
    bwd_and_check(W.make_inputs(wl, 91 + N + d), dev, 92 + N, label=f"bwd_tok N={N} k={top_t}")


def test_backward_token_reduced(dev):
    # the Naive SWA + DSA shape at N = 4096 (16 q heads on 4 kv heads, window
    # 128, top 2048 tokens, sink)
    wl = W.SWA_TOKEN_TOPK.replace(name="bwd_tok_n4096", seq_len=4096)
    bwd_and_check(W.make_inputs(wl, 93), dev, 94, label="bwd_tok_n4096")


def test_backward_ragged(dev):
    wl = W.Workload("bwd_ragged", 1, 3, 1, 300, 80, "bf16", window=37, sink=True)
    bwd_and_check(W.make_inputs(wl, 72), dev, 82, label="bwd_ragged")


def test_backward_bora_all_rows(dev):
    bwd_and_check(W.make_inputs(W.BORA_HYBRID, 102), dev, 83, label="bwd_bora")


@pytest.mark.parametrize("case", [0, 1, 2, 4, 5])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_small_blocks(dev, case, d):
    # blocks of 8, 16 and 32 keys (several per 64-key tile; 128-key dK/dV
    # workgroups meet up to 16 blocks and their far lists)
    kw = dict(SMALL_BLOCK_CASES[case])
    wl = W.Workload("bwd_small_blk", 2, 4, 2, 992, d, "bf16", block_offsets=True, **kw)
    bwd_and_check(W.make_inputs(wl, 161 + case + d), dev, 171 + case, label=f"bwd_small_blk {kw}")


# Seeded random configurations: head dim, GQA ratio, batch, dtype, and the
# branches and their options drawn together (block sizes 8 to 128 with
# windows, every gate variant, the compressed branch, the token gate,
# sinks), at ragged lengths; every row checked.
def random_workload(seed, backward=False):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 80, 128]))
    Hkv, G, Bt = int(rng.choice([1, 2, 4])), int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2]))
    dtype = "bf16" if backward else str(rng.choice(["bf16", "bf16", "f32", "fp8"]))
    kw = dict(sink=bool(rng.random() < 0.4))
    mode = str(rng.choice(["window", "gate", "gate", "token"]))
    if mode == "gate":
        B = int(rng.choice([8, 16, 32, 64, 128]))
        n = int(rng.integers(2, max(3, min(40, 2048 // B))))
        N = B * n
        top_k = int(rng.integers(1, min(n, 33) + 1))
        kw.update(block_size=B, top_k=top_k, block_offsets=True,
                  gate_repr=str(rng.choice(["mean", "minmax"])), gate_shared=bool(rng.random() < 0.4),
                  gate_first=bool(top_k >= 2 and rng.random() < 0.3))
        if rng.random() < 0.6:
            kw["window"] = int(rng.integers(1, min(N, 64 * B) + 1))
    elif mode == "token":
        N = int(rng.integers(1, 1500))
        kw.update(window=int(rng.integers(1, 300)), token_top_k=int(rng.integers(1, 600)), index_dim=64)
    else:
        N = int(rng.integers(1, 1500))
        kw["window"] = int(rng.integers(1, 2000))
    if mode != "token" and rng.random() < 0.35:
        kw["cmp_block"] = int(rng.choice([1, 4, 8, 16, 64]))
    return W.Workload(f"rand{seed}", Bt, Hkv * G, Hkv, N, d, dtype, **kw)


@pytest.mark.parametrize("seed", range(1000, 1064))
def test_random_configs(dev, seed):
    wl = random_workload(seed)
    run_and_check(W.make_inputs(wl, seed), dev, label=f"random {seed}")


@pytest.mark.parametrize("seed", range(2000, 2024))
def test_backward_random_configs(dev, seed):
    wl = random_workload(seed, backward=True)
    bwd_and_check(W.make_inputs(wl, seed), dev, seed + 1, label=f"bwd random {seed}")


# Full-size backward in the benchmark's configuration, checked at listed
# outputs: dq of sampled rows (first/last rows of each head, block and
# window edges, random rows) and dk, dv of keys at window and block edges,
# each against every row that attends it (the device's selection held
# fixed).
def bwd_at_and_check(inp, dev, seed, rows, keys, label):
    from parity import check_grads_at
    wl = inp.wl
    d = wl.head_dim
    log(f"[gpu] {label} {wl} rows={len(rows)} keys={len(keys)}")
    dout, sel, grads = run_backward(inp, dev, seed)
    dq, dk, dv, _ = grads
    tok = wl.token_top_k > 0
    ref = oracle.attend_bwd_at(
        inp.q, inp.k, inp.v, dout, rows=rows, keys=keys, window=wl.window,
        block_size=wl.block_size, sink=inp.sink,
        sel=None if (tok or sel is None) else sel.reshape(-1, wl.top_k),
        tsel=sel.reshape(-1, wl.token_top_k) if tok else None)
    got = (dq.reshape(-1, d)[rows], dk.reshape(-1, d)[keys], dv.reshape(-1, d)[keys])
    for x in got:
        assert np.isfinite(x).all()
    res = check_grads_at(got, ref)
    log(f"[gpu] {label} " + " ".join(f"{k}: max {m:.2e} mean {a:.2e}" for k, (m, a) in res.items()))
    assert grads_ok(res), str(res)


def _keys(wl, pairs):
    return np.array([g * wl.seq_len + j for g, j in pairs], dtype=np.int64)


def test_backward_bitaxon_full_sampled(dev):
    wl = W.BITAXON_SWA   # 32 heads, N 16384, d 80, window 4096
    N = wl.seq_len
    keys = _keys(wl, [(0, 0), (3, 1), (7, 4095), (12, 4096), (20, 8191), (17, 12345), (31, N - 1)])
    bwd_at_and_check(W.make_inputs(wl, 103), dev, 87, W.sample_rows(wl, 96, 5), keys,
                     "bwd_bitaxon_full")


def test_backward_long_moba_full_sampled(dev):
    wl = W.LONG_MOBA     # 32/8 heads, N 131072, d 128, blocks of 512, top 8
    B, N = wl.block_size, wl.seq_len
    keys = _keys(wl, [(0, N - 1), (3, 255 * B + 5), (5, 250 * B + 100), (7, 200 * B + B - 1),
                      (2, 160 * B), (6, 128 * B + 300)])
    bwd_at_and_check(W.make_inputs(wl, 104), dev, 88, W.sample_rows(wl, 96, 6), keys,
                     "bwd_long_moba_full")


def test_backward_token_full_sampled(dev):
    wl = W.SWA_TOKEN_TOPK   # 16/4 heads, N 65536, d 128, window 128, top 2048 tokens, sink
    N = wl.seq_len
    keys = _keys(wl, [(0, N - 1), (1, N - 130), (2, 60000), (3, 40000), (0, 32768)])
    bwd_at_and_check(W.make_inputs(wl, 105), dev, 89, W.sample_rows(wl, 96, 7), keys,
                     "bwd_token_full")


# The compressed branch's gradients (groups of C tokens; GQA 4/2, two
# batches): ragged N and tails past the last group, with a window, block
# gating and its shared variant, a sink; C = 1 (every token also its own
# group), C = 64 (groups as large as the blocks), C = 300 (one group).
CMP_BWD_SHAPES = [
    dict(N=300, window=16, cmp_block=8),
    dict(N=1000, window=64, cmp_block=8, sink=True),
    dict(N=512, block_size=64, top_k=3, window=70, cmp_block=8, gate_shared=True),
    dict(N=257, window=1, cmp_block=1),
    dict(N=512, block_size=64, top_k=4, cmp_block=64, sink=True),
    dict(N=513, window=32, cmp_block=300),
]


@pytest.mark.parametrize("case", range(len(CMP_BWD_SHAPES)))
@pytest.mark.parametrize("d", [64, 80, 128])
def test_backward_compressed(dev, case, d):
    kw = dict(CMP_BWD_SHAPES[case])
    N = kw.pop("N")
    wl = W.Workload("bwd_cmp", 2, 4, 2, N, d, "bf16", block_offsets="block_size" in kw, **kw)
    bwd_and_check(W.make_inputs(wl, 121 + case + d), dev, 131 + case, label=f"bwd_cmp N={N} {kw}")


def test_backward_bora_nsa_all_rows(dev):
    # the BORA NSA layout: 8:1 compression, one selection per kv group
    wl = W.BORA_HYBRID.replace(name="bwd_bora_nsa", cmp_block=8, gate_shared=True)
    bwd_and_check(W.make_inputs(wl, 103), dev, 84, label="bwd_bora_nsa")


# Value ranges past fp16 for the backward's fp16 operands (q, k, dO and the
# score gradients): (name, workload options, q scale, k scale, v scale, dO scale).
BWD_RANGE_CASES = [
    ("v_big", dict(window=64), 1.0, 1.0, 1e5, 1.0),
    ("do_big_v_big", dict(block_size=64, top_k=3, window=40), 1.0, 1.0, 300.0, 1e3),
    ("do_tiny", dict(window=64), 1.0, 1.0, 1.0, 1e-6),
    ("v_tiny_do_tiny", dict(block_size=64, top_k=4), 1.0, 1.0, 1e-4, 1e-4),
    ("q_big_k_tiny", dict(block_size=64, top_k=3, window=50), 1e5, 1e-5, 1.0, 1.0),
]


@pytest.mark.parametrize("case", range(len(BWD_RANGE_CASES)), ids=[c[0] for c in BWD_RANGE_CASES])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_value_range(dev, case, d):
    name, kw, qs, ks, vs, dos = BWD_RANGE_CASES[case]
    wl = W.Workload("bwd_range_" + name, 1, 4, 2, 512, d, "bf16", sink=True,
                    block_offsets="block_size" in kw, **kw)
    inp = W.make_inputs(wl, 300 + case)
    rb = lambda a, c: W._round(a * np.float32(c), "bf16")
    inp = W.Inputs(wl, rb(inp.q, qs), rb(inp.k, ks), rb(inp.v, vs), inp.sink, None, None)
    log(f"[gpu] bwd range {name} d={d}")
    dout, bsel, grads = run_backward(inp, dev, 85 + case, do_scale=dos)
    for x in grads:
        assert x is None or np.isfinite(x).all()
    res = check_grads(inp, dout, bsel, grads, sink=inp.sink, joint_floor=False)
    log(f"[gpu] bwd range {name} d={d} " + " ".join(f"{k}: max {m:.2e} mean {a:.2e}" for k, (m, a) in res.items()))
    assert grads_ok(res), str(res)


def test_backward_deterministic(dev):
    # Every gradient is bitwise reproducible: the compaction writes its far
    # lists in a fixed order (so dk, dv sum the far rows in the same order on
    # every call), and the sink gradient is a fixed-order reduction.  Long
    # enough (N 2048, block 64) that each list spans several row tiles of the
    # compaction and several chunks of the far kernels.
    for kw, far in ((dict(window=50), False),
                    (dict(block_size=64, top_k=3, window=50), True),
                    (dict(block_size=64, top_k=5, sink=True), True)):
        wl = W.Workload("bwd_det", 1, 4, 2, 2048, 64, "bf16", block_offsets=far, **kw)
        inp = W.make_inputs(wl, 73)
        a = run_backward(inp, dev, 84)[2]
        b = run_backward(inp, dev, 84)[2]
        log(f"[gpu] bwd_det {kw}: dq, dk, dv" + (", dsink" if kw.get("sink") else ""))
        for x, y in zip(a, b):
            if x is None:
                assert y is None
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
    # Outputs and lse on sampled rows; the token selection (made per
    # position, shared by the heads) on 2048 random positions plus every
    # position of one 128-row tile in each 8192.
    from parity import check_token_selection
    wl = W.SWA_TOKEN_TOPK
    inp = W.make_inputs(wl, 105)
    log(f"[gpu] swa_token_full {wl}")
    out, lse, bsel, tsel = run_device(inp, dev)
    rep = check(inp, out, lse, W.sample_rows(wl, 160, 5), bsel, tsel)
    log(f"[gpu] swa_token_full outputs {rep}")
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert rep.ok(), str(rep)
    N = wl.seq_len
    rng = np.random.default_rng(55)
    pos = set(rng.choice(N, size=2048, replace=False).tolist())
    for t0 in range(0, N, 8192):
        start = t0 + 128 * int(rng.integers(0, 64))
        pos.update(range(start, start + 128))
    pos = np.array(sorted(pos), dtype=np.int64)
    srep = check_token_selection(inp, tsel, pos)
    log(f"[gpu] swa_token_full selection on {len(pos)} positions: {srep}")
    assert len(pos) >= 2048 + 1024 - 64
    assert srep.mismatched == 0 and srep.invalid == 0, str(srep)


def test_token_history_past_16_bits(dev):
    # Token ids past 2^16: N = 131072 with 2 q heads on 1 kv head.  4096 equal
    # indexer keys straddle id 65536 and score above every other key for the
    # rows from 67584 on (their indexer queries equal that key: score 256
    # against at most ~80 for the N(0,1) keys), so those rows must keep
    # exactly the 2048 lowest of the tied ids, 63488 .. 65535 -- a 16-bit id
    # field would rank 65536 .. 67583 (as 0 .. 2047) above them.  Other rows:
    # the usual sampled selection and output checks.
    from parity import check_token_selection
    wl = W.Workload("swa_token_n131072", 1, 2, 1, 131072, 64, "bf16", window=128,
                    token_top_k=2048, index_dim=64, sink=True)
    inp = W.make_inputs(wl, 131)
    lo, hi = 63488, 67584
    inp.idx_k[0, lo:hi] = 2.0
    inp.idx_q[0, hi:] = 2.0
    log(f"[gpu] token_past_16_bits {wl}")
    out, lse, bsel, tsel = run_device(inp, dev)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    rng = np.random.default_rng(9)
    tied_rows = np.concatenate([[hi, hi + 1, 98304, wl.seq_len - 1],
                                rng.integers(hi, wl.seq_len, size=60)])
    want = np.arange(lo, lo + 2048)
    for r in tied_rows:
        np.testing.assert_array_equal(tsel[0, r], want, err_msg=f"row {r}")
    pos = np.unique(np.concatenate([rng.choice(lo, size=400, replace=False),
                                    np.arange(lo - 2, lo + 40), np.arange(65530, 65542),
                                    np.arange(hi - 3, hi + 3), rng.integers(hi, wl.seq_len, 60)]))
    srep = check_token_selection(inp, tsel, pos)
    log(f"[gpu] token_past_16_bits selection on {len(pos)} positions: {srep}")
    assert srep.mismatched == 0 and srep.invalid == 0, str(srep)
    rows = np.unique(np.concatenate([W.sample_rows(wl, 40, 3),
                                     [h * wl.seq_len + i for h in range(2) for i in (65535, 65536, hi, 100000)]]))
    rep = check(inp, out, lse, rows, bsel, tsel)
    log(f"[gpu] token_past_16_bits outputs {rep}")
    assert rep.ok(), str(rep)


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
    # slice of 8192 ids and merges (65536: every slice full); 17000 keys with
    # top 2048 (three slices passing on at most 3 x 576 ids, fewer than
    # top_t), top_t 3000, and 40 queries (enough workgroups to spread), take
    # the one-workgroup-per-query selection.
    wl = W.Workload("dec_long", 1, 2, 1, Nk, 64, "bf16", window=window, token_top_k=top_t,
                    index_dim=64, sink=True)
    run_and_check(decode_inputs(wl, nq, 7 + nq + top_t), dev, label=f"decode_long Nk={Nk} k={top_t}")


def test_decode_token_long_history_batch(dev):
    # Two sequences: the slice lists, counts and redo flags of each
    # (sequence, query) are kept apart.
    wl = W.Workload("dec_long_b2", 2, 2, 1, 20000, 64, "bf16", window=16, token_top_k=300,
                    index_dim=64, sink=True)
    run_and_check(decode_inputs(wl, 3, 77), dev, label="decode_long batch 2")


# --- decode step under the block gate: every new query is gated as that
# position of a prefill over the cache (own block, the best k - 1 complete
# earlier blocks by their mean keys, the window); the cache need not end on a
# block boundary ---
@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("Nk,nq,B,top_k,window,offs", [(1024, 1, 64, 4, 0, True),
                                                      (1000, 5, 64, 3, 100, False),
                                                      (704, 64, 16, 6, 20, True),
                                                      (4096, 3, 128, 16, 512, True),
                                                      (513, 2, 8, 40, 0, False)])
def test_decode_blocks(dev, d, Nk, nq, B, top_k, window, offs):
    wl = W.Workload("dec_blk", 2, 4, 2, Nk, d, "bf16", block_size=B, top_k=top_k, window=window,
                    sink=True, block_offsets=offs)
    run_and_check(decode_inputs(wl, nq, 41 + d + Nk + nq), dev, label=f"decode_blocks nq={nq} B={B}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("repr_,shared,first", [("minmax", False, False), ("mean", True, False),
                                                ("mean", False, True), ("minmax", True, True)])
def test_decode_blocks_variants(dev, d, repr_, shared, first):
    # the gate variants during decode: min/max summaries, one selection per
    # kv group (GQA 8/2), block 0 always kept
    wl = W.Workload("dec_blk_var", 1, 8, 2, 2000, d, "bf16", block_size=64, top_k=5, window=40,
                    sink=True, gate_repr=repr_, gate_shared=shared, gate_first=first)
    run_and_check(decode_inputs(wl, 3, 13 + d), dev, label=f"decode_blocks {repr_} shared={shared} first={first}")


@pytest.mark.parametrize("dtype", ["f32", "fp8"])
def test_decode_blocks_dtypes(dev, dtype):
    wl = W.Workload("dec_blk_dt", 1, 8, 2, 2048, 128, dtype, block_size=64, top_k=5, window=64,
                    block_offsets=dtype == "f32")
    run_and_check(decode_inputs(wl, 7, 5), dev, label=f"decode_blocks {dtype}")


def test_decode_blocks_long_moba_cache(dev):
    # The long-MoBA layout (32 query / 8 kv heads, d 128, blocks of 512, top
    # 8) after a full 131072-token cache: 4 new tokens, every row checked.
    run_and_check(decode_inputs(W.LONG_MOBA, 4, 8), dev, label="decode_blocks long_moba")


@pytest.mark.parametrize("Nk", [1024, 1000])
def test_decode_blocks_caller_means(dev, Nk):
    # Block means kept by the caller (here from the pooling entry point over
    # the complete blocks) give the same step, bit for bit, as pooling the
    # cache inside the call.
    import torch
    import sliding_window_long_amd as sa
    wl = W.Workload("dec_blk_means", 2, 4, 2, Nk, 128, "bf16", block_size=64, top_k=4, window=32,
                    sink=True)
    inp = decode_inputs(wl, 3, 9)
    g = {k_: (None if v_ is None else v_.to(dev)) for k_, v_ in inp.tensors().items()}
    kw = dict(block_size=64, top_k=4, window=32, sink=g["sink"])
    ro, rl = sa.forward(g["q"], g["k"], g["v"], **kw)
    nb = Nk // 64
    means = sa.block_pool(g["k"][:, :, :nb * 64].contiguous(), 64)
    o, l = sa.forward(g["q"], g["k"], g["v"], block_means=means, **kw)
    torch.cuda.synchronize()
    log(f"[gpu] decode_blocks caller means Nk={Nk}")
    assert torch.equal(o.view(torch.int16), ro.view(torch.int16))
    assert torch.equal(l.view(torch.int32), rl.view(torch.int32))


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


# --- binding checks on device tensors: each malformed call raises before any launch
@pytest.mark.parametrize("which", ["forward", "backward"])
def test_binding_rejects_on_device(dev, which, monkeypatch):
    import torch
    import sliding_window_long_amd as sa
    from binding_cases import bad_backward_args, bad_forward_args
    cases = bad_forward_args(dev) if which == "forward" else bad_backward_args(dev)
    torch.cuda.synchronize()

    def no_library():
        raise AssertionError("the library was reached")
    monkeypatch.setattr(sa.binding, "load_library", no_library)
    for name, a in cases:
        with pytest.raises((ValueError, TypeError)):
            if which == "forward":
                sa.forward(a.pop("q"), a.pop("k"), a.pop("v"), **a)
            else:
                sa.backward(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("out"), a.pop("lse"),
                            a.pop("dout"))
    torch.cuda.synchronize()


# --- value range: bf16 inputs far outside the fp16 range, or tiny ----------
# out(q, k, c v) = c out(q, k, v): the output bar is applied in units of the
# largest |v| (max |out - out*| <= 1e-2 max|v|, mean <= 1e-3 max|v|); lse
# does not depend on v.  q and k scaled: the logits scale (peaked or flat
# softmax), the bar is as is.
RANGE_CASES = [
    ("v_big", dict(window=64), 1.0, 1e5),
    ("v_tiny", dict(window=64), 1.0, 1e-6),
    ("v_big_gate", dict(block_size=64, top_k=3, window=70, block_offsets=True), 1.0, 3e5),
    ("v_tiny_gate_cmp", dict(block_size=64, top_k=3, window=70, block_offsets=True, cmp_block=8),
     1.0, 2e-6),
    ("qk_peaked", dict(window=100), 4.0, 1e5),
    ("qk_tiny", dict(block_size=64, top_k=4, window=16, block_offsets=True), 1e-6, 1.0),
]


@pytest.mark.parametrize("case", range(len(RANGE_CASES)), ids=[c[0] for c in RANGE_CASES])
@pytest.mark.parametrize("d", [80, 128])
def test_value_range(dev, case, d):
    name, kw, qk_scale, v_scale = RANGE_CASES[case]
    wl = W.Workload("range_" + name, 1, 4, 2, 640, d, "bf16", sink=True, **kw)
    inp = W.make_inputs(wl, 200 + case)
    rb = lambda a, c: W._round(a * np.float32(c), "bf16")
    inp = W.Inputs(wl, rb(inp.q, qk_scale), rb(inp.k, qk_scale), rb(inp.v, v_scale), inp.sink,
                   inp.idx_q, inp.idx_k)
    # one row of V with mixed magnitudes: its big entries set the scale
    inp.v[0, 0, 5, :8] = W._round(np.full(8, 3e4 * v_scale, np.float32), "bf16")
    log(f"[gpu] range {name} d={d} max|v|={np.abs(inp.v).max():.3e}")
    out, lse, bsel, tsel = run_device(inp, dev)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    vmax = float(np.abs(inp.v).max())
    rows = np.arange(wl.batch * wl.n_q_heads * wl.seq_len)
    unit = W.Inputs(wl, inp.q, inp.k, (inp.v / vmax).astype(np.float32), inp.sink, None, None)
    rep = check(unit, out / vmax, lse, rows, bsel, tsel)
    log(f"[gpu] range {name} d={d} (units of max|v|) {rep}")
    assert rep.ok(), str(rep)
