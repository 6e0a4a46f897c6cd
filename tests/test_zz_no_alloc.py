"""The allocation-free forward (sparse_attn_fwd_noalloc: static device
scratch, no workspace) against sparse_attn_fwd, through the C ABI: two calls
in a row, the second with a smaller input, each bitwise equal to the
workspace entry point and within the parity bar against the oracle."""
import numpy as np
import pytest

import workloads as W
from parity import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import sliding_window_long_amd as sa
    sa.load_library()
    return torch.device("cuda:0")


def both(inp, dev):
    import torch
    import sliding_window_long_amd as sa
    wl = inp.wl
    g = {k_: (None if v_ is None else v_.to(dev)) for k_, v_ in inp.tensors().items()}
    kw = dict(block_size=wl.block_size, top_k=wl.top_k, window=wl.window, sink=g["sink"],
              return_selection=True)
    a = sa.forward(g["q"], g["k"], g["v"], **kw)
    b = sa.forward(g["q"], g["k"], g["v"], noalloc=True, **kw)
    torch.cuda.synchronize()
    conv = lambda t: None if t is None else t.float().cpu().numpy()
    return [conv(x) for x in a], [conv(x) for x in b]


def test_noalloc_matches_workspace_entry_point(dev):
    import sliding_window_long_amd as sa
    cases = [
        # the headline shape (96 MiB of scratch), then a smaller block-gated
        # call with far blocks, a window and a sink on the same scratch
        (W.BITAXON_SWA, W.sample_rows(W.BITAXON_SWA, 1500, 9)),
        (W.BORA_HYBRID.replace(name="bora_n1024", seq_len=1024, top_k=4, sink=True), None),
    ]
    for wl, rows in cases:
        cfg = sa.Params(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.seq_len, wl.head_dim,
                        block_size=wl.block_size, top_k=wl.top_k, window=wl.window).cfg()
        assert 0 < sa.sparse_attn_workspace_bytes(cfg) <= 128 << 20
        inp = W.make_inputs(wl, 17)
        ref, got = both(inp, dev)
        for x, y in zip(ref, got):
            if x is not None:
                np.testing.assert_array_equal(x, y)
        out, lse, bsel, _ = got
        if rows is None:
            rows = np.arange(wl.batch * wl.n_q_heads * wl.seq_len)
        rep = check(inp, out, lse, rows, None if bsel is None else bsel.astype(np.int32))
        print(f"[gpu] noalloc {wl.name}: {rep}", flush=True)
        assert rep.ok(), str(rep)


def test_noalloc_rejects_oversized(dev):
    import torch
    import sliding_window_long_amd as sa
    wl = W.LONG_MOBA.replace(n_q_heads=4, n_kv_heads=1)
    q = torch.zeros((1, 4, wl.seq_len, 128), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((1, 1, wl.seq_len, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(sa.SparseAttnError, match="SCRATCH_LIMIT"):
        sa.forward(q, k, k, block_size=512, top_k=8, noalloc=True)


def test_noalloc_under_graph_capture(dev):
    """The callers this entry point is for include HIP graph capture: one
    call captured into a graph (inputs, out and lse in fixed buffers), then
    replayed three times with new inputs copied into those buffers, eager
    calls and synchronisations between the replays; every replay must equal
    an eager call on the same inputs bit for bit."""
    import torch
    import sliding_window_long_amd as sa
    for wl in (W.BORA_HYBRID.replace(name="bora_n2048", seq_len=2048, top_k=6, sink=True),
               W.BITAXON_SWA.replace(name="swa_n2048", seq_len=2048, n_q_heads=4, n_kv_heads=4,
                                     window=512)):
        seeds = (31, 32, 33, 34)
        inps = [W.make_inputs(wl, s) for s in seeds]
        dv = [{k_: (None if v_ is None else v_.to(dev)) for k_, v_ in i.tensors().items()} for i in inps]
        kw = dict(block_size=wl.block_size, top_k=wl.top_k, window=wl.window)
        # fixed buffers the graph reads and writes
        q, k, v = (dv[0][n].clone() for n in ("q", "k", "v"))
        sink = None if dv[0]["sink"] is None else dv[0]["sink"].clone()
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        sa.forward(q, k, v, sink=sink, noalloc=True, out=out, lse=lse, **kw)   # warm-up, eager
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                sa.forward(q, k, v, sink=sink, noalloc=True, out=out, lse=lse, **kw)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for rep, d_in in enumerate(dv[1:]):
            q.copy_(d_in["q"]); k.copy_(d_in["k"]); v.copy_(d_in["v"])
            if sink is not None:
                sink.copy_(d_in["sink"])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got_o, got_l = out.clone(), lse.clone()
            # eager call on the same inputs (its own buffers; same static scratch)
            ro, rl = sa.forward(d_in["q"], d_in["k"], d_in["v"], sink=d_in["sink"], noalloc=True, **kw)
            torch.cuda.synchronize()
            print(f"[gpu] graph replay {rep} {wl.name}", flush=True)
            assert torch.equal(got_o.view(torch.int16), ro.view(torch.int16)), f"{wl.name} replay {rep}: out"
            assert torch.equal(got_l.view(torch.int32), rl.view(torch.int32)), f"{wl.name} replay {rep}: lse"
