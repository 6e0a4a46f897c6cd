"""Non-finite inputs propagate; they never make a call fail or fault.

A NaN or an infinity in q, k or v is an ordinary input value for the
library: the call returns SA_OK, the rows whose attended set meets the bad
value come out non-finite, and every row that cannot see it (every earlier
position: attention is causal, and under block gating a later block is
never a candidate) is bitwise equal to a clean run.  One exception is
stated exactly: a non-finite value in v also reaches, in its own head
dimension only, the earlier rows of its 64-key tile (they mask that key to
weight 0, and the P V product forms 0 * inf = NaN); rows before the tile
and the other dimensions stay bitwise equal.  Covered: the window-only
path (Bit-Axon layout, head dim 80) and block gating with far blocks, a
window and a sink (BORA layout), each with NaN in one query row, NaN in one
key, and +inf in one value.  The token gate's indexer inputs must be finite
and are not varied here."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import sliding_window_long_amd as sa
    sa.load_library()
    return torch.device("cuda:0")


CASES = [
    ("window_d80", W.Workload("nf_swa", 1, 4, 4, 1200, 80, "bf16", window=300)),
    ("blocks_window_sink", W.Workload("nf_bora", 1, 4, 2, 1024, 128, "bf16", block_size=64,
                                      top_k=4, window=100, sink=True, block_offsets=True)),
]
POISON = [("q_nan", "q", float("nan")), ("k_nan", "k", float("nan")), ("v_inf", "v", float("inf"))]


def run(g, wl):
    import torch
    import sliding_window_long_amd as sa
    out, lse = sa.forward(g["q"], g["k"], g["v"], block_size=wl.block_size, top_k=wl.top_k,
                          window=wl.window, sink=g["sink"])
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("pname,tensor,val", POISON, ids=[p[0] for p in POISON])
@pytest.mark.parametrize("name,wl", CASES, ids=[c[0] for c in CASES])
def test_nonfinite_input_propagates(dev, name, wl, pname, tensor, val):
    inp = W.make_inputs(wl, 17)
    g = {k: (None if v is None else v.to(dev)) for k, v in inp.tensors().items()}
    out0, lse0 = run(g, wl)
    pos = 700   # a position in the middle of a block and of the sequence
    bad = {k: (None if v is None else v.clone()) for k, v in g.items()}
    bad[tensor][0, 1, pos, 5] = val
    print(f"[gpu] nonfinite {name} {pname} at position {pos}", flush=True)
    out1, lse1 = run(bad, wl)
    G = wl.n_q_heads // wl.n_kv_heads
    heads = [1] if tensor == "q" else list(range(G, 2 * G))   # heads reading kv head 1
    # every earlier position, of every head, is untouched (bitwise); for v,
    # rows before the 64-key tile of the bad value, and the other dims of
    # the tile's earlier rows
    first = pos - pos % 64 if tensor == "v" else pos
    np.testing.assert_array_equal(out1[:, :, :first].view(np.uint32), out0[:, :, :first].view(np.uint32))
    np.testing.assert_array_equal(lse1[:, :, :pos].view(np.uint32), lse0[:, :, :pos].view(np.uint32))
    if tensor == "v":
        dims = [e for e in range(wl.head_dim) if e != 5]
        np.testing.assert_array_equal(out1[:, :, first:pos][..., dims].view(np.uint32),
                                      out0[:, :, first:pos][..., dims].view(np.uint32))
    # the poisoned position itself attends the bad value (it is in its own
    # window / own block): non-finite output in the affected heads
    for h in heads:
        assert not np.isfinite(out1[0, h, pos]).all(), (name, pname, h)
    # heads that never read the bad tensor row are untouched everywhere
    other = [h for h in range(wl.n_q_heads) if h not in heads]
    if tensor != "q":
        other = [h for h in range(wl.n_q_heads) if h // G != 1]
    np.testing.assert_array_equal(out1[:, other].view(np.uint32), out0[:, other].view(np.uint32))
