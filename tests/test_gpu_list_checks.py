"""The device's far-block lists under the library's own checks.

With sparse_attn_set_checks(1) every call that regroups rows by far block
copies the selection and the lists back and verifies them on the host
(sparse_attn_check_far_lists: offsets, chunk table, every entry a far slot
of its row under the right block, every far slot listed exactly once, and
for the backward's lists the fixed order).  The forward's fast scatter and
the backward's ordered scatter run at the BORA hybrid shape, at the full
long-MoBA shape the benchmark times, with each gate variant, and with blocks
of 16 keys; every call must return SA_OK (a violation raises
SparseAttnError with SA_E_CHECK)."""
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


@pytest.fixture
def checks():
    """Checks on for the test; afterwards, the stage record must show that a
    check ran."""
    import sliding_window_long_amd as sa
    sa.sparse_attn_set_checks(True)
    sa.sparse_attn_set_timing(True)
    try:
        yield
        names = [n for n, _ in sa.sparse_attn_stage_times(1024)]
        assert "far_list_check" in names, names
    finally:
        sa.sparse_attn_set_timing(False)
        sa.sparse_attn_set_checks(False)


def kw_of(wl, g):
    return dict(block_size=wl.block_size, top_k=wl.top_k, window=wl.window, sink=g["sink"],
                gate_repr=wl.gate_repr, gate_shared=wl.gate_shared, gate_first=wl.gate_first,
                cmp_block=wl.cmp_block)


FWD = [
    ("bora_hybrid", W.BORA_HYBRID),
    ("bora_shared_first", W.BORA_HYBRID.replace(gate_shared=True, gate_first=True)),
    ("bora_minmax_sink", W.BORA_HYBRID.replace(gate_repr="minmax", sink=True)),
    ("long_moba_full", W.LONG_MOBA),
    ("long_moba_n16384_shared", W.LONG_MOBA.replace(seq_len=16384, gate_shared=True)),
    ("blocks16_window", W.Workload("b16", 2, 4, 2, 2048, 64, "bf16", block_size=16, top_k=12,
                                   window=100, block_offsets=True)),
    ("no_window", W.Workload("nw", 1, 8, 2, 4096, 128, "bf16", block_size=64, top_k=16,
                             block_offsets=True)),
]


@pytest.mark.parametrize("name,wl", FWD, ids=[c[0] for c in FWD])
def test_forward_lists_checked(dev, checks, name, wl):
    import torch
    import sliding_window_long_amd as sa
    inp = W.make_inputs(wl, 21)
    g = {k: (None if v is None else v.to(dev)) for k, v in inp.tensors().items()}
    print(f"[gpu] list checks forward {name} {wl}", flush=True)
    out, lse = sa.forward(g["q"], g["k"], g["v"], **kw_of(wl, g))
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()


BWD = [
    ("bora_hybrid", W.BORA_HYBRID.replace(sink=True)),
    ("blocks16_window", W.Workload("b16", 1, 4, 2, 2048, 64, "bf16", block_size=16, top_k=12,
                                   window=100, block_offsets=True)),
    ("long_moba_n16384", W.LONG_MOBA.replace(seq_len=16384)),
]


@pytest.mark.parametrize("name,wl", BWD, ids=[c[0] for c in BWD])
def test_backward_lists_checked(dev, checks, name, wl):
    import torch
    import sliding_window_long_amd as sa
    inp = W.make_inputs(wl, 22)
    g = {k: (None if v is None else v.to(dev)) for k, v in inp.tensors().items()}
    kw = kw_of(wl, g)
    print(f"[gpu] list checks backward {name} {wl}", flush=True)
    out, lse = sa.forward(g["q"], g["k"], g["v"], **kw)
    dout = torch.from_numpy(W._round(np.random.default_rng(3).standard_normal(inp.q.shape,
                                                                              dtype=np.float32), "bf16"))
    grads = sa.backward(g["q"], g["k"], g["v"], out, lse, dout.to(torch.bfloat16).to(dev), **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(grads[0].float()).all()
