"""Canary bytes around the workspace and the outputs; a poisoned workspace.

The library may write only inside the workspace it is handed and inside its
outputs, and may not read a workspace byte that the same call has not
written first.  Each case runs one call twice:

  * the workspace sits inside a larger buffer whose 64 KiB on either side
    hold a byte pattern; it is filled with 0x00 before the first run and
    with 0xFF (NaN in every float view, -1 in every integer view) before the
    second;
  * out and lse (forward) sit inside guarded buffers the same way;

and requires every guard byte unchanged after each run and the two runs'
results bitwise equal (both paths are deterministic, so a difference can
only come from reading stale workspace bytes).  The cases cover every
branch of the path: block gating with far blocks (blocks of 128 and of 16
keys, mean and min/max summaries), the token gate, the compressed branch,
fp32 and FP8 inputs, a decode step, and the backward of the gated, token
and compressed branches."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

GUARD = 65536
PAT_LO, PAT_HI = 0xA5, 0x5A


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import sliding_window_long_amd as sa
    sa.load_library()
    return torch.device("cuda:0")


class Guarded:
    """A device buffer of `nbytes` between two guard regions."""

    def __init__(self, nbytes, device, fill):
        import torch
        self.n = nbytes
        self.big = torch.empty(nbytes + 2 * GUARD, dtype=torch.uint8, device=device)
        self.big[:GUARD].fill_(PAT_LO)
        self.big[GUARD + nbytes:].fill_(PAT_HI)
        self.big[GUARD:GUARD + nbytes].fill_(fill)

    def inner(self):
        return self.big[GUARD:GUARD + self.n]

    def intact(self):
        import torch
        lo = self.big[:GUARD]
        hi = self.big[GUARD + self.n:]
        return bool(torch.all(lo == PAT_LO).item()) and bool(torch.all(hi == PAT_HI).item())


class GuardedWorkspace:
    """Stands in for the binding's Workspace: every call gets a fresh guarded
    buffer filled with `fill`."""

    def __init__(self, fill):
        self.fill = fill
        self.bufs = []

    def get(self, nbytes, device):
        if nbytes == 0:
            return None
        g = Guarded(nbytes, device, self.fill)
        self.bufs.append(g)
        return g.inner()

    def intact(self):
        return all(g.intact() for g in self.bufs)


def guarded_tensor(shape, dtype, device, fill=0):
    import torch
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    g = Guarded(n, device, fill)
    return g, g.inner().view(dtype).view(shape)


def to_dev(inp, dev):
    t = inp.tensors()
    return {k: (None if v is None else v.to(dev)) for k, v in t.items()}


def fwd_kw(wl, g):
    return dict(block_size=wl.block_size, top_k=wl.top_k, window=wl.window, idx_q=g["idx_q"],
                idx_k=g["idx_k"], token_top_k=wl.token_top_k, sink=g["sink"],
                gate_repr=wl.gate_repr, gate_shared=wl.gate_shared, gate_first=wl.gate_first,
                cmp_block=wl.cmp_block)


def decode_inputs(wl, nq, seed):
    inp = W.make_inputs(wl, seed)
    off = wl.seq_len - nq
    iq = None if inp.idx_q is None else np.ascontiguousarray(inp.idx_q[:, off:])
    return W.Inputs(wl, np.ascontiguousarray(inp.q[:, :, off:]), inp.k, inp.v, inp.sink, iq,
                    inp.idx_k)


FWD_CASES = [
    ("blocks_window_sink", W.Workload("c_bora", 2, 8, 4, 1024, 128, "bf16", block_size=128,
                                      top_k=4, window=200, sink=True, block_offsets=True), 0),
    ("blocks16_minmax", W.Workload("c_b16", 1, 4, 2, 700 - 700 % 16, 64, "bf16", block_size=16,
                                   top_k=6, window=40, gate_repr="minmax", block_offsets=True), 0),
    ("token_gate", W.Workload("c_tok", 1, 4, 1, 3000, 128, "bf16", window=64, token_top_k=300,
                              index_dim=64, sink=True), 0),
    ("compressed_shared", W.Workload("c_nsa", 1, 4, 2, 1024, 64, "bf16", block_size=64, top_k=4,
                                     window=128, gate_shared=True, gate_first=True, cmp_block=8,
                                     sink=True, block_offsets=True), 0),
    ("fp32_blocks", W.Workload("c_f32", 1, 2, 1, 512, 64, "f32", block_size=64, top_k=3,
                               block_offsets=True), 0),
    ("window_d80", W.Workload("c_swa", 1, 4, 4, 1000, 80, "bf16", window=300), 0),
    ("fp8_window_sink", W.Workload("c_fp8", 1, 4, 2, 900, 128, "fp8", window=100, sink=True), 0),
    ("decode_token", W.Workload("c_dec", 1, 4, 1, 3000, 128, "bf16", window=64, token_top_k=300,
                                index_dim=64, sink=True), 5),
]


@pytest.mark.parametrize("name,wl,nq", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_canaries(dev, name, wl, nq):
    import torch
    import sliding_window_long_amd as sa
    inp = decode_inputs(wl, nq, 5) if nq else W.make_inputs(wl, 5)
    g = to_dev(inp, dev)
    out_dt = torch.bfloat16 if g["q"].dtype == torch.float8_e4m3fn else g["q"].dtype
    res = []
    for fill in (0x00, 0xFF):
        ws = GuardedWorkspace(fill)
        go, out = guarded_tensor(tuple(g["q"].shape), out_dt, dev, fill)
        gl, lse = guarded_tensor(tuple(g["q"].shape[:3]), torch.float32, dev, fill)
        print(f"[gpu] canaries {name} fill=0x{fill:02x} {wl}", flush=True)
        sa.forward(g["q"], g["k"], g["v"], workspace=ws, out=out, lse=lse, **fwd_kw(wl, g))
        torch.cuda.synchronize()
        assert ws.bufs or wl.top_k == 0, "a gated call must take a workspace"
        assert ws.intact(), f"{name}: a workspace guard changed (fill 0x{fill:02x})"
        assert go.intact() and gl.intact(), f"{name}: an output guard changed (fill 0x{fill:02x})"
        res.append((out.clone(), lse.clone()))
    (o0, l0), (o1, l1) = res
    assert torch.isfinite(o0.float()).all() and torch.isfinite(l0).all()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)), f"{name}: out depends on stale workspace bytes"
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32)), f"{name}: lse depends on stale workspace bytes"


BWD_CASES = [
    ("blocks_far_sink", W.Workload("cb_bora", 1, 4, 2, 1024, 128, "bf16", block_size=64, top_k=4,
                                   window=100, sink=True, block_offsets=True)),
    ("token_gate", W.Workload("cb_tok", 1, 4, 1, 2000, 64, "bf16", window=32, token_top_k=200,
                              index_dim=64, sink=True)),
    ("compressed", W.Workload("cb_nsa", 1, 4, 2, 1024, 64, "bf16", block_size=64, top_k=3,
                              window=100, gate_shared=True, cmp_block=8, block_offsets=True)),
]


@pytest.mark.parametrize("name,wl", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_canaries(dev, name, wl):
    import torch
    import sliding_window_long_amd as sa
    inp = W.make_inputs(wl, 9)
    g = to_dev(inp, dev)
    kw = fwd_kw(wl, g)
    out, lse = sa.forward(g["q"], g["k"], g["v"], **kw)
    dout = torch.from_numpy(W._round(np.random.default_rng(2).standard_normal(inp.q.shape,
                                                                              dtype=np.float32), "bf16"))
    dout = dout.to(torch.bfloat16).to(dev)
    res = []
    for fill in (0x00, 0xFF):
        ws = GuardedWorkspace(fill)
        print(f"[gpu] canaries backward {name} fill=0x{fill:02x} {wl}", flush=True)
        grads = sa.backward(g["q"], g["k"], g["v"], out, lse, dout, workspace=ws, **kw)
        torch.cuda.synchronize()
        assert ws.bufs, "the backward takes a workspace"
        assert ws.intact(), f"{name}: a backward workspace guard changed (fill 0x{fill:02x})"
        res.append([None if x is None else x.clone() for x in grads])
    for a_, b_, nm in zip(res[0], res[1], ("dq", "dk", "dv", "dsink")):
        if a_ is None:
            continue
        assert torch.isfinite(a_.float()).all(), f"{name}: {nm} not finite"
        iv = torch.int16 if a_.element_size() == 2 else torch.int32
        assert torch.equal(a_.view(iv), b_.view(iv)), f"{name}: {nm} depends on stale workspace bytes"
