"""Seeded synthetic workloads for the causal sparse-attention prefill.

This module only *draws inputs*: it holds the workload shapes and a seeded
generator, and none of the attention method's arithmetic.  Both sides of the
parity check use it -- the fp64 CPU oracle under ``oracle/`` and the HIP
library -- so that they see identical bytes; neither imports the other.

Recipe (the same for every workload):

* random source ``numpy.random.default_rng(seed)`` (PCG64), fp32
  ``standard_normal`` draws in this fixed order: q, k, v, block offsets,
  sink logits, indexer queries, indexer keys (a draw is skipped when the
  workload does not use that tensor);
* "per-block key offset N(0, 0.5^2)": one offset vector per
  (batch, kv head, key block), each component N(0, 0.25), added in fp32 to
  every key of that block before rounding, so that the block means differ
  and the gating is not decided by noise;
* bf16 workloads are rounded to bf16 with round-to-nearest-even
  (``torch.Tensor.to(torch.bfloat16)``), fp8 workloads to OCP E4M3
  (``torch.float8_e4m3fn``, round to nearest even; N(0,1) draws stay far
  below its 448 limit); the fp32 copies handed to the oracle hold exactly
  the rounded values.

Shapes follow the (batch, heads, seq_len, head_dim) layout of the Bit-Axon
"SWA + MoE" page (its q/k/v reshape in the algorithm figure).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_len: int
    head_dim: int
    dtype: str                 # "f32", "bf16" or "fp8" (E4M3, out bf16): dtype of q, k, v
    block_size: int = 0        # B; 0 when block gating is off
    top_k: int = 0             # blocks kept per query, own block included
    window: int = 0            # w: attend iff 0 <= i - j < w; 0 = no window
    token_top_k: int = 0       # tokens kept per query by the indexer
    index_dim: int = 0         # indexer head dim
    sink: bool = False         # per-head sink logit
    block_offsets: bool = False
    gate_repr: str = "mean"    # block summary for the gate: "mean" or "minmax"
    gate_shared: bool = False  # one block selection per kv group
    gate_first: bool = False   # block 0 always kept (takes one of the top_k slots)
    cmp_block: int = 0         # compressed branch: tokens per compressed key/value; 0 = off

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def n_blocks(self) -> int:
        return self.seq_len // self.block_size if self.block_size else 0


# The five synthetic workloads (sizes as stated with the benchmark metric).
TINY_MOBA = Workload("tiny_moba_n512", 1, 1, 1, 512, 64, "f32",
                     block_size=64, top_k=3, block_offsets=True)
BORA_HYBRID = Workload("bora_hybrid_n4096", 2, 8, 4, 4096, 128, "bf16",
                       block_size=128, top_k=16, window=512, block_offsets=True)
BITAXON_SWA = Workload("bitaxon_swa_n16384", 1, 32, 32, 16384, 80, "bf16",
                       window=4096)
LONG_MOBA = Workload("long_moba_n131072", 1, 32, 8, 131072, 128, "bf16",
                     block_size=512, top_k=8, block_offsets=True)
SWA_TOKEN_TOPK = Workload("swa_tokentopk_sink_n65536", 1, 16, 4, 65536, 128, "bf16",
                          window=128, token_top_k=2048, index_dim=64, sink=True)

WORKLOADS = {1: TINY_MOBA, 2: BORA_HYBRID, 3: BITAXON_SWA, 4: LONG_MOBA,
             5: SWA_TOKEN_TOPK}


@dataclass
class Inputs:
    """Inputs of one workload.  ``*_f32`` arrays hold exactly the values the
    device sees (bf16 values widened to fp32 losslessly); ``tensors()``
    gives the device-dtype torch tensors on the CPU."""
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    sink: np.ndarray | None
    idx_q: np.ndarray | None
    idx_k: np.ndarray | None

    def tensors(self):
        import torch
        dt = {"bf16": torch.bfloat16, "f32": torch.float32,
              "fp8": torch.float8_e4m3fn}[self.wl.dtype]
        conv = lambda a: None if a is None else torch.from_numpy(a).to(dt)
        return dict(q=conv(self.q), k=conv(self.k), v=conv(self.v),
                    idx_q=conv(self.idx_q), idx_k=conv(self.idx_k),
                    sink=None if self.sink is None else torch.from_numpy(self.sink))


def _round(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    low = torch.float8_e4m3fn if dtype == "fp8" else torch.bfloat16
    return t.to(low).to(torch.float32).numpy()


def make_inputs(wl: Workload, seed: int) -> Inputs:
    rng = np.random.default_rng(seed)
    Bt, Hq, Hkv, N, d = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.seq_len, wl.head_dim
    q = rng.standard_normal((Bt, Hq, N, d), dtype=np.float32)
    k = rng.standard_normal((Bt, Hkv, N, d), dtype=np.float32)
    v = rng.standard_normal((Bt, Hkv, N, d), dtype=np.float32)
    if wl.block_offsets:
        if not wl.block_size or N % wl.block_size:
            raise ValueError("block offsets need a block size dividing N")
        n = N // wl.block_size
        off = 0.5 * rng.standard_normal((Bt, Hkv, n, d), dtype=np.float32)
        k = (k.reshape(Bt, Hkv, n, wl.block_size, d) + off[:, :, :, None, :]).reshape(Bt, Hkv, N, d)
    sink = rng.standard_normal((Hq,), dtype=np.float32) if wl.sink else None
    iq = ik = None
    if wl.token_top_k:
        iq = rng.standard_normal((Bt, N, wl.index_dim), dtype=np.float32)
        ik = rng.standard_normal((Bt, N, wl.index_dim), dtype=np.float32)
    return Inputs(wl, _round(q, wl.dtype), _round(k, wl.dtype), _round(v, wl.dtype),
                  sink, None if iq is None else _round(iq, wl.dtype),
                  None if ik is None else _round(ik, wl.dtype))


def sample_rows(wl: Workload, count: int, seed: int) -> np.ndarray:
    """Sorted, distinct flat row ids r = (b*Hq + h)*N + i for sampled checks.
    Always includes the first and last row of every head and the rows around
    block and window edges, plus uniform random rows."""
    rng = np.random.default_rng(seed)
    Bt, Hq, N = wl.batch, wl.n_q_heads, wl.seq_len
    special = {0, 1, N - 1, N - 2}
    for edge in (wl.block_size, wl.window):
        if edge:
            for e in (edge - 1, edge, edge + 1, 2 * edge - 1, 2 * edge):
                if 0 <= e < N:
                    special.add(e)
    rows = set()
    for bh in range(Bt * Hq):
        for i in special:
            rows.add(bh * N + i)
    extra = rng.integers(0, Bt * Hq * N, size=max(0, count - len(rows)))
    rows.update(int(r) for r in extra)
    return np.array(sorted(rows), dtype=np.int64)
