"""Exact brute-force version of the method for tiny inputs (N <= ~32).

TEST INFRASTRUCTURE: a second, independent statement of the definitions,
used only to pin the C oracle.  It shares nothing with it: gate scores are
exact rationals (``fractions.Fraction``), the block selection is found by
enumerating every admissible subset of past blocks, and the attended set is
built pair by pair from the three clauses of the mask predicate.

Sources: the MoBA summary page (discuss.pytorch.kr), sections "블록 분할과
top-k 게이팅" and "인과성 보존", and its remark casting attention sinks and
Quest as MoBA with other gates; the Bit-Axon "SWA + MoE" page, section
"슬라이딩 윈도우 마스크"; the Naive-N0.5-Flash page, section "SWA와 DSA를
결합한 어텐션".

Gate variants, stated here independently of the C oracle:
* min/max blocks: a block is the box spanned by its keys' per-dimension
  minima and maxima; its score is the largest <q, x> over the box's 2^d
  corners (enumerated);
* shared: the score of a block for query position i of kv group g is the
  sum over the group's heads of that head's score; all of them keep the
  same blocks;
* first: block 0 is kept like the own block and takes one of the k slots.

Compressed branch (BORA model card, NSA: 8 tokens -> 1 compressed key and
value): with cmp_block = C, every complete group c of C tokens whose last
token is at or before i adds one column to the softmax: the exact mean of
its keys as the key and the mean of its values as the value.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction

import numpy as np


def _frac(x) -> Fraction:
    return Fraction(float(x))


def best_subset(scores: dict[int, Fraction], m: int) -> tuple[int, ...]:
    """Among all m-subsets of the candidate ids, the one with the largest exact
    score sum; among equal sums the lexicographically smallest sorted tuple
    (so a tie is resolved toward lower ids)."""
    best, best_sum = None, None
    for sub in itertools.combinations(sorted(scores), m):
        s = sum((scores[c] for c in sub), Fraction(0))
        if best is None or s > best_sum or (s == best_sum and sub < best):
            best, best_sum = sub, s
    return best if best is not None else ()


def _box_score(qv, lo, hi) -> Fraction:
    """max <q, x> over the corners x of the box [lo, hi] (exact)."""
    best = None
    for corner in itertools.product((0, 1), repeat=len(qv)):
        s = sum(((hi[e] if bit else lo[e]) * qv[e] for e, bit in enumerate(corner)),
                Fraction(0))
        if best is None or s > best:
            best = s
    return best


def forward(q, k, v, *, block_size=0, top_k=0, window=0, idx_q=None, idx_k=None,
            token_top_k=0, sink=None, scale=None, gate_repr="mean", gate_shared=False,
            gate_first=False, cmp_block=0):
    """Returns (out [Bt,Hq,Nq,d], lse [Bt,Hq,Nq], sel dict, tsel dict, count).

    q may hold fewer rows (Nq) than k, v (Nk): query row iq is then the token
    at position iq + Nk - Nq of the history (the causal offset of the
    Bit-Axon page); under block gating it is gated as that position of a
    prefill (candidates: the complete blocks before its own)."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    Bt, Hq, Nq, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    off = N - Nq
    assert off >= 0
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = np.zeros((Bt, Hq, Nq, d))
    lse = np.zeros((Bt, Hq, Nq))
    count = np.zeros((Bt, Hq, Nq), dtype=np.int64)
    sels, tsels = {}, {}
    for b in range(Bt):
        tok = {}
        if token_top_k:
            for iq in range(Nq):
                i = iq + off
                sc = {j: sum((_frac(idx_q[b, iq, e]) * _frac(idx_k[b, j, e])
                              for e in range(idx_q.shape[2])), Fraction(0))
                      for j in range(i)}
                tok[i] = set(best_subset(sc, min(token_top_k, i)))
                tsels[(b, iq)] = tok[i]
        def head_score(h, iq, c):
            """Exact gate score of query iq of head h against block c."""
            g = h // G
            rows = range(c * block_size, (c + 1) * block_size)
            qv = [_frac(q[b, h, iq, e]) for e in range(d)]
            if gate_repr == "minmax":
                lo = [min(_frac(k[b, g, j, e]) for j in rows) for e in range(d)]
                hi = [max(_frac(k[b, g, j, e]) for j in rows) for e in range(d)]
                return _box_score(qv, lo, hi)
            mean = [sum((_frac(k[b, g, j, e]) for j in rows), Fraction(0)) / block_size
                    for e in range(d)]
            return sum((qv[e] * mean[e] for e in range(d)), Fraction(0))

        for h in range(Hq):
            g = h // G
            for iq in range(Nq):
                i = iq + off
                chosen = set()
                if top_k:
                    own = i // block_size
                    forced = {own} | ({0} if gate_first and own > 0 else set())
                    heads = range(g * G, (g + 1) * G) if gate_shared else (h,)
                    sc = {c: sum((head_score(hh, iq, c) for hh in heads), Fraction(0))
                          for c in range(own) if c not in forced}
                    m = min(top_k - len(forced), len(sc))
                    chosen = set(best_subset(sc, m)) | forced
                    sels[(b, h, iq)] = chosen
                keys = []
                for j in range(N):
                    causal = j <= i
                    in_window = window > 0 and i - j < window
                    in_block = bool(top_k) and (j // block_size) in chosen
                    in_tokens = bool(token_top_k) and j in tok[i]
                    if causal and (in_window or in_block or in_tokens):
                        keys.append(j)
                logits = [scale * sum(q[b, h, iq, e] * k[b, g, j, e] for e in range(d))
                          for j in keys]
                vals = [[v[b, g, j, e] for e in range(d)] for j in keys]
                if cmp_block:
                    for c in range(N // cmp_block):
                        grp = range(c * cmp_block, (c + 1) * cmp_block)
                        if grp[-1] > i:
                            continue
                        kc = [float(sum((_frac(k[b, g, j, e]) for j in grp), Fraction(0)) / cmp_block)
                              for e in range(d)]
                        vc = [float(sum((_frac(v[b, g, j, e]) for j in grp), Fraction(0)) / cmp_block)
                              for e in range(d)]
                        logits.append(scale * sum(q[b, h, iq, e] * kc[e] for e in range(d)))
                        vals.append(vc)
                z = None if sink is None else float(sink[h])
                M = max(logits + ([z] if z is not None else []), default=-math.inf)
                w = [math.exp(x - M) for x in logits]
                L = sum(w) + (math.exp(z - M) if z is not None else 0.0)
                for e in range(d):
                    out[b, h, iq, e] = sum(wj * vj[e] for wj, vj in zip(w, vals)) / L
                lse[b, h, iq] = M + math.log(L)
                count[b, h, iq] = len(logits)
    return out, lse, sels, tsels, count
