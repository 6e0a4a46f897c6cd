"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, and rejects bad arguments with the documented codes before any
GPU work.  No kernel is launched here."""
import ctypes
import os
import re

import pytest

import sliding_window_long_amd as sa
from sliding_window_long_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from sliding_window_long_amd.build import build_library
        build_library()
    return sa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(sa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def a256(n):
    return (n + 255) // 256 * 256


def v_copy_bytes(heads, N, row):
    """The fp16 V copy (rows of `row` elements), its per-128-row chunk maxima
    and the per-head scale exponents, each region 256-byte aligned."""
    return a256(heads * N * row * 2) + a256(heads * ((N + 127) // 128) * 4) + a256(heads * 4)


def test_struct_layout_matches(lib):
    # The library rejects any struct_size other than its own sizeof.
    cfg = sa.Params(1, 4, 4, 256, 64, window=16).cfg()
    assert sa.sparse_attn_workspace_bytes(cfg) == v_copy_bytes(4, 256, 64)
    cfg.struct_size = ctypes.sizeof(binding.SparseAttnCfg) - 8
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_workspace_bytes(cfg)
    assert e.value.code == -1


def code_of(params, **cfg_fields):
    cfg = params.cfg()
    for k_, v_ in cfg_fields.items():
        setattr(cfg, k_, v_)
    n = ctypes.c_size_t()
    return sa.load_library().sparse_attn_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n))


@pytest.mark.parametrize("params,code", [
    (sa.Params(0, 4, 4, 256, 64, window=8), -1),                      # batch < 1
    (sa.Params(1, 4, 4, 256, 64, window=-1, top_k=1, block_size=64), -1),
    (sa.Params(1, 4, 4, 256, 64, dtype=7, window=8), -1),
    (sa.Params(1, 4, 4, 256, 96, window=8), -3),                      # head dim
    (sa.Params(1, 6, 4, 256, 64, window=8), -2),                      # Hq % Hkv
    (sa.Params(1, 4, 4, 256, 64), -4),                                # no window, no gate
    (sa.Params(1, 4, 4, 250, 64, block_size=64, top_k=2), -2),        # N % B
    (sa.Params(1, 4, 4, 256, 64, block_size=48, top_k=2), -2),        # B neither 8, 16, 32 nor a multiple of 64
    (sa.Params(1, 4, 4, 256, 64, block_size=4, top_k=2), -2),         # B below 8
    (sa.Params(1, 4, 4, 256, 64, block_size=64, top_k=5), -2),        # top_k > n
    (sa.Params(1, 34, 1, 256, 64, window=8), -8),                     # group > 16
    (sa.Params(1, 4, 4, 64 * 40, 64, block_size=64, top_k=34), -8),   # top_k > 33
    (sa.Params(1, 4, 4, 256, 64, window=8, softmax_scale=-1.0), -1),
    (sa.Params(1, 4, 1, 256, 128, window=8, token_top_k=16, index_dim=32), -3),
    (sa.Params(1, 4, 1, (1 << 24) + 64, 128, window=8, token_top_k=16, index_dim=64), -8),   # ids past 2^24
    (sa.Params(1, 4, 1, 256, 128, window=8, block_size=64, top_k=2, token_top_k=16,
               index_dim=64), -8),
    (sa.Params(1, 1, 1, 1 << 23, 128, window=8), -8),                # one head's K past 2 GiB
    (sa.Params(1, 4, 4, 64 * 80, 64, block_size=64, top_k=3, window=64 * 65 + 1), -8),  # 65 near blocks
    (sa.Params(1, 4, 4, 256, 64, window=8, kv_len=255), -1),          # fewer keys than queries
    (sa.Params(1, 4, 4, 256, 64, window=8, kv_len=-1), -1),
    # decode with a block gate: at most 4096 complete blocks, top 64, and a
    # shared selection over at most 16 heads a group
    (sa.Params(1, 34, 2, 4, 64, block_size=64, top_k=2, kv_len=256, gate_shared=1), -8),
    (sa.Params(1, 4, 4, 4, 64, block_size=64, top_k=1, kv_len=256, gate_first=1), -1),
    (sa.Params(1, 4, 4, 4, 64, block_size=48, top_k=2, kv_len=256), -2),
    (sa.Params(1, 4, 4, 4, 64, block_size=64, top_k=5, kv_len=250), -2),     # 4 blocks
    (sa.Params(1, 1, 1, 1, 64, block_size=8, top_k=2, kv_len=8 * 4097), -8),
    (sa.Params(1, 1, 1, 1, 64, block_size=8, top_k=65, kv_len=8 * 100), -8),
    (sa.Params(1, 4, 4, 65, 64, window=8, kv_len=256), -8),           # decode past 64 queries
    (sa.Params(1, 4, 1, 1, 128, window=8, token_top_k=16, index_dim=64,
               kv_len=65536 + 1), -8),                               # decode: 16-bit token ids
    (sa.Params(1, 4, 4, 1, 64, kv_len=256), -4),                      # decode, no window
    (sa.Params(1, 4, 4, 256, 64, block_size=64, top_k=2, gate_repr=2), -1),   # unknown summary
    (sa.Params(1, 4, 4, 256, 64, block_size=64, top_k=2, gate_shared=2), -1),
    (sa.Params(1, 4, 4, 256, 64, block_size=64, top_k=2, gate_first=-1), -1),
    (sa.Params(1, 4, 4, 256, 64, window=8, gate_repr=1), -1),         # variant without a gate
    (sa.Params(1, 4, 4, 256, 64, window=8, gate_shared=1), -1),
    (sa.Params(1, 4, 4, 256, 64, window=8, gate_first=1), -1),
    (sa.Params(1, 4, 4, 256, 64, block_size=64, top_k=1, gate_first=1), -1),  # no slot for block 0
    (sa.Params(1, 4, 4, 256, 64, window=8, cmp_block=-8), -1),
    (sa.Params(1, 4, 4, 1, 64, window=8, kv_len=256, cmp_block=8), -8),       # decode + compressed
    (sa.Params(1, 4, 1, 256, 128, window=8, token_top_k=16, index_dim=64, cmp_block=8), -8),
])
def test_invalid_configs(lib, params, code):
    assert code_of(params) == code


def test_valid_configs(lib):
    for p in (sa.Params(1, 1, 1, 512, 64, dtype=sa.SA_F32, block_size=64, top_k=3),
              sa.Params(2, 8, 4, 4096, 128, block_size=128, top_k=16, window=512),
              sa.Params(1, 32, 32, 16384, 80, window=4096),
              sa.Params(1, 32, 8, 131072, 128, block_size=512, top_k=8),
              sa.Params(1, 3, 3, 77, 80, window=1),
              sa.Params(1, 16, 4, 65536, 128, window=128, token_top_k=2048, index_dim=64),
              sa.Params(1, 32, 32, 1, 80, window=4096, kv_len=16384),
              sa.Params(4, 16, 4, 64, 128, window=128, token_top_k=2048, index_dim=64,
                        kv_len=65536),
              sa.Params(1, 8, 8, 16, 64, window=4, kv_len=16),      # kv_len = seq_len: prefill
              sa.Params(1, 32, 8, 131072, 128, block_size=512, top_k=8, gate_repr=1),
              sa.Params(2, 8, 4, 4096, 128, block_size=128, top_k=16, window=512,
                        gate_shared=1, gate_first=1),
              sa.Params(1, 1, 1, 512, 64, dtype=sa.SA_F32, block_size=64, top_k=2,
                        gate_repr=1, gate_first=1),
              sa.Params(1, 32, 32, 16384, 80, dtype=sa.SA_FP8, window=4096),
              sa.Params(4, 16, 4, 64, 128, dtype=sa.SA_FP8, window=128, token_top_k=2048,
                        index_dim=64, kv_len=65536)):
        assert code_of(p) == 0


def test_compressed_workspace(lib):
    # compressed K and V [Bt, Hkv, N/C, d] (one 16-bit plane each, two for
    # fp32) plus the other branches' fp32 out [Bt, Hq, N, d]
    base = dict(block_size=128, top_k=16, window=512)
    ws = lambda **kw: sa.sparse_attn_workspace_bytes(sa.Params(2, 8, 4, 4096, 128, **base, **kw).cfg())
    ncmp = 2 * 4 * 512 * 128
    delta = ws(cmp_block=8) - ws()
    assert 2 * ncmp * 2 + 2 * 8 * 4096 * 128 * 4 <= delta <= 2 * ncmp * 2 + 2 * 8 * 4096 * 128 * 4 + 768
    assert code_of(sa.Params(1, 2, 2, 100, 64, window=4, cmp_block=1000)) == 0   # no complete group


def test_gate_variant_workspace(lib):
    # min/max summaries: 2 bf16 planes per block for bf16 keys, as many as
    # the mean's two terms; 6 for fp32 keys (3 for the mean); a shared
    # selection adds the group-summed
    # queries as two bf16 planes [Bt, Hkv, N, d] (four for min/max: the
    # positive and the negative parts)
    base = dict(block_size=128, top_k=4, window=128)
    ws = lambda **kw: sa.sparse_attn_workspace_bytes(sa.Params(2, 8, 4, 4096, 128, **base, **kw).cfg())
    lists = 2 * 4 * 32
    assert ws() == ws(gate_repr=1)
    assert ws(gate_shared=1) - ws() == 2 * 2 * 4 * 4096 * 128 * 2
    assert ws(gate_shared=1, gate_repr=1) - ws(gate_repr=1) == 4 * 2 * 4 * 4096 * 128 * 2
    assert ws(gate_first=1) == ws()
    f32 = lambda **kw: sa.sparse_attn_workspace_bytes(
        sa.Params(1, 2, 2, 512, 64, dtype=sa.SA_F32, block_size=64, top_k=3, **kw).cfg())
    assert f32(gate_repr=1) - f32() == 3 * 2 * 8 * 64 * 2


def test_decode_workspace(lib):
    # partials [rows, ceil((min(w, kv_len) + top_t) / 64), d + 2] fp32 (one
    # per 64-key tile), plus indexer scores [Bt, Nq, kv_len] and the kept lists
    p = sa.Params(1, 32, 32, 1, 80, window=4096, kv_len=16384)
    assert sa.sparse_attn_workspace_bytes(p.cfg()) == 32 * 64 * 82 * 4
    p = sa.Params(2, 16, 4, 3, 128, window=128, token_top_k=2048, index_dim=64, kv_len=65536)
    assert sa.sparse_attn_workspace_bytes(p.cfg()) >= 2 * 3 * 65536 * 4 + 2 * 16 * 3 * 34 * 130 * 4


def test_workspace_sizes_scale(lib):
    # block gating with far blocks: partials
    # [rows, top_k-1, d] fp16 dominate.
    # window only: an fp16 copy of V, rows padded to 96 at d 80 (ones in the
    # padding columns feed the row sums), unpadded at d 64 and 128
    assert sa.sparse_attn_workspace_bytes(sa.Params(1, 32, 32, 16384, 80, window=4096).cfg()) == v_copy_bytes(32, 16384, 96)
    assert sa.sparse_attn_workspace_bytes(sa.Params(1, 8, 8, 4096, 128, window=512).cfg()) == v_copy_bytes(8, 4096, 128)
    assert sa.sparse_attn_workspace_bytes(sa.Params(1, 8, 8, 4096, 64, window=512).cfg()) == v_copy_bytes(8, 4096, 64)
    p = sa.Params(1, 32, 8, 131072, 128, block_size=512, top_k=8)
    rows = 32 * 131072
    assert sa.sparse_attn_workspace_bytes(p.cfg()) >= rows * 7 * 128 * 2


def fwd_code(params, q=0x1000, k=0x2000, v=0x3000, out=0x4000, lse=0x5000, **cfg_fields):
    """Call sparse_attn_fwd with fake device addresses; only checks that
    reject the call before any launch are exercised."""
    cfg = params.cfg()
    for k_, v_ in cfg_fields.items():
        setattr(cfg, k_, v_)
    return sa.load_library().sparse_attn_fwd(
        ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(v), ctypes.byref(cfg),
        ctypes.c_void_p(out), ctypes.c_void_p(lse))


def test_token_workspace(lib):
    # keep-mask words [N/32][N/64][64] plus per-row select state
    p = sa.Params(1, 16, 4, 65536, 128, window=128, token_top_k=2048, index_dim=64)
    assert sa.sparse_attn_workspace_bytes(p.cfg()) >= 2048 * 1024 * 64 * 4 + 65536 * 16


def test_fwd_rejects_before_launch(lib):
    p = sa.Params(1, 4, 4, 256, 64, window=8)
    assert fwd_code(p, q=0) == -1                       # null q
    assert fwd_code(p, lse=0) == -1
    assert fwd_code(p, q=0x1008) == -5                  # misaligned q
    assert fwd_code(p, out=0x4004) == -5
    assert fwd_code(p, lse=0x5002) == -5
    g = sa.Params(1, 4, 4, 256, 64, block_size=64, top_k=2)
    need = sa.sparse_attn_workspace_bytes(g.cfg())
    assert need > 0
    assert fwd_code(g, workspace=0x10000, workspace_bytes=need - 1) == -6
    assert fwd_code(g, workspace=0, workspace_bytes=0) == -6
    t = sa.Params(1, 4, 1, 256, 64, window=8, token_top_k=16, index_dim=64)
    need = sa.sparse_attn_workspace_bytes(t.cfg())
    assert fwd_code(t, workspace=0x10000, workspace_bytes=need) == -1          # no indexer inputs
    assert fwd_code(t) == -1                                # checked before the workspace
    assert fwd_code(t, workspace=0x10000, workspace_bytes=need, idx_q=0x20008,
                    idx_k=0x30000) == -5                                         # misaligned idx_q


def test_strerror_covers_codes(lib):
    for c in range(-9, 1):
        assert sa.sparse_attn_strerror(c) != "unknown status"
    assert sa.sparse_attn_strerror(-99) == "unknown status"


def test_stage_times_without_timing(lib):
    assert isinstance(sa.sparse_attn_stage_times(), list)


def test_backward_configs(lib):
    ws = lambda p: sa.load_library().sparse_attn_bwd_workspace_bytes(
        ctypes.byref(p.cfg()), ctypes.byref(ctypes.c_size_t()))
    assert ws(sa.Params(2, 8, 4, 4096, 128, block_size=128, top_k=16, window=512)) == 0
    assert ws(sa.Params(1, 32, 32, 16384, 80, window=4096)) == 0
    assert ws(sa.Params(1, 2, 2, 512, 64, dtype=sa.SA_F32, window=8)) == -8           # fp32
    assert ws(sa.Params(1, 4, 1, 256, 128, window=8, token_top_k=16, index_dim=64)) == 0
    assert ws(sa.Params(1, 4, 4, 256, 64, window=8, cmp_block=8)) == 0
    assert ws(sa.Params(1, 4, 4, 1, 64, window=8, kv_len=256)) == -8                 # decode
    # fp16 copies of q, k and dO plus the row deltas; no far partials; then
    # the copies' range data: per-128-row maxima of q, dO (4 heads) and k, v
    # (2 kv heads), the largest |dO| and |v| and five exponents per kv head
    # (each region rounded up to 256 bytes)
    p = sa.Params(1, 4, 2, 512, 64, window=16)
    n = ctypes.c_size_t()
    sa.load_library().sparse_attn_bwd_workspace_bytes(ctypes.byref(p.cfg()), ctypes.byref(n))
    a256 = lambda x: (x + 255) // 256 * 256
    ranges = 2 * a256(4 * 4 * 4) + 2 * a256(2 * 4 * 4) + a256(2 * 2 * 4) + a256(2 * 5 * 4)
    base = (2 * 512 * 64 * 2) + 2 * (4 * 512 * 64 * 2) + 4 * 512 * 4 + ranges
    assert n.value == base
    # the compressed branch (groups of 8): bf16 K means and their scaled fp16
    # copy, bf16 V means, and fp32 dK, dV per group from 16 row ranges (two
    # key tiles of 128 groups are far fewer workgroups than the GPU holds)
    p = sa.Params(1, 4, 2, 512, 64, window=16, cmp_block=8)
    sa.load_library().sparse_attn_bwd_workspace_bytes(ctypes.byref(p.cfg()), ctypes.byref(n))
    ncmp = 2 * 64 * 64
    assert n.value == base + 3 * ncmp * 2 + 16 * 2 * ncmp * 4


def test_backward_rejects_before_launch(lib):
    p = sa.Params(1, 4, 4, 256, 64, window=8)
    f = lambda **kw: sa.load_library().sparse_attn_bwd(
        *[ctypes.c_void_p(kw.get(n_, 0x1000 * (i + 1))) for i, n_ in
          enumerate(("q", "k", "v", "out", "lse", "dout"))],
        ctypes.byref(p.cfg()), *[ctypes.c_void_p(kw.get(n_, 0x8000 * (i + 1))) for i, n_ in
                                 enumerate(("dq", "dk", "dv"))], ctypes.c_void_p(kw.get("dsink", 0)))
    assert f(q=0) == -1                        # null pointer
    assert f(dsink=0x9000) == -1               # a sink gradient without a sink
    assert f(q=0x1008) == -5                   # misaligned
    assert f() == -6                           # no workspace
    # the token gate: the indexer tensors are required and checked too
    p = sa.Params(1, 4, 1, 256, 64, window=8, token_top_k=16, index_dim=64)
    assert f() == -1                           # no idx_q / idx_k
    cfg = p.cfg()
    cfg.idx_q, cfg.idx_k = 0x20000, 0x30008
    g = lambda c: sa.load_library().sparse_attn_bwd(
        *[ctypes.c_void_p(0x1000 * (i + 1)) for i in range(6)], ctypes.byref(c),
        *[ctypes.c_void_p(0x8000 * (i + 1)) for i in range(3)], ctypes.c_void_p(0))
    assert g(cfg) == -5                        # misaligned idx_k
    cfg.idx_k = 0x30000
    assert g(cfg) == -6                        # no workspace


def test_fp8_workspace(lib):
    # A window-only FP8 prefill keeps q, k, v in fp8 (the attention kernel's
    # K Q^T on the FP8 matrix cores, V straight to its fp16 copy): the same
    # workspace as bf16.  With block gating, bf16 copies of q, k, v.
    ws = lambda dt, **kw: sa.sparse_attn_workspace_bytes(sa.Params(1, 4, 2, 1024, 64, dtype=dt, **kw).cfg())
    assert ws(sa.SA_FP8, window=16) == ws(sa.SA_BF16, window=16)
    g = dict(window=16, block_size=64, top_k=3)
    assert ws(sa.SA_FP8, **g) - ws(sa.SA_BF16, **g) == (4 + 2 + 2) * 1024 * 64 * 2
    p = sa.Params(1, 4, 2, 1024, 64, dtype=sa.SA_FP8, window=16)
    assert sa.load_library().sparse_attn_bwd_workspace_bytes(
        ctypes.byref(p.cfg()), ctypes.byref(ctypes.c_size_t())) == -8     # no fp8 backward
    p = sa.Params(1, 4, 2, 1024, 64, dtype=sa.SA_FP8, block_size=64, top_k=2)
    assert sa.load_library().sparse_attn_block_pool(
        ctypes.c_void_p(0x1000), ctypes.byref(p.cfg()), ctypes.c_void_p(0x2000)) == -8


def test_noalloc_rejects_before_launch(lib):
    # Too large for the static scratch: rejected before anything is enqueued.
    big = sa.Params(1, 32, 8, 131072, 128, block_size=512, top_k=8).cfg()
    assert sa.sparse_attn_workspace_bytes(big) > 128 << 20
    rc = lib.sparse_attn_fwd_noalloc(ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000),
                                     ctypes.c_void_p(0x30000), ctypes.byref(big),
                                     ctypes.c_void_p(0x40000), ctypes.c_void_p(0x50000))
    assert rc == -9
    # Argument checks as sparse_attn_fwd's.
    bad = sa.Params(1, 4, 3, 256, 64, window=8).cfg()
    assert lib.sparse_attn_fwd_noalloc(None, None, None, ctypes.byref(bad), None, None) == -2


def test_block_means_only_for_block_gated_decode(lib):
    # caller-kept block means serve a decode step under the block gate; any
    # other call with them set is an invalid argument (checked on the host)
    n = ctypes.c_size_t(0)
    for p in (sa.Params(1, 4, 4, 256, 64, block_size=64, top_k=2),         # prefill
              sa.Params(1, 4, 4, 4, 64, window=8, kv_len=256)):             # decode, no block gate
        cfg = p.cfg()
        cfg.block_means = 4096
        assert lib.sparse_attn_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)) == -1
    cfg = sa.Params(1, 4, 4, 4, 64, block_size=64, top_k=2, kv_len=256, gate_repr=1).cfg()
    cfg.block_means = 4096   # min/max summaries: not means
    assert lib.sparse_attn_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)) == -1
    cfg = sa.Params(1, 4, 4, 4, 64, block_size=64, top_k=2, kv_len=256).cfg()
    cfg.block_means = 4096
    assert lib.sparse_attn_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)) == 0
