"""The far-block list checker (sparse_attn_check_far_lists) against planted
faults, on the CPU.

Block gating regroups query rows by kept far block (MoBA summary page, "MoBA의
구현: MoE와 FlashAttention의 결합", steps 1-2).  build_lists below writes such
lists from a selection in plain Python, following the layout stated in the C
header (entry (i G + h_local) kslots + x under list (b, g, block), the chunk
table, the fixed (floor(i/64), h_local, x, i mod 64) order).  The checker
must accept them, accept them shuffled when no order is asked for, and reject
every planted fault: an entry moved to another list, listed twice, naming the
wrong slot, a row past N, a negative entry, shifted offsets or chunk counts,
a wrong chunk table, a truncated chunk count, a missing entry, a near block
listed as far (or a far one left out), too many entries or chunks for the
workspace, and a selection that no longer matches.  Random corruptions must
be rejected without a crash."""
import numpy as np
import pytest

import sliding_window_long_amd as sa

SA_OK, SA_E_CHECK = 0, -10


def make_sel(Bt, Hq, N, B, K, rng):
    """Ascending selections: up to K-1 distinct earlier blocks, then the own
    block, then -1."""
    sel = np.full((Bt, Hq, N, K), -1, dtype=np.int32)
    for b in range(Bt):
        for h in range(Hq):
            for i in range(N):
                bi = i // B
                m = min(K - 1, bi)
                past = np.sort(rng.choice(bi, size=m, replace=False)) if m else np.zeros(0, int)
                sel[b, h, i, :m] = past
                sel[b, h, i, m] = bi
    return sel


def build_lists(sel, Hkv, B, span, kslots, R):
    Bt, Hq, N, K = sel.shape
    G, n = Hq // Hkv, N // B
    lists = [[] for _ in range(Bt * Hkv * n)]
    for b in range(Bt):
        for g in range(Hkv):
            for i64 in range((N + 63) // 64):
                for hl in range(G):
                    for x in range(K):
                        for lane in range(64):
                            i = i64 * 64 + lane
                            if i >= N:
                                continue
                            row = sel[b, g * G + hl, i]
                            far = all(row[xx] >= 0 and i // B - row[xx] > span for xx in range(x + 1))
                            if far:
                                lists[(b * Hkv + g) * n + row[x]].append((i * G + hl) * kslots + x)
    off = np.zeros(len(lists) + 1, dtype=np.int64)
    ch = np.zeros(len(lists) + 1, dtype=np.int64)
    for l, e in enumerate(lists):
        off[l + 1] = off[l] + len(e)
        ch[l + 1] = ch[l] + (len(e) + R - 1) // R
    chunk_list, chunk_start = [], []
    for l in range(len(lists)):
        for q in range(ch[l], ch[l + 1]):
            chunk_list.append(l)
            chunk_start.append(off[l] + (q - ch[l]) * R)
    entries = np.array([x for e in lists for x in e], dtype=np.int32)
    return dict(list_off=off, list_ch=ch, chunk_list=np.array(chunk_list, dtype=np.int32),
                chunk_start=np.array(chunk_start, dtype=np.int32), entries=entries)


SHAPE = dict(batch=2, n_q_heads=4, n_kv_heads=2, seq_len=320, block_size=16, top_k=6)
SPAN, R = 2, 8


@pytest.fixture(scope="module")
def case():
    sa.load_library()
    rng = np.random.default_rng(5)
    sel = make_sel(SHAPE["batch"], SHAPE["n_q_heads"], SHAPE["seq_len"], SHAPE["block_size"],
                   SHAPE["top_k"], rng)
    kslots = SHAPE["top_k"] - 1
    L = build_lists(sel, SHAPE["n_kv_heads"], SHAPE["block_size"], SPAN, kslots, R)
    assert L["entries"].size > 500 and L["chunk_list"].size > 100   # a non-trivial case
    return sel, L


def run(sel, L, *, ordered=True, span=SPAN, max_entries=None, max_chunks=None):
    return sa.sparse_attn_check_far_lists(
        **SHAPE, span=span, kslots=SHAPE["top_k"] - 1, rows_per_chunk=R, ordered=ordered, sel=sel,
        max_entries=L["entries"].size if max_entries is None else max_entries,
        max_chunks=L["chunk_list"].size if max_chunks is None else max_chunks, **L)


def copy(L):
    return {k: v.copy() for k, v in L.items()}


def test_clean_lists_pass(case):
    sel, L = case
    assert run(sel, L) == (SA_OK, "")
    assert run(sel, L, ordered=False) == (SA_OK, "")
    # generous limits pass too
    assert run(sel, L, max_entries=10 ** 7, max_chunks=10 ** 6)[0] == SA_OK


def test_shuffled_lists_need_no_order(case):
    sel, L = case
    L2 = copy(L)
    rng = np.random.default_rng(1)
    off = L2["list_off"]
    for l in range(off.size - 1):
        seg = L2["entries"][off[l]:off[l + 1]]
        rng.shuffle(seg)
    assert run(sel, L2, ordered=False)[0] == SA_OK
    rc, msg = run(sel, L2, ordered=True)
    assert rc == SA_E_CHECK and "out of order" in msg


def nonempty_lists(L):
    off = L["list_off"]
    return [l for l in range(off.size - 1) if off[l + 1] - off[l] >= 3]


def plant(L, sel, fault):
    """Return (lists, selection, kwargs) with one planted fault."""
    L2, sel2, kw = copy(L), sel.copy(), {}
    off, ent = L2["list_off"], L2["entries"]
    ne = nonempty_lists(L2)
    la, lb = ne[3], ne[-2]
    if fault == "moved_to_other_list":
        ea, eb = off[la] + 1, off[lb] + 1
        ent[ea], ent[eb] = ent[eb], ent[ea]
    elif fault == "listed_twice":
        ent[off[la] + 2] = ent[off[la] + 1]
    elif fault == "wrong_slot":
        e = off[la] + 1
        ent[e] = ent[e] + 1 if ent[e] % (SHAPE["top_k"] - 1) < SHAPE["top_k"] - 2 else ent[e] - 1
    elif fault == "row_past_n":
        ent[off[la]] = (SHAPE["seq_len"] * 2 + 1) * (SHAPE["top_k"] - 1)
    elif fault == "negative_entry":
        ent[off[lb]] = -7
    elif fault == "offset_shifted":
        off[la + 1] += 1
    elif fault == "chunk_count_off":
        L2["list_ch"][la + 1] += 1
        L2["list_ch"][la + 2:] += 1
    elif fault == "chunk_start_off":
        L2["chunk_start"][5] += 1
    elif fault == "chunk_list_wrong":
        q = L2["list_ch"][lb]
        L2["chunk_list"][q] = la
    elif fault == "chunks_truncated":
        L2["chunk_list"] = L2["chunk_list"][:-1].copy()
        L2["chunk_start"] = L2["chunk_start"][:-1].copy()
    elif fault == "entry_missing":
        # drop the last entry of list lb, keeping offsets and chunks consistent
        e = off[lb + 1] - 1
        L2["entries"] = np.delete(ent, e)
        off[lb + 1:] -= 1
        R_ = R
        ch = L2["list_ch"]
        for l in range(off.size - 1):
            ch[l + 1] = ch[l] + (off[l + 1] - off[l] + R_ - 1) // R_
        cl, cs = [], []
        for l in range(off.size - 1):
            for q in range(ch[l], ch[l + 1]):
                cl.append(l)
                cs.append(off[l] + (q - ch[l]) * R_)
        L2["chunk_list"], L2["chunk_start"] = np.array(cl, np.int32), np.array(cs, np.int32)
    elif fault == "near_block_listed":
        kw["span"] = SPAN + 1
    elif fault == "far_block_unlisted":
        kw["span"] = SPAN - 1
    elif fault == "too_many_entries":
        kw["max_entries"] = ent.size - 1
    elif fault == "too_many_chunks":
        kw["max_chunks"] = L2["chunk_list"].size - 1
    elif fault == "selection_changed":
        # a listed far slot now holds another block
        e = off[la]
        x = ent[e] % (SHAPE["top_k"] - 1)
        t2 = ent[e] // (SHAPE["top_k"] - 1)
        G = SHAPE["n_q_heads"] // SHAPE["n_kv_heads"]
        hl, i = t2 % G, t2 // G
        n = SHAPE["seq_len"] // SHAPE["block_size"]
        bg = la // n
        b, g = bg // SHAPE["n_kv_heads"], bg % SHAPE["n_kv_heads"]
        sel2[b, g * G + hl, i, x] += 1 if x == 0 else -1
    else:
        raise AssertionError(fault)
    return L2, sel2, kw


FAULTS = ["moved_to_other_list", "listed_twice", "wrong_slot", "row_past_n", "negative_entry",
          "offset_shifted", "chunk_count_off", "chunk_start_off", "chunk_list_wrong",
          "chunks_truncated", "entry_missing", "near_block_listed", "far_block_unlisted",
          "too_many_entries", "too_many_chunks", "selection_changed"]


@pytest.mark.parametrize("fault", FAULTS)
def test_planted_fault_caught(case, fault):
    sel, L = case
    L2, sel2, kw = plant(L, sel, fault)
    for ordered in (True, False):
        rc, msg = run(sel2, L2, ordered=ordered, **kw)
        assert rc == SA_E_CHECK, f"{fault} (ordered={ordered}) not caught"
        assert msg, "a violation comes with a message"


def test_random_corruption_rejected_without_crash(case):
    sel, L = case
    rng = np.random.default_rng(11)
    names = ["entries", "list_off", "list_ch", "chunk_list", "chunk_start"]
    for _ in range(300):
        L2 = copy(L)
        a = L2[names[rng.integers(len(names))]]
        j = rng.integers(a.size)
        v = int(rng.choice([rng.integers(-2 ** 31, 2 ** 31), int(a[j]) + int(rng.integers(1, 5)),
                            int(a[j]) - int(rng.integers(1, 5))]))
        v = max(min(v, 2 ** 31 - 1), -2 ** 31)
        if v == a[j]:
            continue
        a[j] = v
        if int(L2["list_off"][-1]) > L2["entries"].size:
            continue   # the binding refuses entries shorter than list_off says
        rc, _ = run(sel, L2)
        assert rc == SA_E_CHECK


def test_bad_arguments(case):
    sel, L = case
    rc, _ = sa.sparse_attn_check_far_lists(
        **dict(SHAPE, top_k=0), span=SPAN, kslots=5, rows_per_chunk=R, ordered=True, sel=np.zeros(0),
        max_entries=0, max_chunks=0, list_off=L["list_off"], list_ch=L["list_ch"],
        chunk_list=L["chunk_list"], chunk_start=L["chunk_start"], entries=L["entries"])
    assert rc == -1   # SA_E_INVALID_ARG
