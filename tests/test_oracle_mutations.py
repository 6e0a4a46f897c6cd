"""The pins must catch plausible mistakes in the oracle.  Each case plants
one bug into a copy of oracle.c (on the CPU), builds it, and checks that at
least one pin of test_oracle_pins.py fails against it."""
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

MUTATIONS = [
    ("window admits w+1 keys", [("(i - window + 1 > 0 ? i - window + 1 : 0)", "(i - window > 0 ? i - window : 0)")]),
    ("tie goes to the higher index", [("if (a->idx < b->idx) return -1;", "if (a->idx < b->idx) return 1;")]),
    ("own block not counted in k", [("const int64_t m = (top_k - 1 < own) ? top_k - 1 : own;",
                                     "const int64_t m = (top_k < own) ? top_k : own;")]),
    ("own block competes instead of being forced", [
        ("for (int64_t c = 0; c < own; ++c) {\n                cand[c].s",
         "for (int64_t c = 0; c <= own; ++c) {\n                cand[c].s"),
        ("qsort(cand, (size_t)own, sizeof(cand_t), cand_cmp);\n            const int64_t m = (top_k - 1 < own) ? top_k - 1 : own;",
         "qsort(cand, (size_t)(own + 1), sizeof(cand_t), cand_cmp);\n            const int64_t m = (top_k < own + 1) ? top_k : own + 1;"),
        ("out[m] = (int32_t)own;\n            qsort(out, (size_t)(m + 1)", "qsort(out, (size_t)m")]),
    ("sink logit scaled", [("const double z = sink ? (double)sink[h] : -INFINITY;",
                            "const double z = sink ? scale * (double)sink[h] : -INFINITY;")]),
    ("softmax scale dropped", [("x[j] = scale * acc;", "x[j] = acc;")]),
    ("wrong GQA head mapping", [("b = bh / Hq, h = bh % Hq, g = h / G;\n            memset",
                                 "b = bh / Hq, h = bh % Hq, g = h % Hkv;\n            memset")]),
    ("token candidates include j = i", [
        ("for (int64_t j = 0; j < i; ++j) {\n                double acc",
         "for (int64_t j = 0; j <= i; ++j) {\n                double acc"),
        ("qsort(cand, (size_t)i, sizeof(cand_t), cand_cmp);", "qsort(cand, (size_t)(i + 1), sizeof(cand_t), cand_cmp);")]),
    ("token selection keeps one too few", [("const int64_t m = Kt < i ? Kt : i;", "const int64_t m = Kt - 1 < i ? Kt - 1 : i;")]),
    ("lse without the max", [("lse[t] = M + log(L);", "lse[t] = log(L);")]),
    ("pool divides by B - 1", [("dst[e] = acc / (double)B;", "dst[e] = acc / (double)(B - 1);")]),
    ("decode attention ignores the offset", [("const int64_t i = r % Nq + off, bh = r / Nq,",
                                              "const int64_t i = r % Nq, bh = r / Nq,")]),
    ("decode token select ignores the offset", [
        ("i = r % Nq + off, b = r / Nq;\n            for (int64_t j = 0; j < i; ++j) {",
         "i = r % Nq, b = r / Nq;\n            for (int64_t j = 0; j < i; ++j) {")]),
]

PIN_CALLS = [
    lambda: pins.test_p1_all_blocks_is_dense_causal(0),
    lambda: pins.test_p2_window_matches_sdpa_mask(5),
    lambda: pins.test_p3_window_one_is_identity(),
    lambda: pins.test_p4_topk_one_is_blockwise_causal(),
    lambda: pins.test_p5_ties_go_to_lower_block(),
    lambda: pins.test_p6_printed_sparsity(),
] + [
    (lambda c=c, t=t: pins.test_p7_brute_force(c, t))
    for c in range(len(pins.BRUTE_CASES)) for t in (False, True)
] + [
    lambda: pins.test_p8_gqa_is_repeated_mha(),
    lambda: pins.test_p9_sink_closed_form(),
    lambda: pins.test_p10_token_selection_cases(),
    lambda: pins.test_pool_is_block_mean(),
] + [
    (lambda c=c, n=n: pins.test_p15_decode_is_last_prefill_rows(c, n))
    for c in range(len(pins.DECODE_CASES)) for n in (1, 5)
] + [
    (lambda c=c: pins.test_p16_decode_brute_force(c, False)) for c in range(len(pins.DECODE_CASES))
]


@pytest.mark.parametrize("name,edits", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(name, edits, tmp_path):
    src = open(oracle._SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, f"mutation anchor not unique: {name}"
        src = src.replace(old, new)
    c = tmp_path / "mutant.c"
    c.write_text(src)
    so = tmp_path / "mutant.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"])
    caught = []
    with oracle.use_library(str(so)):
        for call in PIN_CALLS:
            try:
                call()
            except (AssertionError, ValueError, IndexError):
                caught.append(call)
    assert caught, f"no pin caught: {name}"
