"""The pins must catch plausible mistakes in the oracle.  Each case plants
one bug into a copy of oracle.c (on the CPU), builds it, and checks that at
least one pin of test_oracle_pins.py fails against it."""
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

MUTATIONS = [
    ("window admits w+1 keys", [("\n            if (window > 0)\n                for (int64_t j = (i - window + 1 > 0 ? i - window + 1 : 0)",
                                 "\n            if (window > 0)\n                for (int64_t j = (i - window > 0 ? i - window : 0)")]),
    ("backward window admits w+1 keys", [("                    if (window > 0)\n                        for (int64_t j = (i - window + 1 > 0 ? i - window + 1 : 0)",
                                          "                    if (window > 0)\n                        for (int64_t j = (i - window > 0 ? i - window : 0)")]),
    ("tie goes to the higher index", [("if (a->idx < b->idx) return -1;", "if (a->idx < b->idx) return 1;")]),
    ("own block not counted in k", [("int64_t m = top_k - 1 - c0;", "int64_t m = top_k - c0;")]),
    ("own block competes instead of being forced", [
        ("const int64_t nc = own - c0;", "const int64_t nc = own + 1 - c0;"),
        ("for (int64_t c = c0; c < own && c < n; ++c) {\n                cand[c - c0].s",
         "for (int64_t c = c0; c <= own && c < n; ++c) {\n                cand[c - c0].s"),
        ("int64_t m = top_k - 1 - c0;", "int64_t m = top_k - c0;"),
        ("if (m < top_k) out[m] = (int32_t)own;\n            if (c0 && m + 1 < top_k) out[m + 1] = 0;\n"
         "            const int64_t kept = m + 1 + c0 < top_k ? m + 1 + c0 : top_k;",
         "if (c0 && m < top_k) out[m] = 0;\n            const int64_t kept = m + c0 < top_k ? m + c0 : top_k;")]),
    ("min/max score keeps only the max corner", [("acc += a > b ? a : b;", "acc += b;")]),
    ("min/max pool swaps min and max", [("lo[e] = mn;\n            hi[e] = mx;",
                                         "lo[e] = mx;\n            hi[e] = mn;")]),
    ("min/max score from the mean formula", [("if (rep == 0) {\n        for (int64_t e = 0; e < d; ++e) acc",
                                              "if (1) {\n        for (int64_t e = 0; e < d; ++e) acc")]),
    ("shared score from the own head only", [("for (int64_t hh = g * G; hh < (g + 1) * G; ++hh)",
                                              "for (int64_t hh = h; hh < h + 1; ++hh)")]),
    ("gate reads the wrong kv group", [("const int64_t G = Hq / Hkv, g = h / G;\n    const double* kbc",
                                        "const int64_t G = Hq / Hkv, g = h % Hkv;\n    const double* kbc")]),
    ("first block not counted in k", [("int64_t m = top_k - 1 - c0;", "int64_t m = top_k - 1;")]),
    ("first block forced as block 1", [("if (c0 && m + 1 < top_k) out[m + 1] = 0;",
                                       "if (c0 && m + 1 < top_k) out[m + 1] = 1;")]),
    ("first block also competes", [("const int64_t c0 = (first && own > 0) ? 1 : 0;\n        for (int64_t c = 0; c < n; ++c)",
                                    "const int64_t c0 = 0;\n        for (int64_t c = 0; c < n; ++c)"),
                                   ("const int64_t c0 = (first && own > 0 && top_k >= 2) ? 1 : 0;",
                                    "const int64_t c0 = 0;\n            if (first && own > 0) sel[t * top_k] = 0;")]),
    ("compressed group seen one token early", [("\n            const int64_t nvis = C > 0 ? (i + 1) / C : 0;",
                                                "\n            const int64_t nvis = C > 0 ? (i + 2) / C : 0;")]),
    ("compressed value is its key", [("\n                for (int64_t e = 0; e < d; ++e) o[e] += p * vcb[c * d + e];",
                                      "\n                for (int64_t e = 0; e < d; ++e) o[e] += p * kcb[c * d + e];")]),
    ("compressed logit unscaled", [("\n                xc[c] = scale * acc;", "\n                xc[c] = acc;")]),
    ("backward compressed group seen one token late", [
        ("\n                    const int64_t nvis = C > 0 ? (i + 1) / C : 0;",
         "\n                    const int64_t nvis = C > 0 ? i / C : 0;")]),
    ("backward compressed logit unscaled", [("\n                        xc[c] = scale * acc;",
                                             "\n                        xc[c] = acc;")]),
    ("backward compressed columns left out of the forward", [
        ("const double p = exp(xc[c] - M);\n                        L += p;",
         "const double p = 0.0 * exp(xc[c] - M);\n                        L += p;")]),
    ("backward compressed score gradient drops D", [("const double dsic = p * (dp - Di);",
                                                     "const double dsic = p * dp;")]),
    ("backward compressed dv from the query", [("dvc[c * d + e] += p * (double)dorow[e];",
                                                "dvc[c * d + e] += p * (double)qrow[e];")]),
    ("backward compressed dq from the group's value", [("dqr[e] += scale * dsic * kcb[c * d + e];",
                                                        "dqr[e] += scale * dsic * vcb[c * d + e];")]),
    ("backward group gradient not shared over its tokens", [
        ("dkb[j * d + e] += dkc[(j / C) * d + e] / (double)C;",
         "dkb[j * d + e] += dkc[(j / C) * d + e];")]),
    ("listed-output backward skips the last row", [("for (int64_t u = 0; u < G * (N - j); ++u) {",
                                                    "for (int64_t u = 0; u < G * (N - j) - 1; ++u) {")]),
    ("listed-output backward reads another head", [("const int64_t h = g * G + u / (N - j), i = j + u % (N - j);",
                                                    "const int64_t h = g + u / (N - j), i = j + u % (N - j);")]),
    ("listed-output dv from the query", [("acc_v[e] += p * (double)dout[r * d + e];",
                                          "acc_v[e] += p * (double)q[r * d + e];")]),
    ("listed-output dq without the D term", [
        ("const double ds = p * (dp - Di);\n                for (int64_t e = 0; e < d; ++e) dqr[e]",
         "const double ds = p * dp;\n                for (int64_t e = 0; e < d; ++e) dqr[e]")]),
    ("listed-output sink left out of the row", [("if (z > -INFINITY) L += exp(z - M);", "")]),
    ("backward group value gradient to the next group", [
        ("dvb[j * d + e] += dvc[(j / C) * d + e] / (double)C;",
         "dvb[j * d + e] += dvc[((j / C + 1) % Nc) * d + e] / (double)C;")]),
    ("compressed columns not counted", [("if (xc[c] > M) M = xc[c];\n                ++cnt;",
                                         "if (xc[c] > M) M = xc[c];")]),
    ("backward drops the D term", [("const double dsij = p * (dp - Di);", "const double dsij = p * dp;")]),
    ("backward dq without the scale", [("dqr[e] += scale * dsij * (double)kb[j * d + e];",
                                        "dqr[e] += dsij * (double)kb[j * d + e];")]),
    ("backward dv from unnormalised weights", [("dvb[j * d + e] += p * (double)dorow[e];",
                                                "dvb[j * d + e] += exp(x[j] - M) * (double)dorow[e];")]),
    ("backward sink gradient sign", [("if (sink) ds_h[h] += -exp(z - lse) * Di;",
                                      "if (sink) ds_h[h] += exp(z - lse) * Di;")]),
    ("sink logit scaled", [("\n            const double z = sink ? (double)sink[h] : -INFINITY;",
                            "\n            const double z = sink ? scale * (double)sink[h] : -INFINITY;")]),
    ("softmax scale dropped", [("\n                x[j] = scale * acc;", "\n                x[j] = acc;")]),
    ("backward softmax scale dropped", [("                        x[j] = scale * acc;",
                                         "                        x[j] = acc;")]),
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
    ("decode block select ignores the offset", [
        ("const int64_t rq = r % Nq, i = rq + off, bh = r / Nq,",
         "const int64_t rq = r % Nq, i = rq, bh = r / Nq,")]),
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
    lambda: pins.test_p17_minmax_block_of_one_is_dot_product(),
    lambda: pins.test_p18_minmax_bounds_and_box_corners(),
    lambda: pins.test_p20_shared_is_summed_query(),
] + [
    (lambda g=g: pins.test_p19_shared_with_one_head_per_group(g)) for g in ("mean", "minmax")
] + [
    (lambda g=g: pins.test_p21_first_block_top2_is_sink_pattern(g)) for g in ("mean", "minmax")
] + [
    (lambda g=g: pins.test_p22_first_block_is_gate_on_shifted_history(g)) for g in ("mean", "minmax")
] + [
    (lambda c=c, t=t: pins.test_p23_variants_brute_force(c, t))
    for c in range(len(pins.VARIANT_CASES)) for t in (False, True)
] + [
    lambda: pins.test_p24_groups_of_one_double_the_causal_keys(),
    lambda: pins.test_p25_compressed_columns_are_group_mean_attention(),
    lambda: pins.test_p26_union_merges_by_lse(),
] + [
    (lambda c=c, t=t: pins.test_p27_compressed_brute_force(c, t))
    for c in range(len(pins.CMP_CASES)) for t in (False, True)
] + [
    (lambda c=c: pins.test_p28_backward_is_autograd(c)) for c in range(len(pins.BWD_CASES))
] + [
    lambda: pins.test_p29_backward_matches_finite_differences(),
    lambda: pins.test_p30_key_gradients_sum_to_sink_term(True, 0),
] + [
    (lambda kw=kw: pins.test_p31_backward_at_listed_outputs(kw))
    for kw in (dict(window=5, sink=True), dict(block_size=4, top_k=3, window=3),
               dict(window=2, token_top_k=5, sink=True))
] + [
    (lambda c=c: pins.test_p28_compressed_backward_is_autograd(c))
    for c in range(len(pins.CMP_BWD_CASES))
] + [
    lambda: pins.test_p29_compressed_backward_matches_finite_differences(),
    lambda: pins.test_p30_key_gradients_sum_to_sink_term(True, 8),
] + [
    (lambda c=c, n=n: pins.test_p15_decode_is_last_prefill_rows(c, n))
    for c in range(len(pins.DECODE_CASES)) for n in (1, 5)
] + [
    (lambda c=c: pins.test_p16_decode_brute_force(c, False)) for c in range(len(pins.DECODE_CASES))
] + [
    (lambda n=n: pins.test_p15_block_decode_over_incomplete_last_block(n)) for n in (1, 3)
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
