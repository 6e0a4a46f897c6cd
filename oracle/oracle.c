/*
 * oracle.c -- plain, slow fp64 CPU definition of the causal sparse-attention
 * prefill: block gating by mean-pooled (or min/max-pooled) keys, per query
 * head or per kv group, optionally always keeping the first block, unioned
 * with a causal sliding window and an optional per-query token selection,
 * under GQA, with an optional per-head sink logit.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no code, header, table or
 * helper with the HIP library and does not include anything from it.
 *
 * Inputs are the exact values the device sees (bf16 or fp32, passed here as
 * fp32, which holds bf16 exactly) and every sum is taken in fp64, one term at
 * a time, in index order.  Loops are the definitions written out; OpenMP only
 * splits independent rows across threads.
 *
 * Layouts (row-major, contiguous):
 *   q   [Bt, Hq,  N, d]     k, v [Bt, Hkv, N, d]
 *   idx_q, idx_k [Bt, N, dI]  (indexer; one head shared by all query heads)
 *   "row" r = (b*Hq + h)*N + i names query i of head h in batch b.
 *   Query head h reads kv head h / (Hq/Hkv) (consecutive grouping).
 *
 * Sources (pages as titled):
 *   [MoBA]  "MoBA: 어텐션에 전문가 혼합을 적용해 긴 문맥을 효율적으로 처리하는
 *           블록 어텐션 (feat. MoonshotAI)", discuss.pytorch.kr summary page.
 *   [SWA]   Bit-Axon docs, "SWA + MoE: 어텐션과 희소 전문가".
 *   [Naive] "Naive-N0.5-Flash -- 100만 토큰 문맥을 지원하는 오픈 가중치 MoE 모델",
 *           section "SWA와 DSA를 결합한 어텐션".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    double s;
    int64_t idx;
} cand_t;

/* Descending score, then ascending index: the lower index wins a tie. */
static int cand_cmp(const void* pa, const void* pb) {
    const cand_t* a = (const cand_t*)pa;
    const cand_t* b = (const cand_t*)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    if (a->idx < b->idx) return -1;
    if (a->idx > b->idx) return 1;
    return 0;
}

static int int32_cmp(const void* pa, const void* pb) {
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

/*
 * Mean-pooled block keys [MoBA, "블록 분할과 top-k 게이팅": the score uses
 * MeanPool(K[I_i]) over the B keys of block i].
 *   kbar[(b*Hkv + g)*n + c][e] = (1/B) * sum_{j=cB}^{cB+B-1} k[b][g][j][e]
 */
void orc_block_pool(const float* k, int64_t n_bh, int64_t N, int64_t d, int64_t B,
                    double* kbar) {
    const int64_t n = N / B;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_bh * n; ++t) {
        const int64_t bh = t / n, c = t % n;
        double* dst = kbar + t * d;
        for (int64_t e = 0; e < d; ++e) {
            double acc = 0.0;
            for (int64_t j = c * B; j < (c + 1) * B; ++j)
                acc += (double)k[(bh * N + j) * d + e];
            dst[e] = acc / (double)B;
        }
    }
}

/*
 * Min/max-pooled block keys [MoBA, the related-work remark: Quest is MoBA
 * with smaller blocks and a block representation by min/max pooling]:
 *   kmm[((b*Hkv + g)*n + c)*2 + 0][e] = min_{j in block c} k[b][g][j][e]
 *   kmm[((b*Hkv + g)*n + c)*2 + 1][e] = max_{j in block c} k[b][g][j][e]
 */
void orc_block_minmax(const float* k, int64_t n_bh, int64_t N, int64_t d, int64_t B,
                      double* kmm) {
    const int64_t n = N / B;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_bh * n; ++t) {
        const int64_t bh = t / n, c = t % n;
        double* lo = kmm + t * 2 * d;
        double* hi = lo + d;
        for (int64_t e = 0; e < d; ++e) {
            double mn = INFINITY, mx = -INFINITY;
            for (int64_t j = c * B; j < (c + 1) * B; ++j) {
                const double x = (double)k[(bh * N + j) * d + e];
                if (x < mn) mn = x;
                if (x > mx) mx = x;
            }
            lo[e] = mn;
            hi[e] = mx;
        }
    }
}

/*
 * Unscaled gate score of one query against one block representation.
 *   rep 0, kb = mean key:         s = <q, kb>  [MoBA, gate score equation]
 *   rep 1, kb = (min row, max row): s = sum_e max(q_e * min_e, q_e * max_e),
 *     the largest <q, x> over all x in the block's per-dimension box
 *     [min, max], which every key of the block lies in.  Reading: the pages
 *     name the min/max representation but no score; this upper bound of
 *     the block's best key score is the plainest score it supports.
 */
static double gate_score(const float* qrow, const double* kb, int64_t d, int rep) {
    double acc = 0.0;
    if (rep == 0) {
        for (int64_t e = 0; e < d; ++e) acc += (double)qrow[e] * kb[e];
    } else {
        for (int64_t e = 0; e < d; ++e) {
            const double a = (double)qrow[e] * kb[e], b = (double)qrow[e] * kb[d + e];
            acc += a > b ? a : b;
        }
    }
    return acc;
}

/*
 * Gate score of query i of head h (batch b) against block c.  Per query
 * head, or -- shared != 0 -- one score per kv group, the sum of the scores
 * of the group's G heads for the same position, so that every head of the
 * group makes the same selection.  Reading: the pages give GQA layers with
 * a block selection (BORA page, NSA layers: 8 heads over 4 kv heads, top
 * 16 blocks) but no rule for sharing it; summing the heads' scores is the
 * plainest one.
 */
static double row_score(const float* q, const double* kb, int64_t Hq, int64_t Hkv, int64_t Nq,
                        int64_t d, int64_t n, int rep, int shared, int64_t b, int64_t h,
                        int64_t rq, int64_t c) {
    /* q [Bt, Hq, Nq, d], query row rq */
    const int64_t G = Hq / Hkv, g = h / G;
    const double* kbc = kb + ((b * Hkv + g) * n + c) * d * (rep ? 2 : 1);
    if (!shared) return gate_score(q + ((b * Hq + h) * Nq + rq) * d, kbc, d, rep);
    double acc = 0.0;
    for (int64_t hh = g * G; hh < (g + 1) * G; ++hh)
        acc += gate_score(q + ((b * Hq + hh) * Nq + rq) * d, kbc, d, rep);
    return acc;
}

/*
 * Gate scores of listed rows against every block: scores[r][c] for the
 * candidates c (first <= c < b(i), first = 1 when block 0 is always kept
 * and b(i) > 0, else 0), -INFINITY for the rest (forced blocks are never
 * candidates, later blocks never seen) [MoBA, "인과성 보존": future blocks
 * get s = -inf and g = 0].
 */
void orc_block_scores(const float* q, const double* kb, int64_t Hq, int64_t Hkv,
                      int64_t N, int64_t d, int64_t B, int64_t rep, int64_t shared,
                      int64_t first, const int64_t* rows, int64_t nrows, double* scores) {
    const int64_t n = N / B;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < nrows; ++t) {
        const int64_t r = rows[t];
        const int64_t i = r % N, bh = r / N, b = bh / Hq, h = bh % Hq;
        const int64_t own = i / B;
        const int64_t c0 = (first && own > 0) ? 1 : 0;
        for (int64_t c = 0; c < n; ++c)
            scores[t * n + c] = (c >= c0 && c < own)
                ? row_score(q, kb, Hq, Hkv, N, d, n, (int)rep, (int)shared, b, h, i, c)
                : -INFINITY;
    }
}

/*
 * Block selection [MoBA, "블록 분할과 top-k 게이팅" (g_i = 1 iff s_i is among
 * the top k) and "인과성 보존" (future blocks excluded; the own block always
 * attended, like a shared expert)].  The own block takes one of the k slots
 * (the sparsity 1 - kB/N printed with the scaling results holds only then).
 * first != 0: block 0 is always kept as well [MoBA, the remark that an
 * attention sink is MoBA whose gate always picks the first block along
 * with the recent one]; reading: like the own block it takes a slot, so
 * top_k >= 2.  Candidates first..b-1 (see orc_block_scores) are ranked by
 * (-s_c, c); the first m = min(k - forced, candidates) are kept.  sel row =
 * ascending block ids of the forced and the kept ones, then -1.
 * s_last[t] = score of the m-th kept candidate (NaN if m == 0);
 * s_next[t] = score of the best candidate not kept (NaN if none).
 */
/*
 * The same for queries q [Bt, Hq, Nq, d] continuing a history of N keys:
 * row r = (b*Hq + h)*Nq + rq sits at position i = rq + off [Bit-Axon page,
 * "슬라이딩 윈도우 마스크": the causal offset during decoding].  kb holds the
 * n = N / B complete blocks of the history; the candidates c < i / B are all
 * complete.  Reading for a decode step: a new query is gated exactly as the
 * same position of a prefill over the same history.  orc_block_select is the
 * case Nq = N, off = 0.
 */
void orc_block_select_at(const float* q, const double* kb, int64_t Hq, int64_t Hkv,
                         int64_t Nq, int64_t N, int64_t d, int64_t off, int64_t B,
                         int64_t top_k, int64_t rep, int64_t shared, int64_t first,
                         const int64_t* rows, int64_t nrows, int32_t* sel, double* s_last,
                         double* s_next) {
    const int64_t n = N / B;
#pragma omp parallel
    {
        /* one spare entry; with the loop bound c < n and the bounded writes
         * below, no selection rule can make this function touch memory
         * outside its arrays */
        cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n + 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < nrows; ++t) {
            const int64_t r = rows[t];
            const int64_t rq = r % Nq, i = rq + off, bh = r / Nq, b = bh / Hq, h = bh % Hq;
            const int64_t own = i / B;
            /* block 0 forced (top_k >= 2 is the caller's contract; the
             * guard only keeps the row's writes in bounds) */
            const int64_t c0 = (first && own > 0 && top_k >= 2) ? 1 : 0;
            const int64_t nc = own - c0;
            for (int64_t c = c0; c < own && c < n; ++c) {
                cand[c - c0].s = row_score(q, kb, Hq, Hkv, Nq, d, n, (int)rep, (int)shared,
                                           b, h, rq, c);
                cand[c - c0].idx = c;
            }
            qsort(cand, (size_t)nc, sizeof(cand_t), cand_cmp);
            int64_t m = top_k - 1 - c0;
            if (m > nc) m = nc;
            if (m < 0) m = 0;
            int32_t* out = sel + t * top_k;
            for (int64_t x = 0; x < top_k; ++x) out[x] = -1;
            for (int64_t x = 0; x < m && x < top_k; ++x) out[x] = (int32_t)cand[x].idx;
            if (m < top_k) out[m] = (int32_t)own;
            if (c0 && m + 1 < top_k) out[m + 1] = 0;
            const int64_t kept = m + 1 + c0 < top_k ? m + 1 + c0 : top_k;
            qsort(out, (size_t)kept, sizeof(int32_t), int32_cmp);
            s_last[t] = m > 0 ? cand[m - 1].s : NAN;
            s_next[t] = m < nc ? cand[m].s : NAN;
        }
        free(cand);
    }
}

void orc_block_select(const float* q, const double* kb, int64_t Hq, int64_t Hkv,
                      int64_t N, int64_t d, int64_t B, int64_t top_k, int64_t rep,
                      int64_t shared, int64_t first, const int64_t* rows, int64_t nrows,
                      int32_t* sel, double* s_last, double* s_next) {
    orc_block_select_at(q, kb, Hq, Hkv, N, N, d, 0, B, top_k, rep, shared, first, rows, nrows,
                        sel, s_last, s_next);
}

/*
 * Token selection by a single-head indexer [Naive, "SWA와 DSA를 결합한 어텐션":
 * a light indexer scores the history and attention runs on the top 2,048
 * tokens].  Reading taken: score = <idx_q_i, idx_k_j> (unscaled), candidates
 * j < i, keep the first min(Kt, i) by (-score, j).  Token rows are
 * r = b*N + i; tsel row = ascending token ids, then -1.
 *
 * The _at form scores Nq queries that continue a history of Nk tokens
 * [Bit-Axon SWA + MoE page, "슬라이딩 윈도우 마스크": the causal offset
 * kv_len - seq_len places query row rq at position rq + off]: row
 * r = b*Nq + rq sits at i = rq + off, keys come from [Bt, Nk, dI].
 */
void orc_token_scores_at(const float* iq, const float* ik, int64_t Nq, int64_t Nk, int64_t dI,
                         int64_t off, const int64_t* rows, int64_t nrows, double* scores) {
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < nrows; ++t) {
        const int64_t r = rows[t], i = r % Nq + off, b = r / Nq;
        for (int64_t j = 0; j < Nk; ++j) {
            if (j >= i) { scores[t * Nk + j] = -INFINITY; continue; }
            double acc = 0.0;
            for (int64_t e = 0; e < dI; ++e)
                acc += (double)iq[r * dI + e] * (double)ik[(b * Nk + j) * dI + e];
            scores[t * Nk + j] = acc;
        }
    }
}

void orc_token_scores(const float* iq, const float* ik, int64_t N, int64_t dI,
                      const int64_t* rows, int64_t nrows, double* scores) {
    orc_token_scores_at(iq, ik, N, N, dI, 0, rows, nrows, scores);
}

void orc_token_select_at(const float* iq, const float* ik, int64_t Nq, int64_t Nk, int64_t dI,
                         int64_t Kt, int64_t off, const int64_t* rows, int64_t nrows,
                         int32_t* tsel, double* s_last, double* s_next) {
#pragma omp parallel
    {
        cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)(Nk > 0 ? Nk : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < nrows; ++t) {
            const int64_t r = rows[t], i = r % Nq + off, b = r / Nq;
            for (int64_t j = 0; j < i; ++j) {
                double acc = 0.0;
                for (int64_t e = 0; e < dI; ++e)
                    acc += (double)iq[r * dI + e] * (double)ik[(b * Nk + j) * dI + e];
                cand[j].s = acc;
                cand[j].idx = j;
            }
            qsort(cand, (size_t)i, sizeof(cand_t), cand_cmp);
            const int64_t m = Kt < i ? Kt : i;
            int32_t* out = tsel + t * Kt;
            for (int64_t x = 0; x < Kt; ++x) out[x] = -1;
            for (int64_t x = 0; x < m; ++x) out[x] = (int32_t)cand[x].idx;
            qsort(out, (size_t)m, sizeof(int32_t), int32_cmp);
            s_last[t] = m > 0 ? cand[m - 1].s : NAN;
            s_next[t] = m < i ? cand[m].s : NAN;
        }
        free(cand);
    }
}

void orc_token_select(const float* iq, const float* ik, int64_t N, int64_t dI, int64_t Kt,
                      const int64_t* rows, int64_t nrows,
                      int32_t* tsel, double* s_last, double* s_next) {
    orc_token_select_at(iq, ik, N, N, dI, Kt, 0, rows, nrows, tsel, s_last, s_next);
}

/*
 * Attention of listed rows under a given selection.
 *
 * Attended set [SWA, "슬라이딩 윈도우 마스크": j <= i and i - j < w;
 * MoBA, "표준 어텐션에서 블록 어텐션으로": softmax over K[I] only]:
 *   A(i) = { j <= i : (w > 0 and i - j < w)  or  j/B in sel(i)
 *                      or  j in tsel(i) }
 * one softmax over the union.  Logits x_j = scale * <q_i, k_j>
 * [SWA, "어텐션 공식": QK^T / sqrt(d_k) plus the additive mask].  A sink
 * [Naive: sink bias in SWA and DSA] is one more logit z = sink[h], not
 * scaled, with a zero value vector:
 *   M = max(max_j x_j, z),  L = sum_j e^(x_j - M) + e^(z - M)
 *   out = sum_j e^(x_j - M) v_j / L,   lse = M + ln L.
 * sel  [nrows, sel_w]  block ids per listed row, -1 ignored (NULL: none)
 * tsel [nrows, tsel_w] token ids per listed row, -1 ignored (NULL: none)
 * count[t] = |A(i)| (compressed columns included).  Returns 0, or -1 if an
 * id is out of range.
 *
 * Compressed columns (C > 0) [BORA model card, NSA: 8 tokens become one
 * compressed key/value (8:1), next to the top-k block selection and the
 * sliding window]: kc, vc [Bt, Hkv, N/C, d] hold the compressed keys and
 * values (orc_block_pool with block C: the mean of each complete group of
 * C tokens).  Reading: the pages give neither the compression function nor
 * how the branches combine; the mean is the parameter-free compression
 * (the same pooling the block gate uses), query i sees group c once all its
 * tokens are at or before i ((c+1)C - 1 <= i), and each visible group is
 * one more column x_c = scale * <q_i, kc_c> with value vc_c in the same
 * softmax as A(i) (the union reading of the other branches).
 *
 * Queries q [Bt, Hq, Nq, d] against keys k, v [Bt, Hkv, N, d]: row
 * r = (b*Hq + h)*Nq + rq sits at position i = rq + off [Bit-Axon page,
 * "슬라이딩 윈도우 마스크": the causal offset kv_len - seq_len during
 * decoding]; orc_attend is the case Nq = N, off = 0.
 */
int orc_attend_at(const float* q, const float* k, const float* v,
                  int64_t Hq, int64_t Hkv, int64_t Nq, int64_t N, int64_t d, int64_t off,
                  double scale, int64_t window, int64_t B,
                  const int32_t* sel, int64_t sel_w,
                  const int32_t* tsel, int64_t tsel_w,
                  const float* sink,
                  const double* kc, const double* vc, int64_t C,
                  const int64_t* rows, int64_t nrows,
                  double* out, double* lse, int64_t* count) {
    const int64_t G = Hq / Hkv;
    const int64_t Nc = C > 0 ? N / C : 0;
    int bad = 0;
#pragma omp parallel
    {
        unsigned char* mark = (unsigned char*)malloc((size_t)(N > 0 ? N : 1));
        double* x = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double* xc = (double*)malloc(sizeof(double) * (size_t)(Nc > 0 ? Nc : 1));
#pragma omp for schedule(dynamic, 8)
        for (int64_t t = 0; t < nrows; ++t) {
            const int64_t r = rows[t];
            const int64_t i = r % Nq + off, bh = r / Nq, b = bh / Hq, h = bh % Hq, g = h / G;
            memset(mark, 0, (size_t)(i + 1));
            if (window > 0)
                for (int64_t j = (i - window + 1 > 0 ? i - window + 1 : 0); j <= i; ++j)
                    mark[j] = 1;
            if (sel)
                for (int64_t s = 0; s < sel_w; ++s) {
                    const int64_t c = sel[t * sel_w + s];
                    if (c < 0) continue;
                    /* blocks of the history; a decode step's last one may be incomplete */
                    if (B <= 0 || c >= (N + B - 1) / B) { bad = 1; continue; }
                    for (int64_t j = c * B; j < (c + 1) * B && j <= i; ++j) mark[j] = 1;
                }
            if (tsel)
                for (int64_t s = 0; s < tsel_w; ++s) {
                    const int64_t j = tsel[t * tsel_w + s];
                    if (j < 0) continue;
                    if (j >= N) { bad = 1; continue; }
                    if (j <= i) mark[j] = 1;
                }
            const float* qrow = q + r * d;
            const float* kb = k + (b * Hkv + g) * N * d;
            const float* vb = v + (b * Hkv + g) * N * d;
            double M = -INFINITY;
            int64_t cnt = 0;
            for (int64_t j = 0; j <= i; ++j) {
                if (!mark[j]) continue;
                double acc = 0.0;
                for (int64_t e = 0; e < d; ++e) acc += (double)qrow[e] * (double)kb[j * d + e];
                x[j] = scale * acc;
                if (x[j] > M) M = x[j];
                ++cnt;
            }
            /* compressed groups c with (c+1)C - 1 <= i */
            const int64_t nvis = C > 0 ? (i + 1) / C : 0;
            const double* kcb = kc ? kc + (b * Hkv + g) * Nc * d : NULL;
            const double* vcb = vc ? vc + (b * Hkv + g) * Nc * d : NULL;
            for (int64_t c = 0; c < nvis; ++c) {
                double acc = 0.0;
                for (int64_t e = 0; e < d; ++e) acc += (double)qrow[e] * kcb[c * d + e];
                xc[c] = scale * acc;
                if (xc[c] > M) M = xc[c];
                ++cnt;
            }
            const double z = sink ? (double)sink[h] : -INFINITY;
            if (z > M) M = z;
            double L = 0.0;
            double* o = out + t * d;
            for (int64_t e = 0; e < d; ++e) o[e] = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                if (!mark[j]) continue;
                const double p = exp(x[j] - M);
                L += p;
                for (int64_t e = 0; e < d; ++e) o[e] += p * (double)vb[j * d + e];
            }
            for (int64_t c = 0; c < nvis; ++c) {
                const double p = exp(xc[c] - M);
                L += p;
                for (int64_t e = 0; e < d; ++e) o[e] += p * vcb[c * d + e];
            }
            if (sink) L += exp(z - M);
            if (L > 0.0) {
                for (int64_t e = 0; e < d; ++e) o[e] /= L;
                lse[t] = M + log(L);
            } else {
                lse[t] = -INFINITY;
            }
            count[t] = cnt;
        }
        free(mark);
        free(x);
        free(xc);
    }
    return bad ? -1 : 0;
}

int orc_attend(const float* q, const float* k, const float* v,
               int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
               double scale, int64_t window, int64_t B,
               const int32_t* sel, int64_t sel_w,
               const int32_t* tsel, int64_t tsel_w,
               const float* sink,
               const int64_t* rows, int64_t nrows,
               double* out, double* lse, int64_t* count) {
    return orc_attend_at(q, k, v, Hq, Hkv, N, N, d, 0, scale, window, B, sel, sel_w, tsel, tsel_w,
                         sink, NULL, NULL, 0, rows, nrows, out, lse, count);
}

/*
 * Backward of the attention for a fixed selection (the gates' top-k choices
 * are not differentiated; MoBA trains through the attention of the chosen
 * blocks, and the DSA hybrid of the Naive-N0.5-Flash page through the
 * attention of its window and selected tokens).  For every row i of A(i)
 * (window, blocks and tokens, as orc_attend) with
 * P_ij = e^(x_ij - lse_i), the sink
 * column P_i0 = e^(z_h - lse_i), loss gradient dO_i:
 *   D_i   = sum_e dO_ie out_ie
 *   dS_ij = P_ij (<dO_i, v_j> - D_i)
 *   dq_i  = scale sum_j dS_ij k_j,   dk_j += scale dS_ij q_i,
 *   dv_j += P_ij dO_i,               dsink_h += -P_i0 D_i
 * (the softmax Jacobian; the sink's value vector is zero).  All rows of q
 * [Bt, Hq, N, d]; sel is [Bt*Hq*N, sel_w] or NULL; tsel is [Bt*N, tsel_w]
 * token ids per position, shared by every head, or NULL; dk, dv [Bt, Hkv,
 * N, d] sum over the kv group's heads.  Returns 0, or -1 if an id is out of
 * range.
 *
 * Compressed columns (C > 0; kc, vc the group means, as orc_attend_at): each
 * visible group c of row i is one more column of the same softmax, so with
 * P_ic = e^(scale <q_i, kc_c> - lse_i) it adds
 *   dS_ic = P_ic (<dO_i, vc_c> - D_i),  dq_i += scale dS_ic kc_c,
 *   dkc_c += scale dS_ic q_i,           dvc_c += P_ic dO_i,
 * and, kc_c and vc_c being means of C tokens, every token j of group c
 * receives dkc_c / C in dk_j and dvc_c / C in dv_j (the chain rule through
 * the mean; tokens past the last complete group receive nothing).
 */
int orc_attend_bwd(const float* q, const float* k, const float* v, const float* dout,
                   int64_t Bt, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                   double scale, int64_t window, int64_t B,
                   const int32_t* sel, int64_t sel_w,
                   const int32_t* tsel, int64_t tsel_w, const float* sink,
                   const double* kc, const double* vc, int64_t C,
                   double* dq, double* dk, double* dv, double* dsink) {
    const int64_t G = Hq / Hkv;
    const int64_t Nc = C > 0 ? N / C : 0;
    int bad = 0;
    for (int64_t h = 0; h < Hq; ++h) dsink[h] = 0.0;
    memset(dk, 0, sizeof(double) * (size_t)(Bt * Hkv * N * d));
    memset(dv, 0, sizeof(double) * (size_t)(Bt * Hkv * N * d));
    /* one (batch, kv group) per thread: its dk, dv rows have one writer */
#pragma omp parallel
    {
        unsigned char* mark = (unsigned char*)malloc((size_t)(N > 0 ? N : 1));
        double* x = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double* o = (double*)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
        double* ds_h = (double*)calloc((size_t)Hq, sizeof(double));
        double* xc = (double*)malloc(sizeof(double) * (size_t)(Nc > 0 ? Nc : 1));
        double* dkc = (double*)malloc(sizeof(double) * (size_t)(Nc > 0 ? Nc * d : 1));
        double* dvc = (double*)malloc(sizeof(double) * (size_t)(Nc > 0 ? Nc * d : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t bg = 0; bg < Bt * Hkv; ++bg) {
            const int64_t b = bg / Hkv, g = bg % Hkv;
            const float* kb = k + bg * N * d;
            const float* vb = v + bg * N * d;
            const double* kcb = Nc > 0 ? kc + bg * Nc * d : NULL;
            const double* vcb = Nc > 0 ? vc + bg * Nc * d : NULL;
            double* dkb = dk + bg * N * d;
            double* dvb = dv + bg * N * d;
            for (int64_t e = 0; e < Nc * d; ++e) dkc[e] = dvc[e] = 0.0;
            for (int64_t h = g * G; h < (g + 1) * G; ++h)
                for (int64_t i = 0; i < N; ++i) {
                    const int64_t r = (b * Hq + h) * N + i;
                    memset(mark, 0, (size_t)(i + 1));
                    if (window > 0)
                        for (int64_t j = (i - window + 1 > 0 ? i - window + 1 : 0); j <= i; ++j)
                            mark[j] = 1;
                    if (sel)
                        for (int64_t s = 0; s < sel_w; ++s) {
                            const int64_t c = sel[r * sel_w + s];
                            if (c < 0) continue;
                            if (B <= 0 || c >= N / B) { bad = 1; continue; }
                            for (int64_t j = c * B; j < (c + 1) * B && j <= i; ++j) mark[j] = 1;
                        }
                    if (tsel)
                        for (int64_t s = 0; s < tsel_w; ++s) {
                            const int64_t j = tsel[(b * N + i) * tsel_w + s];
                            if (j < 0) continue;
                            if (j >= N) { bad = 1; continue; }
                            if (j <= i) mark[j] = 1;
                        }
                    const float* qrow = q + r * d;
                    const float* dorow = dout + r * d;
                    /* forward of the row: logits, lse, out */
                    double M = -INFINITY;
                    for (int64_t j = 0; j <= i; ++j) {
                        if (!mark[j]) continue;
                        double acc = 0.0;
                        for (int64_t e = 0; e < d; ++e) acc += (double)qrow[e] * (double)kb[j * d + e];
                        x[j] = scale * acc;
                        if (x[j] > M) M = x[j];
                    }
                    /* compressed groups c with (c+1)C - 1 <= i */
                    const int64_t nvis = C > 0 ? (i + 1) / C : 0;
                    for (int64_t c = 0; c < nvis; ++c) {
                        double acc = 0.0;
                        for (int64_t e = 0; e < d; ++e) acc += (double)qrow[e] * kcb[c * d + e];
                        xc[c] = scale * acc;
                        if (xc[c] > M) M = xc[c];
                    }
                    const double z = sink ? (double)sink[h] : -INFINITY;
                    if (z > M) M = z;
                    double L = 0.0;
                    for (int64_t e = 0; e < d; ++e) o[e] = 0.0;
                    for (int64_t j = 0; j <= i; ++j) {
                        if (!mark[j]) continue;
                        const double p = exp(x[j] - M);
                        L += p;
                        for (int64_t e = 0; e < d; ++e) o[e] += p * (double)vb[j * d + e];
                    }
                    for (int64_t c = 0; c < nvis; ++c) {
                        const double p = exp(xc[c] - M);
                        L += p;
                        for (int64_t e = 0; e < d; ++e) o[e] += p * vcb[c * d + e];
                    }
                    if (sink) L += exp(z - M);
                    const double lse = M + log(L);
                    double Di = 0.0;
                    for (int64_t e = 0; e < d; ++e) Di += (double)dorow[e] * (o[e] / L);
                    /* gradients */
                    double* dqr = dq + r * d;
                    for (int64_t e = 0; e < d; ++e) dqr[e] = 0.0;
                    for (int64_t j = 0; j <= i; ++j) {
                        if (!mark[j]) continue;
                        const double p = exp(x[j] - lse);
                        double dp = 0.0;
                        for (int64_t e = 0; e < d; ++e) dp += (double)dorow[e] * (double)vb[j * d + e];
                        const double dsij = p * (dp - Di);
                        for (int64_t e = 0; e < d; ++e) {
                            dqr[e] += scale * dsij * (double)kb[j * d + e];
                            dkb[j * d + e] += scale * dsij * (double)qrow[e];
                            dvb[j * d + e] += p * (double)dorow[e];
                        }
                    }
                    for (int64_t c = 0; c < nvis; ++c) {
                        const double p = exp(xc[c] - lse);
                        double dp = 0.0;
                        for (int64_t e = 0; e < d; ++e) dp += (double)dorow[e] * vcb[c * d + e];
                        const double dsic = p * (dp - Di);
                        for (int64_t e = 0; e < d; ++e) {
                            dqr[e] += scale * dsic * kcb[c * d + e];
                            dkc[c * d + e] += scale * dsic * (double)qrow[e];
                            dvc[c * d + e] += p * (double)dorow[e];
                        }
                    }
                    if (sink) ds_h[h] += -exp(z - lse) * Di;
                }
            /* through the means: token j of group c gets 1/C of its gradient */
            for (int64_t j = 0; j < Nc * C; ++j)
                for (int64_t e = 0; e < d; ++e) {
                    dkb[j * d + e] += dkc[(j / C) * d + e] / (double)C;
                    dvb[j * d + e] += dvc[(j / C) * d + e] / (double)C;
                }
        }
#pragma omp critical
        for (int64_t h = 0; h < Hq; ++h) dsink[h] += ds_h[h];
        free(mark);
        free(x);
        free(o);
        free(ds_h);
        free(xc);
        free(dkc);
        free(dvc);
    }
    return bad ? -1 : 0;
}

/*
 * The same gradients as orc_attend_bwd (no compressed columns) at listed
 * outputs only, for shapes where the full backward is out of reach: dq of
 * the listed q rows (rows: flat ids (b*Hq + h)*N + i) and dk, dv of the
 * listed keys (keys: flat ids (b*Hkv + g)*N + j).  dq_i needs row i's
 * attention alone; dk_j and dv_j sum over every row of the kv group's heads
 * whose attended set A(i) holds j (the window, a kept block or a kept
 * token), each with its own lse_i and D_i.  sel [Bt*Hq*N, sel_w] and tsel
 * [Bt*N, tsel_w] are the selections of every row.  Returns 0, or -1 if an id
 * is out of range.
 */
static void row_mark(unsigned char* mark, int64_t r, int64_t i, int64_t b, int64_t N,
                     int64_t window, int64_t B, const int32_t* sel, int64_t sel_w,
                     const int32_t* tsel, int64_t tsel_w, int* bad) {
    memset(mark, 0, (size_t)(i + 1));
    if (window > 0)
        for (int64_t j = (i - window + 1 > 0 ? i - window + 1 : 0); j <= i; ++j) mark[j] = 1;
    if (sel)
        for (int64_t s = 0; s < sel_w; ++s) {
            const int64_t c = sel[r * sel_w + s];
            if (c < 0) continue;
            if (B <= 0 || c >= N / B) { *bad = 1; continue; }
            for (int64_t j = c * B; j < (c + 1) * B && j <= i; ++j) mark[j] = 1;
        }
    if (tsel)
        for (int64_t s = 0; s < tsel_w; ++s) {
            const int64_t j = tsel[(b * N + i) * tsel_w + s];
            if (j < 0) continue;
            if (j >= N) { *bad = 1; continue; }
            if (j <= i) mark[j] = 1;
        }
}

/* Whether row r (position i, batch b) attends key j <= i: the window, a
 * kept block holding j, or j kept as a token (row_mark's rule for one key). */
static int row_attends(int64_t r, int64_t i, int64_t b, int64_t j, int64_t N, int64_t window,
                       int64_t B, const int32_t* sel, int64_t sel_w, const int32_t* tsel,
                       int64_t tsel_w) {
    if (j > i) return 0;
    if (window > 0 && i - j < window) return 1;
    if (sel && B > 0)
        for (int64_t s = 0; s < sel_w; ++s)
            if (sel[r * sel_w + s] == j / B) return 1;
    if (tsel)
        for (int64_t s = 0; s < tsel_w; ++s)
            if (tsel[(b * N + i) * tsel_w + s] == j) return 1;
    return 0;
}

/* Row i of head h over its marked keys: logits x, lse, and D = <dO_i, out_i>. */
static void row_stats(const unsigned char* mark, const float* qrow, const float* dorow,
                      const float* kb, const float* vb, int64_t i, int64_t d, double scale,
                      double z, double* x, double* o, double* lse, double* Di) {
    double M = -INFINITY;
    for (int64_t j = 0; j <= i; ++j) {
        if (!mark[j]) continue;
        double acc = 0.0;
        for (int64_t e = 0; e < d; ++e) acc += (double)qrow[e] * (double)kb[j * d + e];
        x[j] = scale * acc;
        if (x[j] > M) M = x[j];
    }
    if (z > M) M = z;
    double L = 0.0;
    for (int64_t e = 0; e < d; ++e) o[e] = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
        if (!mark[j]) continue;
        const double p = exp(x[j] - M);
        L += p;
        for (int64_t e = 0; e < d; ++e) o[e] += p * (double)vb[j * d + e];
    }
    if (z > -INFINITY) L += exp(z - M);
    *lse = M + log(L);
    double s = 0.0;
    for (int64_t e = 0; e < d; ++e) s += (double)dorow[e] * (o[e] / L);
    *Di = s;
}

int orc_attend_bwd_at(const float* q, const float* k, const float* v, const float* dout,
                      int64_t Bt, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                      double scale, int64_t window, int64_t B,
                      const int32_t* sel, int64_t sel_w,
                      const int32_t* tsel, int64_t tsel_w, const float* sink,
                      const int64_t* rows, int64_t nrows, const int64_t* keys, int64_t nkeys,
                      double* dq, double* dk, double* dv) {
    const int64_t G = Hq / Hkv;
    int bad = 0;
    for (int64_t t = 0; t < nrows; ++t)
        if (rows[t] < 0 || rows[t] >= Bt * Hq * N) return -1;
    for (int64_t t = 0; t < nkeys; ++t)
        if (keys[t] < 0 || keys[t] >= Bt * Hkv * N) return -1;
    memset(dk, 0, sizeof(double) * (size_t)(nkeys * d));
    memset(dv, 0, sizeof(double) * (size_t)(nkeys * d));
#pragma omp parallel
    {
        unsigned char* mark = (unsigned char*)malloc((size_t)(N > 0 ? N : 1));
        double* x = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double* o = (double*)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
        double* acc_k = (double*)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
        double* acc_v = (double*)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
        /* dq of the listed rows */
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < nrows; ++t) {
            const int64_t r = rows[t], i = r % N, bh = r / N, b = bh / Hq, h = bh % Hq, g = h / G;
            const float* kb = k + (b * Hkv + g) * N * d;
            const float* vb = v + (b * Hkv + g) * N * d;
            row_mark(mark, r, i, b, N, window, B, sel, sel_w, tsel, tsel_w, &bad);
            double lse, Di;
            const double zh = sink ? (double)sink[h] : -INFINITY;
            row_stats(mark, q + r * d, dout + r * d, kb, vb, i, d, scale, zh, x, o, &lse, &Di);
            double* dqr = dq + t * d;
            for (int64_t e = 0; e < d; ++e) dqr[e] = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                if (!mark[j]) continue;
                const double p = exp(x[j] - lse);
                double dp = 0.0;
                for (int64_t e = 0; e < d; ++e) dp += (double)dout[r * d + e] * (double)vb[j * d + e];
                const double ds = p * (dp - Di);
                for (int64_t e = 0; e < d; ++e) dqr[e] += scale * ds * (double)kb[j * d + e];
            }
        }
        /* dk, dv of the listed keys: every row of the group's heads attending j */
        for (int64_t t = 0; t < nkeys; ++t) {
            const int64_t bg = keys[t] / N, j = keys[t] % N, b = bg / Hkv, g = bg % Hkv;
            const float* kb = k + bg * N * d;
            const float* vb = v + bg * N * d;
            for (int64_t e = 0; e < d; ++e) acc_k[e] = acc_v[e] = 0.0;
#pragma omp for schedule(dynamic, 16)
            for (int64_t u = 0; u < G * (N - j); ++u) {
                const int64_t h = g * G + u / (N - j), i = j + u % (N - j);
                const int64_t r = (b * Hq + h) * N + i;
                if (!row_attends(r, i, b, j, N, window, B, sel, sel_w, tsel, tsel_w)) continue;
                row_mark(mark, r, i, b, N, window, B, sel, sel_w, tsel, tsel_w, &bad);
                if (!mark[j]) continue;
                double lse, Di;
                const double zh = sink ? (double)sink[h] : -INFINITY;
                row_stats(mark, q + r * d, dout + r * d, kb, vb, i, d, scale, zh, x, o, &lse, &Di);
                const double p = exp(x[j] - lse);
                double dp = 0.0;
                for (int64_t e = 0; e < d; ++e) dp += (double)dout[r * d + e] * (double)vb[j * d + e];
                const double ds = p * (dp - Di);
                for (int64_t e = 0; e < d; ++e) {
                    acc_k[e] += scale * ds * (double)q[r * d + e];
                    acc_v[e] += p * (double)dout[r * d + e];
                }
            }
#pragma omp critical
            for (int64_t e = 0; e < d; ++e) {
                dk[t * d + e] += acc_k[e];
                dv[t * d + e] += acc_v[e];
            }
#pragma omp barrier
        }
        free(mark);
        free(x);
        free(o);
        free(acc_k);
        free(acc_v);
    }
    return bad ? -1 : 0;
}
