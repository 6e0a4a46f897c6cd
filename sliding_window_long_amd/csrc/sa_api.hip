// sa_api.hip -- C ABI: argument checks, workspace plan, launch sequence.
//
// Stage order of one forward call (all on cfg->stream, no host sync):
//   [fp32 only] split q, k, v into hi/lo bf16 planes
//   [block gate] pool (mean or min/max) -> [shared per kv group] group-summed
//                queries -> gate (scores + top-k) -> compaction of far
//                blocks -> far-block attention partials
//   query-centric attention over window / own block / near kept blocks,
//   merging the far partials and the sink -> out, lse
//   [compressed branch] group means of K, V -> attention over the visible
//                compressed columns, merged by lse into out, lse (the
//                query-centric pass then leaves an fp32 out in the workspace)
#include "sparse_attn.h"
#include "sa_internal.hpp"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

namespace {

constexpr size_t kAlign = 256;
constexpr int kRowsPerChunk = 128;     // entries per far-block workgroup
constexpr int kMaxStages = 1024;   // stage records kept per timing session

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
    int Bt, Hq, Hkv, N, D, G;
    bool f32;
    bool fp8;               // FP8 inputs, decoded into bf16 copies first (unless qk8)
    bool qk8;               // FP8 prefill without block gate or compressed branch: the
                            // attention kernel takes fp8 q, k (K Q^T on the FP8 matrix
                            // cores) and V goes straight from fp8 to its fp16 copy
    bool gate;
    int B, n, top_k, span, kslots, idx_bits, lists;
    bool gate_mm, gate_shared, gate_first;   // gate variants
    int gate_planes;
    bool cmp;               // compressed branch
    int C, Nc, cmp_splits;
    bool far;
    long long max_entries;
    int max_chunks;
    bool tok;
    int top_t, nt32, tok_units, tok_nkp;
    bool dec;               // decode/append step: Nk > N
    int Nk, dec_cmax;
    bool dgate;             // decode step with a block gate
    int nb;                 // its complete blocks (Nk / B)
    size_t o_dec_kbar;
    float scale;
    // workspace regions (byte offsets)
    size_t o_sinkterm, o_bmax_q, o_bmax_do, o_bmax_k, o_bmax_v, o_bgmax, o_bexp, o_cmp_grad;
    size_t o_split, o_kb3, o_sel, o_count, o_cursor, o_tilebase, o_listoff, o_listch, o_nchunks, o_chunk_list,
        o_chunk_start, o_entries, o_part_o, o_part_lse, o_tok_split, o_tok_state, o_tok_mask,
        o_tok_qn, o_tok_win, o_tok_kpart, o_tok_scr, o_tok_nslow, o_tok_maskT, o_dec_scores, o_dec_list,
        o_dec_nfar, o_dec_plist, o_dec_pcnt, o_dec_redo, o_dec_part, o_qsum, o_cmp_k, o_cmp_v,
        o_cmp_out, o_k16, o_q16, o_do16, o_delta, o_near, o_f8q, o_f8k, o_f8v, o_f8iq, o_f8ik,
        o_v16, o_vmax, o_vscale, total;
};

bool misaligned(const void* p, size_t a) { return p && (reinterpret_cast<uintptr_t>(p) % a) != 0; }

// bwd: plan of the backward call (the forward's selection and far-row lists,
// no far partials; fp16 copies of q, k, dO and the row deltas).
int make_plan(const sparse_attn_cfg* c, Plan* p, bool bwd = false) {
    if (!c || c->struct_size != sizeof(sparse_attn_cfg)) return SA_E_INVALID_ARG;
    if (c->batch < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->seq_len < 1)
        return SA_E_INVALID_ARG;
    if (c->dtype != SA_BF16 && c->dtype != SA_F32 && c->dtype != SA_FP8) return SA_E_INVALID_ARG;
    if (c->window < 0 || c->top_k < 0 || c->token_top_k < 0 || c->block_size < 0)
        return SA_E_INVALID_ARG;
    if (!(c->softmax_scale >= 0.f) || isinf(c->softmax_scale)) return SA_E_INVALID_ARG;
    if (c->head_dim != 64 && c->head_dim != 80 && c->head_dim != 128)
        return SA_E_UNSUPPORTED_HEAD_DIM;
    if (c->n_q_heads % c->n_kv_heads) return SA_E_SHAPE;
    if (c->n_q_heads / c->n_kv_heads > 16) return SA_E_UNSUPPORTED;
    if (c->window == 0 && c->top_k == 0) return SA_E_NO_SELF;
    // Gate variants: only with block gating; the forced first block needs a
    // slot of its own besides the own block.
    if (c->gate_repr != SA_GATE_MEAN && c->gate_repr != SA_GATE_MINMAX) return SA_E_INVALID_ARG;
    if ((c->gate_shared != 0 && c->gate_shared != 1) || (c->gate_first != 0 && c->gate_first != 1))
        return SA_E_INVALID_ARG;
    if (c->top_k == 0 && (c->gate_repr != SA_GATE_MEAN || c->gate_shared || c->gate_first))
        return SA_E_INVALID_ARG;
    if (c->gate_first && c->top_k < 2) return SA_E_INVALID_ARG;
    if (c->cmp_block < 0) return SA_E_INVALID_ARG;
    // Keys of the history: a decode/append step has more keys than queries.
    if (c->kv_len < 0) return SA_E_INVALID_ARG;
    const int Nk = c->kv_len > 0 ? c->kv_len : c->seq_len;
    if (Nk < c->seq_len) return SA_E_INVALID_ARG;
    const bool dec = Nk > c->seq_len;
    if (dec && (c->seq_len > sa::kDecMaxQ || c->cmp_block > 0)) return SA_E_UNSUPPORTED;
    // Caller-kept block means serve a decode step's mean block gate only.
    if (c->block_means && !(dec && c->top_k > 0 && c->gate_repr == SA_GATE_MEAN))
        return SA_E_INVALID_ARG;
    // A decode step's selection shared by a kv group: at most 16 heads a group.
    if (dec && c->top_k > 0 && c->gate_shared && c->n_kv_heads > 0 &&
        c->n_q_heads / c->n_kv_heads > 16)
        return SA_E_UNSUPPORTED;
    // The compressed branch joins window / block gating (the NSA layout), not
    // the token gate.
    if (c->cmp_block > 0 && c->token_top_k > 0) return SA_E_UNSUPPORTED;
    // The backward covers bf16 prefills (every branch).
    if (bwd && (dec || c->dtype != SA_BF16)) return SA_E_UNSUPPORTED;
    if (c->token_top_k > 0) {
        if (c->index_dim != 64) return SA_E_UNSUPPORTED_HEAD_DIM;
        // Block and token gates are separate methods and are not combined
        // in one call.  Prefill: token ids below 2^24 (the selection packs
        // 24 index bits with a row number in its staging area).  Decode
        // steps: caches of at most 65536 tokens (16 index bits in the decode
        // selection's keys).
        if (c->top_k > 0 || Nk > (1 << 24) || (dec && Nk > 65536)) return SA_E_UNSUPPORTED;
    }

    Plan& P = *p;
    memset(&P, 0, sizeof(P));
    P.Nk = Nk;
    P.dec = dec;
    P.Bt = c->batch; P.Hq = c->n_q_heads; P.Hkv = c->n_kv_heads; P.N = c->seq_len;
    P.D = c->head_dim; P.G = P.Hq / P.Hkv;
    P.f32 = c->dtype == SA_F32;
    P.fp8 = c->dtype == SA_FP8;
    P.scale = c->softmax_scale > 0.f ? c->softmax_scale : 1.0f / sqrtf((float)P.D);
    const long long rows = (long long)P.Bt * P.Hq * P.N;
    const size_t esz = P.f32 ? 4 : (P.fp8 ? 1 : 2);
    if (rows * P.D * (long long)esz > (1LL << 40)) return SA_E_UNSUPPORTED;
    // One head's K or V (16-bit) must be addressable by a 32-bit byte offset.
    if ((long long)P.Nk * P.D * 2 >= (1LL << 31)) return SA_E_UNSUPPORTED;

    if (P.dec) {
        // Decode/append step: its own small workspace (indexer scores, kept
        // lists, chunk partials).
        size_t off = 0;
        auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
        P.tok = c->token_top_k > 0;
        P.top_t = P.tok ? c->token_top_k : 0;
        P.dgate = c->top_k > 0;
        if (P.dgate) {
            // Blocks of the history; the last may be incomplete (it is then
            // the own block of the newest queries, never a candidate).
            P.B = c->block_size;
            if (!(P.B == 8 || P.B == 16 || P.B == 32 || (P.B >= 64 && P.B % 64 == 0))) return SA_E_SHAPE;
            P.top_k = c->top_k;
            if (P.top_k > ((long long)P.Nk + P.B - 1) / P.B) return SA_E_SHAPE;
            P.nb = P.Nk / P.B;
            if (P.nb > sa::kDecMaxBlocks || P.top_k > sa::kDecMaxTopK) return SA_E_UNSUPPORTED;
            P.top_t = (P.top_k - 1) * P.B;   // keys listed per query, at most
            if ((long long)P.Bt * P.Hq * P.N * (P.top_t > 0 ? P.top_t : 1) >= (1LL << 31))
                return SA_E_UNSUPPORTED;
            P.gate_mm = c->gate_repr == SA_GATE_MINMAX;
            P.gate_shared = c->gate_shared != 0;
            P.gate_first = c->gate_first != 0;
            P.o_dec_kbar = take((size_t)P.Bt * P.Hkv * (P.nb > 0 ? P.nb : 1) * P.D * 4 * (P.gate_mm ? 2 : 1));
            P.o_dec_list = take((size_t)P.Bt * P.Hq * P.N * (P.top_t > 0 ? P.top_t : 1) * 4);
            P.o_dec_nfar = take((size_t)P.Bt * P.Hq * P.N * 4);
        }
        if (P.tok) {
            P.o_dec_scores = take((size_t)P.Bt * P.N * P.Nk * 4);
            P.o_dec_list = take((size_t)P.Bt * P.N * P.top_t * 4);
            P.o_dec_nfar = take((size_t)P.Bt * P.N * 4);
            if (sa::dec_split_select((long long)P.Bt * P.N, P.Nk, P.top_t)) {
                P.o_dec_plist = take((size_t)P.Bt * P.N * sa::kDecSelParts * 2 * P.top_t * 4);
                P.o_dec_pcnt = take((size_t)P.Bt * P.N * sa::kDecSelParts * 4);
                P.o_dec_redo = take((size_t)P.Bt * P.N * 4);
            }
        }
        // keys one query attends: its contiguous range (the window, under a
        // block gate joined by the own block) and its list
        long long near = c->window < P.Nk ? c->window : P.Nk;
        if (P.dgate && (P.B < P.Nk ? P.B : P.Nk) > near) near = P.B < P.Nk ? P.B : P.Nk;
        const long long span = near + (long long)P.top_t;
        const int chunk = sa::dec_chunk(P.f32);
        P.dec_cmax = (int)((span + chunk - 1) / chunk);
        P.o_dec_part = take((size_t)P.Bt * P.Hq * P.N * P.dec_cmax * (P.D + 2) * 4);
        if (P.fp8) {
            P.o_f8q = take((size_t)rows * P.D * 2);
            P.o_f8k = take((size_t)P.Bt * P.Hkv * P.Nk * P.D * 2);
            P.o_f8v = take((size_t)P.Bt * P.Hkv * P.Nk * P.D * 2);
            if (P.tok) {
                P.o_f8iq = take((size_t)P.Bt * P.N * 64 * 2);
                P.o_f8ik = take((size_t)P.Bt * P.Nk * 64 * 2);
            }
        }
        P.total = off;
        return SA_OK;
    }

    P.gate = c->top_k > 0;
    if (P.gate) {
        P.B = c->block_size;
        // 64-key tiles: blocks of 8, 16 or 32 keys share a tile; larger
        // blocks are whole tiles.
        if (!(P.B == 8 || P.B == 16 || P.B == 32 || (P.B >= 64 && P.B % 64 == 0)) || P.N % P.B)
            return SA_E_SHAPE;
        P.n = P.N / P.B;
        P.top_k = c->top_k;
        if (P.top_k > P.n) return SA_E_SHAPE;
        if (P.top_k > 33 || P.n > 4096) return SA_E_UNSUPPORTED;
        P.idx_bits = 1;
        while ((1 << P.idx_bits) < P.n) ++P.idx_bits;
        P.gate_mm = c->gate_repr == SA_GATE_MINMAX;
        P.gate_shared = c->gate_shared != 0;
        P.gate_first = c->gate_first != 0;
        P.gate_planes = sa::gate_planes(P.gate_mm, P.f32);
        // Blocks within `span` below the own block overlap the window span of
        // some row of the block and are attended by the query-centric pass.
        long long span = 0;
        if (c->window > 0) span = ((long long)c->window - 1 + P.B - 1) / P.B;
        if (span > P.n) span = P.n;
        if (span > 64 && c->window < P.N) return SA_E_UNSUPPORTED;   // near-block masks of 64
        P.span = (int)span;
        P.kslots = P.top_k > 1 ? P.top_k - 1 : 1;
        P.lists = P.Bt * P.Hkv * P.n;
        long long per_head = 0;   // far entries per head, upper bound
        for (int b = 0; b < P.n; ++b) {
            long long fc = b - P.span;
            if (fc < 0) fc = 0;
            per_head += (fc < P.top_k - 1 ? fc : P.top_k - 1) * (long long)P.B;
        }
        P.max_entries = per_head * P.Bt * P.Hq;
        P.far = P.max_entries > 0;
        if ((long long)P.N * P.G * P.kslots >= (1LL << 31) || P.max_entries >= (1LL << 31) ||
            rows * P.kslots >= (1LL << 31))   // partial slots are indexed with 32 bits
            return SA_E_UNSUPPORTED;
        long long mc = (P.max_entries + kRowsPerChunk - 1) / kRowsPerChunk + P.lists;
        mc = (mc + 7) / 8 * 8;
        P.max_chunks = (int)mc;
    }

    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
    const size_t nq = (size_t)rows * P.D, nkv = (size_t)P.Bt * P.Hkv * P.N * P.D;
    if (bwd) {
        P.o_k16 = take(nkv * 2);
        P.o_q16 = take(nq * 2);
        P.o_do16 = take(nq * 2);
        P.o_delta = take((size_t)rows * 4);
        P.o_sinkterm = take(c->sink ? (size_t)rows * 4 : 0);   // per-row dsink terms
        // Range of the fp16 copies: per-128-row maxima of q, dO (per q head)
        // and k, v (per kv head), then per (batch, kv head) the largest |dO|,
        // |v| and the exponents of q, k, dO and the score gradients.
        const size_t ch = (size_t)sa::f16_chunks(P.N);
        P.o_bmax_q = take((size_t)P.Bt * P.Hq * ch * 4);
        P.o_bmax_do = take((size_t)P.Bt * P.Hq * ch * 4);
        P.o_bmax_k = take((size_t)P.Bt * P.Hkv * ch * 4);
        P.o_bmax_v = take((size_t)P.Bt * P.Hkv * ch * 4);
        P.o_bgmax = take((size_t)P.Bt * P.Hkv * 2 * 4);
        P.o_bexp = take((size_t)P.Bt * P.Hkv * 5 * 4);
        P.o_near = take(P.gate ? (size_t)rows * 8 : 0);
    } else {
        P.o_split = take(P.f32 ? 2 * (nq + 2 * nkv) * 2 : 0);
        // fp16 copy of V for the P V products (rows padded with ones at d 80)
        P.o_v16 = take(P.f32 ? 0 : nkv / P.D * sa::v16_row_of(P.D) * 2);
        // its per-chunk maxima and the per-(batch, kv head) scale exponent
        P.o_vmax = take(P.f32 ? 0 : (size_t)P.Bt * P.Hkv * sa::f16_chunks(P.N) * 4);
        P.o_vscale = take(P.f32 ? 0 : (size_t)P.Bt * P.Hkv * 4);
    }
    if (P.gate) {
        P.o_kb3 = take((size_t)P.gate_planes * P.lists * P.D * 2);
        P.o_qsum = take(P.gate_shared ? (size_t)(P.gate_mm ? 4 : 2) * P.Bt * P.Hkv * P.N * P.D * 2
                                      : 0);
        P.o_sel = take((size_t)rows * P.top_k * 4);
        if (P.far) {
            P.o_count = take((size_t)P.lists * 4);
            P.o_cursor = take(bwd ? 0 : (size_t)P.lists * 4);
            P.o_tilebase = take(bwd ? (size_t)P.lists * ((P.N + 255) / 256) * 4 : 0);
            P.o_listoff = take((size_t)(P.lists + 1) * 4);
            P.o_listch = take((size_t)(P.lists + 1) * 4);
            P.o_nchunks = take(4);
            P.o_chunk_list = take((size_t)P.max_chunks * 4);
            P.o_chunk_start = take((size_t)P.max_chunks * 4);
            P.o_entries = take((size_t)P.max_entries * 4);
            P.o_part_o = take((size_t)rows * P.kslots * P.D * 2);   // backward: dq partials
            if (!bwd) P.o_part_lse = take((size_t)rows * P.kslots * 4);
        }
    }
    P.cmp = c->cmp_block > 0;
    if (P.cmp) {
        P.C = c->cmp_block;
        P.Nc = P.N / P.C;
        const size_t ncmp = (size_t)P.Bt * P.Hkv * P.Nc * P.D;
        const int planes = P.f32 ? 2 : 1;
        if (bwd) {
            // bf16 K means and their scaled fp16 copy; bf16 V means; fp32
            // dK, dV per group from cmp_splits row ranges (enough
            // workgroups to fill the GPU: about 1024, at most 16 ranges)
            P.o_cmp_k = take(2 * ncmp * 2);
            P.o_cmp_v = take(ncmp * 2);
            const long long wgs = (long long)((P.Nc + 127) / 128) * P.Bt * P.Hkv;
            long long sp = wgs > 0 ? (1024 + wgs - 1) / wgs : 1;
            P.cmp_splits = (int)(sp < 1 ? 1 : sp > 16 ? 16 : sp);
            P.o_cmp_grad = take((size_t)P.cmp_splits * 2 * ncmp * 4);
        } else {
            P.o_cmp_k = take(planes * ncmp * 2);
            P.o_cmp_v = take(planes * ncmp * 2);
            P.o_cmp_out = take((size_t)rows * P.D * 4);
        }
    }
    P.tok = c->token_top_k > 0;
    if (P.tok) {
        P.top_t = c->token_top_k;
        P.nt32 = (P.N + 31) / 32;
        const size_t nidx = (size_t)P.Bt * P.N * 64;
        P.o_tok_split = take(P.f32 ? 2 * 2 * nidx * 2 : 0);
        P.o_tok_state = take((size_t)P.Bt * P.N * 16);
        P.o_tok_mask = take((size_t)P.Bt * P.nt32 * ((P.N + 63) / 64) * 64 * 4);
        P.tok_units = sa::tok_units(P.N);
        P.tok_nkp = (P.N + 255) / 256;
        P.o_tok_qn = take((size_t)P.Bt * P.N * 4);
        P.o_tok_win = take((size_t)P.Bt * P.N * 8);
        P.o_tok_kpart = take((size_t)P.Bt * P.tok_nkp * 4);
        // Per-unit bin counts, later reused for the threshold-bin candidates.
        const size_t counts = (size_t)P.Bt * P.tok_units * 64 * 256 * 4;
        const size_t cands = (size_t)P.Bt * P.N * sa::kTokCap * 8;
        P.o_tok_scr = take(counts > cands ? counts : cands);
        P.o_tok_nslow = take(4);
        P.o_tok_maskT = take(bwd ? (size_t)P.Bt * P.nt32 * ((P.N + 63) / 64) * 64 * 4 : 0);
    }
    P.qk8 = P.fp8 && !P.gate && !P.cmp;
    if (P.fp8) {
        if (!P.qk8) {
            P.o_f8q = take(nq * 2);
            P.o_f8k = take(nkv * 2);
            P.o_f8v = take(nkv * 2);
        }
        if (P.tok) {
            P.o_f8iq = take((size_t)P.Bt * P.N * 64 * 2);
            P.o_f8ik = take((size_t)P.Bt * P.N * 64 * 2);
        }
    }
    P.total = off;
    return SA_OK;
}

// ----------------------------------------------------------------------------
// Stage timing (benchmark aid).
// ----------------------------------------------------------------------------
struct Timing {
    bool on = false;
    bool created = false;
    int n = 0;
    const char* names[kMaxStages];
    hipEvent_t ev[kMaxStages][2];
};
// One record per host thread: calls made from other threads are neither
// recorded nor disturbed by it.
thread_local Timing g_timing;

struct StageScope {
    int idx = -1;
    hipStream_t s;
    StageScope(const char* name, hipStream_t st) : s(st) {
        if (!g_timing.on || g_timing.n >= kMaxStages) return;
        idx = g_timing.n++;
        g_timing.names[idx] = name;
        (void)hipEventRecord(g_timing.ev[idx][0], s);   // a failed record only loses the stage's time
    }
    ~StageScope() {
        if (idx >= 0) (void)hipEventRecord(g_timing.ev[idx][1], s);
    }
};


// Block selection (pool, group sums for a shared gate, gate) into sel.
int select_blocks(const Plan& P, const void* q, const void* k, const uint16_t* const* qp, int split,
                  char* ws, int32_t* sel, hipStream_t s) {
    auto ok = [](hipError_t e) { return e == hipSuccess; };
    uint16_t* kb3 = (uint16_t*)(ws + P.o_kb3);
    const size_t plane = (size_t)P.lists * P.D;
    {
        sa::PoolArgs pa{k, P.N, P.B, P.n, nullptr, kb3, plane, P.gate_mm ? 1 : 0};
        StageScope t("block_pool", s);
        if (!ok(sa::launch_pool(pa, P.D, P.f32, P.lists, s))) return SA_E_HIP;
    }
    sa::GateArgs ga{{qp[0], qp[1], nullptr, nullptr}, kb3, plane, sel, P.Bt, P.Hq, P.Hkv,
                    P.N, P.B, P.n, P.top_k, P.idx_bits, 1, P.gate_first ? 1 : 0};
    int gate_split = split;
    if (P.gate_shared) {
        // One gate row per (batch, kv group, position) on the group's summed
        // query (bf16 hi + lo; for min/max the summed positive and negative
        // parts), its selection written to every head of the group.
        const size_t plane_q = (size_t)P.Bt * P.Hkv * P.N * P.D;
        uint16_t* qs = (uint16_t*)(ws + P.o_qsum);
        sa::GroupSumArgs gs{q, {qs, qs + plane_q, qs + 2 * plane_q, qs + 3 * plane_q},
                            P.Bt, P.Hq, P.Hkv, P.N, P.D, P.gate_mm ? 1 : 0};
        StageScope t("group_sum", s);
        if (!ok(sa::launch_group_sum(gs, P.f32, s))) return SA_E_HIP;
        for (int x = 0; x < 4; ++x) ga.q[x] = gs.out[x];
        ga.Hq = P.Hkv; ga.rep = P.G;
        gate_split = P.gate_mm ? 4 : 2;
    }
    StageScope t("block_gate", s);
    return ok(sa::launch_gate(ga, P.D, gate_split, P.gate_planes, P.gate_mm, s)) ? SA_OK : SA_E_HIP;
}

// Token gate: the per-query top-t token selection as the keep mask
// (ta->mask), and the selected ids into cfg->token_sel_out when set.
int select_tokens(const Plan& P, const sparse_attn_cfg* cfg, char* ws, int split, hipStream_t s,
                  sa::TokArgs* out) {
    auto ok = [](hipError_t e) { return e == hipSuccess; };
    sa::TokArgs& ta = *out;
    ta = sa::TokArgs{};
    ta.iq[0] = (const uint16_t*)cfg->idx_q;
    ta.ik[0] = (const uint16_t*)cfg->idx_k;
    if (P.f32) {
        const size_t nidx = (size_t)P.Bt * P.N * 64;
        uint16_t* base = (uint16_t*)(ws + P.o_tok_split);
        StageScope t("split_f32_indexer", s);
        if (!ok(sa::launch_split_f32((const float*)cfg->idx_q, base, base + nidx, nidx, s)) ||
            !ok(sa::launch_split_f32((const float*)cfg->idx_k, base + 2 * nidx, base + 3 * nidx,
                                     nidx, s)))
            return SA_E_HIP;
        ta.iq[0] = base; ta.iq[1] = base + nidx;
        ta.ik[0] = base + 2 * nidx; ta.ik[1] = base + 3 * nidx;
    }
    ta.Bt = P.Bt; ta.N = P.N; ta.top_t = P.top_t;
    ta.state = (int4*)(ws + P.o_tok_state);
    ta.mask = (uint16_t*)(ws + P.o_tok_mask);
    ta.qn = (float*)(ws + P.o_tok_qn);
    ta.win = (float2*)(ws + P.o_tok_win);
    ta.kpart = (float*)(ws + P.o_tok_kpart);
    ta.part = (uint32_t*)(ws + P.o_tok_scr);
    ta.hits = (uint2*)(ws + P.o_tok_scr);
    ta.nslow = (int*)(ws + P.o_tok_nslow);
    ta.units = P.tok_units; ta.nkp = P.tok_nkp;
    {
        StageScope t("token_select", s);
        if (!ok(sa::launch_token_select(ta, split, s))) return SA_E_HIP;
    }
    if (cfg->token_sel_out) {
        StageScope t("token_list", s);
        if (!ok(sa::launch_token_list(ta, cfg->token_sel_out, s))) return SA_E_HIP;
    }
    return SA_OK;
}

// ----------------------------------------------------------------------------
// Invariants of the far-block lists (debugging aid, sparse_attn_set_checks).
// ----------------------------------------------------------------------------
thread_local bool g_checks = false;

int check_fail(const sparse_attn_far_lists* f, const char* fmt, ...) {
    if (f->detail && f->detail_bytes > 0) {
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(f->detail, f->detail_bytes, fmt, ap);
        va_end(ap);
    }
    return SA_E_CHECK;
}

int check_far_lists_impl(const sparse_attn_far_lists* f) {
    if (!f) return SA_E_INVALID_ARG;
    if (f->detail && f->detail_bytes > 0) f->detail[0] = 0;
    const long long Bt = f->batch, Hq = f->n_q_heads, Hkv = f->n_kv_heads, N = f->seq_len;
    const long long B = f->block_size, n = f->n_blocks, K = f->top_k, ks = f->kslots;
    const long long R = f->rows_per_chunk, span = f->span, nch = f->n_chunks;
    if (Bt <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || N <= 0 || B <= 0 || n <= 0 || K <= 0 ||
        ks < 1 || R <= 0 || span < 0 || nch < 0 || f->max_chunks < 0 || f->max_entries < 0)
        return SA_E_INVALID_ARG;
    if (!f->sel || !f->list_off || !f->list_ch || (nch > 0 && (!f->chunk_list || !f->chunk_start)))
        return SA_E_INVALID_ARG;
    const long long G = Hq / Hkv, lists = Bt * Hkv * n;
    const int32_t* off = f->list_off;
    const int32_t* ch = f->list_ch;
    // Offsets and chunking.
    if (off[0] != 0) return check_fail(f, "list_off[0] is %d, not 0", off[0]);
    for (long long l = 0; l < lists; ++l)
        if (off[l + 1] < off[l])
            return check_fail(f, "list_off decreases after list %lld (%d then %d)", l, off[l], off[l + 1]);
    const long long total = off[lists];
    if (total > f->max_entries)
        return check_fail(f, "%lld entries, more than the %lld the workspace holds", total,
                          (long long)f->max_entries);
    if (total > 0 && !f->entries) return SA_E_INVALID_ARG;
    if (ch[0] != 0) return check_fail(f, "list_ch[0] is %d, not 0", ch[0]);
    for (long long l = 0; l < lists; ++l) {
        const long long m = off[l + 1] - off[l];
        if ((long long)ch[l + 1] - ch[l] != (m + R - 1) / R)
            return check_fail(f, "list %lld: %lld entries but %lld chunks", l, m, (long long)ch[l + 1] - ch[l]);
    }
    if (ch[lists] > f->max_chunks)
        return check_fail(f, "%d chunks, more than the chunk table's %d", ch[lists], f->max_chunks);
    if (nch != ch[lists]) return check_fail(f, "n_chunks is %lld, the lists make %d", nch, ch[lists]);
    for (long long q = 0; q < nch; ++q) {
        const long long l = f->chunk_list[q];
        if (l < 0 || l >= lists || q < ch[l] || q >= ch[l + 1])
            return check_fail(f, "chunk %lld names list %lld, which does not own it", q, l);
        if (f->chunk_start[q] != off[l] + (q - ch[l]) * R)
            return check_fail(f, "chunk %lld of list %lld starts at entry %d, not %lld", q, l,
                              f->chunk_start[q], off[l] + (q - ch[l]) * R);
    }
    // Entries: each one a far slot of a row, listed under that slot's block,
    // once; with `ordered`, in the fixed order.
    std::vector<uint8_t> seen((size_t)(Bt * Hq * N * K), 0);
    for (long long l = 0; l < lists; ++l) {
        const long long bg = l / n, c = l % n, b = bg / Hkv, g = bg % Hkv;
        long long prev = -1;
        for (long long e = off[l]; e < off[l + 1]; ++e) {
            const long long ent = f->entries[e];
            if (ent < 0) return check_fail(f, "entry %lld of list %lld is negative (%lld)", e, l, ent);
            const long long x = ent % ks, t2 = ent / ks, hl = t2 % G, i = t2 / G;
            if (i >= N || x >= K)
                return check_fail(f, "entry %lld of list %lld (%lld) decodes to position %lld, slot %lld: "
                                  "out of range", e, l, ent, i, x);
            const long long h = g * G + hl, prow = (b * Hq + h) * N + i, bi = i / B;
            const int32_t* sr = f->sel + prow * K;
            if (sr[x] != c)
                return check_fail(f, "entry %lld of list %lld (block %lld) names slot %lld of row (b %lld, h "
                                  "%lld, i %lld), which holds block %d", e, l, c, x, b, h, i, sr[x]);
            for (long long xx = 0; xx <= x; ++xx)
                if (sr[xx] < 0 || bi - sr[xx] <= span)
                    return check_fail(f, "entry %lld of list %lld: slot %lld of row (b %lld, h %lld, i %lld) "
                                      "is listed but slot %lld (block %d, own block %lld, span %lld) is not far",
                                      e, l, x, b, h, i, xx, sr[xx], bi, span);
            if (seen[prow * K + x]++)
                return check_fail(f, "slot %lld of row (b %lld, h %lld, i %lld) is listed twice", x, b, h, i);
            if (f->ordered) {
                const long long key = (((i / 64) * G + hl) * K + x) * 64 + i % 64;
                if (key <= prev)
                    return check_fail(f, "list %lld: entry %lld (row %lld, head %lld, slot %lld) is out of order",
                                      l, e, i, h, x);
                prev = key;
            }
        }
    }
    for (long long prow = 0; prow < Bt * Hq * N; ++prow) {
        const long long i = prow % N, bi = i / B;
        const int32_t* sr = f->sel + prow * K;
        for (long long x = 0; x < K; ++x) {
            if (sr[x] < 0 || bi - sr[x] <= span) break;
            if (!seen[prow * K + x])
                return check_fail(f, "far slot %lld (block %d) of row (b %lld, h %lld, i %lld) is in no list", x,
                                  sr[x], prow / (Hq * N), (prow / N) % Hq, i);
        }
    }
    return SA_OK;
}

// With checks on: wait for the lists, copy them and the selection to the
// host and check them.
int run_far_checks(const Plan& P, const int32_t* sel, const sa::CompactArgs& ca, bool ordered,
                   hipStream_t s) {
    auto d2h = [](void* dst, const void* src, size_t bytes) {
        return bytes == 0 || hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost) == hipSuccess;
    };
    StageScope t("far_list_check", s);   // shows in the stage record that the check ran
    if (hipStreamSynchronize(s) != hipSuccess) return SA_E_HIP;
    const size_t lists = (size_t)P.lists;
    std::vector<int32_t> off(lists + 1), ch(lists + 1);
    int32_t nch = 0;
    if (!d2h(&nch, ca.n_chunks, 4) || !d2h(off.data(), ca.list_off, off.size() * 4) ||
        !d2h(ch.data(), ca.list_ch, ch.size() * 4))
        return SA_E_HIP;
    char msg[400] = {0};
    const long long total = off[lists];
    if (total < 0 || total > P.max_entries || nch < 0 || nch > P.max_chunks) {
        fprintf(stderr, "sparse_attn: far-list check: %lld entries, %d chunks (limits %lld, %d)\n", total,
                nch, (long long)P.max_entries, P.max_chunks);
        return SA_E_CHECK;
    }
    std::vector<int32_t> cl((size_t)nch), cs((size_t)nch), ent((size_t)total);
    std::vector<int32_t> selh((size_t)P.Bt * P.Hq * P.N * P.top_k);
    if (!d2h(cl.data(), ca.chunk_list, cl.size() * 4) || !d2h(cs.data(), ca.chunk_start, cs.size() * 4) ||
        !d2h(ent.data(), ca.entries, ent.size() * 4) || !d2h(selh.data(), sel, selh.size() * 4))
        return SA_E_HIP;
    sparse_attn_far_lists f{};
    f.batch = P.Bt; f.n_q_heads = P.Hq; f.n_kv_heads = P.Hkv; f.seq_len = P.N;
    f.block_size = P.B; f.n_blocks = P.n; f.top_k = P.top_k; f.span = P.span; f.kslots = P.kslots;
    f.rows_per_chunk = ca.rows_per_chunk; f.ordered = ordered ? 1 : 0; f.n_chunks = nch;
    f.max_entries = P.max_entries; f.max_chunks = P.max_chunks;
    f.sel = selh.data(); f.list_off = off.data(); f.list_ch = ch.data();
    f.chunk_list = cl.data(); f.chunk_start = cs.data(); f.entries = ent.data();
    f.detail = msg; f.detail_bytes = sizeof msg;
    const int rc = check_far_lists_impl(&f);
    if (rc != SA_OK) fprintf(stderr, "sparse_attn: far-list check failed: %s\n", msg);
    return rc;
}

// Per-(batch, kv head, block) lists of the rows that keep that block as a
// far block, and their chunking.
int compact_far(const Plan& P, const int32_t* sel, char* ws, bool ordered, hipStream_t s,
                sa::CompactArgs* out) {
    sa::CompactArgs& ca = *out;
    ca = sa::CompactArgs{};
    ca.sel = sel; ca.Bt = P.Bt; ca.Hq = P.Hq; ca.Hkv = P.Hkv; ca.N = P.N; ca.B = P.B;
    ca.n = P.n; ca.top_k = P.top_k; ca.span = P.span; ca.kslots = P.kslots;
    ca.count = (int32_t*)(ws + P.o_count);
    ca.cursor = ordered ? nullptr : (int32_t*)(ws + P.o_cursor);
    ca.tile_base = ordered ? (int32_t*)(ws + P.o_tilebase) : nullptr;
    ca.ordered = ordered;
    ca.list_off = (int32_t*)(ws + P.o_listoff);
    ca.list_ch = (int32_t*)(ws + P.o_listch);
    ca.entries = (int32_t*)(ws + P.o_entries);
    ca.chunk_list = (int32_t*)(ws + P.o_chunk_list);
    ca.chunk_start = (int32_t*)(ws + P.o_chunk_start);
    ca.n_chunks = (int32_t*)(ws + P.o_nchunks);
    ca.max_chunks = P.max_chunks;
    ca.rows_per_chunk = kRowsPerChunk;
    StageScope t("compact", s);
    if (sa::launch_compact(ca, s) != hipSuccess) return SA_E_HIP;
    return g_checks ? run_far_checks(P, sel, ca, ordered, s) : SA_OK;
}

// ----------------------------------------------------------------------------
// Allocation-free forward: its workspace is a static device array.
// ----------------------------------------------------------------------------
// Largest workspace the allocation-free entry point serves (the headline
// Bit-Axon SWA shape, 32 heads x 16384 x 80, needs 96 MiB).  Every device
// the library runs on holds one such array until the process ends.
constexpr size_t kScratchBytes = (size_t)128 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up once
// per device with that device current.  In host code the array's name only
// stands in for the symbol: kernels get this address, never the name.
int scratch_address(void** addr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SA_E_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SA_E_HIP;
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return SA_OK;
}

}  // namespace

extern "C" {

const char* sparse_attn_strerror(int status) {
    switch (status) {
        case SA_OK: return "success";
        case SA_E_INVALID_ARG: return "invalid argument (null pointer, struct_size, negative size or scale)";
        case SA_E_SHAPE: return "shape mismatch (block_size must be 8, 16, 32 or a multiple of 64, dividing seq_len; n_q_heads a multiple of n_kv_heads; top_k <= seq_len/block_size)";
        case SA_E_UNSUPPORTED_HEAD_DIM: return "unsupported head_dim (64, 80 or 128) or index_dim (64)";
        case SA_E_NO_SELF: return "window == 0 and top_k == 0: a query would have no guaranteed key";
        case SA_E_ALIGNMENT: return "tensor pointer not aligned (16 bytes for q/k/v/out/idx/workspace, 4 for lse/sink/selections)";
        case SA_E_WORKSPACE_TOO_SMALL: return "workspace smaller than sparse_attn_workspace_bytes";
        case SA_E_HIP: return "HIP kernel launch failed";
        case SA_E_UNSUPPORTED: return "configuration outside the supported limits";
        case SA_E_SCRATCH_LIMIT: return "the configuration needs more workspace than the allocation-free entry point's static scratch (128 MiB)";
        case SA_E_CHECK: return "a far-block list invariant failed (sparse_attn_check_far_lists or a checked call)";
        default: return "unknown status";
    }
}

int sparse_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                            const sparse_attn_cfg* cfg, void* out, float* lse) {
    size_t need = 0;
    int rc = sparse_attn_workspace_bytes(cfg, &need);
    if (rc != SA_OK) return rc;
    if (need > kScratchBytes) return SA_E_SCRATCH_LIMIT;
    sparse_attn_cfg c = *cfg;
    c.workspace = nullptr;
    c.workspace_bytes = 0;
    if (need > 0) {
        rc = scratch_address(&c.workspace);
        if (rc != SA_OK) return rc;
        c.workspace_bytes = kScratchBytes;
    }
    return sparse_attn_fwd(q, k, v, &c, out, lse);
}

int sparse_attn_workspace_bytes(const sparse_attn_cfg* cfg, size_t* bytes) {
    if (!bytes) return SA_E_INVALID_ARG;
    Plan P;
    const int rc = make_plan(cfg, &P);
    if (rc != SA_OK) return rc;
    *bytes = P.total;
    return SA_OK;
}

int sparse_attn_check_far_lists(const sparse_attn_far_lists* f) { return check_far_lists_impl(f); }

int sparse_attn_set_checks(int enable) {
    g_checks = enable != 0;
    return SA_OK;
}

int sparse_attn_set_timing(int enable) {
    if (enable && !g_timing.created) {
        for (int i = 0; i < kMaxStages; ++i)
            for (int j = 0; j < 2; ++j)
                if (hipEventCreate(&g_timing.ev[i][j]) != hipSuccess) return SA_E_HIP;
        g_timing.created = true;
    }
    g_timing.on = enable != 0;
    if (g_timing.on) g_timing.n = 0;
    return SA_OK;
}

int sparse_attn_stage_times(int32_t* n_stages, const char** names, float* ms, int32_t capacity) {
    if (!n_stages) return SA_E_INVALID_ARG;
    *n_stages = g_timing.created ? g_timing.n : 0;
    for (int i = 0; i < *n_stages && i < capacity; ++i) {
        if (hipEventSynchronize(g_timing.ev[i][1]) != hipSuccess) return SA_E_HIP;
        float t = 0.f;
        if (hipEventElapsedTime(&t, g_timing.ev[i][0], g_timing.ev[i][1]) != hipSuccess)
            return SA_E_HIP;
        if (names) names[i] = g_timing.names[i];
        if (ms) ms[i] = t;
    }
    return SA_OK;
}

int sparse_attn_block_pool(const void* k, const sparse_attn_cfg* cfg, float* kbar) {
    Plan P;
    int rc = make_plan(cfg, &P);
    if (rc != SA_OK) return rc;
    if (!P.gate) return SA_E_INVALID_ARG;
    if (P.fp8) return SA_E_UNSUPPORTED;
    if (!k || !kbar) return SA_E_INVALID_ARG;
    if (misaligned(k, 16) || misaligned(kbar, 16)) return SA_E_ALIGNMENT;
    hipStream_t s = (hipStream_t)cfg->stream;
    sa::PoolArgs pa{k, P.N, P.B, P.n, kbar, nullptr, 0, P.gate_mm ? 1 : 0};
    StageScope t("block_pool", s);
    return sa::launch_pool(pa, P.D, P.f32, P.lists, s) == hipSuccess ? SA_OK : SA_E_HIP;
}

int sparse_attn_fwd(const void* q, const void* k, const void* v, const sparse_attn_cfg* cfg,
                    void* out, float* lse) {
    Plan P;
    int rc = make_plan(cfg, &P);
    if (rc != SA_OK) return rc;
    if (!q || !k || !v || !out || !lse) return SA_E_INVALID_ARG;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16) ||
        misaligned(cfg->workspace, 16) || misaligned(lse, 4) || misaligned(cfg->sink, 4) ||
        misaligned(cfg->block_sel_out, 4) || misaligned(cfg->token_sel_out, 4) ||
        misaligned(cfg->block_means, 16))
        return SA_E_ALIGNMENT;
    if (P.tok) {
        if (!cfg->idx_q || !cfg->idx_k) return SA_E_INVALID_ARG;
        if (misaligned(cfg->idx_q, 16) || misaligned(cfg->idx_k, 16)) return SA_E_ALIGNMENT;
    }
    if (P.total > 0 && (!cfg->workspace || cfg->workspace_bytes < P.total))
        return SA_E_WORKSPACE_TOO_SMALL;

    hipStream_t s = (hipStream_t)cfg->stream;
    char* ws = (char*)cfg->workspace;
    auto ok = [](hipError_t e) { return e == hipSuccess; };

    // FP8 inputs: decode into bf16 copies, then run as bf16 -- except that
    // an FP8 prefill without block gate or compressed branch keeps q, k, v in
    // fp8 (the attention kernel's K Q^T on the FP8 matrix cores, V straight
    // to its fp16 copy); the indexer tensors are decoded in both cases.
    sparse_attn_cfg c8;
    const void* q_fp8 = P.qk8 ? q : nullptr;
    const void* k_fp8 = P.qk8 ? k : nullptr;
    if (P.fp8) {
        const size_t nkv = (size_t)P.Bt * P.Hkv * P.Nk * P.D;
        if (!P.qk8) {
            StageScope t("fp8_to_bf16", s);
            uint16_t* q8 = (uint16_t*)(ws + P.o_f8q);
            uint16_t* k8 = (uint16_t*)(ws + P.o_f8k);
            uint16_t* v8 = (uint16_t*)(ws + P.o_f8v);
            if (!ok(sa::launch_fp8_to_bf16(q, q8, (size_t)P.Bt * P.Hq * P.N * P.D, s)) ||
                !ok(sa::launch_fp8_to_bf16(k, k8, nkv, s)) || !ok(sa::launch_fp8_to_bf16(v, v8, nkv, s)))
                return SA_E_HIP;
            q = q8; k = k8; v = v8;
        }
        c8 = *cfg;
        if (P.tok) {
            StageScope t("fp8_to_bf16_indexer", s);
            uint16_t* iq8 = (uint16_t*)(ws + P.o_f8iq);
            uint16_t* ik8 = (uint16_t*)(ws + P.o_f8ik);
            if (!ok(sa::launch_fp8_to_bf16(cfg->idx_q, iq8, (size_t)P.Bt * P.N * 64, s)) ||
                !ok(sa::launch_fp8_to_bf16(cfg->idx_k, ik8, (size_t)P.Bt * P.Nk * 64, s)))
                return SA_E_HIP;
            c8.idx_q = iq8;
            c8.idx_k = ik8;
        }
        cfg = &c8;
    }

    if (P.dec) {
        sa::DecArgs da{};
        da.q = q; da.k = k; da.v = v; da.iq = cfg->idx_q; da.ik = cfg->idx_k;
        da.f32 = P.f32 ? 1 : 0;
        da.Bt = P.Bt; da.Hq = P.Hq; da.Hkv = P.Hkv; da.Nq = P.N; da.Nk = P.Nk; da.D = P.D;
        da.top_t = P.top_t; da.window = cfg->window; da.scale = P.scale; da.sink = cfg->sink;
        da.part = (float*)(ws + P.o_dec_part); da.cmax = P.dec_cmax;
        da.out = out; da.lse = lse;
        if (P.tok) {
            da.scores = (float*)(ws + P.o_dec_scores);
            da.list = cfg->token_sel_out ? cfg->token_sel_out : (int32_t*)(ws + P.o_dec_list);
            da.nfar = (int32_t*)(ws + P.o_dec_nfar);
            if (sa::dec_split_select((long long)P.Bt * P.N, P.Nk, P.top_t)) {
                da.plist = (int32_t*)(ws + P.o_dec_plist);
                da.pcnt = (int32_t*)(ws + P.o_dec_pcnt);
                da.redo = (int32_t*)(ws + P.o_dec_redo);
                da.quota = sa::dec_sel_quota(P.top_t);
            }
            StageScope t("decode_token_select", s);
            if (!ok(sa::launch_decode_select(da, s))) return SA_E_HIP;
        }
        if (P.dgate) {
            da.B = P.B; da.top_k = P.top_k; da.nb = P.nb;
            da.gate_mm = P.gate_mm; da.gate_shared = P.gate_shared; da.gate_first = P.gate_first;
            da.list_mode = P.gate_shared ? 2 : 1;
            da.kbar = (const float*)(ws + P.o_dec_kbar);
            da.list = (int32_t*)(ws + P.o_dec_list);
            da.nfar = (int32_t*)(ws + P.o_dec_nfar);
            da.bsel = cfg->block_sel_out;
            if (cfg->block_means) {
                da.kbar = cfg->block_means;   // kept by the caller
            } else if (P.nb > 0) {
                sa::PoolArgs pa{k, P.Nk, P.B, P.nb, (float*)(ws + P.o_dec_kbar), nullptr, 0, P.gate_mm ? 1 : 0};
                StageScope t("decode_block_pool", s);
                if (!ok(sa::launch_pool(pa, P.D, P.f32, P.Bt * P.Hkv * P.nb, s))) return SA_E_HIP;
            }
            StageScope t("decode_block_select", s);
            if (!ok(sa::launch_decode_block_select(da, s))) return SA_E_HIP;
        }
        StageScope t("decode_attn", s);
        return ok(sa::launch_decode_attn(da, s)) ? SA_OK : SA_E_HIP;
    }

    // Operand planes: bf16 inputs are used in place; fp32 inputs are split.
    const uint16_t* qp[2] = {(const uint16_t*)q, nullptr};
    const uint16_t* kp[2] = {(const uint16_t*)k, nullptr};
    const uint16_t* vp[2] = {(const uint16_t*)v, nullptr};
    const int split = P.f32 ? 2 : 1;
    const int32_t* vscale = nullptr;
    if (P.f32) {
        const size_t nq = (size_t)P.Bt * P.Hq * P.N * P.D, nkv = (size_t)P.Bt * P.Hkv * P.N * P.D;
        uint16_t* base = (uint16_t*)(ws + P.o_split);
        uint16_t* qh = base; uint16_t* ql = qh + nq;
        uint16_t* kh = ql + nq; uint16_t* kl = kh + nkv;
        uint16_t* vh = kl + nkv; uint16_t* vl = vh + nkv;
        StageScope t("split_f32", s);
        if (!ok(sa::launch_split_f32((const float*)q, qh, ql, nq, s)) ||
            !ok(sa::launch_split_f32((const float*)k, kh, kl, nkv, s)) ||
            !ok(sa::launch_split_f32((const float*)v, vh, vl, nkv, s)))
            return SA_E_HIP;
        qp[0] = qh; qp[1] = ql; kp[0] = kh; kp[1] = kl; vp[0] = vh; vp[1] = vl;
    } else {
        // fp16 copy of V for the P V products, scaled by a power of two per
        // (batch, kv head) wherever a value would leave the fp16 range.
        uint16_t* v16 = (uint16_t*)(ws + P.o_v16);
        float* vmax = (float*)(ws + P.o_vmax);
        int32_t* vsc = (int32_t*)(ws + P.o_vscale);
        const int heads = P.Bt * P.Hkv, SR = sa::v16_row_of(P.D);
        StageScope t("v_to_f16", s);
        if (!ok(sa::launch_f16_copy(v, P.qk8, v16, vmax, heads, P.N, P.D, SR, s)) ||
            !ok(sa::launch_f16_scale(v, P.qk8, v16, vmax, vsc, heads, 1, P.N, P.D, SR, s)))
            return SA_E_HIP;
        vscale = vsc;
        vp[0] = v16;
    }

    int32_t* sel = nullptr;
    uint16_t* part_o = nullptr;
    float* part_lse = nullptr;
    if (P.gate) {
        sel = cfg->block_sel_out ? cfg->block_sel_out : (int32_t*)(ws + P.o_sel);
        const int rc_gate = select_blocks(P, q, k, qp, split, ws, sel, s);
        if (rc_gate != SA_OK) return rc_gate;
        if (P.far) {
            part_o = (uint16_t*)(ws + P.o_part_o);
            part_lse = (float*)(ws + P.o_part_lse);
            sa::CompactArgs ca{};
            const int rc_comp = compact_far(P, sel, ws, false, s, &ca);
            if (rc_comp != SA_OK) return rc_comp;
            sa::BlocksArgs ba{};
            for (int i = 0; i < 2; ++i) { ba.q[i] = qp[i]; ba.k[i] = kp[i]; ba.v[i] = vp[i]; }
            ba.Bt = P.Bt; ba.Hq = P.Hq; ba.Hkv = P.Hkv; ba.N = P.N; ba.B = P.B; ba.n = P.n;
            ba.scale = P.scale;
            ba.chunk_list = ca.chunk_list; ba.chunk_start = ca.chunk_start;
            ba.list_off = ca.list_off; ba.entries = ca.entries; ba.n_chunks = ca.n_chunks;
            ba.entries_cap = (int)P.max_entries;
            ba.part_o = part_o; ba.part_lse = part_lse; ba.kslots = P.kslots;
            StageScope t("attn_far_blocks", s);
            if (!ok(sa::launch_blocks(ba, P.D, split, P.max_chunks, s))) return SA_E_HIP;
        }
    }

    const uint32_t* tokmask = nullptr;
    if (P.tok) {
        sa::TokArgs ta{};
        const int rc_tok = select_tokens(P, cfg, ws, split, s, &ta);
        if (rc_tok != SA_OK) return rc_tok;
        tokmask = (const uint32_t*)ta.mask;
    }

    sa::RowsArgs ra{};
    for (int i = 0; i < 2; ++i) { ra.q[i] = qp[i]; ra.k[i] = kp[i]; ra.v[i] = vp[i]; }
    ra.out = out; ra.lse = lse;
    ra.Bt = P.Bt; ra.Hq = P.Hq; ra.Hkv = P.Hkv; ra.N = P.N;
    ra.scale = P.scale; ra.window = cfg->window;
    ra.gate = P.gate ? 1 : 0; ra.B = P.B; ra.top_k = P.top_k; ra.span = P.span;
    ra.sel = sel; ra.part_o = part_o; ra.part_lse = part_lse; ra.kslots = P.kslots;
    ra.sink = cfg->sink; ra.out_f32 = P.f32 ? 1 : 0;
    ra.tokmask = tokmask;
    ra.vscale = vscale;
    ra.q8 = (const uint8_t*)q_fp8;
    ra.k8 = (const uint8_t*)k_fp8;
    float* out_r = P.cmp ? (float*)(ws + P.o_cmp_out) : nullptr;
    if (P.cmp) {   // the compressed pass merges into the final out
        ra.out = out_r;
        ra.out_f32 = 1;
    }
    {
        StageScope t("attn_rows", s);
        if (!ok(sa::launch_rows(ra, P.D, split, s))) return SA_E_HIP;
    }
    if (P.cmp) {
        const size_t ncmp = (size_t)P.Bt * P.Hkv * P.Nc * P.D;
        uint16_t* kc = (uint16_t*)(ws + P.o_cmp_k);
        uint16_t* vc = (uint16_t*)(ws + P.o_cmp_v);
        sa::CmpPoolArgs cp{k, v, {kc, P.f32 ? kc + ncmp : nullptr}, {vc, P.f32 ? vc + ncmp : nullptr},
                           P.Bt * P.Hkv, P.N, P.C, P.Nc, P.D, vscale, nullptr, 0};
        {
            StageScope t("cmp_pool", s);
            if (!ok(sa::launch_cmp_pool(cp, P.f32, s))) return SA_E_HIP;
        }
        sa::CmpArgs ca{};
        for (int i = 0; i < 2; ++i) { ca.q[i] = qp[i]; ca.kc[i] = cp.kc[i]; ca.vc[i] = cp.vc[i]; }
        ca.out_r = out_r; ca.out = out; ca.lse = lse;
        ca.Bt = P.Bt; ca.Hq = P.Hq; ca.Hkv = P.Hkv; ca.N = P.N; ca.C = P.C; ca.Nc = P.Nc;
        ca.scale = P.scale; ca.out_f32 = P.f32 ? 1 : 0;
        ca.vscale = vscale;
        StageScope t("attn_compressed", s);
        if (!ok(sa::launch_cmp(ca, P.D, split, s))) return SA_E_HIP;
    }
    return SA_OK;
}

int sparse_attn_bwd_workspace_bytes(const sparse_attn_cfg* cfg, size_t* bytes) {
    if (!bytes) return SA_E_INVALID_ARG;
    Plan P;
    const int rc = make_plan(cfg, &P, true);
    if (rc != SA_OK) return rc;
    *bytes = P.total;
    return SA_OK;
}

int sparse_attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                    const void* dout, const sparse_attn_cfg* cfg, void* dq, void* dk, void* dv,
                    float* dsink) {
    Plan P;
    int rc = make_plan(cfg, &P, true);
    if (rc != SA_OK) return rc;
    if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv) return SA_E_INVALID_ARG;
    if (dsink && !cfg->sink) return SA_E_INVALID_ARG;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16) ||
        misaligned(dout, 16) || misaligned(dq, 16) || misaligned(dk, 16) || misaligned(dv, 16) ||
        misaligned(cfg->workspace, 16) || misaligned(lse, 4) || misaligned(dsink, 4) ||
        misaligned(cfg->sink, 4) || misaligned(cfg->block_sel_out, 4))
        return SA_E_ALIGNMENT;
    if (P.tok) {
        if (!cfg->idx_q || !cfg->idx_k) return SA_E_INVALID_ARG;
        if (misaligned(cfg->idx_q, 16) || misaligned(cfg->idx_k, 16) ||
            misaligned(cfg->token_sel_out, 4))
            return SA_E_ALIGNMENT;
    }
    if ((long long)P.Bt * P.Hq * P.N >= (1LL << 31)) return SA_E_UNSUPPORTED;   // 32-bit row ids
    if (P.total > 0 && (!cfg->workspace || cfg->workspace_bytes < P.total))
        return SA_E_WORKSPACE_TOO_SMALL;
    hipStream_t s = (hipStream_t)cfg->stream;
    char* ws = (char*)cfg->workspace;
    auto ok = [](hipError_t e) { return e == hipSuccess; };

    // The forward's selection and far-row lists (deterministic kernels).
    int32_t* sel = nullptr;
    sa::CompactArgs ca{};
    if (P.gate) {
        sel = cfg->block_sel_out ? cfg->block_sel_out : (int32_t*)(ws + P.o_sel);
        const uint16_t* qp[2] = {(const uint16_t*)q, nullptr};
        rc = select_blocks(P, q, k, qp, 1, ws, sel, s);
        if (rc != SA_OK) return rc;
        if (P.far) {
            rc = compact_far(P, sel, ws, true, s, &ca);
            if (rc != SA_OK) return rc;
        }
    }
    // The forward's token selection (bit-identical), and its key-major copy.
    const uint32_t *tokmask = nullptr, *tokmaskT = nullptr;
    if (P.tok) {
        sa::TokArgs ta{};
        rc = select_tokens(P, cfg, ws, 1, s, &ta);
        if (rc != SA_OK) return rc;
        uint32_t* mt = (uint32_t*)(ws + P.o_tok_maskT);
        StageScope t("bwd_token_mask", s);
        if (!ok(sa::launch_token_mask_transpose(ta, mt, s))) return SA_E_HIP;
        tokmask = (const uint32_t*)ta.mask;
        tokmaskT = mt;
    }
    uint16_t* k16 = (uint16_t*)(ws + P.o_k16);
    uint16_t* q16 = (uint16_t*)(ws + P.o_q16);
    uint16_t* do16 = (uint16_t*)(ws + P.o_do16);
    // fp16 copies of k, q, dO at a power-of-two scale per (batch, kv head)
    // (the rule of the forward's V copy), and the exponent of the score
    // gradients from the largest |dO| and |v|.
    const int groups = P.Bt * P.Hkv;
    int32_t* bexp = (int32_t*)(ws + P.o_bexp);
    int32_t *sq = bexp, *sk = bexp + groups, *sd = bexp + 2 * groups, *es = bexp + 3 * groups,
            *sv = bexp + 4 * groups;
    float* gmax = (float*)(ws + P.o_bgmax);
    {
        StageScope t("bwd_to_f16", s);
        float* mq = (float*)(ws + P.o_bmax_q);
        float* mdo = (float*)(ws + P.o_bmax_do);
        float* mk = (float*)(ws + P.o_bmax_k);
        float* mv = (float*)(ws + P.o_bmax_v);
        const int hq = P.Bt * P.Hq, hkv = P.Bt * P.Hkv;
        if (!ok(sa::launch_f16_copy(k, false, k16, mk, hkv, P.N, P.D, P.D, s)) ||
            !ok(sa::launch_f16_scale(k, false, k16, mk, sk, groups, 1, P.N, P.D, P.D, s)) ||
            !ok(sa::launch_f16_copy(q, false, q16, mq, hq, P.N, P.D, P.D, s)) ||
            !ok(sa::launch_f16_scale(q, false, q16, mq, sq, groups, P.G, P.N, P.D, P.D, s)) ||
            !ok(sa::launch_f16_copy(dout, false, do16, mdo, hq, P.N, P.D, P.D, s)) ||
            !ok(sa::launch_f16_scale(dout, false, do16, mdo, sd, groups, P.G, P.N, P.D, P.D, s,
                                     gmax)) ||
            !ok(sa::launch_f16_copy(v, false, nullptr, mv, hkv, P.N, P.D, P.D, s)) ||
            !ok(sa::launch_f16_scale(v, false, nullptr, mv, sv, groups, 1, P.N, P.D, P.D, s,
                                     gmax + groups)) ||
            !ok(sa::launch_ds_exponent(gmax, gmax + groups, es, groups, P.D, s)))
            return SA_E_HIP;
    }
    sa::BwdArgs ba{};
    ba.q = (const uint16_t*)q; ba.k = (const uint16_t*)k; ba.v = (const uint16_t*)v;
    ba.out = (const uint16_t*)out; ba.dout = (const uint16_t*)dout;
    ba.q16 = q16; ba.k16 = k16; ba.do16 = do16;
    ba.sq = sq; ba.sk = sk; ba.sd = sd; ba.es = es;
    ba.tokmask = tokmask; ba.tokmaskT = tokmaskT;
    ba.lse = lse; ba.delta = (float*)(ws + P.o_delta);
    ba.sink = cfg->sink; ba.dsink = dsink;
    ba.sink_term = dsink ? (float*)(ws + P.o_sinkterm) : nullptr;
    ba.dq = (uint16_t*)dq; ba.dk = (uint16_t*)dk; ba.dv = (uint16_t*)dv;
    ba.sel = sel; ba.top_k = P.top_k; ba.B = P.B; ba.n = P.n; ba.span = P.span;
    ba.near_mask = P.gate ? (uint64_t*)(ws + P.o_near) : nullptr;
    ba.kslots = P.kslots;
    ba.list_off = P.far ? ca.list_off : nullptr; ba.entries = P.far ? ca.entries : nullptr;
    ba.entries_cap = P.far ? (int)P.max_entries : 0;
    ba.chunk_list = ca.chunk_list; ba.chunk_start = ca.chunk_start; ba.n_chunks = ca.n_chunks;
    ba.max_chunks = P.far ? P.max_chunks : 0;
    ba.part_dq = P.far ? (uint16_t*)(ws + P.o_part_o) : nullptr;
    ba.Bt = P.Bt; ba.Hq = P.Hq; ba.Hkv = P.Hkv; ba.N = P.N; ba.D = P.D; ba.window = cfg->window;
    ba.scale = P.scale;
    if (P.cmp && P.Nc > 0) {
        // The compressed columns' operands: the forward's bf16 K means (the
        // same kernel and rounding), bf16 V means, and the K means as fp16 in
        // the units of the K copy.
        StageScope t("bwd_cmp_pool", s);
        const size_t ncmp = (size_t)P.Bt * P.Hkv * P.Nc * P.D;
        uint16_t* kcp = (uint16_t*)(ws + P.o_cmp_k);
        uint16_t* vcp = (uint16_t*)(ws + P.o_cmp_v);
        sa::CmpPoolArgs cp{k, v, {kcp, kcp + ncmp}, {vcp, nullptr}, P.Bt * P.Hkv, P.N, P.C, P.Nc, P.D,
                           nullptr, sk, 1};
        if (!ok(sa::launch_cmp_pool(cp, false, s))) return SA_E_HIP;
        ba.kc = kcp; ba.kc16 = kcp + ncmp; ba.vc = vcp;
        ba.cmp_dk = (float*)(ws + P.o_cmp_grad); ba.cmp_dv = ba.cmp_dk + (size_t)P.cmp_splits * ncmp;
        ba.C = P.C; ba.Nc = P.Nc; ba.cmp_splits = P.cmp_splits;
    }
    {
        StageScope t("bwd_delta", s);
        if (!ok(sa::launch_bwd_delta(ba, s))) return SA_E_HIP;
    }
    StageScope t("bwd_attn", s);
    return ok(sa::launch_bwd(ba, P.D, s)) ? SA_OK : SA_E_HIP;
}

}  // extern "C"
