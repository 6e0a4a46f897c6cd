/*
 * sparse_attn.h -- C ABI of the MI355X (gfx950) causal sparse-attention
 * prefill library.
 *
 * The operation (one call computes all of it):
 *
 *   For query i of head h (block b = i / B, kv head g = h / (Hq/Hkv)):
 *   1. Block gate, when top_k > 0 [MoBA summary page, "블록 분할과 top-k
 *      게이팅" and "인과성 보존"]: each earlier block c < b is scored by
 *      s_c = <q_i, mean of the B keys of block c> (unscaled); the own block b
 *      is always kept and takes one of the top_k slots; the min(top_k-1, b)
 *      best earlier blocks are kept, a tie going to the lower block id.
 *      Gate variants [same page, the remark that attention sinks, Quest
 *      and LongHeads are MoBA with other gates; BORA page, NSA layers with
 *      a block selection under GQA]:
 *      - gate_repr = SA_GATE_MINMAX: block c is summarised by the
 *        per-dimension min and max of its keys and scored by
 *        sum_e max(q_e * min_e, q_e * max_e), the largest <q_i, x> over the
 *        box those bounds span (Quest's block representation);
 *      - gate_shared = 1: one selection per (batch, kv group, position),
 *        scored by the sum of the group's heads' scores; every query head
 *        of the group keeps the same blocks;
 *      - gate_first = 1: block 0 is always kept as well (an attention sink
 *        as a gate rule) and, like the own block, takes one of the top_k
 *        slots (top_k >= 2); candidates are then blocks 1 .. b-1.
 *      top_k = 1 keeps the own block only (LongHeads' top-1 gate).
 *   2. Token gate, when token_top_k > 0 [Naive-N0.5-Flash page, "SWA와 DSA를
 *      결합한 어텐션"]: each earlier token j < i is scored by
 *      <idx_q_i, idx_k_j> (one indexer head shared by all query heads); the
 *      min(token_top_k, i) best are kept, a tie going to the lower token id.
 *   3. One softmax over the union A(i) = { j <= i : (window > 0 and
 *      i - j < window) or block(j) kept or token j kept } [Bit-Axon
 *      "SWA + MoE" page, "어텐션 공식" and "슬라이딩 윈도우 마스크"], logits
 *      softmax_scale * <q_i, k_j>, plus -- when sink != NULL -- one extra
 *      logit sink[h] (not scaled) whose value vector is zero, plus -- when
 *      cmp_block = C > 0 -- the compressed columns [BORA model card, NSA:
 *      8 tokens become one compressed key and value]: every complete group
 *      c of C tokens with (c+1)C - 1 <= i adds the logit
 *      softmax_scale * <q_i, mean of the group's keys> with the mean of its
 *      values as the value.
 *      out_i = sum_j p_j v_j,  lse_i = natural log of the softmax
 *      normaliser (sink included).
 *
 * Decode/append step (kv_len > seq_len) [Bit-Axon "SWA + MoE" page,
 * "슬라이딩 윈도우 마스크": the causal offset kv_len - seq_len during
 * autoregressive decoding with a KV cache]: the seq_len queries are the
 * newest positions of a history of kv_len keys; query row r is position
 * i = kv_len - seq_len + r and the three steps above apply to it over keys
 * 0 .. kv_len-1 (the token gate scans the whole cached history).  Under
 * block gating a new query is gated as that position of a prefill over the
 * history: its own block (the last one may be incomplete) and the best
 * top_k - 1 complete earlier blocks by the dot product with their mean keys
 * (pooled from the cache on every call, or kept by the caller: block_means),
 * per query head, or per kv group with gate_shared (at most 16 heads a
 * group); min/max summaries and block 0 kept work as in the prefill; at most
 * 4096 complete blocks and top_k <= 64.  Full attention (what the MoBA
 * summary page runs for generation) is a window >= kv_len.  Limits:
 * seq_len <= 64.
 *
 * Layouts (row-major, contiguous, device memory; kv_len = seq_len unless a
 * decode step):
 *   q, out  [batch, n_q_heads,  seq_len, head_dim]   dtype cfg->dtype (out bf16
 *                                                     for SA_FP8)
 *   k, v    [batch, n_kv_heads, kv_len,  head_dim]   dtype cfg->dtype
 *   lse     [batch, n_q_heads,  seq_len]              fp32
 *   idx_q   [batch, seq_len, index_dim], idx_k [batch, kv_len, index_dim]
 *                                                     dtype cfg->dtype
 *   sink    [n_q_heads]                               fp32
 *   block_sel_out [batch, n_q_heads, seq_len, top_k]  int32: kept block ids
 *           ascending (the own block is the last valid one), then -1.
 *   token_sel_out [batch, seq_len, token_top_k]       int32: kept token ids
 *           ascending, then -1.
 *
 * Ownership: the caller owns and allocates every buffer, the workspace
 * included (size from sparse_attn_workspace_bytes).  The library allocates
 * no device memory, keeps no per-call state, never synchronises, and
 * enqueues all work on cfg->stream (a hipStream_t; NULL = the default
 * stream).  Calls are reentrant for distinct workspaces.
 *
 * Errors: every entry point returns SA_OK (0) or a negative SA_E_* code.
 * All argument checks happen before anything is enqueued, so every code but
 * SA_E_HIP is returned without touching the GPU.  On error, out, lse and
 * the selection outputs are unspecified.
 *
 * Non-finite inputs: a NaN or an infinity in q, k or v is an ordinary value.
 * The call returns SA_OK and every row whose attended set meets it comes out
 * non-finite; rows that cannot see it are unchanged, except that a
 * non-finite value in v also reaches, in its own head dimension, the earlier
 * rows of its 64-key tile (they weight it 0, and 0 * inf is NaN).  Block
 * selections stay within each row's candidate blocks whatever the scores.
 * The indexer inputs idx_q, idx_k must be finite.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPARSE_ATTN_ABI_VERSION 5

typedef enum {
    SA_BF16 = 0, /* bfloat16 inputs and out; fp32 accumulation.  Q K^T runs on
                    bf16 matrix cores; P V on fp16 ones: V is copied once into
                    the workspace as fp16(v 2^-s), with one power-of-two
                    exponent s per (batch, kv head) chosen from its largest
                    |v| (0 while that lies in [2^-10, 2^15), else the exponent
                    that brings it into [2^14, 2^15)), and the results are
                    scaled back by 2^s.  Every finite bf16 V is covered: the
                    copy is exact wherever |v 2^-s| >= 2^-14 and within
                    2^-15 of the head's largest |v 2^-s| below that. */
    SA_F32 = 1,  /* float32 inputs and out; each operand split into two
                    bf16 terms on the matrix cores (about 16 mantissa bits) */
    SA_FP8 = 2   /* FP8 inputs (OCP E4M3: bias 7, 3 mantissa bits, max 448, no
                    infinities, 0x7F/0xFF = NaN) for q, k, v, idx_q, idx_k; out
                    is bf16.  [Naive-N0.5-Flash page: FP8 mixed-precision
                    inference.]  Prefills without a block or token gate read
                    q and k as E4M3 straight into the FP8 matrix cores for
                    Q K^T (every E4M3 product is exact in the fp32
                    accumulator) and copy V to fp16 with the hardware
                    conversion (exact).  Every other call decodes the inputs
                    exactly into bf16 in the workspace (every E4M3 value is a
                    bf16 value) and computes as SA_BF16.  Not for
                    sparse_attn_block_pool or the backward (SA_E_UNSUPPORTED). */
} sa_dtype;

typedef enum {
    SA_GATE_MEAN = 0,   /* block summary: mean of its keys */
    SA_GATE_MINMAX = 1  /* block summary: per-dimension min and max of its keys */
} sa_gate_repr;

enum {
    SA_OK = 0,
    SA_E_INVALID_ARG = -1,      /* NULL pointer, bad struct_size, negative size */
    SA_E_SHAPE = -2,            /* seq_len % block_size, Hq % Hkv, top_k > n, ... */
    SA_E_UNSUPPORTED_HEAD_DIM = -3, /* head_dim not in {64, 80, 128}, or index_dim != 64 */
    SA_E_NO_SELF = -4,          /* window == 0 and top_k == 0: no key is guaranteed */
    SA_E_ALIGNMENT = -5,        /* a tensor pointer is not 16-byte aligned */
    SA_E_WORKSPACE_TOO_SMALL = -6,
    SA_E_HIP = -7,              /* a kernel launch failed (hipGetLastError) */
    SA_E_UNSUPPORTED = -8,      /* a combination outside the documented limits */
    SA_E_SCRATCH_LIMIT = -9,    /* sparse_attn_fwd_noalloc: the configuration needs
                                   more workspace than its static scratch holds */
    SA_E_CHECK = -10            /* a list invariant failed (sparse_attn_check_far_lists,
                                   or a call made with sparse_attn_set_checks(1)) */
};

typedef struct {
    uint32_t struct_size;   /* = sizeof(sparse_attn_cfg) */
    int32_t batch;
    int32_t n_q_heads;      /* Hq, a multiple of n_kv_heads (GQA: h -> h / (Hq/Hkv)) */
    int32_t n_kv_heads;     /* Hkv; Hq/Hkv <= 16 */
    int32_t seq_len;        /* N >= 1 */
    int32_t head_dim;       /* d in {64, 80, 128} */
    int32_t dtype;          /* sa_dtype */
    int32_t block_size;     /* B: 8, 16, 32 or a multiple of 64, dividing N (else
                               SA_E_SHAPE); ignored if top_k == 0 */
    int32_t top_k;          /* blocks kept per query, own block included; 0 = no
                               block gate; 1 <= top_k <= min(33, N/B) */
    int32_t window;         /* w >= 0: attend iff 0 <= i-j < w; 0 = no window */
    int32_t token_top_k;    /* 0 = no token gate; else tokens kept per query */
    int32_t index_dim;      /* indexer head dim (64) when token_top_k > 0 */
    const void* idx_q;      /* indexer queries, or NULL when token_top_k == 0 */
    const void* idx_k;      /* indexer keys, or NULL when token_top_k == 0 */
    const float* sink;      /* per-head sink logits, or NULL */
    float softmax_scale;    /* logit scale; 0 -> 1/sqrt(head_dim) */
    void* workspace;        /* device scratch, >= sparse_attn_workspace_bytes */
    size_t workspace_bytes;
    int32_t* block_sel_out; /* optional copy-out of the block selection, or NULL */
    int32_t* token_sel_out; /* optional copy-out of the token selection, or NULL */
    void* stream;           /* hipStream_t, NULL = default stream */
    int32_t kv_len;         /* keys of the history: 0 or seq_len for a prefill;
                               > seq_len for a decode/append step (seq_len <= 64;
                               kv_len <= 65536 with a token gate) */
    int32_t gate_repr;      /* sa_gate_repr; SA_GATE_MEAN unless top_k > 0 */
    int32_t gate_shared;    /* 0 or 1: one block selection per kv group; 0 unless top_k > 0 */
    int32_t gate_first;     /* 0 or 1: block 0 always kept (top_k >= 2); 0 unless top_k > 0 */
    int32_t cmp_block;      /* tokens per compressed key/value (the BORA card's 8); 0 = no
                               compressed branch.  Prefill (and its backward) only, not
                               with token_top_k */
    const float* block_means; /* decode step under the block gate: fp32 means of the
                               history's complete blocks [batch, n_kv_heads,
                               kv_len / block_size, head_dim] (block c = keys
                               cB .. cB+B-1), kept by the caller as the cache grows
                               (sparse_attn_block_pool gives them); the step then reads
                               them instead of pooling the cache.  NULL: pooled on every
                               call.  Must be NULL in every other call
                               (SA_E_INVALID_ARG) */
} sparse_attn_cfg;

/* Bytes of device workspace sparse_attn_fwd needs for this configuration
 * (workspace fields of cfg are ignored).  Host only; touches no GPU. */
int sparse_attn_workspace_bytes(const sparse_attn_cfg* cfg, size_t* bytes);

/* The whole forward (a prefill, or a decode/append step when kv_len >
 * seq_len): enqueues every stage on cfg->stream and returns without
 * waiting.  q, k, v, out, lse are device pointers (16-byte aligned). */
int sparse_attn_fwd(const void* q, const void* k, const void* v,
                    const sparse_attn_cfg* cfg, void* out, float* lse);

/* sparse_attn_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, checks and result as sparse_attn_fwd, except
 * that cfg->workspace and cfg->workspace_bytes are ignored: the workspace is
 * a static device array of 128 MiB that the library holds on every device
 * it runs on until the process ends (its address is looked up once per
 * device, on the first call with that device current; cfg->stream must
 * belong to the current device).  A configuration whose
 * sparse_attn_workspace_bytes exceeds 128 MiB returns SA_E_SCRATCH_LIMIT
 * before anything is enqueued.  Nothing is allocated.  Every call on one
 * device shares that device's array and it keeps the last call's contents
 * (the forward initialises whatever it reads before reading it): calls
 * that may overlap on one device -- on different streams, or from different
 * host threads -- race on it and must be serialised by the caller. */
int sparse_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                            const sparse_attn_cfg* cfg, void* out, float* lse);

/* The block pooling stage alone [MoBA summary page, implementation figure:
 * partition into blocks, mean pooling]: kbar[b, g, c, :] = mean of the
 * block_size keys of block c, fp32, [batch, n_kv_heads, seq_len/block_size,
 * head_dim].  With gate_repr = SA_GATE_MINMAX: kbar[b, g, c, 0, :] = the
 * per-dimension min and kbar[b, g, c, 1, :] the max over those keys, fp32,
 * [batch, n_kv_heads, seq_len/block_size, 2, head_dim].  Uses no workspace.
 * Same checks as sparse_attn_fwd. */
int sparse_attn_block_pool(const void* k, const sparse_attn_cfg* cfg, float* kbar);

/* Backward of sparse_attn_fwd for the selection it makes [MoBA summary
 * page: the model trains through the attention of the selected blocks; the
 * gates' top-k choices carry no gradient]: with P_ij = e^(x_ij - lse_i) over
 * the forward's attended set (window, own block, kept blocks, sink column),
 * D_i = <dout_i, out_i> and dS_ij = P_ij (<dout_i, v_j> - D_i):
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i (summed over
 *   the kv group's heads),  dv_j = sum_i P_ij dout_i,
 *   dsink[h] = -sum_i e^(sink[h] - lse_i) D_i.
 * Same cfg as the forward call (the selection is recomputed, bit-identical;
 * block_sel_out, if set, receives it again).  q, k, v, out (the forward's
 * output), dout, dq [batch, n_q_heads, seq_len, head_dim], dk, dv [batch,
 * n_kv_heads, seq_len, head_dim]: bf16, device, 16-byte aligned; lse the
 * forward's fp32 lse; dsink [n_q_heads] fp32 or NULL (needs cfg->sink).
 * Supported: bf16 prefills with a window and/or block gating (any gate
 * variant) or the token gate (cfg->idx_q, cfg->idx_k as for the forward;
 * the selection is recomputed and held fixed), and the compressed branch
 * (cmp_block = C: each visible group c adds the column of its K and V means,
 * and its gradients dkc_c = scale sum_i dS_ic q_i, dvc_c = sum_i P_ic dout_i
 * reach each of its C tokens as dkc_c / C and dvc_c / C, the chain rule
 * through the mean); fp32 or a decode step return SA_E_UNSUPPORTED.  The
 * gradient products run on fp16 matrix cores
 * with fp16 copies of q, k and dout and fp16 score gradients dS_ij, each at
 * a power-of-two scale per (batch, kv head) chosen from the data (the rule
 * of the forward's V copy; for dS from the largest |dout| and |v|), undone
 * exactly in fp32: every finite bf16 input stays inside the fp16 range.
 * Results are the same bits on every call (fixed summation orders).
 * Workspace from sparse_attn_bwd_workspace_bytes; enqueued on cfg->stream,
 * no host sync, nothing allocated. */
int sparse_attn_bwd_workspace_bytes(const sparse_attn_cfg* cfg, size_t* bytes);
int sparse_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                    const float* lse, const void* dout, const sparse_attn_cfg* cfg,
                    void* dq, void* dk, void* dv, float* dsink);

/* Static description of an error code. */
const char* sparse_attn_strerror(int status);

/* Optional per-stage timing for benchmarks.  sparse_attn_set_timing(1)
 * starts a new record (creating the HIP events on first use); from then on
 * every sparse_attn_fwd / sparse_attn_block_pool call records an event pair
 * on cfg->stream around each kernel it enqueues, up to 1024 records.
 * sparse_attn_set_timing(0) stops recording.  sparse_attn_stage_times waits
 * for the recorded events and writes up to `capacity` stage names (static
 * strings) and durations in milliseconds, in enqueue order; *n_stages
 * receives the number recorded.  The record belongs to the calling host
 * thread (only calls made from that thread are recorded): the one piece of
 * state the library keeps between calls, and only while timing is on. */
int sparse_attn_set_timing(int enable);
int sparse_attn_stage_times(int32_t* n_stages, const char** names, float* ms,
                            int32_t capacity);

/* Checks of the far-block lists (a debugging aid; off by default).
 *
 * Block gating regroups query rows by kept far block (MoBA summary page,
 * "MoBA의 구현: MoE와 FlashAttention의 결합", steps 1-2: route each query to
 * its blocks, then reorder the queries by block).  The lists live in the
 * workspace:
 *   list l = (batch b, kv head g, block c), l = (b n_kv_heads + g) n_blocks + c;
 *   list_off[lists + 1]  first entry of each list (exclusive prefix sum);
 *   list_ch[lists + 1]   first chunk of each list: a list of m entries is cut
 *                        into ceil(m / rows_per_chunk) chunks;
 *   chunk_list[n_chunks], chunk_start[n_chunks]  each chunk's list and first
 *                        entry;
 *   entries[list_off[lists]]  one entry per (query row, head, selection slot)
 *                        whose kept block is a far block: (i G + h_local)
 *                        kslots + x for position i, head g G + h_local of the
 *                        kv group (G = n_q_heads / n_kv_heads) and slot x of
 *                        the row's ascending selection sel[b, h, i, x].
 * A slot holds a far block when it and every slot before it hold a block c
 * >= 0 with floor(i / block_size) - c > span (blocks within `span` of the
 * row's own block are attended with the window, not through the lists).
 *
 * sparse_attn_check_far_lists verifies host copies of such lists against
 * the selection: offsets non-decreasing from 0 and at most max_entries; chunk
 * counts, the chunk table and n_chunks (at most max_chunks) consistent with
 * the offsets; every entry decodes to a position, head and slot in range
 * whose selected block is its list's block and is a far block; every far
 * slot of every row listed exactly once; with `ordered`, the entries of each
 * list in increasing (floor(i / 64), h_local, x, i mod 64), the fixed order
 * the backward sums in.  It reads only the arrays it is given (their sizes
 * follow from the fields and from list_off, list_ch and n_chunks, which are
 * range-checked before use) and returns SA_OK or SA_E_CHECK, writing the
 * first violation as a NUL-terminated message into detail (if not NULL).
 *
 * sparse_attn_set_checks(1): from then on, every sparse_attn_fwd and
 * sparse_attn_bwd call on the calling host thread that builds far-block
 * lists waits for them on cfg->stream, copies the selection and the lists
 * to the host and runs sparse_attn_check_far_lists, returning SA_E_CHECK on
 * a violation.  While on, those calls synchronise the stream (the one
 * exception to the no-sync rule above). */
typedef struct {
    int32_t batch, n_q_heads, n_kv_heads, seq_len, block_size, n_blocks, top_k;
    int32_t span;             /* near blocks below the own block (see above) */
    int32_t kslots;           /* slot multiplier of an entry (>= top_k - 1, >= 1) */
    int32_t rows_per_chunk;   /* > 0 */
    int32_t ordered;          /* 1: require the fixed order */
    int32_t n_chunks;
    int64_t max_entries;
    int32_t max_chunks;
    const int32_t* sel;          /* [batch, n_q_heads, seq_len, top_k] */
    const int32_t* list_off;     /* [lists + 1] */
    const int32_t* list_ch;      /* [lists + 1] */
    const int32_t* chunk_list;   /* [n_chunks] */
    const int32_t* chunk_start;  /* [n_chunks] */
    const int32_t* entries;      /* [list_off[lists]] */
    char* detail;                /* out: first violation, or NULL */
    size_t detail_bytes;
} sparse_attn_far_lists;

int sparse_attn_check_far_lists(const sparse_attn_far_lists* f);
int sparse_attn_set_checks(int enable);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
