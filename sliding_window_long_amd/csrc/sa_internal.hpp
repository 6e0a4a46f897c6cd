// sa_internal.hpp -- launch descriptors shared by the host planner and the
// kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sa {

// Query-centric attention over the "near" key range of a row tile: the
// sliding window, the own block and the kept blocks that overlap the window
// span, then the merge of the far-block partials and of the sink.
struct RowsArgs {
    const uint16_t* q[2];   // bf16 planes of q (plane 1 only for split fp32)
    const uint16_t* k[2];
    const uint16_t* v[2];   // fp16 V (bf16 inputs) or bf16 hi/lo planes (fp32)
    void* out;              // bf16 or fp32 (out_f32)
    float* lse;
    int Bt, Hq, Hkv, N;
    float scale;            // softmax scale of the logits
    int window;             // 0 = off
    int gate;               // block gating on
    int B;                  // block size (gate)
    int top_k;
    int span;               // blocks below the own block handled here
    const int32_t* sel;     // [Bt,Hq,N,top_k] kept blocks, ascending, -1 padded
    const uint16_t* part_o; // fp16 [Bt*Hq*N, kslots, D] far-block partials
    const float* part_lse;  // [Bt*Hq*N, kslots]
    int kslots;
    const float* sink;      // [Hq] or nullptr
    int out_f32;
    const uint32_t* tokmask;  // token keep mask words (see sa_token.hip), or nullptr
    const int32_t* vscale;  // [Bt*Hkv] exponent s of the fp16 V copy (v * 2^-s), or nullptr
    const uint8_t* q8;      // FP8 (E4M3) q and k for K Q^T on the FP8 matrix cores, or
    const uint8_t* k8;      // nullptr (then q[0], k[0] are the bf16 planes)
};

// KV-centric attention of one far block against a chunk of gathered rows,
// writing one normalised partial (o, lse) per entry.
struct BlocksArgs {
    const uint16_t* q[2];
    const uint16_t* k[2];
    const uint16_t* v[2];
    int Bt, Hq, Hkv, N, B, n;
    float scale;
    const int32_t* chunk_list;   // [grid] list id of each chunk
    const int32_t* chunk_start;  // [grid] first entry of each chunk
    const int32_t* list_off;     // [lists+1] entry offsets of the lists
    const int32_t* entries;      // (i*G + h_local)*kslots + slot
    const int32_t* n_chunks;     // device count of valid chunks
    int entries_cap;             // capacity of entries
    uint16_t* part_o;
    float* part_lse;
    int kslots;
};

// Block mean-pool: kbar (fp32, optional) and the hi/mid/lo bf16 planes of it
// (optional), both [Bt*Hkv*n, D].
struct PoolArgs {
    const void* k;          // bf16 or fp32 keys [Bt, Hkv, N, D]
    int N, B, n;
    float* kbar;            // fp32 summary: [lists, D] (mean) or [lists, 2, D] (min, max)
    uint16_t* kb3;          // bf16 planes of `plane` elements each (gate_planes of them)
    size_t plane;
    int minmax;             // 0: mean; 1: per-dimension min and max
};

// bf16 planes of the pooled keys the gate reads: the mean split into two
// terms for bf16 keys, three for fp32 keys; min/max as the max terms then
// the min terms, one term each for bf16 keys (exact) and three for fp32.
inline int gate_planes(bool minmax, bool f32) { return minmax ? (f32 ? 6 : 2) : (f32 ? 3 : 2); }

// Block gate: scores against the pooled keys and top-(k-1) earlier blocks.
// Rows are (batch, head, position) over Hq heads of q; each row's selection
// is written to `rep` consecutive heads of sel (rep > 1 when one selection
// per kv group is shared: q then holds the group sums and Hq = Hkv).
// q planes: hi (and lo) of q; for a shared min/max gate the four planes
// hi, lo of the summed positive parts and hi, lo of the summed negative
// parts.
struct GateArgs {
    const uint16_t* q[4];   // bf16 planes of q
    const uint16_t* kb3;
    size_t plane;
    int32_t* sel;           // [Bt, Hq * rep, N, top_k]
    int Bt, Hq, Hkv, N, B, n, top_k, idx_bits;
    int rep;                // heads of sel per gate row
    int first;              // 1: block 0 always kept (takes a slot)
};

// Group sums of the queries for a selection shared per kv group (fp32, head
// order), each split into bf16 hi and lo planes [Bt, Hkv, N, D]:
//   mean gate:    out[0], out[1] = sum_h q_h
//   min/max gate: out[0], out[1] = sum_h max(q_h, 0);
//                 out[2], out[3] = sum_h min(q_h, 0)
// (the min/max score is <q+, max> + <q-, min>, linear in q+ and q-, so the
// group's summed score needs the two parts summed apart).
struct GroupSumArgs {
    const void* q;          // bf16 or fp32 [Bt, Hq, N, D]
    uint16_t* out[4];
    int Bt, Hq, Hkv, N, D;
    int minmax;
};

// Compressed branch: group means of K and V ([lists = Bt*Hkv, Nc, D]; bf16 K
// and fp16 V planes for bf16 inputs, bf16 hi/lo planes of both for fp32).
struct CmpPoolArgs {
    const void* k;
    const void* v;
    uint16_t* kc[2];
    uint16_t* vc[2];
    int lists, N, C, Nc, D;
    const int32_t* vscale;  // [lists] fp16 V means are stored times 2^-s, or nullptr
    // Backward (bwd != 0, bf16 inputs): kc[0] bf16 K means, kc[1] the same
    // values as fp16 times 2^-kscale[list], vc[0] bf16 V means.
    const int32_t* kscale;
    int bwd;
};

// Attention over the compressed columns, merged with the other branches'
// normalised fp32 result out_r and its lse (updated in place).
struct CmpArgs {
    const uint16_t* q[2];
    const uint16_t* kc[2];
    const uint16_t* vc[2];
    const float* out_r;     // [Bt*Hq*N, D] fp32
    void* out;              // final out, bf16 or fp32 (out_f32)
    float* lse;             // in: lse_r; out: the merged lse
    int Bt, Hq, Hkv, N, C, Nc;
    float scale;
    int out_f32;
    const int32_t* vscale;  // [Bt*Hkv] exponent of the compressed V copy, or nullptr
};

// Backward (bf16): inputs, fp16 copies for the P V-style products, the
// forward's lse, the selection and far-row lists, and the gradients.
struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* out;    // forward output
    const uint16_t* dout;   // gradient of the output
    const uint16_t* q16;    // fp16 copies [same layouts]
    const uint16_t* k16;
    const uint16_t* do16;
    const float* lse;       // forward lse [Bt*Hq*N]
    float* delta;           // D_i [Bt*Hq*N]
    const float* sink;      // [Hq] or nullptr
    float* dsink;           // [Hq] or nullptr
    float* sink_term;       // [Bt*Hq*N] per-row terms of dsink (with dsink)
    // Power-of-two exponents per (batch, kv head): the fp16 copies hold
    // q 2^-sq, k 2^-sk, dO 2^-sd; the fp16 score gradients dS 2^-es.
    const int32_t* sq;
    const int32_t* sk;
    const int32_t* sd;
    const int32_t* es;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    const int32_t* sel;     // [Bt*Hq*N, top_k] or nullptr (no block gate)
    // Token gate (else nullptr): the forward's keep mask (query-major, the
    // layout the forward reads) and its key-major copy.
    const uint32_t* tokmask;
    const uint32_t* tokmaskT;
    uint64_t* near_mask;    // [Bt*Hq*N]: bit dlt-1 = block (own - dlt) kept as a near
                            // block (1 <= dlt <= min(span, 64)); nullptr without gate
    const int32_t* list_off;  // far-row lists of the compaction, or nullptr
    const int32_t* entries;
    int entries_cap;            // capacity of entries
    const int32_t* chunk_list;  // their chunking (<= 128 entries per chunk)
    const int32_t* chunk_start;
    const int32_t* n_chunks;
    int max_chunks;
    uint16_t* part_dq;      // bf16 [Bt*Hq*N, kslots, D] far-block dq partials
    // Compressed columns (kc == nullptr: none): group means [Bt*Hkv, Nc, D]
    // of K (bf16, and fp16 times 2^-sk) and V (bf16); the pass over them
    // leaves each group's fp32 dK, dV, already divided by C, for the key
    // pass to add to every token of the group.
    const uint16_t* kc;
    const uint16_t* kc16;
    const uint16_t* vc;
    float* cmp_dk;          // [cmp_splits][Bt*Hkv*Nc, D] partials over row ranges;
    float* cmp_dv;          // summed in order into split 0
    int C, Nc, cmp_splits;
    int top_k, B, n, span, kslots;
    int Bt, Hq, Hkv, N, D, window;
    float scale;
};

hipError_t launch_bwd_delta(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, int head_dim, hipStream_t s);

// FP8 (OCP E4M3) inputs decoded exactly into bf16; n a multiple of 16.
hipError_t launch_fp8_to_bf16(const void* x, uint16_t* y, size_t n, hipStream_t s);

hipError_t launch_cmp_pool(const CmpPoolArgs& a, bool f32_in, hipStream_t s);
hipError_t launch_cmp(const CmpArgs& a, int head_dim, int split, hipStream_t s);

// Inversion of the block selection into per-(batch, kv head, block) lists of
// the rows that keep that block as a far block.
struct CompactArgs {
    const int32_t* sel;
    int Bt, Hq, Hkv, N, B, n, top_k, span, kslots;
    int32_t* count;         // [lists] zeroed before the count pass
    int32_t* cursor;        // [lists] (fast scatter)
    int32_t* tile_base;     // [Bt*Hkv][ceil(N / 256)][n] per row tile: count, then first
                            // position (ordered scatter)
    bool ordered;           // lists in a fixed order (the backward's)
    int32_t* list_off;      // [lists + 1]
    int32_t* list_ch;       // [lists + 1] first chunk of each list (prefix of chunk counts)
    int32_t* entries;
    int32_t* chunk_list;    // [max_chunks]
    int32_t* chunk_start;   // [max_chunks]
    int32_t* n_chunks;      // [1]
    int max_chunks;
    int rows_per_chunk;
};

// Token gate: per-row selection state and the keep mask it produces.
struct TokArgs {
    const uint16_t* iq[2];  // bf16 planes of the indexer queries [Bt, N, 64]
    const uint16_t* ik[2];  // bf16 planes of the indexer keys [Bt, N, 64]
    int Bt, N, top_t;
    int4* state;            // [Bt*N]
    uint16_t* mask;         // keep-mask half-words [Bt][N/32][N/64][64 lanes][2]
    float* qn;              // [Bt*N] indexer query norms
    float2* win;            // [Bt*N] bin map (scale, offset) of the exact pass
    float* kpart;           // [Bt][nkp] largest indexer key norm per 256 keys
    uint32_t* part;         // [Bt][units][64][256] per-unit bin counts (two rows per word);
                            // the sampled pass uses [Bt][NB][64][256] of it first
    uint2* hits;            // [Bt*N][kTokCap] threshold-bin candidates (aliases part)
    int* nslow;             // rows left to the radix fallback
    int units, nkp;
};

// Work units of the binned token passes: 128 query rows (4 waves x 32) by
// a chunk of at most 256 key tiles of 32 keys.  Row block b reads key tiles
// [0, tok_tiles(N, b)), up to the diagonal tile of its last row (every mask
// half a row tile owns is written); key chunk c is present for the blocks
// [64c, NB).
constexpr int kTokRows = 128;
constexpr int kTokChunk = 256;
constexpr int kTokCap = 512;   // threshold-bin candidates a row may collect

__host__ __device__ inline int tok_blocks(int N) { return (N + kTokRows - 1) / kTokRows; }
__host__ __device__ inline int tok_tiles(int N, int b) {
    const int last = (N < (b + 1) * kTokRows ? N : (b + 1) * kTokRows) - 1;   // last row
    return last / 32 + 1;
}
__host__ __device__ inline int tok_chunks(int N, int b) {
    return (tok_tiles(N, b) + kTokChunk - 1) / kTokChunk;
}
// Units before chunk c (chunk-major, blocks descending inside a chunk).
__host__ __device__ inline int tok_unit_base(int N, int c) {
    return c * tok_blocks(N) - 64 * c * (c - 1) / 2;
}
inline int tok_units(int N) { return tok_unit_base(N, tok_chunks(N, tok_blocks(N) - 1)); }

// Decode/append step: Nq (<= kDecMaxQ) queries at positions Nk - Nq + r of
// a history of Nk keys.
constexpr int kDecMaxQ = 64;
// Attended keys per decode attention workgroup (its K and V rows are staged
// in LDS together: 128 rows of 16-bit elements or 64 rows of fp32).
__host__ __device__ constexpr int dec_chunk(bool f32) { return f32 ? 64 : 64; }
struct DecArgs {
    const void* q;          // [Bt, Hq, Nq, D], bf16 or fp32
    const void* k;          // [Bt, Hkv, Nk, D]
    const void* v;
    const void* iq;         // [Bt, Nq, 64] indexer queries, or nullptr
    const void* ik;         // [Bt, Nk, 64] indexer keys, or nullptr
    int f32;                // inputs (and out) are fp32
    int Bt, Hq, Hkv, Nq, Nk, D, top_t, window;
    float scale;
    const float* sink;      // [Hq] or nullptr
    float* scores;          // [Bt, Nq, Nk] indexer scores
    int32_t* list;          // [Bt, Nq, top_t] kept tokens, ascending, -1 padded; nullptr: no gate
    int32_t* nfar;          // [Bt, Nq] kept tokens before the window
    int32_t* plist;         // [Bt, Nq, kDecSelParts, 2, top_t] slice selections (ids, then
                            // their scores' bits), or nullptr
    int32_t* pcnt;          // [Bt, Nq, kDecSelParts] their lengths
    int quota;              // ids kept per slice (dec_sel_quota(top_t))
    int32_t* redo;          // [Bt, Nq] set by the merge when its result may be inexact
    float* part;            // [Bt*Hq*Nq, cmax, D + 2] partials (o, m, l) of each key tile
    int cmax;               // tiles of dec_chunk(f32) attended keys per query, upper bound
    void* out;              // [Bt, Hq, Nq, D], the input dtype
    float* lse;             // [Bt, Hq, Nq]
    // Block gate of a decode step (B > 0): the keys of the kept blocks below
    // the query's range [lo, p] are listed per query head, or per kv group
    // when the group shares its selection.
    int B;                  // block size, 0: no block gate
    int top_k;              // blocks kept per query, the own block (and block 0 with first) included
    int nb;                 // complete blocks of the history (Nk / B)
    const float* kbar;      // [Bt, Hkv, nb, D] fp32 block means, or [.., nb, 2, D] min then max
    int32_t* bsel;          // [Bt, Hq, Nq, top_k] kept blocks (ascending), -1 padded; or nullptr
    int gate_mm, gate_shared, gate_first;   // gate variants
    int list_mode;          // list and nfar rows: 0 (batch, query) -- the token gate;
                            // 1 (batch, q head, query); 2 (batch, kv head, query)
};

// A decode step's block gate scores at most this many complete blocks per
// query (their keys sit in the selecting workgroup's LDS).
constexpr int kDecMaxBlocks = 4096;
constexpr int kDecMaxTopK = 64;

// The decode token selection takes one workgroup per query.  When few
// queries (rows = Bt * Nq <= kDecSplitRows) would leave most of the chip
// idle, a history longer than kDecSplitNk keys is split over kDecSelParts
// slices (one workgroup each) whose selections are then merged, provided
// top_t <= kDecSplitMaxTop; the plan then holds plist and pcnt.
constexpr int kDecSelParts = 8, kDecSplitNk = 16384, kDecSplitMaxTop = 2048, kDecSplitRows = 32;
// Each slice passes on its best dec_sel_quota(top_t) ids: a quarter of
// top_t plus 64 (about twice a slice's expected share of the top_t when the
// best ids spread over the slices).  Where the merge cannot show that no
// slice held back a winner, the query is selected again whole.
__host__ __device__ constexpr int dec_sel_quota(int top_t) {
    return top_t < top_t / 4 + 64 ? top_t : top_t / 4 + 64;
}
// The split pays only when the non-empty slices can pass on more ids than
// top_t: otherwise the merge keeps every id it receives, always asks for a
// whole selection, and the slices and the merge are wasted work.
inline bool dec_split_select(long long rows, int Nk, int top_t) {
    const long long slices = ((long long)Nk + 65536 / kDecSelParts - 1) / (65536 / kDecSelParts);
    return rows <= kDecSplitRows && Nk > kDecSplitNk && top_t > 0 && top_t <= kDecSplitMaxTop &&
           slices * dec_sel_quota(top_t) > top_t;
}
hipError_t launch_decode_select(const DecArgs& a, hipStream_t s);
hipError_t launch_decode_attn(const DecArgs& a, hipStream_t s);
hipError_t launch_decode_block_select(const DecArgs& a, hipStream_t s);

hipError_t launch_token_select(const TokArgs& a, int split, hipStream_t s);
hipError_t launch_token_list(const TokArgs& a, int32_t* out, hipStream_t s);
// Key-major copy of the keep mask (the backward's key-centric pass):
// [Bt][N/32 key groups][N/64 row tiles][64 lanes] words.
hipError_t launch_token_mask_transpose(const TokArgs& a, uint32_t* maskT, hipStream_t s);

hipError_t launch_pool(const PoolArgs& a, int head_dim, bool f32_in, int lists, hipStream_t s);
hipError_t launch_gate(const GateArgs& a, int head_dim, int qsplit, int planes, bool minmax,
                       hipStream_t s);
hipError_t launch_group_sum(const GroupSumArgs& a, bool f32_in, hipStream_t s);
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t value, size_t n, hipStream_t s);

hipError_t launch_rows(const RowsArgs& a, int head_dim, int split, hipStream_t s);
hipError_t launch_blocks(const BlocksArgs& a, int head_dim, int split, int grid, hipStream_t s);
// Row stride of the fp16 V copy that the forward's bf16 path reads: at d 80
// rows of 96 whose columns 80..95 hold fp16 ones (the padding rows of O^T
// then read ones and accumulate the row sums); otherwise D.
__host__ __device__ constexpr int v16_row_of(int D) { return D == 80 ? 96 : D; }
template <int D>
__host__ __device__ constexpr int v16_row() { return v16_row_of(D); }
// fp16 copies of bf16 tensors with a power-of-two scale per head group.
// Rows of D bf16 values, `heads` heads of `rows` rows each; the copy has
// rows of SR >= D elements whose columns D .. SR-1 hold fp16 one.
//   launch_f16_copy: y = fp16(x) (no scale) and, per chunk of kF16ChunkRows
//     rows of a head, the largest |x| into chunk_max
//     [heads][f16_chunks(rows)] (y may be null: the maxima only);
//   launch_f16_scale: per group of `hpg` consecutive heads, the largest
//     |x| m of its chunks and the exponent s (scale[group]): 0 while
//     2^-10 <= m < 2^15, else s = floor(log2 m) - 14 (so m 2^-s lies in
//     [2^14, 2^15)); for s != 0 the group's rows of y are written again as
//     fp16(x 2^-s).  The copy is then exact wherever |x 2^-s| >= 2^-14 and
//     within 2^-25 <= 2^-15 max|x 2^-s| below: no finite bf16 value
//     overflows fp16.
constexpr int kF16ChunkRows = 128;
__host__ __device__ inline int f16_chunks(int rows) { return (rows + kF16ChunkRows - 1) / kF16ChunkRows; }
// (fp8: the source holds OCP E4M3 values, decoded exactly.)
hipError_t launch_f16_copy(const void* x, bool fp8, uint16_t* y, float* chunk_max, int heads,
                           int rows, int D, int SR, hipStream_t s);
// group_max (optional): each group's largest |x|.  y may be null (maxima
// and exponents only).
hipError_t launch_f16_scale(const void* x, bool fp8, uint16_t* y, const float* chunk_max,
                            int32_t* scale, int groups, int hpg, int rows, int D, int SR,
                            hipStream_t s, float* group_max = nullptr);
// Exponent of the backward's fp16 score gradients per group:
// es[g] = e(max|dO|) + e(max|V|) + ceil(log2(2 D)) - 15 with e(m) the
// exponent for which m < 2^e (0 when either maximum is 0), so that
// |dS| 2^-es < 2^15 (|dS| <= 2 D max|dO| max|V| for P <= 1).
hipError_t launch_ds_exponent(const float* do_max, const float* v_max, int32_t* es, int groups,
                              int D, hipStream_t s);
hipError_t launch_split_f32(const float* x, uint16_t* hi, uint16_t* lo, size_t n, hipStream_t s);

}  // namespace sa
