// sa_token.hip -- token gate: single-head dot-product indexer and per-query
// top-k token selection.
//
// [Naive-N0.5-Flash page, "SWA와 DSA를 결합한 어텐션"]: a light indexer scores
// the whole history of each query and attention runs on the top 2,048
// tokens.  Reading taken here: score(i, j) = <idx_q_i, idx_k_j> with no scale,
// candidates j < i, keep the min(top_t, i) best, a tie going to the lower j;
// the selection is shared by every query head.
//
// The selection is exact: "the k best" is the set of the k largest 64-bit keys
//   key = ord(score) << 32 | (0xFFFFFFFF - j)
// where ord maps fp32 to a uint32 with the same order, so the key order is
// (score descending, then j ascending).  Scores are recomputed on the matrix
// core in every pass (same instruction sequence, so bitwise the same values);
// they are never stored.
//
// Binned path (every row unless its threshold bin is crowded):
//   1. prep: |idx_q_i| per row and the largest |idx_k_j| per batch; by
//      Cauchy-Schwarz every score of row i lies in [-B_i, B_i] with
//      B_i = |idx_q_i| max_j |idx_k_j|.
//   2. sample: per-row counts of 256 equal bins over [-B_i, B_i] for key
//      tiles 0, s, 2s, ... with the stride s <= 16 that reads at least 64
//      tiles of the block (all of them for short rows).
//   3. window: from the sample, a score range [L_i, U_i) that holds the
//      k-th best candidate with a wide margin (6 binomial deviations plus
//      16 sample ranks around the expected rank); the exact pass maps it
//      onto bins 1..126, bin 0 below it, bin 127 above it.  Any monotone map of the
//      score to a bin is exact for what follows: the sample only sets how
//      many candidates share the threshold bin.
//   4. hist: exact per-row counts of bins 1..127 over every candidate.
//   5. bin: the bin b* holding the k-th best candidate, the count above it
//      and the rank r still to take inside it.
//   6. mask: keys in bins above b* are kept (mask written whole); the
//      candidates of bin b* are collected as 64-bit keys.
//   7. resolve: radix select of the r best collected keys, whose mask bits
//      are then set.
// Rows whose bin b* holds more than kTokCap candidates, or whose k-th
// candidate lies below the window, are left to the radix fallback: radix select over the 64-bit key one byte per pass (per-row
// 256-bin histograms in LDS), then the mask of those rows.
//
// Output: a keep mask in the layout of the attention kernel's registers.
// For the 32 query rows r0..r0+31 (row tile rt), the 64 keys kt*64 ..
// kt*64+63 (key tile kt) and lane L of the wave that owns those rows, word
// mask[(rt*NT64 + kt)*64 + L] has bit 16*sub + v set iff row r0 + L%32 keeps
// key kt*64 + 32*sub + 8*(v/4) + 4*(L/32) + v%4 -- the key held in register v
// of the sub-th 32-key half of the S^T tile.  The two halves are written as
// separate 16-bit halves of the word; halves past the row tile are not
// written.
#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

constexpr int TOK_WAVES = 4;
constexpr int TOK_THREADS = 64 * TOK_WAVES;
constexpr uint32_t kTokAll = 1u;    // row keeps every candidate
constexpr uint32_t kTokNone = 2u;   // row keeps nothing
constexpr uint32_t kTokDone = 4u;   // radix threshold final
constexpr uint32_t kTokSlow = 8u;   // row resolved by the radix fallback
constexpr uint32_t kTokFast = 16u;  // row's mask already final (radix leaves it)
// Per-row 256-bin histograms in LDS, 257 words apart so that rows adding
// to the same bin hit different banks.
constexpr int HSTRIDE = 257;
constexpr int TK_KS = 72;   // LDS row stride of a staged key, in bf16 (64 dims + 8)
constexpr int kTokSample = 16;   // largest tile stride of the sampled pass

__device__ __forceinline__ uint32_t ord32(float s) {
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 16-bit half of the mask word of (batch, row tile, 32-key tile kc, lane).
__device__ __forceinline__ size_t mask_half(int bt, int nt32, int nt64, int rt, int kc, int lane) {
    return ((((size_t)bt * nt32 + rt) * nt64 + (kc >> 1)) * 64 + lane) * 2 + (kc & 1);
}

// Wave index within the block, as a scalar (wave-uniform) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Indexer scores of one 32-key tile against the wave's 32 query rows:
// acc[v] = score(row r0 + lane%32, key kc*32 + 8*(v/4) + 4*(lane/32) + v%4).
template <int SPLIT>
__device__ __forceinline__ f32x16 index_scores(const TokArgs& a, int bt, int kc,
                                               const bf16x8 (&qf)[SPLIT][4], int lane) {
    const int col = lane & 31, hh = lane >> 5;
    const int key = min(kc * 32 + col, a.N - 1);
    const size_t off = ((size_t)bt * a.N + key) * 64 + 8 * hh;
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 k0 = as_bf16x8(*(const uint4*)(a.ik[0] + off + ks * 16));
        acc = mfma32(k0, qf[0][ks], acc);
        if constexpr (SPLIT == 2) {
            const bf16x8 k1 = as_bf16x8(*(const uint4*)(a.ik[1] + off + ks * 16));
            acc = mfma32(k0, qf[1][ks], acc);
            acc = mfma32(k1, qf[0][ks], acc);
        }
    }
    return acc;
}

// The same scores from a key tile staged in LDS (plane p at kl[p]); the
// instruction sequence matches index_scores, so the values are bitwise equal.
template <int SPLIT>
__device__ __forceinline__ f32x16 index_scores_lds(const uint16_t* kl, const bf16x8 (&qf)[SPLIT][4],
                                                   int lane) {
    const int col = lane & 31, hh = lane >> 5;
    const uint16_t* kb = kl + col * TK_KS + 8 * hh;
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 k0 = as_bf16x8(*(const uint4*)(kb + ks * 16));
        acc = mfma32(k0, qf[0][ks], acc);
        if constexpr (SPLIT == 2) {
            const bf16x8 k1 = as_bf16x8(*(const uint4*)(kb + 32 * TK_KS + ks * 16));
            acc = mfma32(k0, qf[1][ks], acc);
            acc = mfma32(k1, qf[0][ks], acc);
        }
    }
    return acc;
}

template <int SPLIT>
__device__ __forceinline__ void load_qf(bf16x8 (&qf)[SPLIT][4], const TokArgs& a, int bt, int row,
                                        bool row_ok, int hh) {
#pragma unroll
    for (int p = 0; p < SPLIT; ++p)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (row_ok) u = *(const uint4*)(a.iq[p] + ((size_t)bt * a.N + row) * 64 + ks * 16 + 8 * hh);
            qf[p][ks] = as_bf16x8(u);
        }
}

// ---------------------------------------------------------------------------
// Binned path.

// Unit u of a batch -> (row block b, key chunk c).
__device__ __forceinline__ void tok_unit(int N, int u, int& b, int& c) {
    const int nb = tok_blocks(N);
    c = 0;
    int base = 0;
    while (u >= base + nb - 64 * c) {
        base += nb - 64 * c;
        ++c;
    }
    b = nb - 1 - (u - base);
}

// Row norms, per-256-key maxima of the key norms, initial row state and bin map.
__global__ __launch_bounds__(TOK_THREADS) void tok_prep_kernel(TokArgs a) {
    __shared__ float red[TOK_WAVES];
    const int bt = blockIdx.y, tid = threadIdx.x, i = blockIdx.x * TOK_THREADS + tid;
    float kn2 = 0.f;
    if (i < a.N) {
        const size_t r = (size_t)bt * a.N + i;
        const uint4* q = (const uint4*)(a.iq[0] + r * 64);
        const uint4* k = (const uint4*)(a.ik[0] + r * 64);
        float qn2 = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const uint4 uq = q[t], uk = k[t];
            const uint32_t wq[4] = {uq.x, uq.y, uq.z, uq.w}, wk[4] = {uk.x, uk.y, uk.z, uk.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float q0 = bf16_to_f32(wq[e] & 0xffffu), q1 = bf16_to_f32(wq[e] >> 16);
                const float k0 = bf16_to_f32(wk[e] & 0xffffu), k1 = bf16_to_f32(wk[e] >> 16);
                qn2 = fmaf(q0, q0, fmaf(q1, q1, qn2));
                kn2 = fmaf(k0, k0, fmaf(k1, k1, kn2));
            }
        }
        a.qn[r] = sqrtf(qn2);
        const int kk = min(a.top_t, i);
        uint32_t fl = 0;
        if (kk == 0) fl = kTokNone;
        else if (kk == i) fl = kTokAll;
        a.state[r] = make_int4(0, 0, kk, (int)fl);
        a.win[r] = make_float2(0.f, 128.f);   // rows that select get theirs from the sample
    }
    float m = sqrtf(kn2);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    if (tid == 0) {
        a.kpart[(size_t)bt * a.nkp + blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        if (bt == 0 && blockIdx.x == 0) *a.nslow = 0;
    }
}

// Largest key norm of batch bt (every thread of the block gets it).
__device__ __forceinline__ float tok_kmax(const TokArgs& a, int bt, float* red, int tid) {
    float m = 0.f;
    for (int x = tid; x < a.nkp; x += TOK_THREADS) m = fmaxf(m, a.kpart[(size_t)bt * a.nkp + x]);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// x = score * scale + 128 maps [-B_i, B_i] into [0, 256) (B_i widened by
// 1/64 for rounding); bin = trunc(clamp(x, 0, 255)).  Both passes use this
// exact arithmetic, so they agree on every bin.
__device__ __forceinline__ float tok_scale(const TokArgs& a, int bt, int row, bool row_ok, float kmax) {
    if (!row_ok) return 0.f;
    const float bnd = a.qn[(size_t)bt * a.N + row] * kmax * 1.015625f;
    return bnd > 0.f ? 128.f / bnd : 0.f;
}

template <int SPLIT>
struct TokLds {
    uint16_t k[2][SPLIT][32 * TK_KS];   // double-buffered key tile
};

// Key tile t (32 keys x 64 dims per plane): one 16-byte piece per thread;
// keys past N read as zero (the load address is clamped, no branch).
template <int SPLIT>
__device__ __forceinline__ void tok_load(uint4 (&nx)[SPLIT], const TokArgs& a, int bt, int t, int tid) {
    const int key = t * 32 + (tid >> 3);
    const size_t off = ((size_t)bt * a.N + min(key, a.N - 1)) * 64 + (tid & 7) * 8;
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) {
        const uint4 u = *(const uint4*)(a.ik[p] + off);
        nx[p] = key < a.N ? u : make_uint4(0, 0, 0, 0);
    }
}
template <int SPLIT>
__device__ __forceinline__ void tok_store(uint16_t (*dst)[32 * TK_KS], const uint4 (&nx)[SPLIT], int tid) {
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) *(uint4*)(dst[p] + (tid >> 3) * TK_KS + (tid & 7) * 8) = nx[p];
}

// Streams key tiles t0, t0 + step, ... (nt of them) through the LDS double
// buffer, calling body(t, tile) for each with the tile visible to the whole
// block.  Tiles are fetched kTokAhead iterations ahead into registers, so a
// load has that many tiles of work to arrive in.
constexpr int kTokAhead = 4;
template <int SPLIT, typename F>
__device__ __forceinline__ void tok_stream(const TokArgs& a, int bt, int t0, int nt, int step,
                                           TokLds<SPLIT>& lds, int tid, F&& body) {
    constexpr int P = kTokAhead;
    if (nt <= 0) return;
    uint4 pf[P][SPLIT];
#pragma unroll
    for (int s = 0; s < P; ++s) tok_load<SPLIT>(pf[s], a, bt, t0 + min(s, nt - 1) * step, tid);
    tok_store<SPLIT>(lds.k[0], pf[0], tid);
    tok_load<SPLIT>(pf[0], a, bt, t0 + min(P, nt - 1) * step, tid);
    __syncthreads();
    // Whole groups of P iterations, every one storing and fetching (a
    // clamped tile past the end), so the loads stay in flight across the
    // unrolled body and only the oldest is waited for.
    for (int i0 = 0; i0 < nt; i0 += P) {
#pragma unroll
        for (int s = 0; s < P; ++s) {
            const int i = i0 + s;
            if (i < nt) body(t0 + i * step, lds.k[i & 1][0]);
            const int sn = (s + 1) % P;
            tok_store<SPLIT>(lds.k[(i + 1) & 1], pf[sn], tid);
            tok_load<SPLIT>(pf[sn], a, bt, t0 + min(i + 1 + P, nt - 1) * step, tid);
            __syncthreads();
        }
    }
}

// Bins of the counting passes: 256 over the Cauchy-Schwarz range for the
// sample, kTokBins for the exact pass (bin 0 below the window, the last
// above it).  Counts sit bin-major in LDS, word bin * 64 + w for the rows
// 128b + w (low half) and 128b + 64 + w (high half), so the lanes of one
// instruction hit 32 distinct banks.
constexpr int kTokSampleBins = 256;
constexpr int kTokBins = 128;

// Adds one tile's scores to the row's bin counts.  DIAG: the tile holding
// the rows themselves (only keys before the row count); ALL: bin 0 counted
// too.
template <int BINS, bool DIAG, bool ALL>
__device__ __forceinline__ void count_tile(const f32x16& acc, float sa, float sc, uint32_t* hist,
                                           uint32_t woff, uint32_t inc, int col, int hh) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int cv = 8 * (v >> 2) + (v & 3) + 4 * hh;   // key - 32 t
        const float x = fmaf(acc[v], sa, sc);
        const uint32_t bin = (uint32_t)__builtin_amdgcn_fmed3f(x, 0.f, (float)(BINS - 1));
        bool take = ALL || bin != 0;
        if (DIAG) take = take && cv < col;
        if (take) atomicAdd(&hist[(bin << 6) | woff], inc);
    }
}

// Counting pass over one unit.  A unit adds at most 8192 to a count.
// SAMPLE: one unit per row block, key tiles 0, s, 2s, ..., bins over the
// Cauchy-Schwarz range, all bins counted.  Otherwise: the key tiles of the
// unit, bins from the row's window map, bin 0 (below the window) not
// counted.
template <int SPLIT, bool SAMPLE>
__global__ __launch_bounds__(TOK_THREADS) void tok_hist_kernel(TokArgs a) {
    constexpr int BINS = SAMPLE ? kTokSampleBins : kTokBins;
    __shared__ uint32_t hist[BINS * 64];
    __shared__ __attribute__((aligned(16))) TokLds<SPLIT> lds;
    __shared__ float red[TOK_WAVES];
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int bt = blockIdx.y, u = blockIdx.x;
    int b, t0, t1, step;
    if constexpr (SAMPLE) {
        b = tok_blocks(a.N) - 1 - u;
        t0 = 0;
        t1 = tok_tiles(a.N, b);
        step = max(1, min(kTokSample, t1 / 64));   // at least ~64 tiles, or all
    } else {
        int c;
        tok_unit(a.N, u, b, c);
        t0 = c * kTokChunk;
        t1 = min(t0 + kTokChunk, tok_tiles(a.N, b));
        step = 1;
    }
    // A block whose rows all keep every candidate (or none) needs no counts.
    if (min(a.N, (b + 1) * kTokRows) - 1 <= a.top_t) return;
    for (int x = tid; x < BINS * 64; x += TOK_THREADS) hist[x] = 0;

    const int rt = 4 * b + wave, row = rt * 32 + col;
    const bool row_ok = row < a.N;
    float sa = 0.f, sc = 128.f;
    if constexpr (SAMPLE) {
        sa = tok_scale(a, bt, row, row_ok, tok_kmax(a, bt, red, tid));
    } else if (row_ok) {
        const float2 m = a.win[(size_t)bt * a.N + row];
        sa = m.x;
        sc = m.y;
    }
    bf16x8 qf[SPLIT][4];
    load_qf<SPLIT>(qf, a, bt, row, row_ok, hh);
    const uint32_t inc = 1u << (16 * (wave >> 1));
    const uint32_t woff = (uint32_t)(32 * (wave & 1) + col);

    // The stream's first barrier also orders the zeroed counts before the
    // first add.
    tok_stream<SPLIT>(a, bt, t0, (t1 - t0 + step - 1) / step, step, lds, tid,
                      [&](int t, const uint16_t* kl) {
                          if (t < rt) {
                              const f32x16 acc = index_scores_lds<SPLIT>(kl, qf, lane);
                              count_tile<BINS, false, SAMPLE>(acc, sa, sc, hist, woff, inc, col, hh);
                          } else if (t == rt) {
                              const f32x16 acc = index_scores_lds<SPLIT>(kl, qf, lane);
                              count_tile<BINS, true, SAMPLE>(acc, sa, sc, hist, woff, inc, col, hh);
                          }
                      });
    const size_t slot = (size_t)bt * (SAMPLE ? tok_blocks(a.N) : a.units) + (SAMPLE ? b : u);
    uint4* dst = (uint4*)(a.part + slot * (BINS * 64));
    for (int x = tid; x < BINS * 16; x += TOK_THREADS) dst[x] = ((const uint4*)hist)[x];
}

// Bin b* (highest bin whose count from the top reaches k) of a histogram
// spread PER bins per lane (lane l: bins PER*l .. PER*l + PER - 1); above =
// count of the bins over b*, in_bin = count of b*.  Returns false when the
// histogram holds fewer than k entries.
template <int PER>
__device__ __forceinline__ bool tok_find(const uint32_t (&cnt)[PER], uint32_t k, int lane, int& bstar,
                                         uint32_t& above, uint32_t& in_bin) {
    uint32_t tot = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) tot += cnt[i];
    uint32_t incl = tot;   // count of bins >= PER lane
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_down(incl, d);
        if (lane + d < 64) incl += o;
    }
    const uint32_t excl = incl - tot;
    int fb = -1;
    uint32_t fa = 0, fh = 0;
    if (excl < k && incl >= k) {
        uint32_t cum = excl;
#pragma unroll
        for (int i = PER - 1; i >= 0; --i) {
            if (fb < 0 && cum + cnt[i] >= k) {
                fb = PER * lane + i;
                fa = cum;
                fh = cnt[i];
            }
            cum += cnt[i];
        }
    }
    const uint64_t m = __ballot(fb >= 0);
    if (m == 0) return false;
    const int src = __ffsll((unsigned long long)m) - 1;
    bstar = __shfl(fb, src);
    above = __shfl(fa, src);
    in_bin = __shfl(fh, src);
    return true;
}

// Sum of a value over the wave.
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
    return x;
}

// One wave per LDS word row w of block b (rows 128b + w, 128b + 64 + w):
// the window of the exact pass from the sampled counts.  With n candidates,
// s sampled and rank k, the k-th best is expected at sample rank
// k' = k s / n, with binomial deviation sd = sqrt(k' (1 - k'/s)); L is the
// lower edge of the bin where the sampled count from the top reaches
// k' + 6 sd + 16 (or -B), U the upper edge of the bin where it reaches
// k' - 6 sd - 16 (or +B).  win = map of [L, U) onto [1, kTokBins - 1).
__global__ __launch_bounds__(TOK_THREADS) void tok_window_kernel(TokArgs a) {
    __shared__ float red[TOK_WAVES];
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int bt = blockIdx.y, wr = blockIdx.x * TOK_WAVES + wave;
    const float kmax = tok_kmax(a, bt, red, threadIdx.x);
    const int nb = tok_blocks(a.N), b = wr >> 6, w = wr & 63;
    if (b >= nb) return;
    const int r0 = b * kTokRows + w, r1 = r0 + 64;
    int4 s0 = make_int4(0, 0, 0, (int)kTokNone), s1 = s0;
    if (r0 < a.N) s0 = a.state[(size_t)bt * a.N + r0];
    if (r1 < a.N) s1 = a.state[(size_t)bt * a.N + r1];
    const bool need0 = !(s0.w & (kTokAll | kTokNone)), need1 = !(s1.w & (kTokAll | kTokNone));
    if (!need0 && !need1) return;
    constexpr int PER = kTokSampleBins / 64;
    const uint32_t* src = a.part + ((size_t)bt * nb + b) * (kTokSampleBins * 64) + w;
    uint32_t c0[PER], c1[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const uint32_t wd = src[(PER * lane + i) * 64];
        c0[i] = wd & 0xffffu;
        c1[i] = wd >> 16;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (!(h ? need1 : need0)) continue;
        const uint32_t(&cnt)[PER] = h ? c1 : c0;
        const int row = h ? r1 : r0;
        const int k = (h ? s1 : s0).z;
        uint32_t own = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) own += cnt[i];
        const uint32_t ns = wave_sum(own);
        const float rho = (float)k * (float)ns / (float)row;
        const float m = 6.f * sqrtf(fmaxf(rho * (1.f - rho / fmaxf((float)ns, 1.f)), 0.f)) + 16.f;
        const float fhi = ceilf(rho + m), flo = floorf(rho - m);
        float xl = 0.f, xu = 256.f;
        int bs = 0;
        uint32_t ab = 0, ib = 0;
        if (fhi <= (float)ns && tok_find<PER>(cnt, (uint32_t)fhi, lane, bs, ab, ib)) xl = (float)bs;
        if (flo >= 1.f && tok_find<PER>(cnt, (uint32_t)flo, lane, bs, ab, ib)) xu = (float)(bs + 1);
        const float sa = tok_scale(a, bt, row, true, kmax), f = (float)(kTokBins - 2) / (xu - xl);
        if (lane == 0) a.win[(size_t)bt * a.N + row] = make_float2(sa * f, (128.f - xl) * f + 1.f);
    }
}

// Bin step: one wave per LDS word row w of block b (rows 128b + w and
// 128b + 64 + w): sum the unit counts, find b*.  state = {b*, 0 (collect
// counter), rank left inside b*, flags}.
__global__ __launch_bounds__(TOK_THREADS) void tok_bin_kernel(TokArgs a) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int bt = blockIdx.y, wr = blockIdx.x * TOK_WAVES + wave;
    const int nb = tok_blocks(a.N), b = wr >> 6, w = wr & 63;
    if (b >= nb) return;
    const int r0 = b * kTokRows + w, r1 = r0 + 64;
    int4 s0 = make_int4(0, 0, 0, (int)kTokNone), s1 = s0;
    if (r0 < a.N) s0 = a.state[(size_t)bt * a.N + r0];
    if (r1 < a.N) s1 = a.state[(size_t)bt * a.N + r1];
    const bool need0 = !(s0.w & (kTokAll | kTokNone)), need1 = !(s1.w & (kTokAll | kTokNone));
    if (!need0 && !need1) return;
    constexpr int PER = kTokBins / 64;
    uint32_t c0[PER] = {}, c1[PER] = {};
    const int nch = tok_chunks(a.N, b);
    for (int c = 0; c < nch; ++c) {
        const int u = tok_unit_base(a.N, c) + nb - 1 - b;
        const uint32_t* src = a.part + ((size_t)bt * a.units + u) * (kTokBins * 64) + w;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const uint32_t wd = src[(PER * lane + i) * 64];
            c0[i] += wd & 0xffffu;
            c1[i] += wd >> 16;
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (!(h ? need1 : need0)) continue;
        const int4 s = h ? s1 : s0;
        int bstar = 0;
        uint32_t above = 0, in_bin = 0;
        const bool found = tok_find<PER>(h ? c1 : c0, (uint32_t)s.z, lane, bstar, above, in_bin);
        const bool slow = !found || in_bin > (uint32_t)kTokCap;
        if (lane == 0) {
            a.state[(size_t)bt * a.N + (h ? r1 : r0)] =
                make_int4(bstar, 0, s.z - (int)above, s.w | (int)(slow ? kTokSlow : 0u));
            if (slow) atomicAdd(a.nslow, 1);
        }
    }
}

// Mask pass: the keep mask of every binned row: keys in bins above b* kept,
// candidates of b* collected (64-bit key) for the resolve step.  Rows left
// to the radix fallback are not written.
constexpr int kTokStage = 2048;   // candidates one mask unit can hold in LDS
template <int SPLIT>
__global__ __launch_bounds__(TOK_THREADS) void tok_mask_kernel(TokArgs a) {
    __shared__ __attribute__((aligned(16))) TokLds<SPLIT> lds;
    // Candidates of this unit: ord(score), and the low 24 bits of
    // 0xFFFFFFFF - j (j < 2^24: the top 8 bits are ones) under the local row.
    __shared__ uint2 stage[kTokStage];
    __shared__ int s_cnt;
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int bt = blockIdx.y, u = blockIdx.x;
    int b, c;
    tok_unit(a.N, u, b, c);
    const int t0 = c * kTokChunk, t1 = min(t0 + kTokChunk, tok_tiles(a.N, b));

    const int rt = 4 * b + wave, row = rt * 32 + col;
    const bool row_ok = row < a.N;
    const size_t gr = (size_t)bt * a.N + (row_ok ? row : 0);
    const float2 map = row_ok ? a.win[gr] : make_float2(0.f, 0.f);
    const int4 st = row_ok ? a.state[gr] : make_int4(0, 0, 0, (int)kTokNone);
    const uint32_t fl = (uint32_t)st.w;
    const bool write = row_ok && !(fl & kTokSlow);
    // keep <=> x >= keep_x <=> bin > b*; in bin b* <=> !keep && x >= in_x.
    float keep_x = 1e30f, in_x = 1e30f;
    if (fl & kTokAll) {
        keep_x = -1e30f;
    } else if (write && !(fl & kTokNone)) {
        keep_x = st.x < kTokBins - 1 ? (float)(st.x + 1) : 1e30f;
        in_x = st.x > 0 ? (float)st.x : -1e30f;
    }
    bf16x8 qf[SPLIT][4];
    load_qf<SPLIT>(qf, a, bt, row, row_ok, hh);
    const int nt32 = (a.N + 31) / 32, nt64 = (a.N + 63) / 64;
    const uint32_t lr = (uint32_t)(32 * wave + col);
    if (tid == 0) s_cnt = 0;   // ordered before any add by the stream's first barrier

    // Register v of a tile holds key 32 t + cv(v) + 4 hh; on the diagonal
    // tile only keys before the row count.
    uint32_t diag_bits = 0;
#pragma unroll
    for (int v = 0; v < 16; ++v) diag_bits |= (8 * (v >> 2) + (v & 3) + 4 * hh < col ? 1u : 0u) << v;

    // Keep bits of one tile; candidates of bin b* go to the LDS stage (the
    // wave-level test keeps that rare path out of the common one).
    tok_stream<SPLIT>(a, bt, t0, t1 - t0, 1, lds, tid, [&](int t, const uint16_t* kl) {
        if (t > rt) return;
        const f32x16 acc = index_scores_lds<SPLIT>(kl, qf, lane);
        const uint32_t cm = t < rt ? 0xffffu : diag_bits;
        uint32_t bits = 0;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float x = fmaf(acc[v], map.x, map.y);
            const bool keep = x >= keep_x;
            bits |= (keep ? 1u : 0u) << v;
            if (x >= in_x && !keep) {   // rare: a candidate of b*
                if (!((cm >> v) & 1u)) continue;
                const int pos = atomicAdd(&s_cnt, 1);
                const uint32_t o = ord32(acc[v]);
                const uint32_t j = (uint32_t)(t * 32 + 8 * (v >> 2) + (v & 3) + 4 * hh);
                if (pos < kTokStage) {
                    stage[pos] = make_uint2(o, (0xffffffu - j) | (lr << 24));
                } else {   // no room: the radix fallback takes the row
                    atomicOr(&a.state[gr].w, (int)kTokSlow);
                    atomicAdd(a.nslow, 1);
                }
            }
        }
        if (write) a.mask[mask_half(bt, nt32, nt64, rt, t, lane)] = (uint16_t)(bits & cm);
    });
    // Publish the staged candidates to their rows' lists (the stream ends
    // with a barrier).
    const int n = min(s_cnt, kTokStage);
    for (int e = tid; e < n; e += TOK_THREADS) {
        const uint2 h = stage[e];
        const size_t g = (size_t)bt * a.N + b * kTokRows + (h.y >> 24);
        const int pos = atomicAdd(&a.state[g].y, 1);
        // hits: (low word 0xFFFFFFFF - j, high word ord(score)) of the key
        if (pos < kTokCap) a.hits[g * kTokCap + pos] = make_uint2(0xff000000u | (h.y & 0xffffffu), h.x);
    }
}

// Resolve step: one wave per binned row: radix select (one byte per step, from
// the top of the 64-bit key) of the r best collected candidates, then
// their mask bits.
__global__ __launch_bounds__(TOK_THREADS) void tok_resolve_kernel(TokArgs a) {
    __shared__ uint32_t hs[TOK_WAVES][256];
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const long long gi = (long long)blockIdx.x * TOK_WAVES + wave;
    if (gi >= (long long)a.Bt * a.N) return;
    const int4 st = a.state[gi];
    if (st.w & (kTokAll | kTokNone | kTokSlow)) return;
    const int bt = (int)(gi / a.N), row = (int)(gi % a.N);
    const int n = min(st.y, kTokCap);
    constexpr int PER = kTokCap / 64;
    uint64_t key[PER];
    bool val[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        const int e = lane + 64 * m;
        val[m] = e < n;
        uint2 h = make_uint2(0, 0);
        if (val[m]) h = a.hits[gi * kTokCap + e];
        key[m] = ((uint64_t)h.y << 32) | h.x;
    }
    uint32_t* hw = hs[wave];
    uint64_t prefix = 0, pmask = 0;
    uint32_t rem = (uint32_t)st.z;
    bool ok = true;
    for (int d = 7; d >= 0; --d) {
        const int sh = 8 * d;
#pragma unroll
        for (int i = 0; i < 4; ++i) hw[4 * lane + i] = 0;
        wave_sync();
#pragma unroll
        for (int m = 0; m < PER; ++m)
            if (val[m] && (key[m] & pmask) == prefix) atomicAdd(&hw[(uint32_t)(key[m] >> sh) & 255u], 1u);
        wave_sync();
        uint32_t cnt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cnt[i] = hw[4 * lane + i];
        int bstar = 0;
        uint32_t above = 0, in_bin = 0;
        if (!tok_find<4>(cnt, rem, lane, bstar, above, in_bin)) {
            ok = false;   // fewer candidates than the rank: counts disagree
            break;
        }
        prefix |= (uint64_t)bstar << sh;
        pmask |= (uint64_t)0xff << sh;
        rem -= above;
        wave_sync();
        if (in_bin == rem) break;   // every candidate of this bin is kept
    }
    if (!ok) return;
    const int nt32 = (a.N + 31) / 32, nt64 = (a.N + 63) / 64, rt = row >> 5;
    uint32_t* mask32 = (uint32_t*)a.mask;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        if (!val[m] || key[m] < prefix) continue;
        const int j = (int)(0xffffffffu - (uint32_t)key[m]);
        if (j < 0 || j >= row) continue;   // never taken: collected keys are earlier tokens
        const int kc = j >> 5, jl = j & 31;
        const int ln = (row & 31) + 32 * ((jl >> 2) & 1), v = 4 * (jl >> 3) + (jl & 3);
        const size_t hf = mask_half(bt, nt32, nt64, rt, kc, ln);
        atomicOr(&mask32[hf >> 1], 1u << (16 * (hf & 1) + v));
    }
}

// ---------------------------------------------------------------------------
// Radix fallback for the rows flagged kTokSlow: one pass over the
// candidates of a 32-row tile (4 waves split the key tiles).  pass 0..7:
// radix histogram step (score bytes, then bytes of 0xFFFFFFFF - j); pass 8:
// write the keep mask of those rows.
template <int SPLIT>
__global__ __launch_bounds__(TOK_THREADS) void token_select_kernel(TokArgs a, int pass) {
    if (*a.nslow == 0) return;
    __shared__ uint32_t hist[32 * HSTRIDE];
    __shared__ int s_skip;
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int nt = (a.N + 31) / 32;
    // Row tiles with the most candidates first (they run longest).
    const int rt = nt - 1 - (int)(blockIdx.x % nt), bt = blockIdx.x / nt;
    const int r0 = rt * 32;
    const int row = r0 + col;
    const bool row_ok = row < a.N;
    int4* state = a.state + (size_t)bt * a.N;

    // Row state: x = ordered-score prefix, y = index-key prefix, z = keys
    // still to take, w = flags.
    int4 stt = make_int4(0, 0, 0, (int)(kTokNone | kTokDone | kTokFast));
    if (row_ok) {
        stt = state[row];
        if (pass == 0) {
            if (stt.w & kTokSlow) stt = make_int4(0, 0, min(a.top_t, row), 0);
            else stt = make_int4(0, 0, 0, stt.w | (int)(kTokDone | kTokFast));
        }
    }
    const uint32_t flags = (uint32_t)stt.w;
    const uint32_t pre32 = (uint32_t)stt.x, preidx = (uint32_t)stt.y;

    if (tid == 0) s_skip = 1;
    __syncthreads();
    if (!(flags & (pass < 8 ? kTokDone : kTokFast))) s_skip = 0;   // benign race: every writer stores 0
    if (pass < 8)
        for (int x = tid; x < 32 * HSTRIDE; x += TOK_THREADS) hist[x] = 0;
    __syncthreads();
    if (s_skip) {
        if (pass == 0 && tid < 32 && row_ok) state[row] = stt;
        return;
    }

    bf16x8 qf[SPLIT][4];
    load_qf<SPLIT>(qf, a, bt, row, row_ok, hh);

    const bool active = !(flags & kTokDone);
    // Byte of the key examined in this pass and the prefix that must match.
    const int shift = pass < 4 ? 24 - 8 * pass : 24 - 8 * (pass - 4);
    for (int kc = wave; kc <= rt; kc += TOK_WAVES) {
        const f32x16 acc = index_scores<SPLIT>(a, bt, kc, qf, lane);
        const int rj = row - kc * 32 - 4 * hh;   // row - key = rj - cv
        if (pass < 8) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int cv = 8 * (v >> 2) + (v & 3);
                const uint32_t o = ord32(acc[v]);
                bool take = active && rj > cv;
                uint32_t digit;
                if (pass < 4) {
                    if (pass > 0) take = take && ((o ^ pre32) >> (shift + 8)) == 0;
                    digit = (o >> shift) & 0xffu;
                } else {
                    const uint32_t ik = 0xffffffffu - (uint32_t)(kc * 32 + 4 * hh + cv);
                    take = take && o == pre32;
                    if (pass > 4) take = take && ((ik ^ preidx) >> (shift + 8)) == 0;
                    digit = (ik >> shift) & 0xffu;
                }
                if (take) atomicAdd(&hist[col * HSTRIDE + digit], 1u);
            }
        } else if (row_ok && !(flags & kTokFast)) {
            // Keep mask: key >= threshold.
            uint32_t bits = 0;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int cv = 8 * (v >> 2) + (v & 3);
                const uint32_t o = ord32(acc[v]);
                const uint32_t ik = 0xffffffffu - (uint32_t)(kc * 32 + 4 * hh + cv);
                const bool keep = rj > cv && (o > pre32 || (o == pre32 && ik >= preidx));
                bits |= (keep ? 1u : 0u) << v;
            }
            a.mask[mask_half(bt, nt, (a.N + 63) / 64, rt, kc, lane)] = (uint16_t)bits;
        }
    }
    if (pass == 8) return;
    __syncthreads();
    if (tid < 32 && row_ok) {
        if (active) {
            // Bin holding the k-th largest remaining key.
            uint32_t k = (uint32_t)stt.z, cum = 0;
            int b = 255;
            for (; b > 0; --b) {
                const uint32_t h = hist[tid * HSTRIDE + b];
                if (cum + h >= k) break;
                cum += h;
            }
            const uint32_t hb = hist[tid * HSTRIDE + b];
            k -= cum;
            uint32_t fl = flags;
            if (pass < 4) {
                stt.x = (int)(pre32 | ((uint32_t)b << shift));
                // After the last score byte: if every candidate tied at the
                // threshold is kept, the index bits need no selection.
                if (pass == 3 && hb == k) {
                    fl |= kTokDone;
                    stt.y = 0;
                }
            } else {
                stt.y = (int)(preidx | ((uint32_t)b << shift));
                if (pass == 7) fl |= kTokDone;
            }
            stt.z = (int)k;
            stt.w = (int)fl;
        }
        state[row] = stt;
    }
}

// Ascending token ids kept by each row, -1 padded, from the keep mask.
__global__ void token_list_kernel(TokArgs a, int32_t* out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int total = a.Bt * a.N;
    if (i >= total) return;
    const int bt = i / a.N, row = i % a.N;
    const int nt = (a.N + 31) / 32, nt64 = (a.N + 63) / 64, rt = row / 32, L = row % 32;
    int32_t* dst = out + (size_t)i * a.top_t;
    int n = 0;
    for (int kc = 0; kc <= rt && n < a.top_t; ++kc) {
        const uint32_t m0 = a.mask[mask_half(bt, nt, nt64, rt, kc, L)];        // lanes L
        const uint32_t m1 = a.mask[mask_half(bt, nt, nt64, rt, kc, L + 32)];   // and L+32
        for (int jl = 0; jl < 32 && n < a.top_t; ++jl) {
            const int v = 4 * (jl >> 3) + (jl & 3), h = (jl >> 2) & 1;
            if (((h ? m1 : m0) >> v) & 1u) dst[n++] = kc * 32 + jl;
        }
    }
    for (; n < a.top_t; ++n) dst[n] = -1;
}

hipError_t launch_token_select(const TokArgs& a, int split, hipStream_t s) {
    hipLaunchKernelGGL(tok_prep_kernel, dim3((unsigned)a.nkp, (unsigned)a.Bt), dim3(TOK_THREADS), 0, s,
                       a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.units > 0) {
        const dim3 ug((unsigned)a.units, (unsigned)a.Bt), bg((unsigned)tok_blocks(a.N), (unsigned)a.Bt);
        const dim3 wg((unsigned)(tok_blocks(a.N) * 64 / TOK_WAVES), (unsigned)a.Bt);
        if (split == 2)
            hipLaunchKernelGGL((tok_hist_kernel<2, true>), bg, dim3(TOK_THREADS), 0, s, a);
        else
            hipLaunchKernelGGL((tok_hist_kernel<1, true>), bg, dim3(TOK_THREADS), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(tok_window_kernel, wg, dim3(TOK_THREADS), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (split == 2)
            hipLaunchKernelGGL((tok_hist_kernel<2, false>), ug, dim3(TOK_THREADS), 0, s, a);
        else
            hipLaunchKernelGGL((tok_hist_kernel<1, false>), ug, dim3(TOK_THREADS), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(tok_bin_kernel, wg, dim3(TOK_THREADS), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (split == 2)
            hipLaunchKernelGGL(tok_mask_kernel<2>, ug, dim3(TOK_THREADS), 0, s, a);
        else
            hipLaunchKernelGGL(tok_mask_kernel<1>, ug, dim3(TOK_THREADS), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const long long rows = (long long)a.Bt * a.N;
        hipLaunchKernelGGL(tok_resolve_kernel, dim3((unsigned)((rows + TOK_WAVES - 1) / TOK_WAVES)),
                           dim3(TOK_THREADS), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int nt = (a.N + 31) / 32;
    const dim3 grid((unsigned)(nt * a.Bt));
    for (int pass = 0; pass <= 8; ++pass) {
        if (split == 2)
            hipLaunchKernelGGL(token_select_kernel<2>, grid, dim3(TOK_THREADS), 0, s, a, pass);
        else
            hipLaunchKernelGGL(token_select_kernel<1>, grid, dim3(TOK_THREADS), 0, s, a, pass);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

// Key-major copy of the keep mask for the backward's key-centric pass: for
// the 32 keys kc*32 .. kc*32+31, the 64 rows rt*64 .. rt*64+63 and lane L,
// word maskT[((bt*NT32 + kc)*NT64 + rt)*64 + L] has bit 16*sub + v set iff
// row rt*64 + 32*sub + 8*(v/4) + 4*(L/32) + v%4 keeps key kc*32 + L%32 (the
// register layout of S = Q K^T with lane = key).  One workgroup (128
// threads) per (batch, 64-row tile, run of up to 16 64-key tiles): each
// 64 x 64 block goes through LDS as row bitmaps.  Blocks wholly above the
// diagonal are zero; the mask halves the forward layout leaves unwritten
// are read as zero.
constexpr int kTransRun = 16;
__global__ __launch_bounds__(128) void tok_mask_transpose_kernel(TokArgs a, uint32_t* maskT) {
    __shared__ uint32_t rowbits[64][2];
    const int tid = threadIdx.x;
    const int rt = blockIdx.y, bt = blockIdx.z;
    const int nt32 = (a.N + 31) / 32, nt64 = (a.N + 63) / 64;
    const uint32_t* mask32 = (const uint32_t*)a.mask;
    const int kt_begin = blockIdx.x * kTransRun;
    for (int kt = kt_begin; kt < min(kt_begin + kTransRun, nt64); ++kt) {
        // Read: thread t takes forward word (row tile 2 rt + t / 64, key tile
        // kt, lane t % 64): row 32 (t / 64) + t % 32 of the block, the keys
        // 32 sub + 8 (v / 4) + 4 hh + v % 4 with hh = (t / 32) % 2.
        const int r32 = 2 * rt + tid / 64, L = tid & 63, hh = L >> 5;
        uint32_t w = 0;
        if (kt <= r32 / 2 && r32 < nt32) {
            w = mask32[(((size_t)bt * nt32 + r32) * nt64 + kt) * 64 + L];
            if (2 * kt + 1 > r32) w &= 0xffffu;   // the half past the row tile
        }
        uint32_t lo = 0, hi = 0;   // keys 0..31, 32..63 of the block
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int kl = 8 * (v >> 2) + 4 * hh + (v & 3);
            lo |= ((w >> v) & 1u) << kl;
            hi |= ((w >> (16 + v)) & 1u) << kl;
        }
        // Lanes L and L ^ 32 hold the two key halves of the same row.
        lo |= (uint32_t)__shfl_xor((int)lo, 32);
        hi |= (uint32_t)__shfl_xor((int)hi, 32);
        __syncthreads();   // the previous block's reads of rowbits are done
        if (hh == 0) {
            const int row = 32 * (tid / 64) + (L & 31);
            rowbits[row][0] = lo;
            rowbits[row][1] = hi;
        }
        __syncthreads();
        // Write: thread t makes word (key group 2 kt + t / 64, row tile rt,
        // lane t % 64).
        const int kc = 2 * kt + tid / 64, col = L & 31;
        if (kc < nt32) {
            uint32_t o = 0;
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = 32 * sub + 8 * (v >> 2) + (v & 3) + 4 * hh;
                    o |= ((rowbits[row][tid / 64] >> col) & 1u) << (16 * sub + v);
                }
            maskT[(((size_t)bt * nt32 + kc) * nt64 + rt) * 64 + L] = o;
        }
    }
}

hipError_t launch_token_mask_transpose(const TokArgs& a, uint32_t* maskT, hipStream_t s) {
    const int nt64 = (a.N + 63) / 64;
    if (a.Bt == 0 || nt64 == 0) return hipSuccess;
    const dim3 grid((unsigned)((nt64 + kTransRun - 1) / kTransRun), (unsigned)nt64, (unsigned)a.Bt);
    hipLaunchKernelGGL(tok_mask_transpose_kernel, grid, dim3(128), 0, s, a, maskT);
    return hipGetLastError();
}

hipError_t launch_token_list(const TokArgs& a, int32_t* out, hipStream_t s) {
    const int total = a.Bt * a.N;
    hipLaunchKernelGGL(token_list_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a,
                       out);
    return hipGetLastError();
}

}  // namespace sa
