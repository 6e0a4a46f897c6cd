// sa_decode.hip -- decode/append step: a few new queries continuing a cached
// history.
//
// [Bit-Axon SWA + MoE page, "슬라이딩 윈도우 마스크"]: while decoding, the KV
// cache is longer than the queries; the causal offset kv_len - seq_len
// places query row r at position p = r + off, which attends j <= p with
// p - j < w.  [Naive-N0.5-Flash page, "SWA와 DSA를 결합한 어텐션"]: the
// indexer scans the whole cached history and the top tokens join the window
// (same reading as the prefill: candidates j < p, keep min(top_t, p), a tie
// to the lower j).  [MoBA summary page, the long-context experiments]:
// generation runs full attention, i.e. a window of kv_len or more.
//
// Decode reads the cache once and does little arithmetic per byte, so the
// kernels are vector-ALU kernels in fp32:
//   dec_scores  : indexer scores of every (query, key), fp32, to workspace.
//   dec_select  : per query, exact top-k on the 48-bit key
//                 ord(score) << 16 | (0xFFFF - j): 4096 linear score bins
//                 locate the threshold bin, whose few members are resolved
//                 exactly; then the kept ids as an ascending list and the
//                 count below the window.  For a few queries over a long
//                 history: per-slice selections on eight workgroups per
//                 query, then their merge.
//   dec_attn    : per (batch, kv head, query, chunk of 128 attended keys (64
//                 for fp32) -- the window [lo, p] first, then the kept tokens
//                 before lo): the chunk's K and V rows staged in LDS, logits,
//                 chunk max and sum, and the chunk's P V, for every q head of
//                 the kv group from one load of each key and value.
//   dec_combine : merges the chunk partials and the sink column; out, lse.
#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

constexpr int DEC_THREADS = 256;
constexpr int SEL_THREADS = 1024;   // one workgroup per query scans its history

__device__ __forceinline__ float dec_load(const void* p, size_t i, int f32) {
    return f32 ? ((const float*)p)[i] : bf16_to_f32(((const uint16_t*)p)[i]);
}

// Eight consecutive elements starting at element i (a multiple of 8) as fp32.
template <bool F32>
__device__ __forceinline__ void dec_load8(const void* p, size_t i, float (&x)[8]) {
    if constexpr (F32) {
        const float4 a = *(const float4*)((const float*)p + i), b = *(const float4*)((const float*)p + i + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
        const uint4 u = *(const uint4*)((const uint16_t*)p + i);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            x[2 * t] = bf16_to_f32(w[t] & 0xffffu);
            x[2 * t + 1] = bf16_to_f32(w[t] >> 16);
        }
    }
}

__device__ __forceinline__ uint32_t dec_ord32(float s) {
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Indexer scores [Bt, Nq, Nk]: one key per thread against every query.
template <bool F32>
__global__ __launch_bounds__(DEC_THREADS) void dec_scores_kernel(DecArgs a) {
    __shared__ float qs[kDecMaxQ * 64];
    const int bt = blockIdx.y, tid = threadIdx.x, j = blockIdx.x * DEC_THREADS + tid;
    for (int x = tid; x < a.Nq * 64; x += DEC_THREADS)
        qs[x] = dec_load(a.iq, (size_t)bt * a.Nq * 64 + x, a.f32);
    __syncthreads();
    if (j >= a.Nk) return;
    float kj[64];
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
        float x8[8];
        dec_load8<F32>(a.ik, ((size_t)bt * a.Nk + j) * 64 + e8 * 8, x8);
#pragma unroll
        for (int t = 0; t < 8; ++t) kj[e8 * 8 + t] = x8[t];
    }
    for (int r = 0; r < a.Nq; ++r) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 64; ++e) s = fmaf(qs[r * 64 + e], kj[e], s);
        a.scores[((size_t)bt * a.Nq + r) * a.Nk + j] = s;
    }
}

// Block-wide exclusive prefix sum of one value per thread (SEL_THREADS
// threads, 16 waves): wave scans by shuffles, then the wave totals through
// LDS (wsum, 16 entries).  *total receives the sum.
__device__ __forceinline__ int dec_scan(int x, int* wsum, int tid, int* total) {
    const int lane = tid & 63, w = tid >> 6;
    int incl = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < SEL_THREADS / 64; ++i) {
        const int v = wsum[i];
        off += i < w ? v : 0;
        tot += v;
    }
    *total = tot;
    __syncthreads();
    return off + incl - x;
}

// Histogram increment from every active lane; lanes that all hit the same
// bin (ties, narrow ranges) are merged into one atomic.
__device__ __forceinline__ void dec_hist_add(uint32_t* h, uint32_t bin, bool on) {
    const uint64_t act = __ballot(on);
    if (act == 0) return;
    const uint32_t first = (uint32_t)__builtin_amdgcn_readfirstlane(on ? bin : 0xffffffffu);
    const uint64_t same = __ballot(on && bin == first);
    if (same == act) {
        if ((__lane_id() == (uint32_t)__builtin_ctzll(act))) atomicAdd(&h[first], (uint32_t)__popcll(act));
    } else if (on) {
        atomicAdd(&h[bin], 1u);
    }
}

// Highest bin b of a 256-bin histogram whose count from the top reaches k
// (one wave, 4 bins per lane): out = {b, count above b, count of b}.  The
// histogram holds at least k entries.
__device__ __forceinline__ void dec_find(const uint32_t* hist, uint32_t k, int lane, uint32_t* out) {
    uint32_t cnt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cnt[i] = hist[4 * lane + i];
    const uint32_t tot = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    uint32_t incl = tot;   // count of bins >= 4 lane
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_down(incl, d);
        if (lane + d < 64) incl += o;
    }
    const uint32_t excl = incl - tot;
    if (excl < k && incl >= k) {
        uint32_t cum = excl;
        for (int i = 3; i >= 0; --i) {
            if (cum + cnt[i] >= k) {
                out[0] = (uint32_t)(4 * lane + i);
                out[1] = cum;
                out[2] = cnt[i];
                break;
            }
            cum += cnt[i];
        }
    }
}

constexpr int kSelBins = 4096;          // linear score bins
constexpr int kSelRank = 256;           // threshold-bin size resolved by rank counting
constexpr uint16_t kSelKept = 0xffff;   // bin mark of a kept member of b*

// Linear bin of score s over [mn, mn + kSelBins / inv]; inv == 0 puts every
// score in bin 0.  Non-decreasing in s, so bins order the keys.
__device__ __forceinline__ uint32_t dec_bin(float s, float mn, float inv) {
    if (!(inv > 0.f)) return 0u;
    const float t = (s - mn) * inv;
    return t < (float)(kSelBins - 1) ? (uint32_t)t : (uint32_t)(kSelBins - 1);
}

// 48-bit key of token j with score s: ord(score) << 16 | (0xFFFF - j).
__device__ __forceinline__ uint64_t dec_key(float s, int j) {
    return (uint64_t)dec_ord32(s) << 16 | (uint64_t)(0xffffu - (uint32_t)j);
}

// Selection modes of dec_select_kernel.
enum SelMode { kSelWhole = 0, kSelPart = 1, kSelMerge = 2 };
constexpr int kSelParts = kDecSelParts;   // slices of a long history
constexpr int kSelSlice = 65536 / kSelParts;

// Kept tokens of one query: min(top_t, p) best of j < p, ascending, -1
// padded; nfar = how many of them lie before the window start lo.  Keys are
// unique (the index breaks score ties toward the lower j).
//
// The candidates of one selection are n tokens in ascending id order; thread
// t handles candidates x = u * SEL_THREADS + t (u < PT).  MODE kSelWhole: the
// whole history, x = j.  A long history is split: kSelPart selects, for each
// of kSelParts slices of kSelSlice ids (blockIdx.z), the min(quota, slice
// length) best of the slice into plist, ids then their scores (count in
// pcnt); kSelMerge then selects from the concatenated slice lists (ids and
// scores staged in LDS).  A slice
// whose ids were not all passed on dropped only keys below its lowest
// passed key; when that key is not among the merged best (or the slice
// passed on everything, or quota = top_t), nothing dropped can beat the
// merged k-th key and the result is the whole history's.  Otherwise the
// merge sets redo for the query, and kSelWhole, launched with redo, selects
// those queries again (it returns at once for the others).
//   1. the candidates' score range (scores held in registers for 1-2);
//   2. 4096 linear bins over that range: each candidate's bin is kept in
//      LDS (16 bits) and counted in an LDS histogram;
//   3. the bin b* holding the k-th best key and the count above it; the
//      rem = k - above best members of b* are marked kept (bin 0xFFFF):
//      by rank counting over the members gathered in LDS when b* holds at
//      most 256 keys, else by a byte-wise radix select over its members'
//      48-bit keys (6 passes, scores reloaded);
//   4. kept = bin above b* (marks included), written in candidate (= id)
//      order from wave ballots and one block scan.
template <int PT, int MODE>
__global__ __launch_bounds__(SEL_THREADS) void dec_select_kernel(DecArgs a) {
    constexpr int NW = SEL_THREADS / 64;
    constexpr int NC = PT * SEL_THREADS;   // candidate capacity
    __shared__ uint16_t binv[NC];
    __shared__ uint32_t hist[kSelBins];
    __shared__ int sh[SEL_THREADS];
    __shared__ int wsum[NW];
    __shared__ float s_mm[2 * NW];
    __shared__ uint32_t s_b[3];
    __shared__ uint32_t s_n;
    __shared__ uint64_t cand[kSelRank];
    __shared__ int s_ids[MODE == kSelMerge ? NC : 1];
    __shared__ float s_sc[MODE == kSelMerge ? NC : 1];
    __shared__ int s_sel[kSelParts];   // merge: merged best per slice
    const int r = blockIdx.x, bt = blockIdx.y, part = blockIdx.z, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const size_t row = (size_t)bt * a.Nq + r;
    if constexpr (MODE == kSelWhole) {
        if (a.redo && a.redo[row] == 0) return;   // the merge's result stands
    }
    if (tid < kSelParts) s_sel[tid] = 0;
    const int p = a.Nk - a.Nq + r;
    const int lo = a.window > 0 ? max(0, p - a.window + 1) : p;
    const float* sc = a.scores + row * a.Nk;

    // This selection's candidates [0, n), their ids and how many to keep.
    int n, j0 = 0, k;
    if constexpr (MODE == kSelWhole) {
        n = p;
        k = min(a.top_t, p);
    } else if constexpr (MODE == kSelPart) {
        j0 = part * kSelSlice;
        n = max(0, min(p - j0, kSelSlice));
        k = min(a.quota, n);
    } else {
        // concatenate the slice lists (each ascending, slices in order)
        const int32_t* pc = a.pcnt + row * kSelParts;
        int off[kSelParts + 1];
        off[0] = 0;
#pragma unroll
        for (int q = 0; q < kSelParts; ++q) off[q + 1] = off[q] + pc[q];
        n = off[kSelParts];
#pragma unroll
        for (int q = 0; q < kSelParts; ++q) {
            const int32_t* pl = a.plist + (row * kSelParts + q) * 2 * a.top_t;
            for (int x = tid; x < pc[q]; x += SEL_THREADS) {
                s_ids[off[q] + x] = pl[x];
                s_sc[off[q] + x] = __int_as_float(pl[a.top_t + x]);
            }
        }
        k = min(a.top_t, p);
        __syncthreads();
    }
    auto id_of = [&](int x) -> int {
        if constexpr (MODE == kSelMerge) return s_ids[x];
        else return j0 + x;
    };
    auto score_of = [&](int x) -> float {
        if constexpr (MODE == kSelMerge) return s_sc[x];
        else return sc[j0 + x];
    };
    const bool sel = k > 0 && k < n;   // otherwise every candidate (k >= n) or none is kept
    uint32_t bstar = 0;

    if (sel) {
        // 1. range (slots past n re-read candidate n - 1, which leaves it unchanged)
        float sv[PT];
#pragma unroll
        for (int u = 0; u < PT; ++u) sv[u] = score_of(min(u * SEL_THREADS + tid, n - 1));
        float lo_s = sv[0], hi_s = sv[0];
#pragma unroll
        for (int u = 1; u < PT; ++u) {
            lo_s = fminf(lo_s, sv[u]);
            hi_s = fmaxf(hi_s, sv[u]);
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            lo_s = fminf(lo_s, __shfl_xor(lo_s, d));
            hi_s = fmaxf(hi_s, __shfl_xor(hi_s, d));
        }
        if (lane == 0) {
            s_mm[w] = lo_s;
            s_mm[NW + w] = hi_s;
        }
        for (int x = tid; x < kSelBins; x += SEL_THREADS) hist[x] = 0;
        __syncthreads();
        lo_s = s_mm[0];
        hi_s = s_mm[NW];
#pragma unroll
        for (int i = 1; i < NW; ++i) {
            lo_s = fminf(lo_s, s_mm[i]);
            hi_s = fmaxf(hi_s, s_mm[NW + i]);
        }
        const float mn = lo_s;
        float inv = (float)kSelBins / (hi_s - lo_s);
        if (!(inv > 0.f && inv <= 3.0e38f)) inv = 0.f;

        // 2. bins
#pragma unroll
        for (int u = 0; u < PT; ++u) {
            const uint32_t b = dec_bin(sv[u], mn, inv);
            const bool valid = tid < n - u * SEL_THREADS;
            if (valid) binv[u * SEL_THREADS + tid] = (uint16_t)b;
            dec_hist_add(hist, b, valid);
        }
        __syncthreads();

        // 3. threshold bin: thread t holds bins 4095 - 4t - i, highest first
        uint32_t cnt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cnt[i] = hist[kSelBins - 1 - 4 * tid - i];
        const int tot = (int)(cnt[0] + cnt[1] + cnt[2] + cnt[3]);
        int total = 0;
        const int excl = dec_scan(tot, wsum, tid, &total);
        if (excl < k && excl + tot >= k) {
            uint32_t cum = (uint32_t)excl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (cum < (uint32_t)k && cum + cnt[i] >= (uint32_t)k) {
                    s_b[0] = (uint32_t)(kSelBins - 1 - 4 * tid - i);
                    s_b[1] = cum;
                    s_b[2] = cnt[i];
                }
                cum += cnt[i];
            }
        }
        if (tid == 0) s_n = 0;
        __syncthreads();
        bstar = s_b[0];
        const uint32_t in_bin = s_b[2];
        uint32_t rem = (uint32_t)k - s_b[1];   // 1 <= rem <= in_bin

        if (in_bin <= (uint32_t)kSelRank) {
            // gather b* as (48-bit key, candidate) in 64 bits (keys are
            // unique, so the candidate never decides an order); a member is
            // kept when fewer than rem members beat it
            for (int u = 0; u < PT; ++u) {
                const int x = u * SEL_THREADS + tid;
                if (x < n && binv[x] == bstar) {
                    const int j = id_of(x);
                    cand[atomicAdd(&s_n, 1u)] = dec_key(score_of(x), j) << 16 | (uint64_t)x;
                }
            }
            __syncthreads();
            if (tid < (int)in_bin) {
                const uint64_t me = cand[tid];
                uint32_t above = 0;
                for (uint32_t x = 0; x < in_bin; ++x) above += cand[x] > me;
                if (above < rem) binv[(int)(me & 0xffffu)] = kSelKept;
            }
        } else {
            // radix select of the rem-th best member key, then mark
            uint32_t pre_hi = 0, msk_hi = 0, pre_lo = 0, msk_lo = 0;
            for (int d = 5; d >= 0; --d) {
                if (tid < 256) hist[tid] = 0;
                __syncthreads();
                for (int u = 0; u < PT; ++u) {
                    const int x = u * SEL_THREADS + tid;
                    const bool in = x < n && binv[x] == bstar;
                    uint32_t ov = 0, ix = 0;
                    if (in) {
                        const int j = id_of(x);
                        ov = dec_ord32(score_of(x));
                        ix = 0xffffu - (uint32_t)j;
                    }
                    const bool match = in && (ov & msk_hi) == pre_hi && (ix & msk_lo) == pre_lo;
                    const uint32_t digit = d >= 2 ? (ov >> (8 * d - 16)) & 255u : (ix >> (8 * d)) & 255u;
                    dec_hist_add(hist, digit, match);
                }
                __syncthreads();
                if (tid < 64) dec_find(hist, rem, tid, s_b);
                __syncthreads();
                const uint32_t b = s_b[0];
                if (d >= 2) {
                    pre_hi |= b << (8 * d - 16);
                    msk_hi |= 255u << (8 * d - 16);
                } else {
                    pre_lo |= b << (8 * d);
                    msk_lo |= 255u << (8 * d);
                }
                rem -= s_b[1];
                __syncthreads();
            }
            const uint64_t thr = (uint64_t)pre_hi << 16 | pre_lo;
            for (int u = 0; u < PT; ++u) {
                const int x = u * SEL_THREADS + tid;
                if (x < n && binv[x] == bstar) {
                    const int j = id_of(x);
                    if (dec_key(score_of(x), j) >= thr) binv[x] = kSelKept;
                }
            }
        }
        __syncthreads();
    }

    // 4. kept ids in candidate order; lane u of each wave keeps the wave's
    // ballot for slot u
    uint32_t mlo = 0, mhi = 0;
    int nlo = 0;
#pragma unroll
    for (int u = 0; u < PT; ++u) {
        const int x = u * SEL_THREADS + tid;
        bool kp = x < n && k > 0;
        if (sel) kp = kp && binv[min(x, n - 1)] > bstar;
        const uint64_t m = __ballot(kp);
        mlo = lane == u ? (uint32_t)m : mlo;
        mhi = lane == u ? (uint32_t)(m >> 32) : mhi;
        nlo += kp && id_of(min(x, max(n - 1, 0))) < lo;
    }
    sh[lane * NW + w] = __popc(mlo) + __popc(mhi);   // entry (u, w) at u * NW + w
    __syncthreads();
    int total = 0, total_lo = 0;
    const int ex = dec_scan(sh[tid], wsum, tid, &total);
    sh[tid] = ex;
    dec_scan(nlo, wsum, tid, &total_lo);   // its barriers also publish sh
    const int base = sh[lane * NW + w];
    const uint32_t below_lo = lane >= 32 ? 0xffffffffu : (1u << lane) - 1u;
    const uint32_t below_hi = lane < 32 ? 0u : (lane == 63 ? 0x7fffffffu : (1u << (lane - 32)) - 1u);
    int32_t* const list = MODE == kSelPart ? a.plist + (row * kSelParts + part) * 2 * a.top_t
                                           : a.list + row * a.top_t;
    int scnt[kSelParts] = {};   // merge: this wave's kept ids per slice
#pragma unroll
    for (int u = 0; u < PT; ++u) {
        const uint32_t ml = (uint32_t)__builtin_amdgcn_readlane((int)mlo, u);
        const uint32_t mh = (uint32_t)__builtin_amdgcn_readlane((int)mhi, u);
        const bool kp = ((lane < 32 ? ml >> lane : mh >> (lane - 32)) & 1u) != 0;
        const int pos = __builtin_amdgcn_readlane(base, u) + __popc(ml & below_lo) + __popc(mh & below_hi);
        const int id = kp ? id_of(u * SEL_THREADS + tid) : 0;
        if (kp && pos < a.top_t) {
            list[pos] = id;
            if constexpr (MODE == kSelPart) list[a.top_t + pos] = __float_as_int(sc[id]);
        }
        if constexpr (MODE == kSelMerge) {
#pragma unroll
            for (int q = 0; q < kSelParts; ++q) scnt[q] += (int)__popcll(__ballot(kp && id / kSelSlice == q));
        }
    }
    if constexpr (MODE == kSelPart) {
        if (tid == 0) a.pcnt[row * kSelParts + part] = min(total, a.quota);
    } else {
        for (int x = total + tid; x < a.top_t; x += SEL_THREADS) list[x] = -1;
        if (tid == 0) a.nfar[row] = total_lo;
    }
    if constexpr (MODE == kSelMerge) {
        if (lane == 0) {
#pragma unroll
            for (int q = 0; q < kSelParts; ++q) atomicAdd(&s_sel[q], scnt[q]);
        }
        __syncthreads();
        if (tid == 0) {
            // a slice that held ids back and saw every id it passed on kept
            // may have dropped a better one than the merged k-th
            int redo = 0;
            if (a.quota < a.top_t) {
                for (int q = 0; q < kSelParts; ++q) {
                    const int ns = max(0, min(p - q * kSelSlice, kSelSlice));
                    redo |= ns > a.quota && s_sel[q] >= a.quota;
                }
            }
            a.redo[row] = redo;
        }
    }
}

// Attended keys of query r: the window [lo, p] (nw keys) then the nt kept
// tokens before lo.
// Row of query r's key list for query head h (see list_mode).
__device__ __forceinline__ size_t dec_list_row(const DecArgs& a, int bt, int h, int r) {
    if (a.list_mode == 1) return ((size_t)bt * a.Hq + h) * a.Nq + r;
    if (a.list_mode == 2) return ((size_t)bt * a.Hkv + h / (a.Hq / a.Hkv)) * a.Nq + r;
    return (size_t)bt * a.Nq + r;
}

// Query r of batch bt (query head h) at position p attends the contiguous
// keys lo .. p (nw of them: the window, joined under a block gate by the own
// block from its first key) and nt listed keys before lo.
__device__ __forceinline__ void dec_span(const DecArgs& a, int bt, int h, int r, int& p, int& lo,
                                         int& nw, int& nt) {
    p = a.Nk - a.Nq + r;
    lo = a.window > 0 ? max(0, p - a.window + 1) : p;
    if (a.B > 0) lo = min(lo, (p / a.B) * a.B);
    nw = (a.window > 0 || a.B > 0) ? p - lo + 1 : 0;
    nt = a.list ? a.nfar[dec_list_row(a, bt, h, r)] : 0;
}

// Eight consecutive elements of a row staged in LDS, from byte offset b.
template <bool F32>
__device__ __forceinline__ void lds_load8(const uint8_t* row, int b, float (&x)[8]) {
    if constexpr (F32) {
        const float4 u = *(const float4*)(row + b), v = *(const float4*)(row + b + 16);
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
        x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
    } else {
        const uint4 u = *(const uint4*)(row + b);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            x[2 * t] = bf16_to_f32(w[t] & 0xffffu);
            x[2 * t + 1] = bf16_to_f32(w[t] >> 16);
        }
    }
}

// Attended-key tile c (CH keys: the window [lo, lo + nw) first, then the
// listed tokens) of query r for all G q heads of kv head g.  The tile's K
// and V rows are staged in LDS together (coalesced 16-byte loads, all issued
// before the first store); then logits (one key per thread), per-head max
// and sum, and P V.  q and the logits take G * (D + CH) floats of dynamic
// LDS (G = 1 for multi-head attention), so more workgroups fit on a CU.  Partial per (row, tile): o[D] = sum_j e^(x_j - m) v_j,
// then m, l (x in base-2 units: logit * log2 e).
template <int D, bool F32>
__global__ __launch_bounds__(DEC_THREADS) void dec_attn_kernel(DecArgs a) {
    constexpr int CH = dec_chunk(F32);
    constexpr int ESZ = F32 ? 4 : 2;
    constexpr int RB = D * ESZ;         // bytes of a K or V row
    constexpr int ROWB = RB + 16;       // LDS row stride (keeps per-key reads off one bank)
    constexpr int PIECES = RB / 16;     // 16-byte pieces of a row
    constexpr int NPC = CH * PIECES;    // 16-byte pieces of a tile
    constexpr int PER = (NPC + DEC_THREADS - 1) / DEC_THREADS;   // pieces per thread
    constexpr int DG = D / 8;           // 8-dim groups of a row
    static_assert(CH * ROWB >= DEC_THREADS * 8 * 4, "part sums must fit the K tile");
    __shared__ __align__(16) uint8_t kt[CH * ROWB];   // K rows; at the end the P V part sums
    __shared__ __align__(16) uint8_t vt[CH * ROWB];
    __shared__ int js[CH];
    __shared__ float red[16][2];
    extern __shared__ float dyn[];   // q [G][D], logits [G][CH]: sized per launch
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = blockIdx.x, bt = blockIdx.z;
    // The workgroup's query heads h0 .. h0 + G - 1 share its keys: a kv
    // group, or under per-head lists one query head.
    const int grp = blockIdx.y / a.Nq, r = blockIdx.y % a.Nq;
    const int Gr = a.Hq / a.Hkv;
    const int G = a.list_mode == 1 ? 1 : Gr;
    const int kvh = a.list_mode == 1 ? grp / Gr : grp, h0 = a.list_mode == 1 ? grp : grp * Gr;
    float* const qs = dyn;
    float* const ps = dyn + G * D;
    int p, lo, nw, nt;
    dec_span(a, bt, h0, r, p, lo, nw, nt);
    const int L = nw + nt, key0 = c * CH;
    if (key0 >= L) return;   // whole block: nothing past the attended keys
    const int nk = min(CH, L - key0);

    for (int x = tid; x < G * D; x += DEC_THREADS) {
        const int hl = x / D, e = x % D;
        qs[x] = dec_load(a.q, (((size_t)bt * a.Hq + h0 + hl) * a.Nq + r) * D + e, a.f32);
    }
    if (tid < CH) {
        const int idx = key0 + min(tid, nk - 1);   // rows past nk repeat the last key
        js[tid] = idx < nw ? lo + idx : a.list[dec_list_row(a, bt, h0, r) * a.top_t + (idx - nw)];
    }
    __syncthreads();

    // Stage K and V rows: piece x = row * PIECES + col.
    const size_t kvb = ((size_t)bt * a.Hkv + kvh) * a.Nk;
    const uint8_t* kg = (const uint8_t*)a.k;
    const uint8_t* vg = (const uint8_t*)a.v;
    uint4 kr[PER], vr[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {   // threads past the last piece repeat it
        const int x = min(tid + i * DEC_THREADS, NPC - 1), row = x / PIECES, col = x % PIECES;
        const size_t off = (kvb + js[row]) * RB + col * 16;
        kr[i] = *(const uint4*)(kg + off);
        vr[i] = *(const uint4*)(vg + off);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int x = min(tid + i * DEC_THREADS, NPC - 1), row = x / PIECES, col = x % PIECES;
        *(uint4*)(kt + row * ROWB + col * 16) = kr[i];
        *(uint4*)(vt + row * ROWB + col * 16) = vr[i];
    }
    __syncthreads();

    // Logits: one key per thread, every head of the group against it.
    const float c2 = a.scale * kLog2e;
    if (tid < nk) {
        float sacc[16];
#pragma unroll
        for (int hl = 0; hl < 16; ++hl) sacc[hl] = 0.f;
#pragma unroll
        for (int d8 = 0; d8 < DG; ++d8) {
            float kx[8];
            lds_load8<F32>(kt + tid * ROWB, d8 * 8 * ESZ, kx);
#pragma unroll
            for (int hl = 0; hl < 16; ++hl)
                if (hl < G)
#pragma unroll
                    for (int u = 0; u < 8; ++u) sacc[hl] = fmaf(qs[hl * D + d8 * 8 + u], kx[u], sacc[hl]);
        }
#pragma unroll
        for (int hl = 0; hl < 16; ++hl)
            if (hl < G) ps[hl * CH + tid] = sacc[hl] * c2;
    }
    __syncthreads();
    // Per head: max and sum over the tile (wave w takes heads w, w+4, ...).
    for (int hl = wave; hl < G; hl += 4) {
        float* prow = ps + hl * CH;
        float m = -INFINITY;
        for (int u = lane; u < nk; u += 64) m = fmaxf(m, prow[u]);
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
        float l = 0.f;
        for (int u = lane; u < nk; u += 64) {
            const float e = fast_exp2(prow[u] - m);
            prow[u] = e;
            l += e;
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) l += __shfl_xor(l, d);
        if (lane == 0) {
            red[hl][0] = m;
            red[hl][1] = l;
        }
    }
    __syncthreads();
    // P V: thread (part, head, 8-dim group) sums its share of the keys.
    const int pairs = G * DG, parts = DEC_THREADS / pairs;
    const int part = tid / pairs, pr = tid % pairs, hl = pr / DG, dg = pr % DG;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (part < parts) {
        for (int k = part; k < nk; k += parts) {
            float vx[8];
            lds_load8<F32>(vt + k * ROWB, dg * 8 * ESZ, vx);
            const float pw = ps[hl * CH + k];
#pragma unroll
            for (int u = 0; u < 8; ++u) o[u] = fmaf(pw, vx[u], o[u]);
        }
    }
    float* acc = (float*)kt;   // the K tile is no longer read
    if (part < parts)
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[(part * pairs + pr) * 8 + u] = o[u];
    __syncthreads();
    for (int x = tid; x < G * D; x += DEC_THREADS) {
        const int h2 = x / D, ee = x % D, pr2 = h2 * DG + ee / 8;
        float sum = 0.f;
        for (int q_ = 0; q_ < parts; ++q_) sum += acc[(q_ * pairs + pr2) * 8 + (ee & 7)];
        const size_t row = ((size_t)bt * a.Hq + h0 + h2) * a.Nq + r;
        float* dst = a.part + (row * a.cmax + c) * (D + 2);
        dst[ee] = sum;
        if (ee == 0) {
            dst[D] = red[h2][0];
            dst[D + 1] = red[h2][1];
        }
    }
}

// One workgroup per (batch, head, query): merge the tile partials and the
// sink.  Thread (slice s, dim e) sums partials s, s + S, ...
template <int D>
__global__ __launch_bounds__(DEC_THREADS) void dec_combine_kernel(DecArgs a) {
    constexpr int S = DEC_THREADS / D;   // partial slices
    __shared__ float sm[DEC_THREADS], sl[DEC_THREADS];
    __shared__ float so[S * D];
    const int tid = threadIdx.x;
    const size_t row = blockIdx.x;
    const int r = (int)(row % a.Nq), bt = (int)(row / ((size_t)a.Hq * a.Nq));
    const int h = (int)((row / a.Nq) % a.Hq);
    int p, lo, nw, nt;
    dec_span(a, bt, h, r, p, lo, nw, nt);
    const int chunk = dec_chunk(a.f32 != 0);
    const int nc = (nw + nt + chunk - 1) / chunk;
    const float* src = a.part + row * a.cmax * (D + 2);
    // Largest exponent base over the partials and the sink (base-2 units).
    float m = -INFINITY;
    for (int cc = tid; cc < nc; cc += DEC_THREADS) m = fmaxf(m, src[cc * (D + 2) + D]);
    sm[tid] = m;
    __syncthreads();
    for (int d = DEC_THREADS / 2; d >= 1; d >>= 1) {
        if (tid < d) sm[tid] = fmaxf(sm[tid], sm[tid + d]);
        __syncthreads();
    }
    const float z = a.sink ? a.sink[h] * kLog2e : -INFINITY;
    const float M = fmaxf(sm[0], z);
    float l = 0.f;
    for (int cc = tid; cc < nc; cc += DEC_THREADS)
        l += src[cc * (D + 2) + D + 1] * fast_exp2(src[cc * (D + 2) + D] - M);
    sl[tid] = l;
    __syncthreads();
    for (int d = DEC_THREADS / 2; d >= 1; d >>= 1) {
        if (tid < d) sl[tid] += sl[tid + d];
        __syncthreads();
    }
    const float Ltot = sl[0] + (a.sink ? fast_exp2(z - M) : 0.f);
    const int s = tid / D, e = tid % D;
    if (s < S) {
        float o = 0.f;
#pragma unroll 4
        for (int cc = s; cc < nc; cc += S)
            o += src[cc * (D + 2) + e] * fast_exp2(src[cc * (D + 2) + D] - M);
        so[s * D + e] = o;
    }
    __syncthreads();
    const float inv = Ltot > 0.f ? 1.f / Ltot : 0.f;
    if (tid < D) {
        float o = 0.f;
        for (int s2 = 0; s2 < S; ++s2) o += so[s2 * D + tid];
        o *= inv;
        if (a.f32) ((float*)a.out)[row * D + tid] = o;
        else ((__bf16*)a.out)[row * D + tid] = (__bf16)o;
    }
    if (tid == 0) a.lse[row] = Ltot > 0.f ? (M + fast_log2(Ltot)) * kLn2 : -INFINITY;
}

template <int D>
static hipError_t dec_d(const DecArgs& a, hipStream_t s) {
    const int groups = a.list_mode == 1 ? a.Hq : a.Hkv;
    const dim3 ag((unsigned)a.cmax, (unsigned)(groups * a.Nq), (unsigned)a.Bt);
    const int G = a.list_mode == 1 ? 1 : a.Hq / a.Hkv;
    const size_t dyn = (size_t)G * (D + dec_chunk(a.f32 != 0)) * sizeof(float);   // q, logits
    if (a.f32)
        hipLaunchKernelGGL((dec_attn_kernel<D, true>), ag, dim3(DEC_THREADS), dyn, s, a);
    else
        hipLaunchKernelGGL((dec_attn_kernel<D, false>), ag, dim3(DEC_THREADS), dyn, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t rows = (size_t)a.Bt * a.Hq * a.Nq;
    hipLaunchKernelGGL(dec_combine_kernel<D>, dim3((unsigned)rows), dim3(DEC_THREADS), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode_select(const DecArgs& a, hipStream_t s) {
    const dim3 sg((unsigned)((a.Nk + DEC_THREADS - 1) / DEC_THREADS), (unsigned)a.Bt);
    if (a.f32)
        hipLaunchKernelGGL(dec_scores_kernel<true>, sg, dim3(DEC_THREADS), 0, s, a);
    else
        hipLaunchKernelGGL(dec_scores_kernel<false>, sg, dim3(DEC_THREADS), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (!dec_split_select((long long)a.Bt * a.Nq, a.Nk, a.top_t) || !a.plist || !a.redo) {
        DecArgs b = a;
        b.redo = nullptr;
        hipLaunchKernelGGL((dec_select_kernel<65536 / SEL_THREADS, kSelWhole>),
                           dim3((unsigned)a.Nq, (unsigned)a.Bt), dim3(SEL_THREADS), 0, s, b);
        return hipGetLastError();
    }
    if (a.quota < 1 || a.quota > dec_sel_quota(kDecSplitMaxTop) || a.quota > a.top_t)
        return hipErrorInvalidValue;
    // Long histories: the slices' selections spread over kSelParts
    // workgroups per query, then the merge.
    hipLaunchKernelGGL((dec_select_kernel<kSelSlice / SEL_THREADS, kSelPart>),
                       dim3((unsigned)a.Nq, (unsigned)a.Bt, (unsigned)kSelParts), dim3(SEL_THREADS), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int kMergePT = (kSelParts * dec_sel_quota(kDecSplitMaxTop) + SEL_THREADS - 1) / SEL_THREADS;
    hipLaunchKernelGGL((dec_select_kernel<kMergePT, kSelMerge>), dim3((unsigned)a.Nq, (unsigned)a.Bt),
                       dim3(SEL_THREADS), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // queries whose merge may be inexact, selected again whole
    hipLaunchKernelGGL((dec_select_kernel<65536 / SEL_THREADS, kSelWhole>),
                       dim3((unsigned)a.Nq, (unsigned)a.Bt), dim3(SEL_THREADS), 0, s, a);
    return hipGetLastError();
}

// Block gate of a decode step [MoBA summary page, "블록 분할과 top-k 게이팅"
// and "인과성 보존": score every earlier block by the query's dot product
// with its mean key, keep the top k with the own block always among them;
// read for a decode step as the same position of a prefill over the
// history; the related-work remark for the min/max summary (Quest) and
// block 0 always kept (an attention sink); one selection per kv group from
// the summed scores of its heads].  One 64-lane workgroup per (batch, query
// head, query), or per (batch, kv head, query) for a shared selection: the
// query at position p scores the complete candidate blocks c0 <= c < p / B
// (c0 = 1 when block 0 is forced) against their fp32 summaries, keeps the
// best min(top_k - 1 - c0, p / B - c0) by (score desc, index asc) -- an
// order key ord(score) << 32 | (2^32 - 1 - c), whose wave-wide maximum is
// taken once per kept block -- and lists the keys of the forced and kept
// blocks below lo (the first key of its contiguous range [lo, p]: the own
// block, joined with the window), ascending.  Writes list, nfar and, when
// asked, bsel (for every head of a sharing group).
__global__ __launch_bounds__(64) void dec_block_select_kernel(DecArgs a) {
    __shared__ float qs[16 * 128];
    __shared__ uint64_t keys[kDecMaxBlocks];
    __shared__ int kept[kDecMaxTopK];
    const int lane = threadIdx.x;
    const int Gr = a.Hq / a.Hkv;
    const size_t row = blockIdx.x;   // (bt * heads + head) * Nq + r, heads = Hkv if shared else Hq
    const int heads = a.gate_shared ? a.Hkv : a.Hq;
    const int r = (int)(row % a.Nq), hx = (int)((row / a.Nq) % heads);
    const int bt = (int)(row / ((size_t)a.Nq * heads));
    const int g = a.gate_shared ? hx : hx / Gr;
    const int h_first = a.gate_shared ? g * Gr : hx, nh = a.gate_shared ? min(Gr, 16) : 1;
    const int p = a.Nk - a.Nq + r, own = p / a.B;
    const int c0 = (a.gate_first && own > 0) ? 1 : 0;
    const int ncand = min(own, min(a.nb, kDecMaxBlocks));   // own <= nb, nb <= kDecMaxBlocks (plan)
    for (int x = lane; x < nh * a.D; x += 64)
        qs[x] = dec_load(a.q, (((size_t)bt * a.Hq + h_first + x / a.D) * a.Nq + r) * a.D + x % a.D, a.f32);
    __syncthreads();
    const int R = a.gate_mm ? 2 : 1;   // summary rows per block
    const float* kb = a.kbar + (size_t)(bt * a.Hkv + g) * a.nb * R * a.D;
    for (int c = c0 + lane; c < ncand; c += 64) {
        const float* kr = kb + (size_t)c * R * a.D;
        float sc = 0.f;
        for (int hl = 0; hl < nh; ++hl) {
            const float* qh = qs + hl * a.D;
            for (int e = 0; e < a.D; e += 4) {
                const float4 k4 = *(const float4*)(kr + e);
                if (a.gate_mm) {   // sum_e max(q_e min_e, q_e max_e)
                    const float4 x4 = *(const float4*)(kr + a.D + e);
                    sc += fmaxf(qh[e] * k4.x, qh[e] * x4.x);
                    sc += fmaxf(qh[e + 1] * k4.y, qh[e + 1] * x4.y);
                    sc += fmaxf(qh[e + 2] * k4.z, qh[e + 2] * x4.z);
                    sc += fmaxf(qh[e + 3] * k4.w, qh[e + 3] * x4.w);
                } else {
                    sc = fmaf(qh[e], k4.x, sc);
                    sc = fmaf(qh[e + 1], k4.y, sc);
                    sc = fmaf(qh[e + 2], k4.z, sc);
                    sc = fmaf(qh[e + 3], k4.w, sc);
                }
            }
        }
        keys[c] = (uint64_t)dec_ord32(sc) << 32 | (uint64_t)(0xffffffffu - (uint32_t)c);
    }
    __syncthreads();
    // kept[0] = 0 when block 0 is forced, then the chosen candidates
    const int m = max(0, min(min(a.top_k - 1 - c0, kDecMaxTopK - c0), ncand - c0));
    if (lane == 0 && c0) kept[0] = 0;
    for (int t = 0; t < m; ++t) {
        uint64_t best = 0;
        for (int c = c0 + lane; c < ncand; c += 64) best = keys[c] > best ? keys[c] : best;
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            const uint32_t lo32 = (uint32_t)__shfl_xor((int)(uint32_t)best, d);
            const uint32_t hi32 = (uint32_t)__shfl_xor((int)(uint32_t)(best >> 32), d);
            const uint64_t o = (uint64_t)hi32 << 32 | lo32;
            best = o > best ? o : best;
        }
        // every key not yet taken is nonzero, so best names a candidate
        const int c = min(max((int)(0xffffffffu - (uint32_t)best), c0), ncand - 1);
        if (lane == 0) kept[c0 + t] = c;
        if (lane == ((c - c0) & 63)) keys[c] = 0;   // the lane that scans c
        __syncthreads();
    }
    const int nk = c0 + m;   // forced and kept blocks before the own one
    if (lane == 0)   // ascending
        for (int t = 1; t < nk; ++t) {
            const int x = kept[t];
            int u = t - 1;
            while (u >= 0 && kept[u] > x) {
                kept[u + 1] = kept[u];
                --u;
            }
            kept[u + 1] = x;
        }
    __syncthreads();
    if (a.bsel)
        for (int hl = 0; hl < nh; ++hl) {
            int32_t* o = a.bsel + (((size_t)bt * a.Hq + h_first + hl) * a.Nq + r) * a.top_k;
            for (int t = lane; t < a.top_k; t += 64) o[t] = t < nk ? kept[t] : (t == nk ? own : -1);
        }
    int lo = own * a.B;
    if (a.window > 0) lo = min(lo, max(0, p - a.window + 1));
    int32_t* L = a.list + row * a.top_t;
    int pos = 0;
    for (int t = 0; t < nk; ++t) {
        const int kb0 = kept[t] * a.B;
        const int cnt = max(0, min(a.B, lo - kb0));   // <= B: the list holds (top_k - 1) B keys
        for (int j = lane; j < cnt; j += 64) L[pos + j] = kb0 + j;
        pos += cnt;
    }
    if (lane == 0) a.nfar[row] = pos;
}

hipError_t launch_decode_block_select(const DecArgs& a, hipStream_t s) {
    if (a.B <= 0 || a.D > 128 || a.nb > kDecMaxBlocks || a.top_k > kDecMaxTopK ||
        a.top_t < (a.top_k - 1) * a.B || (a.gate_shared && a.Hq / a.Hkv > 16) ||
        a.list_mode != (a.gate_shared ? 2 : 1))
        return hipErrorInvalidValue;
    const unsigned rows = (unsigned)((size_t)a.Bt * (a.gate_shared ? a.Hkv : a.Hq) * a.Nq);
    hipLaunchKernelGGL(dec_block_select_kernel, dim3(rows), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode_attn(const DecArgs& a, hipStream_t s) {
    if (a.D == 64) return dec_d<64>(a, s);
    if (a.D == 80) return dec_d<80>(a, s);
    if (a.D == 128) return dec_d<128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace sa
