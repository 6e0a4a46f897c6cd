// sa_attn.hip -- flash-style attention kernels on the gfx950 matrix cores.
//
// attn_rows_kernel  : query-centric.  A workgroup owns 128 consecutive query
//                     rows of one head and walks the keys that can be near
//                     them (the sliding window, the own block, and kept
//                     blocks overlapping the window span) in 64-key tiles
//                     staged through LDS.  The epilogue merges the far-block
//                     partials and the sink column and writes out and lse.
// attn_blocks_kernel: KV-centric.  A workgroup owns one chunk (<= 128 entries)
//                     of the list of rows that kept one far block, gathers
//                     those query rows and attends the block's B keys, writing
//                     one normalised partial per entry.
//
// The split between the two follows the implementation section of the MoBA
// summary page ("MoBA의 구현: MoE와 FlashAttention의 결합"): rows are
// regrouped by kept KV block, each block is attended as a variable-length
// batch, the own block is attended causally on its own, and the pieces are
// combined with the online-softmax rule.  The window of the Bit-Axon SWA page
// ("슬라이딩 윈도우 마스크") joins the causal own-block pass.
//
// Every tile does S^T = K Q^T (bf16 MFMA 32x32x16, fp32 accumulation),
// an online softmax in base 2 on the VALU, and O^T += V^T P^T.
#include "sa_device.hpp"
#include "sa_internal.hpp"

#include <math.h>

namespace sa {

constexpr int KT = 64;                 // keys per tile
constexpr int NWAVES = 4;              // waves per workgroup
constexpr int NTHREADS = 64 * NWAVES;
constexpr int RT = 32 * NWAVES;        // query rows per workgroup

template <int D>
struct Tile {
    static constexpr int DK = D / 16;              // contraction steps of K Q^T
    static constexpr int DM = (D + 31) / 32;       // 32-row blocks of O^T
    static constexpr int DPAD = DM * 32;
    static constexpr int KS = D + 8;               // K tile row stride (elements)
    static constexpr int VS = KT + 8;              // V^T tile row stride (elements)
    static constexpr int KELEMS = KT * KS;
    static constexpr int VELEMS = DPAD * VS;
    static constexpr int KCHUNKS = KT * D / 8;     // 16-byte pieces of a K tile
    static constexpr int KPT = (KCHUNKS + NTHREADS - 1) / NTHREADS;
    static constexpr int VTASKS = (KT / 4) * (D / 8);  // 4 keys x 8 dims each
    static constexpr int VPT = (VTASKS + NTHREADS - 1) / NTHREADS;
};

template <int D, int SPLIT>
struct Stage {
    uint4 k[SPLIT][Tile<D>::KPT];
    uint4 v[SPLIT][Tile<D>::VPT][4];
};

__device__ __forceinline__ uint32_t word_of(const uint4& u, int i) {
    return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

// Global -> registers for the 64-key tile starting at kt0 (keys >= kend read
// as zero; they are always masked by causality).
template <int D, int SPLIT>
__device__ __forceinline__ void stage_load(Stage<D, SPLIT>& st, const uint16_t* const* kp,
                                           const uint16_t* const* vp, int kt0, int kend, int tid) {
    using T = Tile<D>;
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) {
#pragma unroll
        for (int c = 0; c < T::KPT; ++c) {
            const int idx = tid + c * NTHREADS;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (idx < T::KCHUNKS) {
                const int row = idx / (D / 8), col = idx % (D / 8);
                const int key = kt0 + row;
                if (key < kend) val = *(const uint4*)(kp[p] + (size_t)key * D + col * 8);
            }
            st.k[p][c] = val;
        }
#pragma unroll
        for (int c = 0; c < T::VPT; ++c) {
            const int task = tid + c * NTHREADS;
            const int kq = task % (KT / 4), dc = task / (KT / 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint4 val = make_uint4(0, 0, 0, 0);
                const int key = kt0 + kq * 4 + r;
                if (task < T::VTASKS && key < kend)
                    val = *(const uint4*)(vp[p] + (size_t)key * D + dc * 8);
                st.v[p][c][r] = val;
            }
        }
    }
}

// Registers -> LDS.  K keeps its row-major layout (padded rows).  V is
// written transposed (one row per head dimension) with the 16 keys of each
// contraction step permuted so that lane half h finds the 8 keys it feeds to
// the matrix core contiguous: positions 8h..8h+7 of a 16-key group hold keys
// {4h..4h+3, 8+4h..8+4h+3}, the order in which the S^T accumulator hands
// them out.
template <int D, int SPLIT>
__device__ __forceinline__ void stage_store(const Stage<D, SPLIT>& st, uint16_t* ks, uint16_t* vt,
                                            int tid) {
    using T = Tile<D>;
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) {
        uint16_t* kdst = ks + p * T::KELEMS;
        uint16_t* vdst = vt + p * T::VELEMS;
#pragma unroll
        for (int c = 0; c < T::KPT; ++c) {
            const int idx = tid + c * NTHREADS;
            if (idx < T::KCHUNKS) {
                const int row = idx / (D / 8), col = idx % (D / 8);
                *(uint4*)(kdst + row * T::KS + col * 8) = st.k[p][c];
            }
        }
#pragma unroll
        for (int c = 0; c < T::VPT; ++c) {
            const int task = tid + c * NTHREADS;
            if (task < T::VTASKS) {
                const int kq = task % (KT / 4), dc = task / (KT / 4);
                const int q4 = kq & 3;
                const int pos = (kq >> 2) * 16 + (((q4 & 1) << 3) | ((q4 >> 1) << 2));
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const uint32_t w0 = word_of(st.v[p][c][0], t >> 1);
                    const uint32_t w1 = word_of(st.v[p][c][1], t >> 1);
                    const uint32_t w2 = word_of(st.v[p][c][2], t >> 1);
                    const uint32_t w3 = word_of(st.v[p][c][3], t >> 1);
                    uint2 pk;
                    if (t & 1) {
                        pk.x = (w0 >> 16) | (w1 & 0xffff0000u);
                        pk.y = (w2 >> 16) | (w3 & 0xffff0000u);
                    } else {
                        pk.x = (w0 & 0xffffu) | (w1 << 16);
                        pk.y = (w2 & 0xffffu) | (w3 << 16);
                    }
                    *(uint2*)(vdst + (dc * 8 + t) * T::VS + pos) = pk;
                }
            }
        }
    }
}

// Per-lane mask state for one query row.
struct RowMask {
    int row;        // query position i
    int window;     // 0 = off
    bool blk_ok;    // the current tile's block is attended by this row
};

// One 64-key tile for one wave (32 query rows, one per lane pair).
//   m: running max of the raw dot products of this row (both lane halves
//      agree), l: this lane's partial sum of exp2((s - m) * c).
template <int D, int SPLIT, bool MASKED>
__device__ __forceinline__ void attend_tile(const uint16_t* ks, const uint16_t* vt,
                                            const bf16x8 (&qf)[SPLIT][Tile<D>::DK],
                                            f32x16 (&o)[Tile<D>::DM], float& m, float& l,
                                            float c, int lane, const RowMask& mk, int kt0) {
    using T = Tile<D>;
    const int col = lane & 31, hh = lane >> 5;
    f32x16 s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
        f32x16 acc = {};
#pragma unroll
        for (int ks_ = 0; ks_ < T::DK; ++ks_) {
            const int off = (sub * 32 + col) * T::KS + ks_ * 16 + 8 * hh;
            const bf16x8 a = *(const bf16x8*)(ks + off);
            acc = mfma32(a, qf[0][ks_], acc);
            if constexpr (SPLIT == 2) {
                const bf16x8 alo = *(const bf16x8*)(ks + T::KELEMS + off);
                acc = mfma32(a, qf[1][ks_], acc);
                acc = mfma32(alo, qf[0][ks_], acc);
            }
        }
        s[sub] = acc;
    }
    if constexpr (MASKED) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = kt0 + sub * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
                const bool ok = key <= mk.row &&
                                ((mk.window > 0 && mk.row - key < mk.window) || mk.blk_ok);
                if (!ok) s[sub][v] = -INFINITY;
            }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[sub][v]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2((m - m_use) * c);
    const float nb = -m_use * c;
    float p[2][16];
    float psum = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            p[sub][v] = fast_exp2(fmaf(s[sub][v], c, nb));
            psum += p[sub][v];
        }
    l = l * alpha + psum;
    m = m_new;
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[mb][v] *= alpha;

    bf16x8 pb[4];
    bf16x8 pl[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        pb[kk] = to_bf16x8(&p[kk >> 1][8 * (kk & 1)]);
        if constexpr (SPLIT == 2) {
            float r[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) r[t] = p[kk >> 1][8 * (kk & 1) + t] - (float)pb[kk][t];
            pl[kk] = to_bf16x8(r);
        }
    }
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int off = (mb * 32 + col) * T::VS + kk * 16 + 8 * hh;
            const bf16x8 a = *(const bf16x8*)(vt + off);
            o[mb] = mfma32(a, pb[kk], o[mb]);
            if constexpr (SPLIT == 2) {
                const bf16x8 alo = *(const bf16x8*)(vt + T::VELEMS + off);
                o[mb] = mfma32(a, pl[kk], o[mb]);
                o[mb] = mfma32(alo, pb[kk], o[mb]);
            }
        }
    }
}

template <int D, int SPLIT>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[SPLIT][Tile<D>::DK], const uint16_t* const* qp,
                                       size_t row_off, bool ok, int hh) {
#pragma unroll
    for (int p = 0; p < SPLIT; ++p)
#pragma unroll
        for (int ks_ = 0; ks_ < Tile<D>::DK; ++ks_) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (ok) u = *(const uint4*)(qp[p] + row_off + ks_ * 16 + 8 * hh);
            qf[p][ks_] = as_bf16x8(u);
        }
}

template <int D>
__device__ __forceinline__ void zero_pad_rows(uint16_t* vt, int planes_x_bufs, int tid) {
    using T = Tile<D>;
    if constexpr (T::DPAD > D) {
        const int n = (T::DPAD - D) * T::VS;
        for (int b = 0; b < planes_x_bufs; ++b)
            for (int x = tid; x < n; x += NTHREADS) vt[b * T::VELEMS + D * T::VS + x] = 0;
    }
}

// ---------------------------------------------------------------------------
// Query-centric kernel.
// ---------------------------------------------------------------------------
template <int D, int SPLIT>
__global__ __launch_bounds__(NTHREADS, 2) void attn_rows_kernel(RowsArgs a) {
    using T = Tile<D>;
    __shared__ __align__(16) uint16_t lds_k[2][SPLIT * T::KELEMS];
    __shared__ __align__(16) uint16_t lds_v[2][SPLIT * T::VELEMS];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int BH = a.Bt * a.Hq;
    const int ntiles = (a.N + RT - 1) / RT;
    const int bh = blockIdx.x % BH;
    const int tile = ntiles - 1 - (int)(blockIdx.x / BH);   // longest rows first
    const int b = bh / a.Hq, h = bh % a.Hq, G = a.Hq / a.Hkv, g = h / G;
    const int N = a.N;
    const int r0 = tile * RT;

    const size_t kvoff = (size_t)(b * a.Hkv + g) * N * D;
    const uint16_t* kp[2] = {a.k[0] + kvoff, SPLIT == 2 ? a.k[1] + kvoff : nullptr};
    const uint16_t* vp[2] = {a.v[0] + kvoff, SPLIT == 2 ? a.v[1] + kvoff : nullptr};

    const int row = r0 + wave * 32 + col;
    const bool row_ok = row < N;
    const size_t prow = (size_t)bh * N + row;   // flat row id
    bf16x8 qf[SPLIT][T::DK];
    load_q<D, SPLIT>(qf, a.q, prow * D, row_ok, hh);

    // Block-gate state of this row: its block, the kept near blocks as a
    // bit mask over (own block - 1 - bit), and the count of far blocks.
    int row_blk = 0, nfar = 0;
    uint32_t near_bits = 0;
    if (a.gate) {
        row_blk = (row_ok ? row : N - 1) / a.B;
        if (row_ok) {
            const int32_t* sr = a.sel + prow * a.top_k;
            for (int x = 0; x < a.top_k; ++x) {
                const int cblk = sr[x];
                if (cblk < 0) break;
                const int dlt = row_blk - cblk;
                if (dlt > a.span) ++nfar;
                else if (dlt >= 1 && dlt <= 32) near_bits |= 1u << (dlt - 1);
            }
        }
    }

    // Key range of the workgroup and of this wave.
    const int r_hi = min(r0 + RT - 1, N - 1);
    auto lower_key = [&](int r) {
        int lo = r;
        if (a.window > 0) lo = min(lo, r - a.window + 1);
        if (a.gate) lo = min(lo, (r / a.B - a.span) * a.B);
        return max(lo, 0);
    };
    const int t_begin = lower_key(r0) / KT, t_end = r_hi / KT;
    const int q0 = r0 + wave * 32;
    const bool wave_rows = q0 < N;
    const int q1 = min(q0 + 31, N - 1);
    const int wlo = lower_key(q0);
    const float c = a.scale * kLog2e;

    zero_pad_rows<D>(&lds_v[0][0], 2 * SPLIT, tid);

    f32x16 o[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) o[mb] = f32x16{};
    float m = -INFINITY, l = 0.f;

    Stage<D, SPLIT> st;
    stage_load<D, SPLIT>(st, kp, vp, t_begin * KT, N, tid);
    stage_store<D, SPLIT>(st, lds_k[0], lds_v[0], tid);
    __syncthreads();

    RowMask mk;
    mk.row = row;
    mk.window = a.window;
    for (int t = t_begin; t <= t_end; ++t) {
        const int buf = (t - t_begin) & 1;
        const bool more = t < t_end;
        if (more) stage_load<D, SPLIT>(st, kp, vp, (t + 1) * KT, N, tid);
        const int kt0 = t * KT;
        if (wave_rows && kt0 <= q1 && kt0 + KT - 1 >= wlo) {
            bool full = kt0 + KT - 1 <= q0 &&
                        ((a.window > 0 && q1 - kt0 < a.window) ||
                         (a.gate && kt0 / a.B == q0 / a.B && q1 / a.B == q0 / a.B));
            if (a.gate) {
                const int dlt = row_blk - kt0 / a.B;
                mk.blk_ok = dlt == 0 || (dlt >= 1 && dlt <= a.span && dlt <= 32 &&
                                         ((near_bits >> (dlt - 1)) & 1u));
            } else {
                mk.blk_ok = false;
            }
            if (full)
                attend_tile<D, SPLIT, false>(lds_k[buf], lds_v[buf], qf, o, m, l, c, lane, mk, kt0);
            else
                attend_tile<D, SPLIT, true>(lds_k[buf], lds_v[buf], qf, o, m, l, c, lane, mk, kt0);
        }
        if (more) stage_store<D, SPLIT>(st, lds_k[buf ^ 1], lds_v[buf ^ 1], tid);
        __syncthreads();
    }

    if (!row_ok) return;

    // Combine: near part (this kernel), far partials, sink.
    const float lt = l + xor32(l);
    const float lse_near = m * a.scale + kLn2 * fast_log2(lt);
    float M = lse_near;
    const size_t pbase = prow * (size_t)a.kslots;
    for (int s_ = 0; s_ < nfar; ++s_) M = fmaxf(M, a.part_lse[pbase + s_]);
    const float z = a.sink ? a.sink[h] : -INFINITY;
    M = fmaxf(M, z);
    float total = __expf(lse_near - M);
    const float wn = total / lt;
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[mb][v] *= wn;
    for (int s_ = 0; s_ < nfar; ++s_) {
        const float w = __expf(a.part_lse[pbase + s_] - M);
        total += w;
        const uint16_t* po = a.part_o + (pbase + s_) * D;
#pragma unroll
        for (int mb = 0; mb < T::DM; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = mb * 32 + 8 * j + 4 * hh;
                if (d0 < D) {
                    const uint2 raw = *(const uint2*)(po + d0);
                    const _Float16* hv = (const _Float16*)&raw;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[mb][4 * j + e] += w * (float)hv[e];
                }
            }
    }
    if (a.sink) total += __expf(z - M);
    const float inv = 1.f / total;
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d0 = mb * 32 + 8 * j + 4 * hh;
            if (d0 < D) {
                const float v0 = o[mb][4 * j] * inv, v1 = o[mb][4 * j + 1] * inv;
                const float v2 = o[mb][4 * j + 2] * inv, v3 = o[mb][4 * j + 3] * inv;
                if (a.out_f32) {
                    *(float4*)((float*)a.out + prow * D + d0) = make_float4(v0, v1, v2, v3);
                } else {
                    __bf16 r[4] = {(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
                    *(uint2*)((uint16_t*)a.out + prow * D + d0) = *(const uint2*)r;
                }
            }
        }
    if (hh == 0) a.lse[prow] = M + kLn2 * fast_log2(total);
}

// ---------------------------------------------------------------------------
// KV-centric far-block kernel.
// ---------------------------------------------------------------------------
template <int D, int SPLIT>
__global__ __launch_bounds__(NTHREADS, 2) void attn_blocks_kernel(BlocksArgs a) {
    using T = Tile<D>;
    __shared__ __align__(16) uint16_t lds_k[2][SPLIT * T::KELEMS];
    __shared__ __align__(16) uint16_t lds_v[2][SPLIT * T::VELEMS];

    // Chunks of one list are contiguous in the table; hand each XCD (the
    // dispatcher deals workgroups to the 8 XCDs in turn) a contiguous range
    // so the block's K/V stays in that XCD's L2.
    const int grid = gridDim.x;
    const int per_xcd = grid / 8;
    const int chunk = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (chunk >= *a.n_chunks) return;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int list = a.chunk_list[chunk];
    const int e0 = a.chunk_start[chunk];
    const int e_end = min(e0 + RT, a.list_off[list + 1]);
    const int cblk = list % a.n, bg = list / a.n;   // bg = b*Hkv + g
    const int b = bg / a.Hkv, g = bg % a.Hkv, G = a.Hq / a.Hkv;
    const int N = a.N;

    const int e = e0 + wave * 32 + col;
    const bool ok = e < e_end;
    int slot = 0;
    size_t prow = 0;
    if (ok) {
        const int ent = a.entries[e];
        slot = ent % a.kslots;
        const int t2 = ent / a.kslots;
        const int hl = t2 % G, i = t2 / G;
        prow = (size_t)(b * a.Hq + g * G + hl) * N + i;
    }
    bf16x8 qf[SPLIT][T::DK];
    load_q<D, SPLIT>(qf, a.q, prow * D, ok, hh);

    const size_t kvoff = (size_t)bg * N * D;
    const uint16_t* kp[2] = {a.k[0] + kvoff, SPLIT == 2 ? a.k[1] + kvoff : nullptr};
    const uint16_t* vp[2] = {a.v[0] + kvoff, SPLIT == 2 ? a.v[1] + kvoff : nullptr};
    const float c = a.scale * kLog2e;

    zero_pad_rows<D>(&lds_v[0][0], 2 * SPLIT, tid);

    f32x16 o[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) o[mb] = f32x16{};
    float m = -INFINITY, l = 0.f;

    const int ntile = a.B / KT;
    const int k_begin = cblk * a.B;
    Stage<D, SPLIT> st;
    stage_load<D, SPLIT>(st, kp, vp, k_begin, N, tid);
    stage_store<D, SPLIT>(st, lds_k[0], lds_v[0], tid);
    __syncthreads();
    RowMask mk{0, 0, true};
    for (int t = 0; t < ntile; ++t) {
        const int buf = t & 1;
        const bool more = t + 1 < ntile;
        if (more) stage_load<D, SPLIT>(st, kp, vp, k_begin + (t + 1) * KT, N, tid);
        attend_tile<D, SPLIT, false>(lds_k[buf], lds_v[buf], qf, o, m, l, c, lane, mk,
                                     k_begin + t * KT);
        if (more) stage_store<D, SPLIT>(st, lds_k[buf ^ 1], lds_v[buf ^ 1], tid);
        __syncthreads();
    }
    if (!ok) return;

    const float lt = l + xor32(l);
    const float inv = 1.f / lt;
    const size_t pidx = prow * (size_t)a.kslots + slot;
    uint16_t* po = a.part_o + pidx * D;
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d0 = mb * 32 + 8 * j + 4 * hh;
            if (d0 < D) {
                _Float16 r[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) r[e2] = (_Float16)(o[mb][4 * j + e2] * inv);
                *(uint2*)(po + d0) = *(const uint2*)r;
            }
        }
    if (hh == 0) a.part_lse[pidx] = m * a.scale + kLn2 * fast_log2(lt);
}

// fp32 -> (hi, lo) bf16 planes: x = hi + lo + O(2^-16 |x|).
__global__ void split_f32_kernel(const float* __restrict__ x, uint16_t* __restrict__ hi,
                                 uint16_t* __restrict__ lo, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float f = x[i];
    const __bf16 h = (__bf16)f;
    const __bf16 r = (__bf16)(f - (float)h);
    hi[i] = __builtin_bit_cast(uint16_t, h);
    lo[i] = __builtin_bit_cast(uint16_t, r);
}

template <int D, int SPLIT>
static hipError_t rows_d(const RowsArgs& a, hipStream_t s) {
    const int ntiles = (a.N + RT - 1) / RT;
    const unsigned grid = (unsigned)(ntiles * a.Bt * a.Hq);
    hipLaunchKernelGGL((attn_rows_kernel<D, SPLIT>), dim3(grid), dim3(NTHREADS), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_rows(const RowsArgs& a, int head_dim, int split, hipStream_t s) {
    if (split == 1) {
        if (head_dim == 64) return rows_d<64, 1>(a, s);
        if (head_dim == 80) return rows_d<80, 1>(a, s);
        if (head_dim == 128) return rows_d<128, 1>(a, s);
    } else {
        if (head_dim == 64) return rows_d<64, 2>(a, s);
        if (head_dim == 80) return rows_d<80, 2>(a, s);
        if (head_dim == 128) return rows_d<128, 2>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int D, int SPLIT>
static hipError_t blocks_d(const BlocksArgs& a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((attn_blocks_kernel<D, SPLIT>), dim3(grid), dim3(NTHREADS), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_blocks(const BlocksArgs& a, int head_dim, int split, int grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if (split == 1) {
        if (head_dim == 64) return blocks_d<64, 1>(a, grid, s);
        if (head_dim == 80) return blocks_d<80, 1>(a, grid, s);
        if (head_dim == 128) return blocks_d<128, 1>(a, grid, s);
    } else {
        if (head_dim == 64) return blocks_d<64, 2>(a, grid, s);
        if (head_dim == 80) return blocks_d<80, 2>(a, grid, s);
        if (head_dim == 128) return blocks_d<128, 2>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_split_f32(const float* x, uint16_t* hi, uint16_t* lo, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const unsigned grid = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(split_f32_kernel, dim3(grid), dim3(256), 0, s, x, hi, lo, n);
    return hipGetLastError();
}

}  // namespace sa
