// sa_bwd.hip -- backward of the attention for the selection the forward
// makes (window, own block, kept blocks; GQA; sink logit).
//
// The gates' top-k choices carry no gradient [MoBA summary page: the model
// is trained through the attention of the selected blocks].  With
// P_ij = e^(x_ij - lse_i), x_ij = scale <q_i, k_j>, D_i = <dO_i, O_i>:
//   dS_ij = P_ij (<dO_i, v_j> - D_i),
//   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
//   dv_j = sum_i P_ij dO_i,        dsink_h = -sum_i e^(sink_h - lse_i) D_i.
//
// bwd_delta  : D_i per row, and the sink gradient.
// bwd_far_dq : far blocks' share of dQ, key-block-centric over the forward's
//              compaction lists (gathered rows), as fp16 partials per slot.
// bwd_dq     : query-centric (lane = query row): per 64-key tile S^T = K Q^T
//              and dP^T = V dO^T on the matrix cores, P^T from the saved lse,
//              dS^T, and dQ^T += K^T dS^T (K in fp16, P V-style product) over
//              the near key range (window, own and near blocks); adds the far
//              partials.
// bwd_dkv    : key-centric (lane = key): per 64-row tile S = Q K^T and
//              dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS; rows are
//              the contiguous span that can reach the keys through the window,
//              the own block or a near kept block (all heads of the kv group),
//              then the rows that kept the keys' block as a far block (the
//              forward's compaction lists), gathered.
#include "sa_attn_common.hpp"

namespace sa {

// ---------------------------------------------------------------------------
// D_i and the sink gradient.  One thread per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
    const size_t rows = (size_t)a.Bt * a.Hq * a.N;
    const size_t r = (size_t)blockIdx.x * 256 + threadIdx.x;
    float dsum = 0.f;
    int h = -1;
    if (r < rows) {
        const uint4* po = (const uint4*)(a.out + r * a.D);
        const uint4* pd = (const uint4*)(a.dout + r * a.D);
        for (int c = 0; c < a.D / 8; ++c) {
            const uint4 u = po[c], w = pd[c];
            const uint32_t uo[4] = {u.x, u.y, u.z, u.w}, ud[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                dsum = fmaf(bf16_to_f32(uo[t] & 0xffffu), bf16_to_f32(ud[t] & 0xffffu), dsum);
                dsum = fmaf(bf16_to_f32(uo[t] >> 16), bf16_to_f32(ud[t] >> 16), dsum);
            }
        }
        a.delta[r] = dsum;
        h = (int)((r / a.N) % a.Hq);
    }
    if (!a.dsink) return;
    float term = (r < rows && a.sink) ? -__expf(a.sink[h] - a.lse[r]) * dsum : 0.f;
    // Lanes of one head add once per wave; mixed waves add per lane.
    const int h0 = __builtin_amdgcn_readfirstlane(h);
    if (__ballot(h != h0 && h >= 0) == 0) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) term += __shfl_xor(term, d);
        if ((threadIdx.x & 63) == 0 && h0 >= 0) atomicAdd(&a.dsink[h0], term);
    } else if (h >= 0) {
        atomicAdd(&a.dsink[h], term);
    }
}

__global__ __launch_bounds__(256) void bwd_zero_kernel(float* x, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) x[i] = 0.f;
}

// Probabilities and score gradients of one tile in the S^T register layout:
// p = 2^(s c - lse2) (0 where s = -inf), ds = p (dp - D).  lse2 and D are
// given per register (per row of the tile) or per lane.
__device__ __forceinline__ void p_ds(f32x16 (&s)[2], const f32x16 (&dp)[2], float c, float lse2,
                                     float dr, uint4 (&pb)[4], uint4 (&db)[4]) {
    float p[2][16], g[2][16];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            p[sub][v] = fast_exp2(fmaf(s[sub][v], c, -lse2));
            g[sub][v] = p[sub][v] * (dp[sub][v] - dr);
        }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        pb[kk] = __builtin_bit_cast(uint4, to_f16x8(&p[kk >> 1][8 * (kk & 1)]));
        db[kk] = __builtin_bit_cast(uint4, to_f16x8(&g[kk >> 1][8 * (kk & 1)]));
    }
}

// Write 32 rows' O^T registers (times f) as bf16 rows of dst (row stride D):
// lane (col, hh) holds dims mb*32 + 8j + 4hh .. +3 of row col.
template <int D>
__device__ __forceinline__ void write_rows_bf16(uint16_t* dst, const f32x16 (&o)[Tile<D>::DM],
                                                float f, int hh) {
#pragma unroll
    for (int mb = 0; mb < Tile<D>::DM; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d0 = mb * 32 + 8 * j + 4 * hh;
            if (d0 < D) {
                __bf16 r[4] = {(__bf16)(o[mb][4 * j] * f), (__bf16)(o[mb][4 * j + 1] * f),
                               (__bf16)(o[mb][4 * j + 2] * f), (__bf16)(o[mb][4 * j + 3] * f)};
                *(uint2*)(dst + d0) = *(const uint2*)r;
            }
        }
}

// ---------------------------------------------------------------------------
// dQ: a workgroup owns 128 query rows of one (batch, head).
// ---------------------------------------------------------------------------
template <int D>
struct DqSmem {
    using T = Tile<D>;
    static constexpr int K = 0;                          // K tile, K layout (bf16)
    static constexpr int V = K + T::KELEMS;              // V tile, K layout (bf16)
    static constexpr int K16 = V + T::KELEMS;            // K tile, V layout (fp16)
    static constexpr int ELEMS = K16 + T::VELEMS;
    static constexpr int BYTES = ELEMS * 2;
};

template <int D>
__global__ __launch_bounds__(NTHREADS, 1) void bwd_dq_kernel(BwdArgs a) {
    using T = Tile<D>;
    using S = DqSmem<D>;
    __shared__ __align__(16) uint8_t smem[S::BYTES];
    uint16_t* const lk = (uint16_t*)smem + S::K;
    uint16_t* const lv = (uint16_t*)smem + S::V;
    uint16_t* const lk16 = (uint16_t*)smem + S::K16;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int N = a.N;
    const int ntiles = (N + RT - 1) / RT;
    const int bh = blockIdx.x / ntiles, rtile = blockIdx.x % ntiles;
    const int b = bh / a.Hq, h = bh % a.Hq, g = h / (a.Hq / a.Hkv);
    const int r0 = rtile * RT;
    const int r_hi = min(r0 + RT - 1, N - 1);
    const int q0 = r0 + __builtin_amdgcn_readfirstlane(wave) * 32;
    const int row = q0 + col;
    const bool ok = row < N;
    const size_t prow = (size_t)bh * N + (ok ? row : 0);

    bf16x8 qf[1][T::DK], df[1][T::DK];
    load_q<D, 1>(qf, &a.q, prow * D, ok, hh);
    load_q<D, 1>(df, &a.dout, prow * D, ok, hh);
    const float c = a.scale * kLog2e;
    const float lse2 = ok ? a.lse[prow] * kLog2e : 0.f;
    const float dr = ok ? a.delta[prow] : 0.f;

    // Kept blocks: own and near ones (within span below the own block) are
    // attended here; far ones come as partials from bwd_far_dq.  nfar = the
    // row's far blocks (slots 0 .. nfar-1 of its partials).
    const int32_t* sr = a.sel ? a.sel + prow * a.top_k : nullptr;
    const int row_blk = a.sel ? min(row, N - 1) / a.B : 0;
    int nfar = 0;
    if (a.sel && ok)
        for (int x = 0; x < a.top_k; ++x) {
            const int cb = sr[x];
            if (cb < 0) break;
            nfar += row_blk - cb > a.span;
        }
    const uint32_t wl_window = a.window > 0 ? (uint32_t)a.window : 0u;
    int cur = 0;   // this row's cursor into its ascending kept-block list

    f32x16 o[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) o[mb] = f32x16{};
    int voff[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) voff[mb] = v_lane_offset<D>(lane, mb);
    const size_t kvoff = (size_t)(b * a.Hkv + g) * N * D;
    const uint16_t* kp[1] = {a.k + kvoff};
    const uint16_t* vp[1] = {a.v + kvoff};
    const uint16_t* k16p[1] = {a.k16 + kvoff};
    const TileSrc<D, 1> ksrc = tile_src<D, 1>(kp, N, tid), vsrc = tile_src<D, 1>(vp, N, tid);
    const TileSrc<D, 1> k16src = tile_src<D, 1>(k16p, N, tid);

    // Near key range of the workgroup: the window span and the blocks within
    // span below the rows' own blocks.
    int lo = r0;
    if (a.window > 0) lo = min(lo, r0 - a.window + 1);
    if (a.sel) lo = min(lo, (r0 / a.B - a.span) * a.B);
    const int t_begin = max(lo, 0) / KT, t_end = r_hi / KT;
    for (int t = t_begin; t <= t_end; ++t) {
        const int kt0 = t * KT;
        Stage<D, 1> st;
        load_tile<D, 1>(st, ksrc, kt0);
        store_tile<D, 1, T::KS, T::KELEMS>(st, lk, tid);
        load_tile<D, 1>(st, vsrc, kt0);
        store_tile<D, 1, T::KS, T::KELEMS>(st, lv, tid);
        load_tile<D, 1>(st, k16src, kt0);
        store_tile<D, 1, T::VS, T::VELEMS>(st, lk16, tid);
        __syncthreads();
        // Mask: window keys, and every causal key of a kept block.
        uint32_t wl = wl_window;
        if (a.sel && ok) {
            const int blk = kt0 / a.B;
            while (cur < a.top_k && sr[cur] >= 0 && sr[cur] < blk) ++cur;
            if (cur < a.top_k && sr[cur] == blk && row_blk - blk <= a.span) wl = 0x80000000u;
        }
        f32x16 s[2], dp[2];
        qk_tile<D, 1>(lk, qf, s, lane);
        qk_tile<D, 1>(lv, df, dp, lane);
        mask_tile(s, row - kt0 - 4 * hh, wl);
        uint4 pb[4], db[4], dl[4];
        p_ds(s, dp, c, lse2, dr, pb, db);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) dl[kk] = make_uint4(0, 0, 0, 0);
        pv_tile<D, 1>(lk16, db, dl, o, voff);
        __syncthreads();
    }
    if (!ok) return;
    // dq = scale * near part + the far blocks' partials (already scaled).
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[mb][v] *= a.scale;
    for (int s_ = 0; s_ < nfar; ++s_) {
        const uint16_t* po = a.part_dq + (prow * (size_t)a.kslots + s_) * D;
#pragma unroll
        for (int mb = 0; mb < T::DM; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = mb * 32 + 8 * j + 4 * hh;
                if (d0 < D) {
                    const uint2 raw = *(const uint2*)(po + d0);
                    const _Float16* hv = (const _Float16*)&raw;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[mb][4 * j + e] += (float)hv[e];
                }
            }
    }
    write_rows_bf16<D>(a.dq + prow * D, o, 1.f, hh);
}

// ---------------------------------------------------------------------------
// Far blocks' share of dQ: a workgroup owns one chunk (<= 128 entries) of
// the list of rows that kept one block as a far block (the forward's
// compaction), gathers those rows and walks the block's keys; every key of a
// far block is attended.  Writes scale * sum_j dS_ij k_j per (row, slot),
// fp16.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(NTHREADS, 1) void bwd_far_dq_kernel(BwdArgs a) {
    using T = Tile<D>;
    using S = DqSmem<D>;
    __shared__ __align__(16) uint8_t smem[S::BYTES];
    uint16_t* const lk = (uint16_t*)smem + S::K;
    uint16_t* const lv = (uint16_t*)smem + S::V;
    uint16_t* const lk16 = (uint16_t*)smem + S::K16;

    // Chunks of one list are contiguous: give each XCD a contiguous range.
    const int grid = gridDim.x;
    const int per_xcd = grid / 8;
    const int chunk = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (chunk >= *a.n_chunks) return;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int N = a.N, G = a.Hq / a.Hkv;
    const int list = a.chunk_list[chunk];
    const int e0 = a.chunk_start[chunk];
    const int e_end = min(e0 + RT, a.list_off[list + 1]);
    const int cblk = list % a.n, bg = list / a.n;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int e = e0 + wave * 32 + col;
    const bool ok = e < e_end;
    int slot = 0;
    size_t prow = 0;
    if (ok) {   // entry = (i*G + head in group)*kslots + slot
        const int ent = a.entries[e];
        slot = ent % a.kslots;
        const int t2 = ent / a.kslots;
        prow = (size_t)(b * a.Hq + g * G + t2 % G) * N + t2 / G;
    }
    bf16x8 qf[1][T::DK], df[1][T::DK];
    load_q<D, 1>(qf, &a.q, prow * D, ok, hh);
    load_q<D, 1>(df, &a.dout, prow * D, ok, hh);
    const float c = a.scale * kLog2e;
    const float lse2 = ok ? a.lse[prow] * kLog2e : INFINITY;
    const float dr = ok ? a.delta[prow] : 0.f;

    f32x16 o[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) o[mb] = f32x16{};
    int voff[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) voff[mb] = v_lane_offset<D>(lane, mb);
    const size_t kvoff = (size_t)bg * N * D;
    const uint16_t* kp[1] = {a.k + kvoff};
    const uint16_t* vp[1] = {a.v + kvoff};
    const uint16_t* k16p[1] = {a.k16 + kvoff};
    const TileSrc<D, 1> ksrc = tile_src<D, 1>(kp, N, tid), vsrc = tile_src<D, 1>(vp, N, tid);
    const TileSrc<D, 1> k16src = tile_src<D, 1>(k16p, N, tid);
    const uint4 zero4[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                            make_uint4(0, 0, 0, 0)};
    for (int t = 0; t < a.B / KT; ++t) {
        const int kt0 = cblk * a.B + t * KT;
        Stage<D, 1> st;
        load_tile<D, 1>(st, ksrc, kt0);
        store_tile<D, 1, T::KS, T::KELEMS>(st, lk, tid);
        load_tile<D, 1>(st, vsrc, kt0);
        store_tile<D, 1, T::KS, T::KELEMS>(st, lv, tid);
        load_tile<D, 1>(st, k16src, kt0);
        store_tile<D, 1, T::VS, T::VELEMS>(st, lk16, tid);
        __syncthreads();
        f32x16 s[2], dp[2];
        qk_tile<D, 1>(lk, qf, s, lane);
        qk_tile<D, 1>(lv, df, dp, lane);
        uint4 pb[4], db[4];
        p_ds(s, dp, c, lse2, dr, pb, db);
        pv_tile<D, 1>(lk16, db, zero4, o, voff);
        __syncthreads();
    }
    if (!ok) return;
    _Float16* dst = (_Float16*)a.part_dq + (prow * (size_t)a.kslots + slot) * D;
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d0 = mb * 32 + 8 * j + 4 * hh;
            if (d0 < D) {
                _Float16 r[4] = {(_Float16)(o[mb][4 * j] * a.scale), (_Float16)(o[mb][4 * j + 1] * a.scale),
                                 (_Float16)(o[mb][4 * j + 2] * a.scale), (_Float16)(o[mb][4 * j + 3] * a.scale)};
                *(uint2*)(dst + d0) = *(const uint2*)r;
            }
        }
}

// ---------------------------------------------------------------------------
// dK, dV: a workgroup owns 128 keys of one (batch, kv head).
// ---------------------------------------------------------------------------
template <int D>
struct DkvSmem {
    using T = Tile<D>;
    static constexpr int Q = 0;                          // Q rows, K layout (bf16)
    static constexpr int DO = Q + T::KELEMS;             // dO rows, K layout (bf16)
    static constexpr int Q16 = DO + T::KELEMS;           // Q rows, V layout (fp16)
    static constexpr int DO16 = Q16 + T::VELEMS;         // dO rows, V layout (fp16)
    static constexpr int ELEMS = DO16 + T::VELEMS;
    static constexpr int BYTES = ELEMS * 2 + 4 * KT * 4; // + lse2, D, row info, row ids
};

// Gathered 64-row tile: row x of the tile is global row ids[x] (-1: zeros).
template <int D>
__device__ __forceinline__ void gather_tile(const uint16_t* base, const int* ids, uint16_t* dst,
                                            int stride, int tid) {
    using T = Tile<D>;
#pragma unroll
    for (int cc = 0; cc < T::CPT; ++cc) {
        const int idx = min(tid + cc * NTHREADS, T::CHUNKS - 1);
        const int r = idx / (D / 8), c8 = idx % (D / 8);
        const int id = ids[r];
        uint4 u = make_uint4(0, 0, 0, 0);
        if (id >= 0) u = *(const uint4*)(base + (size_t)id * D + c8 * 8);
        *(uint4*)(dst + r * stride + c8 * 8) = u;
    }
}

// Mask of an S tile in the key-centric layout (lane = key j, registers =
// rows i = rt0 + cv + 4hh): keep iff (unsigned)(i - j) < w, or i >= j and
// the row's info bit for the key's block is set.  rj = rt0 + 4hh - j.
__device__ __forceinline__ void mask_rows(f32x16 (&s)[2], int rj, uint32_t w, const int* info,
                                          int kb, int hh) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int cv = sub * 32 + 8 * (v >> 2) + (v & 3);
            const int dif = rj + cv;
            const bool keep = (uint32_t)dif < w || (dif >= 0 && ((info[cv + 4 * hh] >> kb) & 1));
            if (!keep) s[sub][v] = -INFINITY;
        }
}

template <int D>
__global__ __launch_bounds__(NTHREADS, 1) void bwd_dkv_kernel(BwdArgs a) {
    using T = Tile<D>;
    using S = DkvSmem<D>;
    __shared__ __align__(16) uint8_t smem[S::BYTES];
    uint16_t* const lq = (uint16_t*)smem + S::Q;
    uint16_t* const ldo = (uint16_t*)smem + S::DO;
    uint16_t* const lq16 = (uint16_t*)smem + S::Q16;
    uint16_t* const ldo16 = (uint16_t*)smem + S::DO16;
    float* const l_lse = (float*)((uint16_t*)smem + S::ELEMS);
    float* const l_d = l_lse + KT;
    int* const l_info = (int*)(l_d + KT);
    int* const l_ids = l_info + KT;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int N = a.N, G = a.Hq / a.Hkv;
    const int ntiles = (N + RT - 1) / RT;
    const int bg = blockIdx.x / ntiles, ktile = blockIdx.x % ntiles;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int k0 = ktile * RT;
    const int k_hi = min(k0 + RT - 1, N - 1);
    const int j0 = k0 + __builtin_amdgcn_readfirstlane(wave) * 32;
    const int key = j0 + col;
    const bool ok = key < N;
    const size_t pkey = (size_t)bg * N + (ok ? key : 0);

    bf16x8 kf[1][T::DK], vf[1][T::DK];
    load_q<D, 1>(kf, &a.k, pkey * D, ok, hh);
    load_q<D, 1>(vf, &a.v, pkey * D, ok, hh);
    const float c = a.scale * kLog2e;
    const uint32_t wl = a.window > 0 ? (uint32_t)a.window : 0u;
    const int blk0 = a.B > 0 ? k0 / a.B : 0;
    const int kb = a.B > 0 ? min(key, N - 1) / a.B - blk0 : 0;   // 0 or 1 (B >= 64)

    f32x16 dv[T::DM], dk[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) dv[mb] = dk[mb] = f32x16{};
    int voff[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) voff[mb] = v_lane_offset<D>(lane, mb);
    const uint4 zero4[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                            make_uint4(0, 0, 0, 0)};

    // One 64-row tile staged in LDS (rows by id; lse2, D and the info bits
    // per row set by the caller) against this wave's 32 keys.
    auto rows_step = [&](int rt0, bool far, int far_kb) {
        f32x16 s[2], dp[2];
        qk_tile<D, 1>(lq, kf, s, lane);
        qk_tile<D, 1>(ldo, vf, dp, lane);
        if (far) {
            // every key of the far block, none of the other block
            if (kb != far_kb) {
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int v = 0; v < 16; ++v) s[sub][v] = -INFINITY;
            }
        } else {
            mask_rows(s, rt0 + 4 * hh - key, wl, l_info, kb, hh);
        }
        // p and ds with per-register rows
        float p[2][16], gds[2][16];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int rr = sub * 32 + 8 * (v >> 2) + (v & 3) + 4 * hh;
                p[sub][v] = fast_exp2(fmaf(s[sub][v], c, -l_lse[rr]));
                gds[sub][v] = p[sub][v] * (dp[sub][v] - l_d[rr]);
            }
        uint4 pb[4], db[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            pb[kk] = __builtin_bit_cast(uint4, to_f16x8(&p[kk >> 1][8 * (kk & 1)]));
            db[kk] = __builtin_bit_cast(uint4, to_f16x8(&gds[kk >> 1][8 * (kk & 1)]));
        }
        pv_tile<D, 1>(ldo16, pb, zero4, dv, voff);
        pv_tile<D, 1>(lq16, db, zero4, dk, voff);
    };

    // (1) contiguous rows of every head of the group: window, own block and
    // near kept blocks.
    int r_end = a.window > 0 ? min(N - 1, k_hi + a.window - 1) : -1;
    if (a.sel) r_end = max(r_end, min(N - 1, (k_hi / a.B + a.span + 1) * a.B - 1));
    for (int hl = 0; hl < G; ++hl) {
        const int h = g * G + hl;
        const size_t hbase = (size_t)(b * a.Hq + h) * N;
        for (int rt0 = k0; rt0 <= r_end; rt0 += KT) {
            if (tid < KT) {
                const int r = rt0 + tid;
                const bool rok = r < N;
                l_ids[tid] = rok ? (int)(hbase + r) : -1;
                l_lse[tid] = rok ? a.lse[hbase + r] * kLog2e : INFINITY;
                l_d[tid] = rok ? a.delta[hbase + r] : 0.f;
                int info = 0;
                if (rok && a.sel) {
                    const int rb = r / a.B;
                    const int32_t* sr = a.sel + (hbase + r) * a.top_k;
                    for (int x = 0; x < a.top_k; ++x) {
                        const int cb = sr[x];
                        if (cb < 0) break;
                        const int dl = cb - blk0;
                        if ((dl == 0 || dl == 1) && rb - cb <= a.span) info |= 1 << dl;
                    }
                }
                l_info[tid] = info;
            }
            __syncthreads();
            gather_tile<D>(a.q, l_ids, lq, T::KS, tid);
            gather_tile<D>(a.dout, l_ids, ldo, T::KS, tid);
            gather_tile<D>(a.q16, l_ids, lq16, T::VS, tid);
            gather_tile<D>(a.do16, l_ids, ldo16, T::VS, tid);
            __syncthreads();
            rows_step(rt0, false, 0);
            __syncthreads();
        }
    }

    // (2) rows that kept a block of these keys as a far block.
    if (a.sel && a.list_off) {
        for (int fb = 0; fb < 2; ++fb) {
            const int cb = blk0 + fb;
            if (cb * a.B > k_hi || cb >= a.n) break;
            const int list = bg * a.n + cb;
            const int e0 = a.list_off[list], e1 = a.list_off[list + 1];
            for (int e = e0; e < e1; e += KT) {
                if (tid < KT) {
                    const int ee = e + tid;
                    int id = -1;
                    if (ee < e1) {   // entry = (i*G + head in group)*kslots + slot
                        const int t2 = a.entries[ee] / a.kslots;
                        const int hl = t2 % G, i = t2 / G;
                        id = (int)((size_t)(b * a.Hq + g * G + hl) * N + i);
                    }
                    l_ids[tid] = id;
                    l_lse[tid] = id >= 0 ? a.lse[id] * kLog2e : INFINITY;
                    l_d[tid] = id >= 0 ? a.delta[id] : 0.f;
                    l_info[tid] = 0;
                }
                __syncthreads();
                gather_tile<D>(a.q, l_ids, lq, T::KS, tid);
                gather_tile<D>(a.dout, l_ids, ldo, T::KS, tid);
                gather_tile<D>(a.q16, l_ids, lq16, T::VS, tid);
                gather_tile<D>(a.do16, l_ids, ldo16, T::VS, tid);
                __syncthreads();
                rows_step(0, true, fb);
                __syncthreads();
            }
        }
    }
    if (ok) {
        write_rows_bf16<D>(a.dk + pkey * D, dk, a.scale, hh);
        write_rows_bf16<D>(a.dv + pkey * D, dv, 1.f, hh);
    }
}

template <int D>
static hipError_t bwd_d(const BwdArgs& a, hipStream_t s) {
    const int nt = (a.N + RT - 1) / RT;
    if (a.list_off && a.max_chunks > 0) {
        hipLaunchKernelGGL((bwd_far_dq_kernel<D>), dim3(a.max_chunks), dim3(NTHREADS), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3(nt * a.Bt * a.Hq), dim3(NTHREADS), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkv_kernel<D>), dim3(nt * a.Bt * a.Hkv), dim3(NTHREADS), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bwd_delta(const BwdArgs& a, hipStream_t s) {
    const size_t rows = (size_t)a.Bt * a.Hq * a.N;
    if (a.dsink) {
        hipLaunchKernelGGL(bwd_zero_kernel, dim3((a.Hq + 255) / 256), dim3(256), 0, s, a.dsink, a.Hq);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int head_dim, hipStream_t s) {
    if (head_dim == 64) return bwd_d<64>(a, s);
    if (head_dim == 80) return bwd_d<80>(a, s);
    if (head_dim == 128) return bwd_d<128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace sa
