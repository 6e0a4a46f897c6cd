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
        if (a.near_mask) {   // the row's kept near blocks, as the forward attends them
            const int rb = (int)(r % a.N) / a.B;
            const int32_t* sr = a.sel + r * a.top_k;
            uint32_t nm = 0;
            for (int x = 0; x < a.top_k; ++x) {
                const int cb = sr[x];
                if (cb < 0) break;
                const int dlt = rb - cb;
                if (dlt >= 1 && dlt <= a.span && dlt <= 32) nm |= 1u << (dlt - 1);
            }
            a.near_mask[r] = nm;
        }
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
// dQ.  Both dQ kernels walk 64-key tiles of contiguous keys; the K, V and
// fp16 K tiles go straight from global memory into LDS, double-buffered (one
// LDS array per buffer, the loop unrolled by two), so the next tile loads
// while the current one is computed.
// ---------------------------------------------------------------------------
template <int D>
struct DqTiles {
    using T = Tile<D>;
    static constexpr int VS = dma_vs<D>();
    static constexpr int VEL = KT * VS;
    TileDma<D, T::KS> kd;
    TileDma<D, VS> vd;
    uint64_t kb[1], vb[1], k16b[1];
    int N;
    __device__ __forceinline__ void init(const BwdArgs& a, size_t kvoff, int wave, int lane) {
        kd.init(wave, lane);
        vd.init(wave, lane);
        kb[0] = uniform_u64((uint64_t)(a.k + kvoff));
        vb[0] = uniform_u64((uint64_t)(a.v + kvoff));
        k16b[0] = uniform_u64((uint64_t)(a.k16 + kvoff));
        N = a.N;
    }
    // Issue the loads of the tile at key kt0 (0 <= kt0 < N).
    __device__ __forceinline__ void load(int kt0, uint16_t* lk, uint16_t* lv, uint16_t* lk16, int wave) const {
        dma_tile<D, 1, T::KELEMS>(kd, kb, N, kt0, lk, wave);
        dma_tile<D, 1, T::KELEMS>(kd, vb, N, kt0, lv, wave);
        dma_tile<D, 1, VEL>(vd, k16b, N, kt0, lk16, wave);
    }
};

// dQ^T += K^T dS^T for one tile (lane = query row): S^T = K Q^T and dP^T =
// V dO^T on the bf16 matrix cores, P^T and dS^T, then the fp16 product.
template <int D>
__device__ __forceinline__ void dq_tile(const uint16_t* lk, const uint16_t* lv, const uint16_t* lk16,
                                        const bf16x8 (&qf)[1][Tile<D>::DK], const bf16x8 (&df)[1][Tile<D>::DK],
                                        f32x16 (&o)[Tile<D>::DM], const int (&voff)[Tile<D>::DM],
                                        float c, float lse2, float dr, bool masked, int rk, uint32_t wl,
                                        int lane) {
    f32x16 s[2], dp[2];
    qk_tile<D, 1>(lk, qf, s, lane);
    qk_tile<D, 1>(lv, df, dp, lane);
    if (masked) mask_tile(s, rk, wl);
    uint4 pb[4], db[4];
    p_ds(s, dp, c, lse2, dr, pb, db);
    const uint4 zero4[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                            make_uint4(0, 0, 0, 0)};
    pv_tile<D, 1, DqTiles<D>::VS>(lk16, db, zero4, o, voff);
}

// ---------------------------------------------------------------------------
// dQ: a workgroup owns 128 query rows of one (batch, head).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(NTHREADS, 1) void bwd_dq_kernel(BwdArgs a) {
    using T = Tile<D>;
    using DT = DqTiles<D>;
    __shared__ __align__(16) uint16_t lk0[T::KELEMS], lk1[T::KELEMS], lv0[T::KELEMS], lv1[T::KELEMS];
    __shared__ __align__(16) uint16_t lk16_0[DT::VEL], lk16_1[DT::VEL];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int N = a.N;
    const int ntiles = (N + RT - 1) / RT;
    const int bh = blockIdx.x / ntiles, rtile = blockIdx.x % ntiles;
    const int b = bh / a.Hq, h = bh % a.Hq, g = h / (a.Hq / a.Hkv);
    const int r0 = rtile * RT;
    const int r_hi = min(r0 + RT - 1, N - 1);
    const int q0 = r0 + wu * 32;
    const int row = q0 + col;
    const bool ok = row < N;
    const size_t prow = (size_t)bh * N + (ok ? row : 0);

    // Near key range of the workgroup: the window span and the blocks within
    // span below the rows' own blocks.
    int lo = r0;
    if (a.window > 0) lo = min(lo, r0 - a.window + 1);
    if (a.sel) lo = min(lo, (r0 / a.B - a.span) * a.B);
    const int t_begin = max(lo, 0) / KT, t_end = r_hi / KT;
    const int n_t = t_end - t_begin + 1;
    DT dt;
    dt.init(a, (size_t)(b * a.Hkv + g) * N * D, wu, lane);
    dt.load(t_begin * KT, lk0, lv0, lk16_0, wu);

    bf16x8 qf[1][T::DK], df[1][T::DK];
    load_q<D, 1>(qf, &a.q, prow * D, ok, hh);
    load_q<D, 1>(df, &a.dout, prow * D, ok, hh);
    const float c = a.scale * kLog2e;
    const float lse2 = ok ? a.lse[prow] * kLog2e : 0.f;
    const float dr = ok ? a.delta[prow] : 0.f;

    // Kept blocks: own and near ones (the near mask of the delta pass) are
    // attended here; far ones come as partials from bwd_far_dq.  nfar = the
    // row's far blocks (slots 0 .. nfar-1 of its partials).
    const int row_blk = a.sel ? min(row, N - 1) / a.B : 0;
    const uint32_t near_bits = a.near_mask && ok ? a.near_mask[prow] : 0u;
    int nfar = 0;
    if (a.sel && ok) {
        const int32_t* sr = a.sel + prow * a.top_k;
        for (int x = 0; x < a.top_k; ++x) {
            const int cb = sr[x];
            if (cb < 0) break;
            nfar += row_blk - cb > a.span;
        }
    }
    const uint32_t wl_window = a.window > 0 ? (uint32_t)a.window : 0u;

    f32x16 o[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) o[mb] = f32x16{};
    int voff[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) voff[mb] = v_lane_offset<D, DT::VS>(lane, mb);
    __syncthreads();

    // Mask of tile t: window keys, and every causal key of a kept block.
    auto compute = [&](int t, const uint16_t* lk, const uint16_t* lv, const uint16_t* lk16)
                       __attribute__((always_inline)) {
        const int kt0 = t * KT;
        uint32_t wl = wl_window;
        if (a.sel) {
            const int dlt = row_blk - kt0 / a.B;
            if (dlt == 0 || (dlt >= 1 && dlt <= 32 && ((near_bits >> (dlt - 1)) & 1u))) wl = 0x80000000u;
        }
        dq_tile<D>(lk, lv, lk16, qf, df, o, voff, c, lse2, dr, true, row - kt0 - 4 * hh, wl, lane);
    };
    auto step = [&](auto par, int it) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par)::value;
        if (it + 1 < n_t) {
            if (PAR) dt.load((t_begin + it + 1) * KT, lk0, lv0, lk16_0, wu);
            else dt.load((t_begin + it + 1) * KT, lk1, lv1, lk16_1, wu);
        }
        if (PAR) compute(t_begin + it, lk1, lv1, lk16_1);
        else compute(t_begin + it, lk0, lv0, lk16_0);
        __syncthreads();
    };
    int it = 0;
    for (; it + 1 < n_t; it += 2) {
        step(Par<0>{}, it);
        step(Par<1>{}, it + 1);
    }
    if (it < n_t) step(Par<0>{}, it);
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
    using DT = DqTiles<D>;
    __shared__ __align__(16) uint16_t lk0[T::KELEMS], lk1[T::KELEMS], lv0[T::KELEMS], lv1[T::KELEMS];
    __shared__ __align__(16) uint16_t lk16_0[DT::VEL], lk16_1[DT::VEL];

    // Chunks of one list are contiguous: give each XCD a contiguous eighth
    // of the valid chunks.
    const int nch = *a.n_chunks;
    const int per_xcd = (nch + 7) / 8;
    const int slot8 = (int)(blockIdx.x / 8);
    const int chunk = (int)(blockIdx.x % 8) * per_xcd + slot8;
    if (slot8 >= per_xcd || chunk >= nch) return;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int N = a.N, G = a.Hq / a.Hkv;
    const int list = a.chunk_list[chunk];
    const int e0 = a.chunk_start[chunk];
    const int e = e0 + wu * 32 + col;
    const int ent = a.entries[min(e, a.entries_cap - 1)];   // used only below the list end
    const int e_end = min(e0 + RT, a.list_off[list + 1]);
    const int cblk = list % a.n, bg = list / a.n;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int ntile = a.B / KT;
    DT dt;
    dt.init(a, (size_t)bg * N * D, wu, lane);
    dt.load(cblk * a.B, lk0, lv0, lk16_0, wu);

    const bool ok = e < e_end;
    int slot = 0;
    size_t prow = 0;
    if (ok) {   // entry = (i*G + head in group)*kslots + slot
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
    for (int mb = 0; mb < T::DM; ++mb) voff[mb] = v_lane_offset<D, DT::VS>(lane, mb);
    __syncthreads();

    auto step = [&](auto par, int t) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par)::value;
        if (t + 1 < ntile) {
            if (PAR) dt.load(cblk * a.B + (t + 1) * KT, lk0, lv0, lk16_0, wu);
            else dt.load(cblk * a.B + (t + 1) * KT, lk1, lv1, lk16_1, wu);
        }
        if (PAR) dq_tile<D>(lk1, lv1, lk16_1, qf, df, o, voff, c, lse2, dr, false, 0, 0u, lane);
        else dq_tile<D>(lk0, lv0, lk16_0, qf, df, o, voff, c, lse2, dr, false, 0, 0u, lane);
        __syncthreads();
    };
    int t = 0;
    for (; t + 1 < ntile; t += 2) {
        step(Par<0>{}, t);
        step(Par<1>{}, t + 1);
    }
    if (t < ntile) step(Par<0>{}, t);
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

// Lane offsets of a gathered 64-row tile in an LDS image of row stride S
// (the layout of TileDma): instruction j of this wave writes chunk p = 64 i +
// lane, i = min(wave + NWAVES j, S/8 - 1), of row p / (S/8); chunks past the
// row's D elements repeat its last one.  row_c packs (row << 8) | element
// offset of the chunk.
template <int D, int S>
struct GatherDma {
    static constexpr int NI = S / 8;
    static constexpr int PER = (NI + NWAVES - 1) / NWAVES;
    int row_c[PER];
    __device__ __forceinline__ static int inst(int wave, int j) { return min(wave + NWAVES * j, NI - 1); }
    __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int p = 64 * inst(wave, j) + lane;
            row_c[j] = ((p / NI) << 8) | (min(p % NI, D / 8 - 1) * 8);
        }
    }
};

// Issue the gather of one [N, D] plane's rows ids[0..63] into an LDS image
// (global_load_lds, 16 bytes per lane, per-lane 64-bit addresses).  A row id
// < 0 loads row 0 instead: such rows carry lse = +inf and D = 0, so their P
// and dS are zero and the data never counts.
template <int D, int S>
__device__ __forceinline__ void gather_dma(const GatherDma<D, S>& gd, const uint16_t* base,
                                           const int* ids, uint16_t* lds, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass rejects the LDS-pointer builtin
#pragma unroll
    for (int j = 0; j < GatherDma<D, S>::PER; ++j) {
        const int id = ids[gd.row_c[j] >> 8];
        const uint16_t* src = base + (size_t)(id >= 0 ? id : 0) * D + (gd.row_c[j] & 0xff);
        __builtin_amdgcn_global_load_lds((const void*)src,
                                         (lds_ptr_t)(lds + GatherDma<D, S>::inst(wave, j) * 512), 16, 0, 0);
    }
#endif
}

// ---------------------------------------------------------------------------
// dK, dV: a workgroup owns 128 keys of one (batch, kv head) and walks 64-row
// tiles: (1) the contiguous rows of every head of the group that can reach
// the keys through the window, the own block or a near kept block; (2) the
// rows that kept the keys' block as a far block (the forward's compaction
// lists).  The tile after the current one is gathered straight into the
// other LDS buffer while the current one is computed, and wave 0 fetches the
// per-row data (id, lse, D, kept-block bits) two tiles ahead into a ring of
// three slots.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(NTHREADS, 1) void bwd_dkv_kernel(BwdArgs a) {
    using T = Tile<D>;
    constexpr int VS = dma_vs<D>();
    constexpr int VEL = KT * VS;
    __shared__ __align__(16) uint16_t lq0[T::KELEMS], lq1[T::KELEMS], ldo0[T::KELEMS], ldo1[T::KELEMS];
    __shared__ __align__(16) uint16_t lq16_0[VEL], lq16_1[VEL], ldo16_0[VEL], ldo16_1[VEL];
    __shared__ float s_lse[3][KT], s_d[3][KT];
    __shared__ int s_info[3][KT], s_ids[3][KT];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int N = a.N, G = a.Hq / a.Hkv;
    const int ntiles = (N + RT - 1) / RT;
    const int bg = blockIdx.x / ntiles, ktile = blockIdx.x % ntiles;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int k0 = ktile * RT;
    const int k_hi = min(k0 + RT - 1, N - 1);
    const int j0 = k0 + wu * 32;
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
    for (int mb = 0; mb < T::DM; ++mb) voff[mb] = v_lane_offset<D, VS>(lane, mb);
    const uint4 zero4[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                            make_uint4(0, 0, 0, 0)};
    GatherDma<D, T::KS> gk;
    GatherDma<D, VS> gv;
    gk.init(wu, lane);
    gv.init(wu, lane);

    // The row tiles: n_rt contiguous tiles per head of the group, then the
    // far lists of the keys' (at most two) blocks.
    int r_end = a.window > 0 ? min(N - 1, k_hi + a.window - 1) : -1;
    if (a.sel) r_end = max(r_end, min(N - 1, (k_hi / a.B + a.span + 1) * a.B - 1));
    const int n_rt = r_end >= k0 ? (r_end - k0) / KT + 1 : 0;
    const int n1 = G * n_rt;
    // (Scalars, not arrays: a runtime-indexed array would live in scratch,
    // whose loads wait for every tile load in flight.)
    int fa0 = 0, fa1 = 0, fb0 = 0, fb1 = 0;   // entry ranges of blocks blk0, blk0 + 1
    if (a.sel && a.list_off) {
        const int list = bg * a.n + blk0;
        if (blk0 * a.B <= k_hi && blk0 < a.n) {
            fa0 = a.list_off[list];
            fa1 = a.list_off[list + 1];
        }
        if ((blk0 + 1) * a.B <= k_hi && blk0 + 1 < a.n) {
            fb0 = a.list_off[list + 1];
            fb1 = a.list_off[list + 2];
        }
    }
    const int fn0 = (fa1 - fa0 + KT - 1) / KT, fn1 = (fb1 - fb0 + KT - 1) / KT;
    const int n_tiles = n1 + fn0 + fn1;

    // Per-row data of row r of tile i, fetched by wave 0 (r = lane) in three
    // parts so that no load is waited for before the step's closing barrier:
    // the far-list entry one step early (ent_of), the row's loads (fetch,
    // unconditional at a clamped id) and the values into their slot (put).
    auto ent_of = [&](int i, int r) __attribute__((always_inline)) -> int {
        if (i < n1 || i >= n_tiles) return -1;
        const bool second = i - n1 >= fn0;
        const int ee = (second ? fb0 + (i - n1 - fn0) * KT : fa0 + (i - n1) * KT) + r;
        return ee < (second ? fb1 : fa1) ? a.entries[min(ee, a.entries_cap - 1)] : -1;
    };
    struct RowData {
        int id, rr;
        float lse, d;
        uint32_t nm;
    };
    auto fetch = [&](int i, int r, int ent) __attribute__((always_inline)) -> RowData {
        RowData rd{-1, 0, 0.f, 0.f, 0u};
        if (i < n1) {
            const int hl = i / n_rt, rr = k0 + (i % n_rt) * KT + r;
            rd.rr = rr;
            if (rr < N) rd.id = (int)((size_t)(b * a.Hq + g * G + hl) * N + rr);
        } else if (ent >= 0) {   // entry = (i*G + head in group)*kslots + slot
            const int t2 = ent / a.kslots;
            rd.id = (int)((size_t)(b * a.Hq + g * G + t2 % G) * N + t2 / G);
        }
        const int idc = max(rd.id, 0);
        rd.lse = a.lse[idc];
        rd.d = a.delta[idc];
        if (a.near_mask && i < n1) rd.nm = a.near_mask[idc];
        return rd;
    };
    auto put = [&](const RowData& rd, int i, int sl) __attribute__((always_inline)) {
        int info = 0;
        if (a.near_mask && i < n1 && rd.id >= 0) {
            // Blocks blk0 and blk0 + 1 kept for this row by the forward: its
            // own block, or a near block it selected.
            const int rb = rd.rr / a.B;
#pragma unroll
            for (int dl = 0; dl < 2; ++dl) {
                const int dlt = rb - (blk0 + dl);
                if (dlt == 0 || (dlt >= 1 && dlt <= 32 && ((rd.nm >> (dlt - 1)) & 1u))) info |= 1 << dl;
            }
        }
        s_ids[sl][lane] = rd.id;
        s_lse[sl][lane] = rd.id >= 0 ? rd.lse * kLog2e : INFINITY;
        s_d[sl][lane] = rd.id >= 0 ? rd.d : 0.f;
        s_info[sl][lane] = info;
    };
    auto gather = [&](int sl, uint16_t* q_, uint16_t* do_, uint16_t* q16_, uint16_t* do16_) __attribute__((always_inline)) {
        gather_dma<D, T::KS>(gk, a.q, s_ids[sl], q_, wu);
        gather_dma<D, T::KS>(gk, a.dout, s_ids[sl], do_, wu);
        gather_dma<D, VS>(gv, a.q16, s_ids[sl], q16_, wu);
        gather_dma<D, VS>(gv, a.do16, s_ids[sl], do16_, wu);
    };

    // Tile i from its buffers against this wave's 32 keys.
    auto compute = [&](int i, int sl, const uint16_t* q_, const uint16_t* do_, const uint16_t* q16_,
                       const uint16_t* do16_) __attribute__((always_inline)) {
        f32x16 s[2], dp[2];
        qk_tile<D, 1>(q_, kf, s, lane);
        qk_tile<D, 1>(do_, vf, dp, lane);
        if (i >= n1) {
            // every key of the far block, none of the other block
            const int far_kb = i - n1 < fn0 ? 0 : 1;
            if (kb != far_kb) {
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int v = 0; v < 16; ++v) s[sub][v] = -INFINITY;
            }
        } else {
            const int rt0 = k0 + (i % n_rt) * KT;
            mask_rows(s, rt0 + 4 * hh - key, wl, s_info[sl], kb, hh);
        }
        float p[2][16], gds[2][16];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int rr = sub * 32 + 8 * (v >> 2) + (v & 3) + 4 * hh;
                p[sub][v] = fast_exp2(fmaf(s[sub][v], c, -s_lse[sl][rr]));
                gds[sub][v] = p[sub][v] * (dp[sub][v] - s_d[sl][rr]);
            }
        uint4 pb[4], db[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            pb[kk] = __builtin_bit_cast(uint4, to_f16x8(&p[kk >> 1][8 * (kk & 1)]));
            db[kk] = __builtin_bit_cast(uint4, to_f16x8(&gds[kk >> 1][8 * (kk & 1)]));
        }
        pv_tile<D, 1, VS>(do16_, pb, zero4, dv, voff);
        pv_tile<D, 1, VS>(q16_, db, zero4, dk, voff);
    };

    if (n_tiles > 0) {
        int ent2 = -1;   // wave 0: this lane's entry of tile i + 2 (far tiles)
        if (wu == 0) {
            put(fetch(0, lane, ent_of(0, lane)), 0, 0);
            if (n_tiles > 1) put(fetch(1, lane, ent_of(1, lane)), 1, 1);
            ent2 = ent_of(2, lane);
        }
        __syncthreads();
        gather(0, lq0, ldo0, lq16_0, ldo16_0);
        __syncthreads();

        // Step of tile i (buffer parity PAR = i & 1, data slot i % 3).
        auto step = [&](auto par, int i) __attribute__((always_inline)) {
            constexpr int PAR = decltype(par)::value;
            const bool ahead = wu == 0 && i + 2 < n_tiles;
            RowData rd{-1, 0, 0.f, 0.f, 0u};
            int ent3 = -1;
            if (ahead) {   // loads first: their data is not needed before the barrier
                rd = fetch(i + 2, lane, ent2);
                ent3 = ent_of(i + 3, lane);
            }
            if (i + 1 < n_tiles) {
                const int sl1 = (i + 1) % 3;
                if (PAR) gather(sl1, lq0, ldo0, lq16_0, ldo16_0);
                else gather(sl1, lq1, ldo1, lq16_1, ldo16_1);
            }
            const int sl = i % 3;
            if (PAR) compute(i, sl, lq1, ldo1, lq16_1, ldo16_1);
            else compute(i, sl, lq0, ldo0, lq16_0, ldo16_0);
            if (ahead) {
                put(rd, i + 2, (i + 2) % 3);
                ent2 = ent3;
            }
            __syncthreads();
        };
        int i = 0;
        for (; i + 1 < n_tiles; i += 2) {
            step(Par<0>{}, i);
            step(Par<1>{}, i + 1);
        }
        if (i < n_tiles) step(Par<0>{}, i);
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
