// sa_blocks.hip -- KV-centric far-block attention kernel.
//
// A workgroup owns one chunk (<= 128 entries) of the list of rows that kept
// one far block, gathers those query rows and attends the block's B keys,
// writing one normalised partial per entry.  The query-centric kernel merges
// the partials of each row.  This is the variable-length per-block step of
// the implementation section of the MoBA summary page ("MoBA의 구현: MoE와
// FlashAttention의 결합").
#include "sa_attn_common.hpp"

namespace sa {

// Staging area of one wave's 32 output rows after the key loop (it reuses
// the workgroup's K/V buffers): fp32 rows D + 4 apart (16-byte writes of 32
// rows land on distinct banks), then 4 words of per-row data.
template <int D>
struct EpiStage {
    static constexpr int RS = D + 4;
    static constexpr int INFO = 32 * RS;           // float offset of the per-row words
    static constexpr int FLOATS = INFO + 4 * 32;
    static constexpr int BYTES = FLOATS * 4;
};

// Row-owner lanes put their O^T registers (times f) into the stage: lane
// (col, hh) holds dims mb*32 + 8j + 4hh .. +3 of row col.
template <int D>
__device__ __forceinline__ void stage_rows(float* st, const f32x16 (&o)[Tile<D>::DM], float f,
                                           int col, int hh) {
    using E = EpiStage<D>;
#pragma unroll
    for (int mb = 0; mb < Tile<D>::DM; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d0 = mb * 32 + 8 * j + 4 * hh;
            if (d0 < D)
                *(float4*)(st + col * E::RS + d0) =
                    make_float4(o[mb][4 * j] * f, o[mb][4 * j + 1] * f, o[mb][4 * j + 2] * f,
                                o[mb][4 * j + 3] * f);
        }
}

// The writes of other lanes of this wave to the stage are visible to its
// reads from here on.
__device__ __forceinline__ void stage_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// KV-centric far-block kernel.
//
// The key loop is the query-centric kernel's (sa_attn.hip) without masks:
// K/V tiles straight from global memory into LDS, one buffer per LDS array
// and the loop unrolled by two; S_{t+1} = K_{t+1} Q^T, then O += V_t P_t
// beside the row max and exp of S_{t+1}.  The first K/V tile is requested
// before the query rows are gathered, and every load that only needs the
// chunk table is issued before the ones that need the list end.
// ---------------------------------------------------------------------------
template <int D, int SPLIT>
__global__ __launch_bounds__(NTHREADS, rows_waves(D, SPLIT)) void attn_blocks_kernel(BlocksArgs a) {
    using T = Tile<D>;
    constexpr bool ONES = T::DPAD > D;
    constexpr int VS = dma_vs<D>();
    constexpr int VELEMS = KT * VS;
    // After the key loop, wave w stages its rows in buffer w: a K buffer
    // holds exactly one stage (64 (D + 8) 16-bit elements = 32 (D + 4) + 128
    // floats), a V buffer more.
    static_assert(EpiStage<D>::BYTES <= T::KELEMS * 2, "stage must fit a K buffer");
    __shared__ __align__(16) uint16_t lds_k0[SPLIT * T::KELEMS], lds_k1[SPLIT * T::KELEMS];
    __shared__ __align__(16) uint16_t lds_v0[SPLIT * VELEMS], lds_v1[SPLIT * VELEMS];

    // Chunks of one list are contiguous in the table; hand each XCD (the
    // dispatcher deals workgroups to the 8 XCDs in turn) a contiguous eighth
    // of the valid chunks, so the block's K/V stays in that XCD's L2 and the
    // XCDs get equal shares.
    const int nch = *a.n_chunks;
    const int per_xcd = (nch + 7) / 8;
    const int slot = (int)(blockIdx.x / 8);
    const int chunk = (int)(blockIdx.x % 8) * per_xcd + slot;
    if (slot >= per_xcd || chunk >= nch) return;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int list = a.chunk_list[chunk];
    const int e0 = a.chunk_start[chunk];
    const int e = e0 + wu * 32 + col;
    // Both depend on the chunk table only: the entry (clamped into the
    // array; used only below the list end) and the list end.
    const int ent = a.entries[min(e, a.entries_cap - 1)];
    const int e_end = min(e0 + RT, a.list_off[list + 1]);
    const int cblk = list % a.n, bg = list / a.n;   // bg = b*Hkv + g
    const int b = bg / a.Hkv, g = bg % a.Hkv, G = a.Hq / a.Hkv;
    const int N = a.N;
    const int ntile = a.B >= KT ? a.B / KT : 1;   // a block smaller than a tile: one masked tile
    const int k_begin = cblk * a.B;

    // V rows: the fp16 copy's stride (bf16 path; ones past D at d 80) or D.
    constexpr int VSRC = SPLIT == 1 ? v16_row<D>() : D;
    constexpr bool ONES_SEL = ONES && VSRC == D;   // padding lanes select ones
    const size_t kvoff = (size_t)bg * N * D;
    uint64_t kb[SPLIT], vb[SPLIT];   // workgroup-uniform byte addresses
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) {
        kb[p] = uniform_u64((uint64_t)(a.k[p] + kvoff));
        vb[p] = uniform_u64((uint64_t)(a.v[p] + (size_t)bg * N * VSRC));
    }
    TileDma<D, T::KS> kd;
    TileDma<D, VS, VSRC> vd;
    kd.init(wu, lane);
    vd.init(wu, lane);
    auto load_k = [&](int t, uint16_t* dst) { dma_tile<D, SPLIT, T::KELEMS>(kd, kb, N, k_begin + t * KT, dst, wu); };
    auto load_v = [&](int t, uint16_t* dst) { dma_tile<D, SPLIT, VELEMS>(vd, vb, N, k_begin + t * KT, dst, wu); };
    load_k(0, lds_k0);
    load_v(0, lds_v0);

    const bool ok = e < e_end;
    int slot_ = 0;
    size_t prow = 0;
    if (ok) {
        slot_ = ent % a.kslots;
        const int t2 = ent / a.kslots;
        const int hl = t2 % G, i = t2 / G;
        prow = (size_t)(b * a.Hq + g * G + hl) * N + i;
    }
    bf16x8 qf[SPLIT][T::DK];
    load_q<D, SPLIT>(qf, a.q, prow * D, ok, hh);
    const float c = a.scale * kLog2e;

    f32x16 o[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) o[mb] = f32x16{};
    RowState rs{-INFINITY, 0.f, 1.f, false};
    uint4 pb[4], pl[4];
    int voff[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) voff[mb] = v_lane_offset<D, VS, ONES>(lane, mb);
    const bool pad = ONES && ((lane >> 4) & 1);   // lanes of the padding dims in the last row block

    __syncthreads();
    load_k(min(1, ntile - 1), lds_k1);
    f32x16 s0[2];
    qk_tile<D, SPLIT>(lds_k0, qf, s0, lane);
    if (a.B < KT) mask_tile(s0, a.B - 1 - 4 * hh, (uint32_t)a.B);   // keys past the block
    max_tile(s0, rs, c);
    exp_tile<SPLIT, !ONES>(s0, rs, c, pb, pl);
    __syncthreads();

    // Step of tile it < ntile - 1 (buffer parity PAR = it & 1): consumes
    // P_it, produces S_{it+1} and P_{it+1}.
    auto step = [&](auto par, int it) {
        constexpr int PAR = decltype(par)::value;
        uint16_t* const k_next = PAR ? lds_k0 : lds_k1;   // K_{it+1}
        uint16_t* const k_free = PAR ? lds_k1 : lds_k0;   // K_it: done
        uint16_t* const v_cur = PAR ? lds_v1 : lds_v0;    // V_it
        uint16_t* const v_free = PAR ? lds_v0 : lds_v1;   // V_{it-1}: done
        load_k(min(it + 2, ntile - 1), k_free);
        load_v(it + 1, v_free);
        apply_rescale<D>(o, rs);
        qk_tile<D, SPLIT>(k_next, qf, s0, lane);
        pv_tile<D, SPLIT, VS, ONES_SEL>(v_cur, pb, pl, o, voff, pad);
        max_tile(s0, rs, c);
        exp_tile<SPLIT, !ONES>(s0, rs, c, pb, pl);
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 4, 0);
#pragma unroll
        for (int i = 0; i < T::DM * 4 * (SPLIT == 2 ? 3 : 1); ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedVALU, 8, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            pin(pb[kk]);
            if constexpr (SPLIT == 2) pin(pl[kk]);
        }
        __syncthreads();
    };
    auto last = [&](auto par) {
        constexpr int PAR = decltype(par)::value;
        apply_rescale<D>(o, rs);
        pv_tile<D, SPLIT, VS, ONES_SEL>(PAR ? lds_v1 : lds_v0, pb, pl, o, voff, pad);
    };
    int it = 0;
    for (; it + 2 < ntile; it += 2) {
        step(Par<0>{}, it);
        step(Par<1>{}, it + 1);
    }
    if (it + 1 < ntile) {
        step(Par<0>{}, it);
        last(Par<1>{});
    } else {
        last(Par<0>{});
    }

    // Normalised partial of each row, staged row-major and written in
    // 16-byte chunks by all lanes (each row's D fp16 values are contiguous
    // at part_o[pidx]); the lse by the row-owner lanes.
    __syncthreads();   // every wave is done with the K/V buffers
    using E = EpiStage<D>;
    float* const st = (float*)(wu == 0 ? lds_k0 : wu == 1 ? lds_k1 : wu == 2 ? lds_v0 : lds_v1);
    float lt;
    if constexpr (ONES) lt = o[T::DM - 1][8];   // O^T row D (hh 0) or D + 4 (hh 1)
    else lt = pair_sum(rs.l);
    const size_t pidx = prow * (size_t)a.kslots + slot_;
    stage_rows<D>(st, o, 1.f / lt, col, hh);
    if (hh == 0) {
        st[E::INFO + 4 * col] = __int_as_float(ok ? (int)pidx : -1);
        if (ok) a.part_lse[pidx] = rs.m * a.scale + kLn2 * fast_log2(lt);
    }
    stage_fence();
    constexpr int CPR = D / 8;
#pragma unroll
    for (int it2 = 0; it2 < (32 * CPR + 63) / 64; ++it2) {
        const int q = lane + 64 * it2;
        const int r = q / CPR, c8 = q % CPR;
        if (q < 32 * CPR) {
            const int pr = __float_as_int(st[E::INFO + 4 * r]);
            if (pr >= 0) {
                const float* sr = st + r * E::RS + 8 * c8;
                const float4 x0 = *(const float4*)sr, x1 = *(const float4*)(sr + 4);
                const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                _Float16 hv[8];
#pragma unroll
                for (int e2 = 0; e2 < 8; ++e2) hv[e2] = (_Float16)x[e2];
                *(uint4*)(a.part_o + (size_t)pr * D + 8 * c8) = *(const uint4*)hv;
            }
        }
    }
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

}  // namespace sa
