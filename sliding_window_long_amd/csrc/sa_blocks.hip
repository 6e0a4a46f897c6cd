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

// LDS of the attention kernels: double-buffered K and V tiles during the
// key loop, the per-wave output stages after it (far-block kernel).
template <int D, int SPLIT>
struct AttnSmem {
    static constexpr int KV = 2 * SPLIT * (Tile<D>::KELEMS + Tile<D>::VELEMS) * 2;
    static constexpr int EPI = NWAVES * EpiStage<D>::BYTES;
    static constexpr int BYTES = KV > EPI ? KV : EPI;
};

// ---------------------------------------------------------------------------
// KV-centric far-block kernel.
// ---------------------------------------------------------------------------
template <int D, int SPLIT>
__global__ __launch_bounds__(NTHREADS, 2) void attn_blocks_kernel(BlocksArgs a) {
    using T = Tile<D>;
    __shared__ __align__(16) uint8_t smem[AttnSmem<D, SPLIT>::BYTES];
    uint16_t* const lds_k = (uint16_t*)smem;                  // [2][SPLIT * KELEMS]
    uint16_t* const lds_v = lds_k + 2 * SPLIT * T::KELEMS;    // [2][SPLIT * VELEMS]
    auto kbuf = [&](int i) { return lds_k + i * (SPLIT * T::KELEMS); };
    auto vbuf = [&](int i) { return lds_v + i * (SPLIT * T::VELEMS); };

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

    zero_v_init<D, SPLIT>(lds_v, tid);

    f32x16 o[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) o[mb] = f32x16{};
    RowState rs{-INFINITY, 0.f, 1.f, false};
    uint4 pb[4], pl[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) pb[kk] = pl[kk] = make_uint4(0, 0, 0, 0);

    const int ntile = a.B / KT;
    const int k_begin = cblk * a.B;
    int voff[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) voff[mb] = v_lane_offset<D>(lane, mb);
    Stage<D, SPLIT> kst, vst;
    const TileSrc<D, SPLIT> ksrc = tile_src<D, SPLIT>(kp, N, tid), vsrc = tile_src<D, SPLIT>(vp, N, tid);
    load_tile<D, SPLIT>(kst, ksrc, k_begin);
    store_tile<D, SPLIT, T::KS, T::KELEMS>(kst, kbuf(0), tid);
    __syncthreads();
    for (int t = 0; t < ntile; ++t) {
        load_tile<D, SPLIT>(kst, ksrc, k_begin + min(t + 1, ntile - 1) * KT);
        load_tile<D, SPLIT>(vst, vsrc, k_begin + t * KT);
        kv_step<D, SPLIT>(kbuf(t & 1), vbuf((t + 1) & 1), qf, o, rs, pb, pl, c, lane, voff);
        store_tile<D, SPLIT, T::KS, T::KELEMS>(kst, kbuf((t + 1) & 1), tid);
        store_tile<D, SPLIT, T::VS, T::VELEMS>(vst, vbuf(t & 1), tid);
        __syncthreads();
    }
    apply_rescale<D>(o, rs);
    pv_tile<D, SPLIT>(vbuf((ntile - 1) & 1), pb, pl, o, voff);

    // Normalised partial of each row, staged row-major and written in
    // 16-byte chunks by all lanes (each row's D fp16 values are contiguous
    // at part_o[pidx]); the lse by the row-owner lanes.
    __syncthreads();   // every wave is done with the K/V buffers
    using E = EpiStage<D>;
    float* st = (float*)smem + wave * E::FLOATS;
    const float lt = pair_sum(rs.l);
    const size_t pidx = prow * (size_t)a.kslots + slot;
    stage_rows<D>(st, o, 1.f / lt, col, hh);
    if (hh == 0) {
        st[E::INFO + 4 * col] = __int_as_float(ok ? (int)pidx : -1);
        if (ok) a.part_lse[pidx] = rs.m * a.scale + kLn2 * fast_log2(lt);
    }
    stage_fence();
    constexpr int CPR = D / 8;
#pragma unroll
    for (int it = 0; it < (32 * CPR + 63) / 64; ++it) {
        const int q = lane + 64 * it;
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
