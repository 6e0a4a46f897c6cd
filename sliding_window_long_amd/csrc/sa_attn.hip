// sa_attn.hip -- query-centric attention kernel on the gfx950 matrix cores,
// and the small conversion kernels of the attention inputs.
//
// attn_rows_kernel: a workgroup owns 128 consecutive query rows of one head
// and walks the keys that can be near them (the sliding window, the own
// block, kept blocks overlapping the window span, or every earlier key under
// the token gate) in 64-key tiles staged through LDS.  The epilogue merges
// the far-block partials (sa_blocks.hip) and the sink column and writes out
// and lse.
//
// The split between the two kernels follows the implementation section of
// the MoBA summary page ("MoBA의 구현: MoE와 FlashAttention의 결합"): rows are
// regrouped by kept KV block, each block is attended as a variable-length
// batch, the own block is attended causally on its own, and the pieces are
// combined with the online-softmax rule.  The window of the Bit-Axon SWA page
// ("슬라이딩 윈도우 마스크") joins the causal own-block pass.
#include "sa_attn_common.hpp"

namespace sa {

// Epilogue of the query-centric kernels: combine the near part (o, row sum
// lt, exponent base m), the far-block partials of the row and the sink
// column; write out and lse.
template <int D>
__device__ __forceinline__ void finish_rows(const RowsArgs& a, f32x16 (&o)[Tile<D>::DM], float lt,
                                            float m, size_t prow, int h, int nfar, int hh) {
    using T = Tile<D>;
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
// Query-centric kernel.
// ---------------------------------------------------------------------------

// A workgroup owns 128 consecutive query rows of one head; wave w holds rows
// 32w .. 32w + 31, one row per lane pair.
//
// The key loop runs over 64-key tiles, skewed by one so that the matrix-core
// products of one tile have independent vector work beside them:
//   S_{t+1} = K_{t+1} Q^T, then  O += V_t P_t  with  the mask, row max and
//   exp2((S_{t+1} - m) c) of S_{t+1} (which give P_{t+1}).
// K_{t+1} and V_t are in LDS when the step of tile t starts; the step loads
// K_{t+2} and V_{t+1} straight from global memory into the LDS buffers that
// tiles t and t - 1 used, and its closing barrier waits for them.  Each
// buffer is its own LDS array and the loop is unrolled by two, so every
// access names its buffer at compile time (the compiler then knows that the
// loads in flight never alias the tiles being read).  With no staging
// registers, head dims up to 80 fit three workgroups per CU (three waves
// per SIMD): 11 % faster at d 80 than two workgroups with an extra S tile in
// registers that moved the exp beside the K Q^T products.
//
// Head dims that are not a multiple of 32 (80) pad O^T to 96 rows; those
// rows take constant ones as their V^T operand (columns 80..95 of the fp16 V
// copy hold ones; the fp32 path selects them), so the matrix cores produce
// the softmax row sums (of the same fp16 P that weights V) and no vector ops
// are spent on them.
template <int D, int SPLIT, bool TOK>
__global__ __launch_bounds__(NTHREADS, D <= 80 && SPLIT == 1 ? 3 : 2) void attn_rows_kernel(RowsArgs a) {
    using T = Tile<D>;
    constexpr bool ONES = T::DPAD > D;
    constexpr int VS = dma_vs<D>();
    constexpr int VELEMS = KT * VS;
    __shared__ __align__(16) uint16_t lds_k0[SPLIT * T::KELEMS], lds_k1[SPLIT * T::KELEMS];
    __shared__ __align__(16) uint16_t lds_v0[SPLIT * VELEMS], lds_v1[SPLIT * VELEMS];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int BH = a.Bt * a.Hq;
    const int ntiles = (a.N + RT - 1) / RT;
    const int bh = blockIdx.x % BH;
    const int tile = ntiles - 1 - (int)(blockIdx.x / BH);   // longest rows first
    const int b = bh / a.Hq, h = bh % a.Hq, G = a.Hq / a.Hkv, g_kv = h / G;
    const int N = a.N;
    const int r0 = tile * RT;

    // V rows: the fp16 copy's stride (bf16 path; ones past D at d 80) or D.
    constexpr int VSRC = SPLIT == 1 ? v16_row<D>() : D;
    constexpr bool ONES_SEL = ONES && VSRC == D;   // padding lanes select ones
    const size_t kvoff = (size_t)(b * a.Hkv + g_kv) * N * D;
    const size_t voff_src = (size_t)(b * a.Hkv + g_kv) * N * VSRC;
    uint64_t kb[SPLIT], vb[SPLIT];   // workgroup-uniform byte addresses
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) {
        kb[p] = uniform_u64((uint64_t)(a.k[p] + kvoff));
        vb[p] = uniform_u64((uint64_t)(a.v[p] + voff_src));
    }

    const int wu = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform
    const int q0 = r0 + wu * 32, q1 = min(q0 + 31, N - 1);
    const int row = q0 + col;
    const bool row_ok = row < N;
    const size_t prow = (size_t)bh * N + row;   // flat row id
    bf16x8 qf[SPLIT][T::DK];
    load_q<D, SPLIT>(qf, a.q, prow * D, row_ok, hh);

    // Block-gate state of the row: its block, the kept near blocks as a bit
    // mask over (own block - 1 - bit), and the count of far blocks.
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

    // Key range of the workgroup.
    const int r_hi = min(r0 + RT - 1, N - 1);
    auto lower_key = [&](int r) {
        if (TOK) return 0;   // selected tokens can be anywhere before r
        int lo = r;
        if (a.window > 0) lo = min(lo, r - a.window + 1);
        if (a.gate) lo = min(lo, (r / a.B - a.span) * a.B);
        return max(lo, 0);
    };
    const int t_begin = lower_key(r0) / KT, t_end = r_hi / KT;
    const int n_t = t_end - t_begin + 1;
    const float c = a.scale * kLog2e;
    const uint32_t wl_window = a.window > 0 ? (uint32_t)a.window : 0u;

    f32x16 o[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) o[mb] = f32x16{};
    RowState rs{-INFINITY, 0.f, 1.f, false};
    uint4 pb[4], pl[4];

    int voff[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) voff[mb] = v_lane_offset<D, VS, ONES>(lane, mb);
    const bool pad = ONES && ((lane >> 4) & 1);   // lanes of the padding dims in the last row block
    TileDma<D, T::KS> kd;
    TileDma<D, VS, VSRC> vd;
    kd.init(wu, lane);
    vd.init(wu, lane);
    auto load_k = [&](int t, uint16_t* dst) { dma_tile<D, SPLIT, T::KELEMS>(kd, kb, N, t * KT, dst, wu); };
    auto load_v = [&](int t, uint16_t* dst) { dma_tile<D, SPLIT, VELEMS>(vd, vb, N, t * KT, dst, wu); };

    // Mask of key tile t: keys the row does not attend become -inf (a tile
    // past the wave's rows is fully masked).  Tiles that are entirely inside
    // every row's window, or inside every row's own block, need no mask
    // (wave-uniform test).
    // Token gate: this lane's keep bits for key tile t; key tiles past the
    // wave's rows hold no kept key, and a wave past the last row has no mask.
    // Only 32-key halves kc <= rt are written; a half past the row tile (kc
    // = rt + 1 when rt is even) is all future keys: cleared.
    auto tok_word = [&](int t) -> uint32_t {
        if constexpr (!TOK) return 0u;
        const int nt32 = (N + 31) / 32, nt64 = (N + KT - 1) / KT, rt = q0 / 32;
        uint32_t tword = t <= rt / 2 && q0 < N
                             ? a.tokmask[(((size_t)b * nt32 + rt) * nt64 + t) * 64 + lane]
                             : 0u;
        if (2 * t + 1 > rt) tword &= 0xffffu;
        return tword;
    };
    auto mask_t = [&](f32x16 (&sv)[2], int t, uint32_t tword) {
        const int kt0 = t * KT;
        const int rk = row - kt0 - 4 * hh;
        if constexpr (TOK) {
            const bool near = kt0 + KT - 1 >= q0 - a.window + 1;   // tile meets a window
            mask_tile_tok(sv, rk, wl_window, near, tword);
        } else {
            const bool full = kt0 + KT - 1 <= q0 &&
                              ((a.window > 0 && q1 - kt0 < a.window) ||
                               (a.gate && kt0 / a.B == q0 / a.B && q1 / a.B == q0 / a.B));
            if (!full) {
                uint32_t wl = wl_window;
                if (a.gate) {
                    const int dlt = row_blk - kt0 / a.B;
                    const bool blk_ok = dlt == 0 || (dlt >= 1 && dlt <= a.span && dlt <= 32 &&
                                                     ((near_bits >> (dlt - 1)) & 1u));
                    if (blk_ok) wl = 0x80000000u;
                }
                mask_tile(sv, rk, wl);
            }
        }
    };

    // Prologue: K_0 and V_0 into LDS; S_0 with its mask and max while K_1
    // loads.
    const uint32_t tw0 = tok_word(t_begin);
    load_k(t_begin, lds_k0);
    load_v(t_begin, lds_v0);
    __syncthreads();
    load_k(min(t_begin + 1, t_end), lds_k1);
    f32x16 s0[2];
    qk_tile<D, SPLIT>(lds_k0, qf, s0, lane);
    mask_t(s0, t_begin, tw0);
    max_tile(s0, rs, c);
    exp_tile<SPLIT, !ONES>(s0, rs, c, pb, pl);
    __syncthreads();

    // Step of relative tile it < n_t - 1 (buffer parity PAR = it & 1):
    // consumes P_it, produces S_{it+1} and P_{it+1} (in sn and pb, pl).
    auto step = [&](auto par, int it, f32x16 (&sn)[2]) {
        constexpr int PAR = decltype(par)::value;
        uint16_t* const k_next = PAR ? lds_k0 : lds_k1;   // K_{it+1}
        uint16_t* const k_free = PAR ? lds_k1 : lds_k0;   // K_it: done
        uint16_t* const v_cur = PAR ? lds_v1 : lds_v0;    // V_it
        uint16_t* const v_free = PAR ? lds_v0 : lds_v1;   // V_{it-1}: done
        const int t = t_begin + it;
        // The mask word first: waiting for it then does not wait for the
        // tile loads issued after it.
        const uint32_t tw = tok_word(t + 1);
        load_k(min(t + 2, t_end), k_free);
        load_v(t + 1, v_free);
        apply_rescale<D>(o, rs);
        qk_tile<D, SPLIT>(k_next, qf, sn, lane);
        mask_t(sn, t + 1, tw);
        pv_tile<D, SPLIT, VS, ONES_SEL>(v_cur, pb, pl, o, voff, pad);
        max_tile(sn, rs, c);
        exp_tile<SPLIT, !ONES>(sn, rs, c, pb, pl);
        // 12 (d 80) matrix-core ops and 24 transposing reads with about 90
        // vector ops.
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
    // Last tile: its P V only.
    auto last = [&](auto par) {
        constexpr int PAR = decltype(par)::value;
        apply_rescale<D>(o, rs);
        pv_tile<D, SPLIT, VS, ONES_SEL>(PAR ? lds_v1 : lds_v0, pb, pl, o, voff, pad);
    };
    // Unrolled by two so that the buffer parity is a constant.
    int it = 0;
    for (; it + 2 < n_t; it += 2) {
        step(Par<0>{}, it, s0);
        step(Par<1>{}, it + 1, s0);
    }
    if (it + 1 < n_t) {
        step(Par<0>{}, it, s0);
        last(Par<1>{});
    } else {
        last(Par<0>{});
    }

    if (row_ok) {
        float lt;
        if constexpr (ONES) lt = o[T::DM - 1][8];   // O^T row D (hh 0) or D + 4 (hh 1)
        else lt = pair_sum(rs.l);
        finish_rows<D>(a, o, lt, rs.m, prow, h, nfar, hh);
    }
}


// bf16 -> fp16, exact for |x| in the fp16 normal range [2^-14, 65504].
__global__ void bf16_to_f16_kernel(const uint4* __restrict__ x, uint4* __restrict__ y, size_t n8) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n8) return;
    const uint4 u = x[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    uint32_t r[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const _Float16 lo = (_Float16)bf16_to_f32(w[t] & 0xffffu);
        const _Float16 hi = (_Float16)bf16_to_f32(w[t] >> 16);
        r[t] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    y[i] = make_uint4(r[0], r[1], r[2], r[3]);
}

// bf16 rows of D -> fp16 rows of SR (> D) whose columns D .. SR-1 hold
// fp16 one; one thread per 8 output elements.
__global__ void bf16_to_f16_rows_kernel(const uint16_t* __restrict__ x, uint4* __restrict__ y,
                                        size_t rows, int D, int SR) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int cpr = SR / 8;
    if (i >= rows * cpr) return;
    const size_t r = i / cpr;
    const int c = (int)(i % cpr);
    uint32_t o[4] = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
    if (c < D / 8) {
        const uint4 u = *(const uint4*)(x + r * D + c * 8);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const _Float16 lo = (_Float16)bf16_to_f32(w[t] & 0xffffu);
            const _Float16 hi = (_Float16)bf16_to_f32(w[t] >> 16);
            o[t] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
    }
    y[i] = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_v_to_f16(const uint16_t* v, uint16_t* y, size_t rows, int D, hipStream_t s) {
    const int SR = v16_row_of(D);
    if (SR == D) return launch_bf16_to_f16(v, y, rows * D, s);
    const size_t n8 = rows * (SR / 8);
    if (n8 == 0) return hipSuccess;
    hipLaunchKernelGGL(bf16_to_f16_rows_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, v,
                       (uint4*)y, rows, D, SR);
    return hipGetLastError();
}

hipError_t launch_bf16_to_f16(const uint16_t* x, uint16_t* y, size_t n, hipStream_t s) {
    const size_t n8 = n / 8;   // n is a multiple of the head dim, hence of 8
    if (n8 == 0) return hipSuccess;
    hipLaunchKernelGGL(bf16_to_f16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                       (const uint4*)x, (uint4*)y, n8);
    return hipGetLastError();
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
    // One 32-row group per wave.  Two (every K/V fragment read from LDS
    // feeding 64 rows) leave room for one wave per SIMD and measured slower
    // on every shape (d = 80 window: 1.20 vs 0.94 ms).
    const int ntiles = (a.N + RT - 1) / RT;
    const unsigned grid = (unsigned)(ntiles * a.Bt * a.Hq);
    if (a.tokmask)
        hipLaunchKernelGGL((attn_rows_kernel<D, SPLIT, true>), dim3(grid), dim3(NTHREADS), 0, s, a);
    else
        hipLaunchKernelGGL((attn_rows_kernel<D, SPLIT, false>), dim3(grid), dim3(NTHREADS), 0, s, a);
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

hipError_t launch_split_f32(const float* x, uint16_t* hi, uint16_t* lo, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const unsigned grid = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(split_f32_kernel, dim3(grid), dim3(256), 0, s, x, hi, lo, n);
    return hipGetLastError();
}

}  // namespace sa
