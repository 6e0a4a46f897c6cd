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

// S^T tiles of NG 32-row groups of one wave: every K fragment read from LDS
// feeds the matrix-core ops of all groups.
template <int D, int SPLIT, int NG>
__device__ __forceinline__ void qk_tiles(const uint16_t* ks, const bf16x8 (&qf)[NG][SPLIT][Tile<D>::DK],
                                         f32x16 (&s)[NG][2], int lane) {
    using T = Tile<D>;
    const int col = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int g = 0; g < NG; ++g) s[g][0] = s[g][1] = f32x16{};
#pragma unroll
    for (int k_ = 0; k_ < T::DK; ++k_)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int off = (sub * 32 + col) * T::KS + k_ * 16 + 8 * hh;
            const bf16x8 a = *(const bf16x8*)(ks + off);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                s[g][sub] = mfma32(a, qf[g][0][k_], s[g][sub]);
                if constexpr (SPLIT == 2) {
                    s[g][sub] = mfma32(a, qf[g][1][k_], s[g][sub]);
                    s[g][sub] = mfma32(*(const bf16x8*)(ks + T::KELEMS + off), qf[g][0][k_], s[g][sub]);
                }
            }
        }
}

// O^T += V^T P^T for NG row groups; every V^T fragment feeds all groups.
template <int D, int SPLIT, int NG>
__device__ __forceinline__ void pv_tiles(const uint16_t* vs, const uint4 (&pb)[NG][4],
                                         const uint4 (&pl)[NG][4], f32x16 (&o)[NG][Tile<D>::DM],
                                         const int (&voff)[Tile<D>::DM]) {
    using T = Tile<D>;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int mb = 0; mb < T::DM; ++mb) {
            const uint16_t* p0 = vs + voff[mb] + 16 * kk * T::VS;
            const v4i16 lo = read_tr(p0), hi = read_tr(p0 + 8 * T::VS);
            const auto a8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            if constexpr (SPLIT == 1) {
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    o[g][mb] = mfma32_f16(__builtin_bit_cast(f16x8, a8),
                                          __builtin_bit_cast(f16x8, pb[g][kk]), o[g][mb]);
            } else {
                const bf16x8 av = __builtin_bit_cast(bf16x8, a8);
                const v4i16 lo2 = read_tr(p0 + T::VELEMS), hi2 = read_tr(p0 + T::VELEMS + 8 * T::VS);
                const bf16x8 a2 = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(lo2, hi2, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    o[g][mb] = mfma32(av, __builtin_bit_cast(bf16x8, pb[g][kk]), o[g][mb]);
                    o[g][mb] = mfma32(av, __builtin_bit_cast(bf16x8, pl[g][kk]), o[g][mb]);
                    o[g][mb] = mfma32(a2, __builtin_bit_cast(bf16x8, pb[g][kk]), o[g][mb]);
                }
            }
        }
}

// A workgroup owns NG * 128 consecutive query rows of one head: wave w holds
// the 32-row groups w*NG .. w*NG + NG - 1, one row per lane pair in each.
template <int D, int SPLIT, bool TOK, int NG>
__global__ __launch_bounds__(NTHREADS, NG == 1 ? 2 : 1) void attn_rows_kernel(RowsArgs a) {
    using T = Tile<D>;
    constexpr int RTW = RT * NG;   // query rows per workgroup
    __shared__ __align__(16) uint16_t lds_k[2][SPLIT * T::KELEMS];
    __shared__ __align__(16) uint16_t lds_v[2][SPLIT * T::VELEMS];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int BH = a.Bt * a.Hq;
    const int ntiles = (a.N + RTW - 1) / RTW;
    const int bh = blockIdx.x % BH;
    const int tile = ntiles - 1 - (int)(blockIdx.x / BH);   // longest rows first
    const int b = bh / a.Hq, h = bh % a.Hq, G = a.Hq / a.Hkv, g_kv = h / G;
    const int N = a.N;
    const int r0 = tile * RTW;

    const size_t kvoff = (size_t)(b * a.Hkv + g_kv) * N * D;
    const uint16_t* kp[2] = {a.k[0] + kvoff, SPLIT == 2 ? a.k[1] + kvoff : nullptr};
    const uint16_t* vp[2] = {a.v[0] + kvoff, SPLIT == 2 ? a.v[1] + kvoff : nullptr};

    const int wu = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform
    int row[NG], q0[NG], q1[NG];
    bool row_ok[NG];
    size_t prow[NG];   // flat row ids
    bf16x8 qf[NG][SPLIT][T::DK];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        q0[g] = r0 + (wu * NG + g) * 32;
        q1[g] = min(q0[g] + 31, N - 1);
        row[g] = q0[g] + col;
        row_ok[g] = row[g] < N;
        prow[g] = (size_t)bh * N + row[g];
        load_q<D, SPLIT>(qf[g], a.q, prow[g] * D, row_ok[g], hh);
    }

    // Block-gate state of each row: its block, the kept near blocks as a
    // bit mask over (own block - 1 - bit), and the count of far blocks.
    int row_blk[NG], nfar[NG];
    uint32_t near_bits[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        row_blk[g] = 0;
        nfar[g] = 0;
        near_bits[g] = 0;
        if (a.gate) {
            row_blk[g] = (row_ok[g] ? row[g] : N - 1) / a.B;
            if (row_ok[g]) {
                const int32_t* sr = a.sel + prow[g] * a.top_k;
                for (int x = 0; x < a.top_k; ++x) {
                    const int cblk = sr[x];
                    if (cblk < 0) break;
                    const int dlt = row_blk[g] - cblk;
                    if (dlt > a.span) ++nfar[g];
                    else if (dlt >= 1 && dlt <= 32) near_bits[g] |= 1u << (dlt - 1);
                }
            }
        }
    }

    // Key range of the workgroup.
    const int r_hi = min(r0 + RTW - 1, N - 1);
    auto lower_key = [&](int r) {
        if (TOK) return 0;   // selected tokens can be anywhere before r
        int lo = r;
        if (a.window > 0) lo = min(lo, r - a.window + 1);
        if (a.gate) lo = min(lo, (r / a.B - a.span) * a.B);
        return max(lo, 0);
    };
    const int t_begin = lower_key(r0) / KT, t_end = r_hi / KT;
    const float c = a.scale * kLog2e;
    const uint32_t wl_window = a.window > 0 ? (uint32_t)a.window : 0u;

    zero_v_init<D, SPLIT>(&lds_v[0][0], tid);

    f32x16 o[NG][T::DM];
    RowState rs[NG];
    uint4 pb[NG][4], pl[NG][4];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
        for (int mb = 0; mb < T::DM; ++mb) o[g][mb] = f32x16{};
        rs[g] = RowState{-INFINITY, 0.f, 1.f, false};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) pb[g][kk] = pl[g][kk] = make_uint4(0, 0, 0, 0);
    }

    int voff[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) voff[mb] = v_lane_offset<D>(lane, mb);
    Stage<D, SPLIT> kst, vst;
    const TileSrc<D, SPLIT> ksrc = tile_src<D, SPLIT>(kp, N, tid), vsrc = tile_src<D, SPLIT>(vp, N, tid);
    load_tile<D, SPLIT>(kst, ksrc, t_begin * KT);
    store_tile<D, SPLIT, T::KS, T::KELEMS>(kst, lds_k[0], tid);
    __syncthreads();

    // Mask of key tile t for the rows of group g: keys a row does not attend
    // become -inf (a tile past a group's rows is fully masked).  Tiles that
    // are entirely inside every row's window, or inside every row's own
    // block, need no mask (wave-uniform test).
    auto mask_t = [&](f32x16 (&sv)[2], int t, int g) {
        const int kt0 = t * KT;
        const int rk = row[g] - kt0 - 4 * hh;
        if constexpr (TOK) {
            // This lane's keep bits for the tile; key tiles past the group's
            // rows hold no kept key, and a group past the last row has no
            // mask.  Only 32-key halves kc <= rt are written; a half past the
            // row tile (kc = rt + 1 when rt is even) is all future keys:
            // cleared.
            const int nt32 = (N + 31) / 32, nt64 = (N + KT - 1) / KT, rt = q0[g] / 32;
            uint32_t tword = t <= rt / 2 && q0[g] < N
                                 ? a.tokmask[(((size_t)b * nt32 + rt) * nt64 + t) * 64 + lane]
                                 : 0u;
            if (2 * t + 1 > rt) tword &= 0xffffu;
            const bool near = kt0 + KT - 1 >= q0[g] - a.window + 1;   // tile meets a window
            mask_tile_tok(sv, rk, wl_window, near, tword);
        } else {
            const bool full = kt0 + KT - 1 <= q0[g] &&
                              ((a.window > 0 && q1[g] - kt0 < a.window) ||
                               (a.gate && kt0 / a.B == q0[g] / a.B && q1[g] / a.B == q0[g] / a.B));
            if (!full) {
                uint32_t wl = wl_window;
                if (a.gate) {
                    const int dlt = row_blk[g] - kt0 / a.B;
                    const bool blk_ok = dlt == 0 || (dlt >= 1 && dlt <= a.span && dlt <= 32 &&
                                                     ((near_bits[g] >> (dlt - 1)) & 1u));
                    if (blk_ok) wl = 0x80000000u;
                }
                mask_tile(sv, rk, wl);
            }
        }
    };

    // One-stage skew: the step of tile t computes S_t, O += V_{t-1} P_{t-1}
    // and P_t; V is staged one tile behind K.
    for (int t = t_begin; t <= t_end; ++t) {
        const int it = t - t_begin;
        load_tile<D, SPLIT>(kst, ksrc, min(t + 1, t_end) * KT);
        load_tile<D, SPLIT>(vst, vsrc, t * KT);
#pragma unroll
        for (int g = 0; g < NG; ++g) apply_rescale<D>(o[g], rs[g]);
        f32x16 sv[NG][2];
        qk_tiles<D, SPLIT, NG>(lds_k[it & 1], qf, sv, lane);
#pragma unroll
        for (int g = 0; g < NG; ++g) mask_t(sv[g], t, g);
        pv_tiles<D, SPLIT, NG>(lds_v[(it + 1) & 1], pb, pl, o, voff);
#pragma unroll
        for (int g = 0; g < NG; ++g) softmax_tile<SPLIT>(sv[g], rs[g], c, pb[g], pl[g]);
        store_tile<D, SPLIT, T::KS, T::KELEMS>(kst, lds_k[(it + 1) & 1], tid);
        store_tile<D, SPLIT, T::VS, T::VELEMS>(vst, lds_v[it & 1], tid);
        __syncthreads();
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) apply_rescale<D>(o[g], rs[g]);
    pv_tiles<D, SPLIT, NG>(lds_v[(t_end - t_begin) & 1], pb, pl, o, voff);

#pragma unroll
    for (int g = 0; g < NG; ++g)
        if (row_ok[g]) finish_rows<D>(a, o[g], pair_sum(rs[g].l), rs[g].m, prow[g], h, nfar[g], hh);
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
    constexpr int NG = 1;
    const int ntiles = (a.N + RT * NG - 1) / (RT * NG);
    const unsigned grid = (unsigned)(ntiles * a.Bt * a.Hq);
    if (a.tokmask)
        hipLaunchKernelGGL((attn_rows_kernel<D, SPLIT, true, NG>), dim3(grid), dim3(NTHREADS), 0, s, a);
    else
        hipLaunchKernelGGL((attn_rows_kernel<D, SPLIT, false, NG>), dim3(grid), dim3(NTHREADS), 0, s, a);
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
