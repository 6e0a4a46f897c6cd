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

#include <type_traits>

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
    // Far partials two at a time: both slots' loads are issued before either
    // is accumulated.
    auto add_part = [&](float w, const uint2 (&raw)[T::DM][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < T::DM; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (mb * 32 + 8 * j + 4 * hh < D) {
                    const _Float16* hv = (const _Float16*)&raw[mb][j];
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[mb][4 * j + e] += w * (float)hv[e];
                }
            }
    };
    auto load_part = [&](int s_, uint2 (&raw)[T::DM][4]) __attribute__((always_inline)) {
        const uint16_t* po = a.part_o + (pbase + s_) * D;
#pragma unroll
        for (int mb = 0; mb < T::DM; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = mb * 32 + 8 * j + 4 * hh;
                raw[mb][j] = d0 < D ? *(const uint2*)(po + d0) : make_uint2(0, 0);
            }
    };
    int s_ = 0;
    for (; s_ + 1 < nfar; s_ += 2) {
        uint2 r0[T::DM][4], r1[T::DM][4];
        const float l0 = a.part_lse[pbase + s_], l1 = a.part_lse[pbase + s_ + 1];
        load_part(s_, r0);
        load_part(s_ + 1, r1);
        const float w0 = __expf(l0 - M), w1 = __expf(l1 - M);
        total += w0 + w1;
        add_part(w0, r0);
        add_part(w1, r1);
    }
    if (s_ < nfar) {
        uint2 r0[T::DM][4];
        const float l0 = a.part_lse[pbase + s_];
        load_part(s_, r0);
        const float w0 = __expf(l0 - M);
        total += w0;
        add_part(w0, r0);
    }
    if (a.sink) total += __expf(z - M);
    const float inv = 1.f / total;
    // V (and the far partials) were taken in units of 2^s.
    const int vs = a.vscale ? a.vscale[prow / a.N / (a.Hq / a.Hkv)] : 0;
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d0 = mb * 32 + 8 * j + 4 * hh;
            if (d0 < D) {
                const float v0 = ldexpf(o[mb][4 * j] * inv, vs), v1 = ldexpf(o[mb][4 * j + 1] * inv, vs);
                const float v2 = ldexpf(o[mb][4 * j + 2] * inv, vs), v3 = ldexpf(o[mb][4 * j + 3] * inv, vs);
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

// Pieces of the staged epilogue below (finish_rows_lds).  rows_begin: the common exponent base M of the row's parts (near lse, far
// partials' lse, sink), the near part's weight applied to o; returns the
// running weight sum.  rows_end: the sink's weight, then out and lse.
template <int D>
__device__ __forceinline__ float rows_begin(const RowsArgs& a, f32x16 (&o)[Tile<D>::DM], float lt,
                                            float m, size_t pbase, int h, int nfar, float& M, float& z) {
    using T = Tile<D>;
    const float lse_near = m * a.scale + kLn2 * fast_log2(lt);
    M = lse_near;
    for (int s_ = 0; s_ < nfar; ++s_) M = fmaxf(M, a.part_lse[pbase + s_]);
    z = a.sink ? a.sink[h] : -INFINITY;
    M = fmaxf(M, z);
    const float total = __expf(lse_near - M);
    const float wn = total / lt;
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[mb][v] *= wn;
    return total;
}

template <int D>
__device__ __forceinline__ void rows_end(const RowsArgs& a, f32x16 (&o)[Tile<D>::DM], float M,
                                         float total, float z, size_t prow, int hh) {
    using T = Tile<D>;
    if (a.sink) total += __expf(z - M);
    const float inv = 1.f / total;
    // V (and the far partials) were taken in units of 2^s.
    const int vs = a.vscale ? a.vscale[prow / a.N / (a.Hq / a.Hkv)] : 0;
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d0 = mb * 32 + 8 * j + 4 * hh;
            if (d0 < D) {
                const float v0 = ldexpf(o[mb][4 * j] * inv, vs), v1 = ldexpf(o[mb][4 * j + 1] * inv, vs);
                const float v2 = ldexpf(o[mb][4 * j + 2] * inv, vs), v3 = ldexpf(o[mb][4 * j + 3] * inv, vs);
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

// Add the fp16 partial raw (this lane's dims of one row) with weight w.
template <int D>
__device__ __forceinline__ void add_part(f32x16 (&o)[Tile<D>::DM], float w, const uint2 (&raw)[Tile<D>::DM][4],
                                         int hh) {
#pragma unroll
    for (int mb = 0; mb < Tile<D>::DM; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (mb * 32 + 8 * j + 4 * hh < D) {
                const _Float16* hv = (const _Float16*)&raw[mb][j];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[mb][4 * j + e] += w * (float)hv[e];
            }
        }
}

// The far partials staged through LDS (block gate, after the key loop): a
// wave's 32 rows hold their partials in one contiguous run of memory (kslots
// slots per row), so two slots of every row are loaded straight into the
// wave's own LDS buffer with coalesced 16-byte loads (global_load_lds), then
// read back one row per lane.  In LDS each row takes 2 (D / 8) + 1 chunks of
// 16 bytes (one chunk of padding: an odd stride, so the 32 rows' reads of a
// chunk spread over the banks).  Called by every lane of the workgroup (the
// batch loop holds barriers); ok: the lane's row exists.
template <int D>
__device__ __forceinline__ void finish_rows_lds(const RowsArgs& a, f32x16 (&o)[Tile<D>::DM], float lt,
                                                float m, size_t prow, int h, int nfar, int hh, bool ok,
                                                int col, int lane, uint16_t* buf) {
    using T = Tile<D>;
    constexpr int CH = D / 8, CPR = 2 * CH + 1;
    const size_t pbase = prow * (size_t)a.kslots;
    float M = 0.f, z = 0.f, total = 0.f;
    if (ok) total = rows_begin<D>(a, o, lt, m, pbase, h, nfar, M, z);
    for (int s0 = 0; __syncthreads_or(ok && nfar > s0); s0 += 2) {
        // (the barrier above: every wave is done with the buffers it reads)
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass rejects the LDS-pointer builtin
        constexpr int NI = (32 * CPR + 63) / 64;
        const size_t wrow0 = (size_t)__builtin_amdgcn_readfirstlane((int)(prow - col));   // the wave's first row
        const size_t last_el = (size_t)a.Bt * a.Hq * a.N * a.kslots * D - 8;
#pragma unroll 2
        for (int j = 0; j < NI; ++j) {
            const int qc = 64 * j + lane, r = qc / CPR, c = qc % CPR;
            size_t el = wrow0 * a.kslots * D;   // padding and past the rows: any chunk in bounds
            if (r < 32 && c < 2 * CH) el = ((wrow0 + r) * a.kslots + s0 + c / CH) * D + (c % CH) * 8;
            el = el < last_el ? el : last_el;
            __builtin_amdgcn_global_load_lds((const void*)(a.part_o + el), (lds_ptr_t)(buf + j * 512), 16, 0,
                                             0);
        }
#else
        (void)lane;
#endif
        const bool in0 = ok && s0 < nfar, in1 = ok && s0 + 1 < nfar;
        const float l0 = in0 ? a.part_lse[pbase + s0] : 0.f, l1 = in1 ? a.part_lse[pbase + s0 + 1] : 0.f;
        __syncthreads();   // the loads above have landed
#pragma unroll 1
        for (int sb = 0; sb < 2; ++sb) {
            if (sb == 0 ? in0 : in1) {
                uint2 raw[T::DM][4];
#pragma unroll
                for (int mb = 0; mb < T::DM; ++mb)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        raw[mb][j] = mb * 32 + 8 * j + 4 * hh < D
                                         ? *(const uint2*)(buf + (col * CPR + sb * CH + 4 * mb + j) * 8 + 4 * hh)
                                         : make_uint2(0, 0);
                const float w = __expf((sb == 0 ? l0 : l1) - M);
                total += w;
                add_part<D>(o, w, raw, hh);
            }
        }
    }
    if (ok) rows_end<D>(a, o, M, total, z, prow, hh);
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
// FP8 (QK8): q and k arrive as OCP E4M3 and S^T = K Q^T runs on the FP8
// matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4 at twice the bf16 rate,
// unit scales; the 16 dims past a multiple of 64 on the 32x32x16 FP8 op);
// every E4M3 product is exact in the fp32 accumulator, as the bf16 products
// of the decoded values would be.  K tiles hold fp8 rows of K8S<D>() bytes.
// NEAR: 0 no block gate; 3 block gate, the near-block mask holding 32
// blocks; 1 the mask holding 64 (a window of 33..64 blocks); 2 as 1, with
// blocks smaller than the 64-key tile (B = 8, 16, 32), whose tiles get
// per-key block bits.
template <int D, int SPLIT, bool TOK, bool QK8, int NEAR = 0>
__global__ __launch_bounds__(NTHREADS, rows_waves(D, SPLIT)) void attn_rows_kernel(RowsArgs a) {
    using T = Tile<D>;
    constexpr bool ONES = T::DPAD > D;
    constexpr int VS = dma_vs<D>();
    constexpr int VELEMS = KT * VS;
    constexpr int KE = QK8 ? KT * K8S<D>() / 2 : SPLIT * T::KELEMS;   // K buffer, 16-bit units
    __shared__ __align__(16) uint16_t lds_k0[KE], lds_k1[KE];
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
        kb[p] = uniform_u64(QK8 ? (uint64_t)(a.k8 + kvoff) : (uint64_t)(a.k[p] + kvoff));
        vb[p] = uniform_u64((uint64_t)(a.v[p] + voff_src));
    }

    const int wu = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform
    const int q0 = r0 + wu * 32, q1 = min(q0 + 31, N - 1);
    const int row = q0 + col;
    const bool row_ok = row < N;
    const size_t prow = (size_t)bh * N + row;   // flat row id
    bf16x8 qf[SPLIT][QK8 ? 1 : T::DK];
    Q8Frag<D> q8f;
    if constexpr (QK8) q8f.load(a.q8 + prow * D, row_ok, hh);
    else load_q<D, SPLIT>(qf, a.q, prow * D, row_ok, hh);

    // Block-gate state of the row: its block, the kept near blocks as a bit
    // mask over (own block - 1 - bit), and the count of far blocks.
    constexpr bool WIDE = NEAR == 1 || NEAR == 2, SMALLB = NEAR == 2, GATED = NEAR != 0;
    using NearT = typename std::conditional<WIDE, uint64_t, uint32_t>::type;
    constexpr int kNear = WIDE ? 64 : 32;
    int row_blk = 0, nfar = 0;
    NearT near_bits = 0;
    if (a.gate) {
        row_blk = (row_ok ? row : N - 1) / a.B;
        if (row_ok) {
            const int32_t* sr = a.sel + prow * a.top_k;
            for (int x = 0; x < a.top_k; ++x) {
                const int cblk = sr[x];
                if (cblk < 0) break;
                const int dlt = row_blk - cblk;
                if (dlt > a.span) ++nfar;
                else if (dlt >= 1 && dlt <= kNear) near_bits |= NearT(1) << (dlt - 1);
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
    // fp8 K rows are D bytes: 16-bit units of D / 2 in the DMA's bookkeeping
    TileDma<D, QK8 ? K8S<D>() / 2 : T::KS, QK8 ? D / 2 : D> kd;
    TileDma<D, VS, VSRC> vd;
    kd.init(wu, lane);
    vd.init(wu, lane);
    auto load_k = [&](int t, uint16_t* dst) { dma_tile<D, SPLIT, KE / SPLIT>(kd, kb, N, t * KT, dst, wu); };
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
        } else if (SMALLB) {
            // blocks smaller than the tile: per-block key bits of the own
            // block and the kept near blocks
            uint32_t word = 0;
            for (int bo = 0; bo < KT / a.B; ++bo) {
                const int dlt = row_blk - (kt0 / a.B + bo);
                if (dlt == 0 || (dlt >= 1 && dlt <= a.span && dlt <= kNear &&
                                 ((near_bits >> (dlt - 1)) & 1u)))
                    word |= block_bits(a.B, bo);
            }
            mask_tile_blocks(sv, rk, wl_window, word);
        } else {
            const bool full = kt0 + KT - 1 <= q0 &&
                              ((a.window > 0 && q1 - kt0 < a.window) ||
                               (a.gate && kt0 / a.B == q0 / a.B && q1 / a.B == q0 / a.B));
            if (!full) {
                uint32_t wl = wl_window;
                if (a.gate) {
                    const int dlt = row_blk - kt0 / a.B;
                    const bool blk_ok = dlt == 0 || (dlt >= 1 && dlt <= a.span && dlt <= kNear &&
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
    if constexpr (QK8) qk_tile8<D>(lds_k0, q8f, s0, lane);
    else qk_tile<D, SPLIT>(lds_k0, qf, s0, lane);
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
        if constexpr (QK8) qk_tile8<D>(k_next, q8f, sn, lane);
        else qk_tile<D, SPLIT>(k_next, qf, sn, lane);
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

    if constexpr (GATED && !TOK && !QK8) {
        if (a.part_o) {   // far partials exist (workgroup-uniform)
            float lt = 0.f;
            if (row_ok) {
                if constexpr (ONES) lt = o[T::DM - 1][8];
                else lt = pair_sum(rs.l);
            }
            uint16_t* const buf = wu == 0 ? lds_k0 : wu == 1 ? lds_k1 : wu == 2 ? lds_v0 : lds_v1;
            static_assert((32 * (2 * (D / 8) + 1) + 63) / 64 * 512 <= KE, "a K buffer holds two slots");
            finish_rows_lds<D>(a, o, lt, rs.m, prow, h, nfar, hh, row_ok, col, lane, buf);
            return;
        }
    }
    if (row_ok) {
        float lt;
        if constexpr (ONES) lt = o[T::DM - 1][8];   // O^T row D (hh 0) or D + 4 (hh 1)
        else lt = pair_sum(rs.l);
        finish_rows<D>(a, o, lt, rs.m, prow, h, nfar, hh);
    }
}


// Largest |x| of 8 bf16 values (sign bits cleared; NaN-free compares).
__device__ __forceinline__ float absmax8(const uint4& u, float m) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        m = fmaxf(m, bf16_to_f32(w[t] & 0x7fffu));
        m = fmaxf(m, bf16_to_f32((w[t] >> 16) & 0x7fffu));
    }
    return m;
}

// 8 bf16 values times 2^-e as fp16 (exact for results in the fp16 normal
// range; ldexp is exact in fp32).
__device__ __forceinline__ uint4 f16x8_scaled(const uint4& u, int e) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    uint32_t r[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const _Float16 lo = (_Float16)ldexpf(bf16_to_f32(w[t] & 0xffffu), -e);
        const _Float16 hi = (_Float16)ldexpf(bf16_to_f32(w[t] >> 16), -e);
        r[t] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    return make_uint4(r[0], r[1], r[2], r[3]);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// 8 consecutive source values of row r as fp16 times 2^-e (exact for results
// in the fp16 normal range), and the running largest |source value| in m
// (for FP8 sources only when e = 0).
// bf16 source: widened to fp32 and scaled exactly with ldexp.  FP8 (OCP
// E4M3) source: the gfx950 conversion to fp16 with scale 2^-e (exact for
// every E4M3 code at e = 0: checked against the format's definition for all
// 256 codes).
template <bool FP8>
__device__ __forceinline__ uint4 f16x8_from(const void* x, size_t r, int D, int cc, int e,
                                            float& m) {
    if constexpr (FP8) {
        const uint2 b = *(const uint2*)((const unsigned char*)x + r * D + cc * 8);
        const float sc = ldexpf(1.f, -e);
        const f16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)b.x, sc, false);
        const f16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)b.x, sc, true);
        const f16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)b.y, sc, false);
        const f16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)b.y, sc, true);
        const uint4 u = make_uint4(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1),
                                   __builtin_bit_cast(uint32_t, h2), __builtin_bit_cast(uint32_t, h3));
        // Largest |x| from the converted values (exact at e = 0; every
        // caller that needs it converts unscaled).
        const f16x2 hs[4] = {h0, h1, h2, h3};
#pragma unroll
        for (int t = 0; t < 4; ++t)
            m = fmaxf(m, fmaxf(fabsf((float)hs[t][0]), fabsf((float)hs[t][1])));
        return u;
    } else {
        const uint4 u = *(const uint4*)((const uint16_t*)x + r * D + cc * 8);
        m = absmax8(u, m);
        return f16x8_scaled(u, e);
    }
}

// One workgroup per (chunk of kF16ChunkRows rows, head): the fp16 copy of
// the chunk (rows of D -> rows of SR, columns D .. SR-1 fp16 one) and the
// chunk's largest |x|.  Every chunk writes its maximum (no zeroing needed).
// FP8: the source is OCP E4M3, decoded exactly.
template <bool FP8>
__global__ __launch_bounds__(256) void f16_copy_kernel(const void* __restrict__ x,
                                                       uint4* __restrict__ y, float* chunk_max,
                                                       int rows, int D, int SR) {
    const int c = blockIdx.x, h = blockIdx.y, nch = gridDim.x;
    const int r0 = c * kF16ChunkRows, nr = min(kF16ChunkRows, rows - r0);
    const int cpr = SR / 8, dpr = D / 8;
    const size_t row0 = (size_t)h * rows + r0;
    float m = 0.f;
    const int n = nr * cpr;
    // Four 16-byte output pieces per thread in flight at a time.
    for (int i0 = threadIdx.x; i0 < n; i0 += 4 * 256) {
        uint4 o[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int i = i0 + t * 256;
            const int r = i / cpr, cc = i % cpr;
            o[t] = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
            if (i < n && cc < dpr) o[t] = f16x8_from<FP8>(x, row0 + r, D, cc, 0, m);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int i = i0 + t * 256;
            if (i >= n) break;
            if (y) y[(row0 + i / cpr) * cpr + i % cpr] = o[t];
        }
    }
    __shared__ float red[4];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0)
        chunk_max[(size_t)h * nch + c] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// One workgroup per group of hpg heads: the group's largest |x|, its
// exponent s, and (s != 0 only) the group's copy written again at 2^-s.
template <bool FP8>
__global__ __launch_bounds__(256) void f16_scale_kernel(const void* __restrict__ x,
                                                        uint4* __restrict__ y,
                                                        const float* __restrict__ chunk_max,
                                                        int32_t* scale, float* group_max, int hpg,
                                                        int rows, int D, int SR) {
    const int grp = blockIdx.x, nch = f16_chunks(rows);
    const float* cm = chunk_max + (size_t)grp * hpg * nch;
    float m = 0.f;
    for (int i = threadIdx.x; i < hpg * nch; i += 256) m = fmaxf(m, cm[i]);
    __shared__ float red[4];
    __shared__ int s_sh;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        const float mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        int sc = 0;
        if (mx > 0.f && mx < INFINITY && (mx < 0x1p-10f || mx >= 0x1p15f)) {
            int e;
            frexpf(mx, &e);   // mx = f 2^e, f in [0.5, 1): floor(log2 mx) = e - 1
            sc = e - 1 - 14;
        }
        s_sh = sc;
        scale[grp] = sc;
        if (group_max) group_max[grp] = mx;
    }
    __syncthreads();
    const int sc = s_sh;
    if (sc == 0 || !y) return;
    const int cpr = SR / 8, dpr = D / 8;
    const size_t row0 = (size_t)grp * hpg * rows;
    const size_t n = (size_t)hpg * rows * dpr;
    for (size_t i = threadIdx.x; i < n; i += 256) {
        const size_t r = i / dpr;
        const int cc = (int)(i % dpr);
        float unused = 0.f;
        y[(row0 + r) * cpr + cc] = f16x8_from<FP8>(x, row0 + r, D, cc, sc, unused);
    }
}

hipError_t launch_f16_copy(const void* x, bool fp8, uint16_t* y, float* chunk_max, int heads,
                           int rows, int D, int SR, hipStream_t s) {
    if (heads == 0 || rows == 0) return hipSuccess;
    const dim3 grid((unsigned)f16_chunks(rows), (unsigned)heads);
    if (fp8)
        hipLaunchKernelGGL(f16_copy_kernel<true>, grid, dim3(256), 0, s, x, (uint4*)y, chunk_max,
                           rows, D, SR);
    else
        hipLaunchKernelGGL(f16_copy_kernel<false>, grid, dim3(256), 0, s, x, (uint4*)y, chunk_max,
                           rows, D, SR);
    return hipGetLastError();
}

hipError_t launch_f16_scale(const void* x, bool fp8, uint16_t* y, const float* chunk_max,
                            int32_t* scale, int groups, int hpg, int rows, int D, int SR,
                            hipStream_t s, float* group_max) {
    if (groups == 0 || rows == 0) return hipSuccess;
    if (fp8)
        hipLaunchKernelGGL(f16_scale_kernel<true>, dim3((unsigned)groups), dim3(256), 0, s, x,
                           (uint4*)y, chunk_max, scale, group_max, hpg, rows, D, SR);
    else
        hipLaunchKernelGGL(f16_scale_kernel<false>, dim3((unsigned)groups), dim3(256), 0, s, x,
                           (uint4*)y, chunk_max, scale, group_max, hpg, rows, D, SR);
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
    if constexpr (SPLIT == 1) {
        if (a.q8) {
            if (a.tokmask)
                hipLaunchKernelGGL((attn_rows_kernel<D, 1, true, true>), dim3(grid), dim3(NTHREADS), 0, s, a);
            else
                hipLaunchKernelGGL((attn_rows_kernel<D, 1, false, true>), dim3(grid), dim3(NTHREADS), 0, s, a);
            return hipGetLastError();
        }
    }
    if (a.tokmask)
        hipLaunchKernelGGL((attn_rows_kernel<D, SPLIT, true, false>), dim3(grid), dim3(NTHREADS), 0, s, a);
    else if (a.gate && a.B < KT)
        hipLaunchKernelGGL((attn_rows_kernel<D, SPLIT, false, false, 2>), dim3(grid), dim3(NTHREADS), 0, s, a);
    else if (a.gate && a.span > 32)
        hipLaunchKernelGGL((attn_rows_kernel<D, SPLIT, false, false, 1>), dim3(grid), dim3(NTHREADS), 0, s, a);
    else if (a.gate)
        hipLaunchKernelGGL((attn_rows_kernel<D, SPLIT, false, false, 3>), dim3(grid), dim3(NTHREADS), 0, s, a);
    else
        hipLaunchKernelGGL((attn_rows_kernel<D, SPLIT, false, false>), dim3(grid), dim3(NTHREADS), 0, s, a);
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
