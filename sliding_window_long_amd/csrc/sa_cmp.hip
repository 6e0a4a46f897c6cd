// sa_cmp.hip -- compressed-KV branch: compression of K and V into group
// means, and the attention of every query over the compressed keys it may
// see, merged into the result of the other branches.
//
// [BORA model card, NSA]: eight tokens become one compressed key and value,
// next to the top-k block selection and the sliding window.  Readings taken
// (the pages give neither the compression function nor the combination):
//   * compressed key / value of group c = the mean of the keys / values of
//     tokens cC .. cC+C-1 (complete groups only);
//   * query i sees group c iff (c+1)C - 1 <= i;
//   * each visible group is one more column of the same softmax as the
//     window / block / sink columns.
// The query-centric kernel (sa_attn.hip) leaves its normalised fp32 output
// and lse; attn_cmp_kernel attends the compressed columns and merges the two
// parts by their lse:
//   M = max(lse_r, lse_c),  w_r = e^(lse_r - M),  w_c = e^(lse_c - M),
//   out = (w_r out_r + w_c out_c) / (w_r + w_c),  lse = M + ln(w_r + w_c).
#include "sa_attn_common.hpp"

namespace sa {

// ---------------------------------------------------------------------------
// Compression: one thread per 8 consecutive dims of one (batch, kv head,
// group) row of K and of V.
// ---------------------------------------------------------------------------
template <bool F32IN>
__device__ __forceinline__ void load8(const void* p, size_t i, float (&x)[8]) {
    if constexpr (F32IN) {
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

// 8 values as one 16-byte chunk of bf16 (hi, or lo = x - hi) or fp16.
__device__ __forceinline__ uint4 pack_bf16(const float (&x)[8], bool lo) {
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float a = x[2 * t], b = x[2 * t + 1];
        if (lo) {
            a -= (float)(__bf16)a;
            b -= (float)(__bf16)b;
        }
        w[t] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint4 pack_f16(const float (&x)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        w[t] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x[2 * t]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x[2 * t + 1]) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

template <bool F32IN>
__global__ __launch_bounds__(256) void cmp_pool_kernel(CmpPoolArgs a) {
    const size_t oct = (size_t)a.D / 8;
    const size_t total = (size_t)a.lists * a.Nc * oct;
    const size_t x = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (x >= total) return;
    const size_t row = x / oct, e0 = (x % oct) * 8;     // row = (b*Hkv + g)*Nc + c
    const size_t bg = row / a.Nc, c = row % a.Nc;
    const size_t src = (bg * a.N + c * a.C) * a.D + e0;
    float sk[8] = {0, 0, 0, 0, 0, 0, 0, 0}, sv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < a.C; ++j) {
        float xk[8], xv[8];
        load8<F32IN>(a.k, src + (size_t)j * a.D, xk);
        load8<F32IN>(a.v, src + (size_t)j * a.D, xv);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            sk[t] += xk[t];
            sv[t] += xv[t];
        }
    }
    const float inv = 1.f / (float)a.C;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        sk[t] *= inv;
        sv[t] *= inv;
    }
    const size_t o = row * a.D + e0;
    *(uint4*)(a.kc[0] + o) = pack_bf16(sk, false);
    if (!F32IN && a.bwd) {   // backward operands: bf16 V, and the bf16 K means as scaled fp16
        *(uint4*)(a.vc[0] + o) = pack_bf16(sv, false);
        const int e = a.kscale[bg];
        float kr[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) kr[t] = ldexpf((float)(__bf16)sk[t], -e);
        *(uint4*)(a.kc[1] + o) = pack_f16(kr);
        return;
    }
    if constexpr (F32IN) {   // split operands: hi and lo bf16 terms of K and V
        *(uint4*)(a.kc[1] + o) = pack_bf16(sk, true);
        *(uint4*)(a.vc[0] + o) = pack_bf16(sv, false);
        *(uint4*)(a.vc[1] + o) = pack_bf16(sv, true);
    } else {                 // bf16 K, fp16 V as in the other kernels' P V
        // the V copy's power-of-two scale of this (batch, kv head)
        if (a.vscale) {
            const int e = a.vscale[bg];
#pragma unroll
            for (int t = 0; t < 8; ++t) sv[t] = ldexpf(sv[t], -e);
        }
        *(uint4*)(a.vc[0] + o) = pack_f16(sv);
    }
}

hipError_t launch_cmp_pool(const CmpPoolArgs& a, bool f32_in, hipStream_t s) {
    const size_t total = (size_t)a.lists * a.Nc * (a.D / 8);
    if (total == 0) return hipSuccess;
    const unsigned grid = (unsigned)((total + 255) / 256);
    if (f32_in)
        hipLaunchKernelGGL(cmp_pool_kernel<true>, dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(cmp_pool_kernel<false>, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Attention over the compressed columns and the merge.  A workgroup owns 128
// consecutive query rows of one (batch, head); in compressed coordinates
// row i's last visible group is i' = (i+1)/C - 1, a causal mask.
// ---------------------------------------------------------------------------
template <int D, int SPLIT>
struct CmpSmem {
    static constexpr int BYTES = 2 * SPLIT * (Tile<D>::KELEMS + Tile<D>::VELEMS) * 2;
};

template <int D, int SPLIT>
__global__ __launch_bounds__(NTHREADS, SPLIT == 2 && D >= 80 ? 1 : 2) void attn_cmp_kernel(CmpArgs a) {
    using T = Tile<D>;
    __shared__ __align__(16) uint8_t smem[CmpSmem<D, SPLIT>::BYTES];
    uint16_t* const lds_k = (uint16_t*)smem;                  // [2][SPLIT * KELEMS]
    uint16_t* const lds_v = lds_k + 2 * SPLIT * T::KELEMS;    // [2][SPLIT * VELEMS]
    auto kbuf = [&](int i) { return lds_k + i * (SPLIT * T::KELEMS); };
    auto vbuf = [&](int i) { return lds_v + i * (SPLIT * T::VELEMS); };

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int N = a.N, C = a.C;
    const int ntiles = (N + RT - 1) / RT;
    const int bh = blockIdx.x / ntiles, rtile = blockIdx.x % ntiles;
    const int b = bh / a.Hq, h = bh % a.Hq, g = h / (a.Hq / a.Hkv);
    const int r0 = rtile * RT;
    const int q0 = r0 + __builtin_amdgcn_readfirstlane(wave) * 32;
    const int row = q0 + col;
    const bool ok = row < N;
    const size_t prow = (size_t)bh * N + (ok ? row : 0);
    const int ip = (min(row, N - 1) + 1) / C - 1;                    // last visible group
    const int ip_lo = (min(q0, N - 1) + 1) / C - 1;                  // of the wave's first row
    const int r_hi = min(r0 + RT - 1, N - 1);
    const int t_end = ((r_hi + 1) / C - 1) >= 0 ? ((r_hi + 1) / C - 1) / KT : -1;

    bf16x8 qf[SPLIT][T::DK];
    load_q<D, SPLIT>(qf, a.q, prow * D, ok, hh);
    f32x16 o[T::DM];
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb) o[mb] = f32x16{};
    RowState rs{-INFINITY, 0.f, 1.f, false};

    if (t_end >= 0) {   // workgroup-uniform: some row sees a group
        const size_t kvoff = (size_t)(b * a.Hkv + g) * a.Nc * D;
        const uint16_t* kp[2] = {a.kc[0] + kvoff, SPLIT == 2 ? a.kc[1] + kvoff : nullptr};
        const uint16_t* vp[2] = {a.vc[0] + kvoff, SPLIT == 2 ? a.vc[1] + kvoff : nullptr};
        const float c = a.scale * kLog2e;
        zero_v_init<D, SPLIT>(lds_v, tid);
        uint4 pb[4], pl[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) pb[kk] = pl[kk] = make_uint4(0, 0, 0, 0);
        int voff[T::DM];
#pragma unroll
        for (int mb = 0; mb < T::DM; ++mb) voff[mb] = v_lane_offset<D>(lane, mb);
        Stage<D, SPLIT> kst, vst;
        const TileSrc<D, SPLIT> ksrc = tile_src<D, SPLIT>(kp, a.Nc, tid);
        const TileSrc<D, SPLIT> vsrc = tile_src<D, SPLIT>(vp, a.Nc, tid);
        load_tile<D, SPLIT>(kst, ksrc, 0);
        store_tile<D, SPLIT, T::KS, T::KELEMS>(kst, kbuf(0), tid);
        __syncthreads();
        for (int t = 0; t <= t_end; ++t) {
            load_tile<D, SPLIT>(kst, ksrc, min(t + 1, t_end) * KT);
            load_tile<D, SPLIT>(vst, vsrc, t * KT);
            apply_rescale<D>(o, rs);
            f32x16 sv[2];
            qk_tile<D, SPLIT>(kbuf(t & 1), qf, sv, lane);
            const int kt0 = t * KT;
            if (kt0 + KT - 1 > ip_lo) mask_tile(sv, ip - kt0 - 4 * hh, 0x80000000u);
            pv_tile<D, SPLIT>(vbuf((t + 1) & 1), pb, pl, o, voff);
            softmax_tile<SPLIT>(sv, rs, c, pb, pl);
            store_tile<D, SPLIT, T::KS, T::KELEMS>(kst, kbuf((t + 1) & 1), tid);
            store_tile<D, SPLIT, T::VS, T::VELEMS>(vst, vbuf(t & 1), tid);
            __syncthreads();
        }
        apply_rescale<D>(o, rs);
        pv_tile<D, SPLIT>(vbuf(t_end & 1), pb, pl, o, voff);
    }
    if (!ok) return;

    // Merge with the other branches' normalised fp32 result (out_r, lse_r).
    const float lt = pair_sum(rs.l);
    const float lse_c = lt > 0.f ? rs.m * a.scale + kLn2 * fast_log2(lt) : -INFINITY;
    const float lse_r = a.lse[prow];
    const float M = fmaxf(lse_r, lse_c);
    const float wr = __expf(lse_r - M);
    const float wc = lt > 0.f ? __expf(lse_c - M) : 0.f;
    const float inv = 1.f / (wr + wc);
    const float fc = lt > 0.f ? wc * inv / lt : 0.f, fr = wr * inv;
    // the compressed values were taken in units of 2^vs
    const int vs = a.vscale ? a.vscale[prow / a.N / (a.Hq / a.Hkv)] : 0;
#pragma unroll
    for (int mb = 0; mb < T::DM; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d0 = mb * 32 + 8 * j + 4 * hh;
            if (d0 < D) {
                const float4 r = *(const float4*)(a.out_r + prow * D + d0);
                const float v0 = fr * r.x + ldexpf(fc * o[mb][4 * j], vs);
                const float v1 = fr * r.y + ldexpf(fc * o[mb][4 * j + 1], vs);
                const float v2 = fr * r.z + ldexpf(fc * o[mb][4 * j + 2], vs);
                const float v3 = fr * r.w + ldexpf(fc * o[mb][4 * j + 3], vs);
                if (a.out_f32) {
                    *(float4*)((float*)a.out + prow * D + d0) = make_float4(v0, v1, v2, v3);
                } else {
                    __bf16 rr[4] = {(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
                    *(uint2*)((uint16_t*)a.out + prow * D + d0) = *(const uint2*)rr;
                }
            }
        }
    if (hh == 0) a.lse[prow] = M + kLn2 * fast_log2(wr + wc);
}

template <int D, int SPLIT>
static hipError_t cmp_d(const CmpArgs& a, hipStream_t s) {
    const int grid = (a.N + RT - 1) / RT * a.Bt * a.Hq;
    hipLaunchKernelGGL((attn_cmp_kernel<D, SPLIT>), dim3(grid), dim3(NTHREADS), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_cmp(const CmpArgs& a, int head_dim, int split, hipStream_t s) {
    if (split == 1) {
        if (head_dim == 64) return cmp_d<64, 1>(a, s);
        if (head_dim == 80) return cmp_d<80, 1>(a, s);
        if (head_dim == 128) return cmp_d<128, 1>(a, s);
    } else {
        if (head_dim == 64) return cmp_d<64, 2>(a, s);
        if (head_dim == 80) return cmp_d<80, 2>(a, s);
        if (head_dim == 128) return cmp_d<128, 2>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace sa
