// sa_attn_common.hpp -- tile machinery shared by the attention kernels
// (query-centric in sa_attn.hip, KV-centric in sa_blocks.hip, compressed
// branch in sa_cmp.hip, backward in sa_bwd.hip).
//
// Every tile does S^T = K Q^T (bf16 MFMA 32x32x16, fp32 accumulation), an
// online softmax in base 2 on the VALU, and O^T += V^T P^T.  K and V tiles sit
// row-major in LDS; the V^T operand comes from the transposing LDS reads of
// gfx950 (ds_read_b64_tr_b16).  Key loops are skewed by one tile, so that the
// P V products of one tile run beside the softmax of the next.  Tiles reach
// LDS either through registers (load_tile / store_tile) or straight from
// global memory (TileDma / dma_tile, at the end of this file).
#pragma once

#include "sa_device.hpp"
#include "sa_internal.hpp"

#include <math.h>

namespace sa {

constexpr int KT = 64;                 // keys per tile
constexpr int NWAVES = 4;              // waves per workgroup
constexpr int NTHREADS = 64 * NWAVES;
constexpr int RT = 32 * NWAVES;        // query rows per workgroup
constexpr int kMaxKeyBlocks = RT / 8;  // blocks met by RT consecutive keys (smallest block: 8)

// Waves per SIMD the attention kernels ask for: three for one bf16 plane at
// head dims up to 80 (168 registers), one for split fp32 operands past 64
// (more than 256 registers), else two.
__host__ __device__ constexpr int rows_waves(int D, int SPLIT) {
    return SPLIT == 1 ? (D <= 80 ? 3 : 2) : (D >= 80 ? 1 : 2);
}

template <int D>
struct Tile {
    static constexpr int DK = D / 16;              // contraction steps of K Q^T
    static constexpr int DM = (D + 31) / 32;       // 32-row blocks of O^T
    static constexpr int DPAD = DM * 32;
    // Row strides (elements) of the K and V tiles in LDS, both row-major
    // [key][dim].  K rows are read 16 bytes per lane by 32 consecutive keys:
    // D + 8 puts those reads on distinct banks.  V rows are read by the
    // transposing LDS loads, 4 keys x 32 bytes per 16-lane group: a stride of
    // 8 (mod 32) dwords keeps the 4 rows on distinct banks.
    static constexpr int KS = D + 8;
    static constexpr int VS = D == 128 ? 144 : 80;
    static constexpr int KELEMS = KT * KS;
    static constexpr int VELEMS = KT * VS;
    static constexpr int CHUNKS = KT * D / 8;      // 16-byte pieces of a tile
    static constexpr int CPT = (CHUNKS + NTHREADS - 1) / NTHREADS;
};

// Registers holding one K or V tile between its global load and LDS store.
template <int D, int SPLIT>
struct Stage {
    uint4 x[SPLIT][Tile<D>::CPT];
};

// Source of the K or V tiles of one head ([N, D] 16-bit planes) and this
// thread's byte offsets within a 64-key tile.  Each tile load builds a
// buffer descriptor in scalar registers whose base is the tile's first key
// and whose size is what is left of the head, so a tile costs scalar work
// only; keys at or past N fall outside the descriptor and read as zero
// (finite data that causality always masks).  Threads past the last chunk
// repeat it (they later write the same bytes to the same LDS address).
template <int D, int SPLIT>
struct TileSrc {
    uint64_t base[SPLIT];   // byte addresses, workgroup-uniform
    int N;
    int off[Tile<D>::CPT];
};

__device__ __forceinline__ uint64_t uniform_u64(uint64_t u) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    return ((uint64_t)hi << 32) | (uint64_t)lo;
}

template <int D, int SPLIT>
__device__ __forceinline__ TileSrc<D, SPLIT> tile_src(const uint16_t* const* base, int N, int tid) {
    using T = Tile<D>;
    TileSrc<D, SPLIT> ts;
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) ts.base[p] = uniform_u64((uint64_t)base[p]);
    ts.N = N;
#pragma unroll
    for (int c = 0; c < T::CPT; ++c) {
        const int idx = min(tid + c * NTHREADS, T::CHUNKS - 1);
        ts.off[c] = ((idx / (D / 8)) * D + (idx % (D / 8)) * 8) * 2;
    }
    return ts;
}

// Global -> registers for the 64-key tile starting at key kt0 (K or V);
// requires 0 <= kt0 < N.
template <int D, int SPLIT>
__device__ __forceinline__ void load_tile(Stage<D, SPLIT>& st, const TileSrc<D, SPLIT>& ts, int kt0) {
    using T = Tile<D>;
    const int k0 = __builtin_amdgcn_readfirstlane(kt0);   // wave-uniform
    const int bytes = (ts.N - k0) * D * 2;
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(ts.base[p] + (uint64_t)k0 * D * 2), (short)0, bytes, 0x00020000);
#pragma unroll
        for (int c = 0; c < T::CPT; ++c)
            st.x[p][c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, ts.off[c], 0, 0));
    }
}

// Registers -> LDS, row-major with row stride STRIDE; planes PLANE apart.
template <int D, int SPLIT, int STRIDE, int PLANE>
__device__ __forceinline__ void store_tile(const Stage<D, SPLIT>& st, uint16_t* dst, int tid) {
    using T = Tile<D>;
#pragma unroll
    for (int p = 0; p < SPLIT; ++p)
#pragma unroll
        for (int c = 0; c < T::CPT; ++c) {
            const int idx = min(tid + c * NTHREADS, T::CHUNKS - 1);
            const int row = idx / (D / 8), col = idx % (D / 8);
            *(uint4*)(dst + p * PLANE + row * STRIDE + col * 8) = st.x[p][c];
        }
}

// Before the key loop: V buffer 1 is read by the first iteration's P V,
// whose P is zero; it is zeroed so no stale LDS bits (possibly NaN) meet it.
template <int D, int SPLIT>
__device__ __forceinline__ void zero_v_init(uint16_t* vs, int tid) {
    using T = Tile<D>;
    uint32_t* b1 = (uint32_t*)(vs + SPLIT * T::VELEMS);
    for (int x = tid; x < SPLIT * T::VELEMS / 2; x += NTHREADS) b1[x] = 0u;
}

// Softmax state of one query row in one lane (the lane pair l, l^32 shares
// the row and keeps the same m).
struct RowState {
    float m;      // exponent base, raw dot-product units; lags the running max
                  // by less than kLazy / c (rescaling is deferred until then)
    float l;      // this lane's partial sum of exp2((s - m) c)
    float alpha;  // pending rescale of O from the last softmax
    bool need;    // alpha != 1 for this row
};

// Rescale the accumulators only when the row max grew by more than 2^8 in
// the exponent: until then exp2((s - m) c) <= 256, harmless in fp32 and bf16,
// and the final normalisation uses the same base.
constexpr float kLazy = 8.f;

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// v_permlane32_swap gives every lane the pair {x of lane l%32, x of lane
// l%32+32}, lower lane first, so both lanes of a row compute the same value.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float tree_max32(const f32x16& x, const f32x16& y) {
    float t[11];
#pragma unroll
    for (int i = 0; i < 5; ++i) t[i] = max3f(x[3 * i], x[3 * i + 1], x[3 * i + 2]);
    t[5] = max3f(x[15], y[0], y[1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) t[6 + i] = max3f(y[2 + 3 * i], y[3 + 3 * i], y[4 + 3 * i]);
    t[10] = fmaxf(y[14], y[15]);
    const float u0 = max3f(t[0], t[1], t[2]), u1 = max3f(t[3], t[4], t[5]);
    const float u2 = max3f(t[6], t[7], t[8]), u3 = fmaxf(t[9], t[10]);
    return fmaxf(max3f(u0, u1, u2), u3);
}

__device__ __forceinline__ float tree_sum32(const float (&p)[2][16]) {
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = p[0][i] + p[1][i];
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) t[i] += t[i + w];
    return t[0];
}

// S^T tile (64 keys x 32 queries) of one wave: s[sub] covers keys
// sub*32 .. sub*32+31; the two halves are interleaved so consecutive
// matrix-core ops are independent.
template <int D, int SPLIT>
__device__ __forceinline__ void qk_tile(const uint16_t* ks, const bf16x8 (&qf)[SPLIT][Tile<D>::DK],
                                        f32x16 (&s)[2], int lane) {
    using T = Tile<D>;
    const int col = lane & 31, hh = lane >> 5;
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int k_ = 0; k_ < T::DK; ++k_)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int off = (sub * 32 + col) * T::KS + k_ * 16 + 8 * hh;
            const bf16x8 a = *(const bf16x8*)(ks + off);
            s[sub] = mfma32(a, qf[0][k_], s[sub]);
            if constexpr (SPLIT == 2) {
                s[sub] = mfma32(a, qf[1][k_], s[sub]);
                s[sub] = mfma32(*(const bf16x8*)(ks + T::KELEMS + off), qf[0][k_], s[sub]);
            }
        }
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// 4 keys x 1 dim per lane from row-major V (ds_read_b64_tr_b16): within each
// 16-lane group, lane i receives the i%4-th 16-bit column of the 8 bytes
// addressed by lanes 4r + i/4, r = 0..3.
__device__ __forceinline__ v4i16 read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
}

// Per-lane offset (elements) into a V tile of row stride VS for the V^T
// operand of O^T row block mb: lane group G = lane/16 covers dims mb*32 +
// 16*(G%2) .. +15 and key half h = G/2; source lane 4r + q of the group
// points at key 4h + r, dims +4q, so lane i of the group receives keys
// 4h..4h+3 of dim +i.  Dims past D (padding rows of O^T) read dim 0 and are
// discarded, or, with PAD_READ, read their own columns (which then must exist
// in the tile: the row-sum columns of the query-centric kernel).
template <int D, int VS = Tile<D>::VS, bool PAD_READ = false>
__device__ __forceinline__ int v_lane_offset(int lane, int mb) {
    const int j = lane & 15, r = j >> 2, q = j & 3, G = lane >> 4, h = G >> 1;
    int dim = mb * 32 + 16 * (G & 1) + 4 * q;
    if (!PAD_READ && dim >= D) dim = 0;
    return (4 * h + r) * VS + dim;
}

// O^T += V^T P^T for one tile.  For contraction step kk (keys 16kk..16kk+15)
// lane half h feeds keys {4h..4h+3, 8+4h..8+4h+3}: two transposing reads.
// bf16 inputs: V (converted once) and P are fp16 -- P keeps 11 significant
// bits, which the few-key rows need to stay within the output tolerance.
// fp32 inputs: hi/lo bf16 splits of V and P, three products.
//
// ONES (head dims with padding rows in O^T): lanes with pad set (the padding
// dims of the last row block) take constant ones (zero in the low plane)
// instead of what they read, so those rows of O^T accumulate the row sums of
// P.  Their reads must stay inside the tile.
template <int D, int SPLIT, int VS = Tile<D>::VS, bool ONES = false>
__device__ __forceinline__ void pv_tile(const uint16_t* vs, const uint4 (&pb)[4],
                                        const uint4 (&pl)[4], f32x16 (&o)[Tile<D>::DM],
                                        const int (&voff)[Tile<D>::DM], bool pad = false) {
    using T = Tile<D>;
    constexpr int VELEMS = KT * VS;
    constexpr uint32_t one2 = SPLIT == 1 ? 0x3C003C00u : 0x3F803F80u;   // fp16 / bf16 1.0 pairs
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int mb = 0; mb < T::DM; ++mb) {
            const uint16_t* p0 = vs + voff[mb] + 16 * kk * VS;
            const v4i16 lo = read_tr(p0), hi = read_tr(p0 + 8 * VS);
            uint4 u = __builtin_bit_cast(uint4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            if (ONES && mb == T::DM - 1) {
                u.x = pad ? one2 : u.x;
                u.y = pad ? one2 : u.y;
                u.z = pad ? one2 : u.z;
                u.w = pad ? one2 : u.w;
            }
            if constexpr (SPLIT == 1) {
                o[mb] = mfma32_f16(__builtin_bit_cast(f16x8, u), __builtin_bit_cast(f16x8, pb[kk]),
                                   o[mb]);
            } else {
                const bf16x8 a = __builtin_bit_cast(bf16x8, u);
                const v4i16 lo2 = read_tr(p0 + VELEMS), hi2 = read_tr(p0 + VELEMS + 8 * VS);
                uint4 u2 = __builtin_bit_cast(uint4, __builtin_shufflevector(lo2, hi2, 0, 1, 2, 3, 4, 5, 6, 7));
                if (ONES && mb == T::DM - 1) {
                    u2.x = pad ? 0u : u2.x;
                    u2.y = pad ? 0u : u2.y;
                    u2.z = pad ? 0u : u2.z;
                    u2.w = pad ? 0u : u2.w;
                }
                const bf16x8 a2 = __builtin_bit_cast(bf16x8, u2);
                o[mb] = mfma32(a, __builtin_bit_cast(bf16x8, pb[kk]), o[mb]);
                o[mb] = mfma32(a, __builtin_bit_cast(bf16x8, pl[kk]), o[mb]);
                o[mb] = mfma32(a2, __builtin_bit_cast(bf16x8, pb[kk]), o[mb]);
            }
        }
}

// Mask of an S^T tile: key j stays for this lane's row i iff
// (unsigned)(i - j) < wl: wl = 2^31 keeps every causal key (an attended
// block), wl = w the window.  rk = i - kt0 - 4*(lane/32), so i - j = rk - (a
// constant of the accumulator register).
//
// Online softmax of the tile: produces the bf16 operand P (and its low part
// for split fp32 operands) and leaves in st the factor by which O must be
// rescaled once the previous tile's P V is in.
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int rk, uint32_t wl) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int cv = sub * 32 + 8 * (v >> 2) + (v & 3);
            if ((uint32_t)(rk - cv) >= wl) s[sub][v] = -INFINITY;
        }
}

// Token-gate mask of an S^T tile: key j stays iff its bit is set in this
// lane's mask word (bit 16*sub + v for register v of half sub) or, on tiles
// that meet a window, it passes the same unsigned window test as mask_tile.
__device__ __forceinline__ void mask_tile_tok(f32x16 (&s)[2], int rk, uint32_t wl, bool window,
                                              uint32_t word) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            bool keep = (word >> (16 * sub + v)) & 1u;
            if (window) {
                const int cv = sub * 32 + 8 * (v >> 2) + (v & 3);
                keep = keep || (uint32_t)(rk - cv) < wl;
            }
            if (!keep) s[sub][v] = -INFINITY;
        }
}

// Block-gate mask of an S^T tile with blocks smaller than the tile: key j
// stays iff it is causal (j <= i) and either its bit is set in this lane's
// word (bit 16*sub + v for register v of half sub: the key's block is the
// row's own block or a kept near block) or it passes the window test.
__device__ __forceinline__ void mask_tile_blocks(f32x16 (&s)[2], int rk, uint32_t wl, uint32_t word) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int cv = sub * 32 + 8 * (v >> 2) + (v & 3);
            const int dif = rk - cv;   // i - j
            const bool keep = dif >= 0 && (((word >> (16 * sub + v)) & 1u) || (uint32_t)dif < wl);
            if (!keep) s[sub][v] = -INFINITY;
        }
}

// This lane's key bits of one block of a tile when blocks are smaller than
// the tile: for block size B in {8, 16, 32}, the lane's keys of block bo
// (key offsets 32 sub + 8 (v/4) + v%4 + 4 (lane/32)) are bits
// B/2 * bo .. B/2 * (bo + 1) - 1 of the word.
__device__ __forceinline__ uint32_t block_bits(int B, int bo) {
    const int w = B / 2;
    return (w >= 32 ? 0xffffffffu : ((1u << w) - 1u)) << (w * bo);
}

// Row max of an S^T tile (both lanes of a row get it).
__device__ __forceinline__ float tile_max(const f32x16 (&s)[2]) {
    return pair_max(tree_max32(s[0], s[1]));
}

// Max phase of the online softmax of a tile: the new exponent base and the
// pending rescale factor.
__device__ __forceinline__ void max_tile(const f32x16 (&s)[2], RowState& st, float c) {
    const float mx = tile_max(s);
    // NaN-free test: true while m is still -inf and mx is finite; false when
    // both are -inf (a fully masked tile before the row's first key).
    st.need = mx > st.m + kLazy / c;
    st.alpha = st.need ? fast_exp2((st.m - mx) * c) : 1.f;
    st.m = st.need ? mx : st.m;
}

// Exp phase: P = exp2((s - m) c) as the P V operand(s), and (LSUM) the row
// sum, rescaled by the pending factor.  Without LSUM the caller gets the row
// sum elsewhere (from constant-one rows of V^T).
template <int SPLIT, bool LSUM = true>
__device__ __forceinline__ void exp_tile(const f32x16 (&s)[2], RowState& st, float c,
                                         uint4 (&pb)[4], uint4 (&pl)[4]) {
    const float nb = st.m == -INFINITY ? 0.f : -st.m * c;
    float p[2][16];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 16; ++v) p[sub][v] = fast_exp2(fmaf(s[sub][v], c, nb));
    if constexpr (LSUM) st.l = fmaf(st.l, st.alpha, tree_sum32(p));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const float* pk = &p[kk >> 1][8 * (kk & 1)];
        if constexpr (SPLIT == 1) {
            pb[kk] = __builtin_bit_cast(uint4, to_f16x8(pk));
        } else {
            const bf16x8 hb = to_bf16x8(pk);
            float r[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) r[t] = pk[t] - (float)hb[t];
            pb[kk] = __builtin_bit_cast(uint4, hb);
            pl[kk] = __builtin_bit_cast(uint4, to_bf16x8(r));
        }
    }
}

template <int SPLIT>
__device__ __forceinline__ void softmax_tile(const f32x16 (&s)[2], RowState& st, float c,
                                             uint4 (&pb)[4], uint4 (&pl)[4]) {
    max_tile(s, st, c);
    exp_tile<SPLIT>(s, st, c, pb, pl);
}

// Rescale O by the factor the last softmax left pending (rare: only when a
// row max grew past the lazy threshold).
template <int D>
__device__ __forceinline__ void apply_rescale(f32x16 (&o)[Tile<D>::DM], RowState& st) {
    if (__any(st.need)) {
#pragma unroll
        for (int mb = 0; mb < Tile<D>::DM; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[mb][v] *= st.alpha;
    }
    st.need = false;
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

// ---------------------------------------------------------------------------
// Direct global -> LDS tiles and key-loop helpers of the attention kernels.
// ---------------------------------------------------------------------------

// Masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008, kSchedDSRead = 0x100;

// An empty asm that reads x: its computation stays before this point (the
// compiler would otherwise sink the softmax of a key-loop step past the
// step's closing barrier, next to its only use in the following step, where
// nothing runs beside it on the matrix cores).
__device__ __forceinline__ void pin(const uint4& x) {
    asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Direct global -> LDS loads of a 64-key tile (buffer_load ... lds, 16 bytes
// per lane) into an LDS image with row stride S elements: instruction i
// writes LDS bytes 1024 i .. 1024 i + 1023 of the image, lane l the 16-byte
// chunk p = 64 i + l = row * (S / 8) + c.  Chunks past the row's D elements
// (padding, never read) get a copy of the row's last chunk, so every lane
// loads and no lane masking is needed.  The S / 8 instructions of a plane are
// dealt round-robin to the waves; where they do not divide evenly, the waves
// past the last one repeat it (the same bytes to the same LDS address), so
// every wave issues the same count with no branches.
//
// SRC is the source's row stride (elements, >= D): columns D .. SRC-1 of a
// source row are copied too (up to the image's row length).
template <int D, int S, int SRC = D>
struct TileDma {
    static constexpr int NI = S / 8;                           // instructions per plane
    static constexpr int PER = (NI + NWAVES - 1) / NWAVES;     // per wave
    static constexpr int ROW = SRC;                            // source row stride
    int voff[PER];   // byte offset of this lane's chunk from the tile's first key
    __device__ __forceinline__ static int inst(int wave, int j) { return min(wave + NWAVES * j, NI - 1); }
    __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int p = 64 * inst(wave, j) + lane, row = p / NI, c = min(p % NI, SRC / 8 - 1);
            voff[j] = (row * SRC + c * 8) * 2;
        }
    }
};

// Issue the loads of the tile starting at key kt0 (0 <= kt0 < N) of SPLIT
// [N, TD::ROW] planes (byte addresses base[]) into lds (planes PLANE elements
// apart).  Keys at or past N fall outside the buffer descriptor and load
// zero (finite data that causality always masks).  Completion is awaited
// with the memory counter (the barrier at the end of a step).
template <int D, int SPLIT, int PLANE, class TD>
__device__ __forceinline__ void dma_tile(const TD& td, const uint64_t* base, int N, int kt0,
                                         uint16_t* lds, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass rejects the LDS-pointer builtin
    const int k0 = __builtin_amdgcn_readfirstlane(kt0);
    const int bytes = (N - k0) * TD::ROW * 2;
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(base[p] + (uint64_t)k0 * TD::ROW * 2), (short)0, bytes, 0x00020000);
#pragma unroll
        for (int j = 0; j < TD::PER; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (lds_ptr_t)(lds + p * PLANE + TD::inst(wave, j) * 512), 16, td.voff[j], 0, 0, 0);
    }
#else
    (void)td; (void)base; (void)N; (void)kt0; (void)lds; (void)wave;
#endif
}

// V row stride of the directly loaded tiles: measured fastest for the
// transposing reads of the P V operand on gfx950 (96 at d 80, 160 at d 128:
// 11 % and 18 % faster than 80 and 144; 120 and 128 are twice as slow).  At
// d 80 the columns past D feed the padding rows of O^T.
template <int D>
__host__ __device__ constexpr int dma_vs() {
    return D == 80 ? 96 : D == 128 ? 160 : Tile<D>::VS;
}

// ---------------------------------------------------------------------------
// FP8 (OCP E4M3) K Q^T.
// ---------------------------------------------------------------------------
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Row stride (bytes) of an fp8 K tile in LDS: 32 lanes read 16 bytes at
// keys 32 apart; a stride of 20 dwords (80 bytes) or 36 (144) puts those
// reads on distinct banks (128-byte rows would not).
template <int D>
__host__ __device__ constexpr int K8S() { return D == 128 ? 144 : 80; }

// One query row's fp8 fragments as the B operand of S^T = K Q^T: per 64 dims
// the 32 bytes 32*(lane/32) .. +31 (32x32x64 op), and for D = 80 the 8 bytes
// of dims 64 + 8*(lane/32) .. +7 (32x32x16 op).  Lane l supplies column l % 32.
template <int D>
struct Q8Frag {
    static constexpr int NB = D / 64;          // 32x32x64 steps
    static constexpr bool TAIL = D % 64 == 16; // one 32x32x16 step
    i32x8 b[NB > 0 ? NB : 1];
    long t;
    __device__ __forceinline__ void load(const uint8_t* row, bool ok, int hh) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
            if (ok) {
                lo = *(const uint4*)(row + 64 * j + 32 * hh);
                hi = *(const uint4*)(row + 64 * j + 32 * hh + 16);
            }
            b[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
                         (int)hi.w};
        }
        t = 0;
        if constexpr (TAIL) {
            if (ok) t = *(const long*)(row + 64 * NB + 8 * hh);
        }
    }
};

// S^T tile (64 keys x 32 queries) of one wave from an fp8 K tile.
template <int D>
__device__ __forceinline__ void qk_tile8(const uint16_t* ks, const Q8Frag<D>& qf, f32x16 (&s)[2],
                                         int lane) {
    constexpr int S8 = K8S<D>();
    const int col = lane & 31, hh = lane >> 5;
    const uint8_t* kb = (const uint8_t*)ks;
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int j = 0; j < Q8Frag<D>::NB; ++j)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const uint8_t* p = kb + (sub * 32 + col) * S8 + 64 * j + 32 * hh;
            const uint4 lo = *(const uint4*)p, hi = *(const uint4*)(p + 16);
            const i32x8 av = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                              (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            s[sub] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qf.b[j], s[sub], 0, 0, 0, 127,
                                                                     0, 127);
        }
    if constexpr (Q8Frag<D>::TAIL) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const long av = *(const long*)(kb + (sub * 32 + col) * S8 + 64 * Q8Frag<D>::NB + 8 * hh);
            s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(av, qf.t, s[sub], 0, 0, 0);
        }
    }
}

template <int V>
struct Par {
    static constexpr int value = V;
};

}  // namespace sa
