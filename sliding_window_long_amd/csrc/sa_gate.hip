// sa_gate.hip -- block mean-pool and block gate (score GEMM + top-k).
//
// Block gate [MoBA summary page, "블록 분할과 top-k 게이팅" and "인과성
// 보존"]: every key block c is summarised by the mean of its B keys; query i
// of block b scores each earlier block by <q_i, mean_c> (no scale), keeps its
// own block plus the min(top_k-1, b) best earlier ones (ties toward the
// lower block id), and never sees a later block.
//
// Accuracy: the pooled keys are split into bf16 terms so the score GEMM runs
// on bf16 matrix cores with fp32 accumulation -- a single bf16 rounding of
// the mean (2^-9 relative) would flip selections whose top-k margin is far
// larger than the accepted tolerance.  For bf16 queries two terms (mean = hi
// + lo to about 17 bits) match what the order key keeps of a score (its
// low idx_bits carry the block index: 23 - idx_bits mantissa bits); fp32
// queries take three (hi + mid + lo, about 24 bits).  This is the bf16x3
// splitting of Henry, Tang and Heinecke (ARITH 2019).
//
// Top-k: each lane owns one query row (lane pair l, l^32 split the blocks),
// packs every score into a 32-bit key that orders like the float and breaks
// ties toward the lower block id (the low idx_bits of the mantissa are
// replaced by (mask - c), costing 2^-(23-idx_bits) of relative precision),
// and keeps a sorted top-M list in registers with a max/min insertion chain.
#include <type_traits>

#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

// ---------------------------------------------------------------------------
// Pool: one workgroup per (batch, kv head, block).  MM = false: the mean of
// the block's keys; MM = true: their per-dimension min and max [MoBA summary
// page, the remark on Quest's min/max-pooled block representation].
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split2(float x, uint16_t* dst, size_t plane, size_t o) {
    const __bf16 hi = (__bf16)x;
    const __bf16 lo = (__bf16)(x - (float)hi);
    dst[o] = __builtin_bit_cast(uint16_t, hi);
    dst[plane + o] = __builtin_bit_cast(uint16_t, lo);
}

__device__ __forceinline__ void split3(float x, uint16_t* dst, size_t plane, size_t o) {
    const __bf16 hi = (__bf16)x;
    const float r1 = x - (float)hi;
    const __bf16 mid = (__bf16)r1;
    const __bf16 lo = (__bf16)(r1 - (float)mid);
    dst[o] = __builtin_bit_cast(uint16_t, hi);
    dst[plane + o] = __builtin_bit_cast(uint16_t, mid);
    dst[2 * plane + o] = __builtin_bit_cast(uint16_t, lo);
}

template <int D, bool F32IN, bool MM>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
    constexpr int OCT = D / 8;            // 8-element column groups
    constexpr int NG = 256 / OCT;         // row groups
    constexpr int NR = MM ? 2 : 1;        // reductions: sum, or min and max
    __shared__ float red[NR][NG * D];
    const int tid = threadIdx.x;
    const int list = blockIdx.x;          // (b*Hkv + g)*n + c
    const int bg = list / a.n, cblk = list % a.n;
    const int co = tid % OCT, rg = tid / OCT;
    float acc[NR][8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        acc[0][t] = MM ? INFINITY : 0.f;
        acc[NR - 1][t] = MM ? -INFINITY : acc[0][t];
    }
    if (rg < NG) {
        const size_t base = ((size_t)bg * a.N + (size_t)cblk * a.B) * D + co * 8;
        for (int j = rg; j < a.B; j += NG) {
            float x[8];
            if constexpr (F32IN) {
                const float4* p = (const float4*)((const float*)a.k + base + (size_t)j * D);
                const float4 x0 = p[0], x1 = p[1];
                x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
                x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
            } else {
                const uint4 u = *(const uint4*)((const uint16_t*)a.k + base + (size_t)j * D);
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    x[2 * t] = bf16_to_f32(w[t] & 0xffffu);
                    x[2 * t + 1] = bf16_to_f32(w[t] >> 16);
                }
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if constexpr (MM) {
                    acc[0][t] = fminf(acc[0][t], x[t]);
                    acc[NR - 1][t] = fmaxf(acc[NR - 1][t], x[t]);
                } else {
                    acc[0][t] += x[t];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int t = 0; t < 8; ++t) red[r][rg * D + co * 8 + t] = acc[r][t];
    }
    __syncthreads();
    if (tid < D) {
        const size_t o = (size_t)list * D + tid;
        if constexpr (MM) {
            float mn = INFINITY, mx = -INFINITY;
            for (int r = 0; r < NG; ++r) {
                mn = fminf(mn, red[0][r * D + tid]);
                mx = fmaxf(mx, red[NR - 1][r * D + tid]);
            }
            if (a.kbar) {
                a.kbar[((size_t)list * 2) * D + tid] = mn;
                a.kbar[((size_t)list * 2 + 1) * D + tid] = mx;
            }
            if (a.kb3) {
                if constexpr (F32IN) {   // max terms in planes 0-2, min terms in 3-5
                    split3(mx, a.kb3, a.plane, o);
                    split3(mn, a.kb3 + 3 * a.plane, a.plane, o);
                } else {                 // bf16 keys: both bounds are bf16 values
                    a.kb3[o] = __builtin_bit_cast(uint16_t, (__bf16)mx);
                    a.kb3[a.plane + o] = __builtin_bit_cast(uint16_t, (__bf16)mn);
                }
            }
        } else {
            float sum = 0.f;
            for (int r = 0; r < NG; ++r) sum += red[0][r * D + tid];
            const float mean = sum / (float)a.B;
            if (a.kbar) a.kbar[o] = mean;
            if (a.kb3) {
                if constexpr (F32IN) split3(mean, a.kb3, a.plane, o);
                else split2(mean, a.kb3, a.plane, o);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Gate: one wave per 32 query rows of one head; the waves of a workgroup
// share each staged candidate tile.  Eight waves when q is one bf16 term
// (at most 128 registers: four waves per SIMD), four otherwise (the split
// queries need more registers).
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int gate_waves(int qsplit) { return qsplit == 1 ? 8 : 4; }

// lo = mask - cblk, the block's index field.
__device__ __forceinline__ uint32_t order_key_lo(float s, uint32_t lo, uint32_t mask) {
    const uint32_t u = __float_as_uint(s);
    const uint32_t ord = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);   // ~u if negative
    return (ord & ~mask) | lo;
}

// Median of three: one v_med3_u32 (written out as min/max, the compiler's
// combiner runs for a very long time on these kernels).
__device__ __forceinline__ uint32_t med3u(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Insert x into the descending list L (top M kept).  Slot t of the new list
// is the median of the old L[t-1], L[t] and x: x itself where it lands, the
// shifted L[t-1] below that, L[t] above.  Slots are independent (one median
// each); a key below L[M-1] changes nothing.
template <int M>
__device__ __forceinline__ void insert_desc(uint32_t (&L)[M], uint32_t x) {
#pragma unroll
    for (int t = M - 1; t >= 1; --t) L[t] = med3u(L[t - 1], L[t], x);
    L[0] = max(L[0], x);
}

template <int M>
__device__ __forceinline__ void sort_asc(int (&x)[M]) {
#pragma unroll
    for (int k = 2; k <= M; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < M; ++i) {
                const int p = i ^ j;
                if (p > i) {
                    const bool up = (i & k) == 0;
                    const int lo = min(x[i], x[p]), hi = max(x[i], x[p]);
                    x[i] = up ? lo : hi;
                    x[p] = up ? hi : lo;
                }
            }
}

// Candidate blocks are scored 32 at a time.  The NP planes of those 32
// pooled keys go through LDS (double buffered, rows D + 8 elements apart so
// the 16-byte reads of 32 consecutive rows hit distinct banks); every wave
// of the workgroup reads them from there as the A operand of
// S^T = Kbar Q^T.
// The staging registers are a native vector type: with HIP's uint4 (a struct)
// the copies become memcpy calls that keep the array in scratch memory.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int D, int NP, int NT>
struct GateTile {
    static constexpr int RS = D + 8;                 // LDS row stride
    static constexpr int PLANE = 32 * RS;            // one plane of 32 rows
    static constexpr int CHUNKS = NP * 32 * D / 8;   // 16-byte pieces per tile
    static constexpr int CPT = (CHUNKS + NT - 1) / NT;
};

// Positive and negative parts of eight bf16 values, selected by the signs of
// `sgn` (the hi term of the same values): pos + neg = x, exactly.
__device__ __forceinline__ void sign_split(const bf16x8& x, const bf16x8& sgn, bf16x8& pos,
                                           bf16x8& neg) {
    const uint4 u = __builtin_bit_cast(uint4, x), g = __builtin_bit_cast(uint4, sgn);
    const uint32_t m0 = ((g.x >> 15) & 0x00010001u) * 0xffffu, m1 = ((g.y >> 15) & 0x00010001u) * 0xffffu;
    const uint32_t m2 = ((g.z >> 15) & 0x00010001u) * 0xffffu, m3 = ((g.w >> 15) & 0x00010001u) * 0xffffu;
    neg = as_bf16x8(make_uint4(u.x & m0, u.y & m1, u.z & m2, u.w & m3));
    pos = as_bf16x8(make_uint4(u.x & ~m0, u.y & ~m1, u.z & ~m2, u.w & ~m3));
}

// MM = false: NP planes of the mean (2 for bf16 keys, 3 for fp32).  MM = true: the min/max summary,
// NP / 2 planes of the max then of the min; the score
// sum_e max(q_e min_e, q_e max_e) is <q+, max> + <q-, min> with q+ and q-
// the positive and negative parts of q, two exact products on the matrix
// cores.  QSPLIT: bf16 terms of q (1 or 2); 4 = the parts come split
// already (q+ hi, lo, q- hi, lo: group sums of a shared min/max gate).
template <int D, int M, int QSPLIT, int NP, bool MM>
__global__ __launch_bounds__(64 * gate_waves(QSPLIT)) void gate_kernel(GateArgs a) {
    constexpr int kGateThreads = 64 * gate_waves(QSPLIT), kGateRows = 32 * gate_waves(QSPLIT);
    using GT = GateTile<D, NP, kGateThreads>;
    constexpr int DK = D / 16;
    __shared__ __align__(16) uint16_t lds[2][NP * GT::PLANE];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int BH = a.Bt * a.Hq;
    const int ntiles = (a.N + kGateRows - 1) / kGateRows;
    const int bh = blockIdx.x % BH;
    const int tile = ntiles - 1 - (int)(blockIdx.x / BH);
    const int b = bh / a.Hq, h = bh % a.Hq, g = h / (a.Hq / a.Hkv);
    const int q0 = tile * kGateRows + __builtin_amdgcn_readfirstlane(wave) * 32;
    const int row = q0 + col;
    const bool row_ok = row < a.N;
    const size_t prow = (size_t)bh * a.N + row;

    bf16x8 qf[QSPLIT][DK];
#pragma unroll
    for (int p = 0; p < QSPLIT; ++p)
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (row_ok) u = *(const uint4*)(a.q[p] + prow * D + ks * 16 + 8 * hh);
            qf[p][ks] = as_bf16x8(u);
        }

    const int row_blk = (row_ok ? row : a.N - 1) / a.B;
    const int last = min(tile * kGateRows + kGateRows - 1, a.N - 1);
    const int ncand_wg = last / a.B;                           // candidates: blocks < own block
    const int ncand_wave = q0 < a.N ? min(q0 + 31, a.N - 1) / a.B : 0;
    const int ntc = (ncand_wg + 31) / 32;
    const uint32_t mask = (1u << a.idx_bits) - 1u;
    // Block 0 forced (first block always kept, rows past block 0): not a
    // candidate, and one slot fewer for the candidates.
    const int c0 = (a.first && row_blk > 0) ? 1 : 0;
    const uint16_t* kb = a.kb3 + (size_t)(b * a.Hkv + g) * a.n * D;

    // Staging of candidate tile mt: chunk x = (plane, row, 16-byte column).
    u32x4 st[GT::CPT];
    auto load = [&](int mt) {
#pragma unroll
        for (int c = 0; c < GT::CPT; ++c) {
            const int x = min(tid + kGateThreads * c, GT::CHUNKS - 1);
            const int pl = x / (32 * D / 8), r = (x / (D / 8)) % 32, cc = x % (D / 8);
            const int cblk = min(mt * 32 + r, a.n - 1);
            st[c] = *(const u32x4*)(kb + pl * a.plane + (size_t)cblk * D + cc * 8);
        }
    };
    auto store = [&](uint16_t* dst) {
#pragma unroll
        for (int c = 0; c < GT::CPT; ++c) {
            const int x = min(tid + kGateThreads * c, GT::CHUNKS - 1);
            const int pl = x / (32 * D / 8), r = (x / (D / 8)) % 32, cc = x % (D / 8);
            *(u32x4*)(dst + pl * GT::PLANE + r * GT::RS + cc * 8) = st[c];
        }
    };

    uint32_t L[M];
#pragma unroll
    for (int t = 0; t < M; ++t) L[t] = 0u;

    if (ntc > 0) {
        load(0);
        store(lds[0]);
    }
    __syncthreads();
    for (int mt = 0; mt < ntc; ++mt) {
        if (mt + 1 < ntc) load(mt + 1);
        if (mt * 32 < ncand_wave) {
            const uint16_t* src = lds[mt & 1] + col * GT::RS + 8 * hh;
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < DK; ++ks) {
                if constexpr (!MM) {
                    // NP terms of the mean against q (and q's lo term against
                    // all but the last)
#pragma unroll
                    for (int p = 0; p < NP; ++p) {
                        const bf16x8 av = *(const bf16x8*)(src + p * GT::PLANE + ks * 16);
                        acc = mfma32(av, qf[0][ks], acc);
                        if constexpr (QSPLIT >= 2) {
                            if (p < NP - 1) acc = mfma32(av, qf[1][ks], acc);
                        }
                    }
                } else {
                    constexpr int NH = NP / 2;
                    constexpr int QT = QSPLIT == 4 ? 2 : QSPLIT;   // terms per part
                    bf16x8 qp[QT], qn[QT];
                    if constexpr (QSPLIT == 4) {
                        qp[0] = qf[0][ks]; qp[1] = qf[1][ks];
                        qn[0] = qf[2][ks]; qn[1] = qf[3][ks];
                    } else {
#pragma unroll
                        for (int x = 0; x < QT; ++x) sign_split(qf[x][ks], qf[0][ks], qp[x], qn[x]);
                    }
#pragma unroll
                    for (int p = 0; p < NH; ++p) {
                        const bf16x8 amax = *(const bf16x8*)(src + p * GT::PLANE + ks * 16);
                        const bf16x8 amin = *(const bf16x8*)(src + (NH + p) * GT::PLANE + ks * 16);
                        acc = mfma32(amax, qp[0], acc);
                        acc = mfma32(amin, qn[0], acc);
                        if constexpr (QT == 2) {
                            if (p < 2) {
                                acc = mfma32(amax, qp[1], acc);
                                acc = mfma32(amin, qn[1], acc);
                            }
                        }
                    }
                }
            }
            // Insert the 16 scores of this lane, four at a time; a score
            // that does not beat the lane's current M-th key cannot enter its
            // list (inserting it changes nothing), and a wave in which no
            // lane has such a score among the four skips their insertion.
            // Every candidate of the tile is valid for every row of the
            // wave when the tile ends before the wave's first row block and
            // holds no forced block 0 (wave-uniform).
            const bool all_ok = mt * 32 + 31 < q0 / a.B && (mt > 0 || !a.first);
            const uint32_t kbase = mask - (uint32_t)(mt * 32 + 4 * hh);
            auto insert_tile = [&](auto check) __attribute__((always_inline)) {
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    uint32_t keys[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int v = 4 * v4 + u;
                        const int vo = 8 * (v >> 2) + (v & 3);
                        uint32_t key = order_key_lo(acc[v], kbase - (uint32_t)vo, mask);
                        if constexpr (decltype(check)::value) {
                            const int cblk = mt * 32 + vo + 4 * hh;
                            key = cblk < row_blk && cblk >= c0 ? key : 0u;
                        }
                        keys[u] = key;
                    }
                    const uint32_t top = max(max(keys[0], keys[1]), max(keys[2], keys[3]));
                    if (__any(top > L[M - 1])) {
#pragma unroll
                        for (int u = 0; u < 4; ++u) insert_desc<M>(L, keys[u]);
                    }
                }
            };
            if (all_ok) insert_tile(std::false_type{});
            else insert_tile(std::true_type{});
        }
        if (mt + 1 < ntc) store(lds[(mt + 1) & 1]);
        __syncthreads();
    }
    // Merge with the partner lane, which scored the other half of the blocks.
    uint32_t P[M];
#pragma unroll
    for (int t = 0; t < M; ++t) P[t] = (uint32_t)__shfl_xor((int)L[t], 32);
#pragma unroll
    for (int t = 0; t < M; ++t) insert_desc<M>(L, P[t]);

    // Both lanes of a row hold the merged list; each writes half of the row
    // (16-byte pieces when top_k is a multiple of 4), so a wave's stores
    // cover its 32 rows' selections contiguously.
    if (!row_ok) return;
    const int m = max(0, min(a.top_k - 1 - c0, row_blk - c0));
    constexpr int MP = M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : M <= 16 ? 16 : 32;   // sorting width
    int ids[MP];
#pragma unroll
    // Clamped to the candidate range: with finite inputs every kept key is
    // a candidate's and the clamp changes nothing; NaN scores can leave keys
    // that decode past the last block, and a selection must stay in range.
    for (int t = 0; t < MP; ++t)
        ids[t] = t < m && t < M ? min(max((int)(mask - (L[t] & mask)), c0), row_blk - 1) : 0x7fffffff;
    sort_asc<MP>(ids);
    // Ascending: block 0 when forced, the m kept candidates, the own block.
    auto val_at = [&](int t) {
        int val = -1;
        if (t < c0) {
            val = 0;
        } else if (t < c0 + m) {
#pragma unroll
            for (int u = 0; u < MP; ++u)
                if (u == t - c0) val = ids[u];
        } else if (t == c0 + m) {
            val = row_blk;
        }
        return val;
    };
    for (int r = 0; r < a.rep; ++r) {
        int32_t* out = a.sel + (((size_t)b * a.Hq + h) * a.rep + r) * a.N * a.top_k +
                       (size_t)row * a.top_k;
        if ((a.top_k & 3) == 0 && ((uintptr_t)a.sel & 15) == 0) {
            for (int q = hh; q < a.top_k / 4; q += 2)
                *(int4*)(out + 4 * q) =
                    make_int4(val_at(4 * q), val_at(4 * q + 1), val_at(4 * q + 2), val_at(4 * q + 3));
        } else {
            for (int t = hh; t < a.top_k; t += 2) out[t] = val_at(t);
        }
    }
}

template <int D, bool F32IN>
static hipError_t pool_d(const PoolArgs& a, int lists, hipStream_t s) {
    if (a.minmax)
        hipLaunchKernelGGL((pool_kernel<D, F32IN, true>), dim3(lists), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((pool_kernel<D, F32IN, false>), dim3(lists), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pool(const PoolArgs& a, int head_dim, bool f32_in, int lists, hipStream_t s) {
    if (lists <= 0) return hipSuccess;
    if (f32_in) {
        if (head_dim == 64) return pool_d<64, true>(a, lists, s);
        if (head_dim == 80) return pool_d<80, true>(a, lists, s);
        if (head_dim == 128) return pool_d<128, true>(a, lists, s);
    } else {
        if (head_dim == 64) return pool_d<64, false>(a, lists, s);
        if (head_dim == 80) return pool_d<80, false>(a, lists, s);
        if (head_dim == 128) return pool_d<128, false>(a, lists, s);
    }
    return hipErrorInvalidValue;
}

template <int D, int M, int QS, int NP, bool MM>
static hipError_t gate_dm(const GateArgs& a, hipStream_t s) {
    const int rows = 32 * gate_waves(QS);
    const int ntiles = (a.N + rows - 1) / rows;
    hipLaunchKernelGGL((gate_kernel<D, M, QS, NP, MM>), dim3(ntiles * a.Bt * a.Hq), dim3(2 * rows), 0, s,
                       a);
    return hipGetLastError();
}

template <int D, int QS, int NP, bool MM>
static hipError_t gate_d(const GateArgs& a, hipStream_t s) {
    const int need = a.top_k - 1;
    if (need <= 2) return gate_dm<D, 2, QS, NP, MM>(a, s);
    if (need <= 4) return gate_dm<D, 4, QS, NP, MM>(a, s);
    if (need == 7) return gate_dm<D, 7, QS, NP, MM>(a, s);   // top 8 blocks: seven slots
    if (need <= 8) return gate_dm<D, 8, QS, NP, MM>(a, s);
    if (need == 15) return gate_dm<D, 15, QS, NP, MM>(a, s);  // top 16
    if (need <= 16) return gate_dm<D, 16, QS, NP, MM>(a, s);
    if (need <= 32) return gate_dm<D, 32, QS, NP, MM>(a, s);
    return hipErrorInvalidValue;
}

template <int QS, int NP, bool MM>
static hipError_t gate_v(const GateArgs& a, int head_dim, hipStream_t s) {
    if (head_dim == 64) return gate_d<64, QS, NP, MM>(a, s);
    if (head_dim == 80) return gate_d<80, QS, NP, MM>(a, s);
    if (head_dim == 128) return gate_d<128, QS, NP, MM>(a, s);
    return hipErrorInvalidValue;
}

// planes: the gate_planes() of the summary; qsplit: bf16 terms of q (1 or
// 2), or 4 for the pre-split parts of a shared min/max gate.  fp32 min/max
// planes come with fp32 (split) queries only.
hipError_t launch_gate(const GateArgs& a, int head_dim, int qsplit, int planes, bool minmax,
                       hipStream_t s) {
    if (!minmax && planes == 2) {   // bf16 keys
        if (qsplit == 1) return gate_v<1, 2, false>(a, head_dim, s);
        if (qsplit == 2) return gate_v<2, 2, false>(a, head_dim, s);
    }
    if (!minmax && planes == 3) {   // fp32 keys
        if (qsplit == 2) return gate_v<2, 3, false>(a, head_dim, s);
    }
    if (minmax && planes == 2) {
        if (qsplit == 1) return gate_v<1, 2, true>(a, head_dim, s);
        if (qsplit == 2) return gate_v<2, 2, true>(a, head_dim, s);
        if (qsplit == 4) return gate_v<4, 2, true>(a, head_dim, s);
    }
    if (minmax && planes == 6) {
        if (qsplit == 2) return gate_v<2, 6, true>(a, head_dim, s);
        if (qsplit == 4) return gate_v<4, 6, true>(a, head_dim, s);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Group sums of the queries (selection shared per kv group): one thread per
// 8 consecutive elements of one (batch, kv group, position) row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_split8(const float (&s)[8], uint16_t* hi, uint16_t* lo,
                                             size_t o) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const __bf16 h0 = (__bf16)s[2 * t], h1 = (__bf16)s[2 * t + 1];
        const __bf16 l0 = (__bf16)(s[2 * t] - (float)h0), l1 = (__bf16)(s[2 * t + 1] - (float)h1);
        hw[t] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        lw[t] = (uint32_t)__builtin_bit_cast(uint16_t, l0) |
                ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
    }
    *(uint4*)(hi + o) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    *(uint4*)(lo + o) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
}

template <bool F32IN, bool MM>
__global__ __launch_bounds__(256) void group_sum_kernel(GroupSumArgs a) {
    const size_t oct = (size_t)a.D / 8;
    const size_t total = (size_t)a.Bt * a.Hkv * a.N * oct;
    const size_t x = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (x >= total) return;
    const size_t row = x / oct, e0 = (x % oct) * 8;      // row = (b*Hkv + g)*N + i
    const int i = (int)(row % a.N), bg = (int)(row / a.N);
    const int b = bg / a.Hkv, g = bg % a.Hkv, G = a.Hq / a.Hkv;
    float sp[8] = {0, 0, 0, 0, 0, 0, 0, 0}, sn[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int h = g * G; h < (g + 1) * G; ++h) {
        const size_t src = (((size_t)b * a.Hq + h) * a.N + i) * a.D + e0;
        float v[8];
        if constexpr (F32IN) {
            const float4 p0 = *(const float4*)((const float*)a.q + src);
            const float4 p1 = *(const float4*)((const float*)a.q + src + 4);
            v[0] = p0.x; v[1] = p0.y; v[2] = p0.z; v[3] = p0.w;
            v[4] = p1.x; v[5] = p1.y; v[6] = p1.z; v[7] = p1.w;
        } else {
            const uint4 u = *(const uint4*)((const uint16_t*)a.q + src);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                v[2 * t] = bf16_to_f32(w[t] & 0xffffu);
                v[2 * t + 1] = bf16_to_f32(w[t] >> 16);
            }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if constexpr (MM) {
                sp[t] += fmaxf(v[t], 0.f);
                sn[t] += fminf(v[t], 0.f);
            } else {
                sp[t] += v[t];
            }
        }
    }
    const size_t o = row * a.D + e0;
    store_split8(sp, a.out[0], a.out[1], o);
    if constexpr (MM) store_split8(sn, a.out[2], a.out[3], o);
}

hipError_t launch_group_sum(const GroupSumArgs& a, bool f32_in, hipStream_t s) {
    const size_t total = (size_t)a.Bt * a.Hkv * a.N * (a.D / 8);
    if (total == 0) return hipSuccess;
    const unsigned grid = (unsigned)((total + 255) / 256);
    if (f32_in) {
        if (a.minmax) hipLaunchKernelGGL((group_sum_kernel<true, true>), dim3(grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((group_sum_kernel<true, false>), dim3(grid), dim3(256), 0, s, a);
    } else {
        if (a.minmax) hipLaunchKernelGGL((group_sum_kernel<false, true>), dim3(grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((group_sum_kernel<false, false>), dim3(grid), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace sa
