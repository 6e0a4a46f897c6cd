// sa_gate.hip -- block mean-pool and block gate (score GEMM + top-k).
//
// Block gate [MoBA summary page, "블록 분할과 top-k 게이팅" and "인과성
// 보존"]: every key block c is summarised by the mean of its B keys; query i
// of block b scores each earlier block by <q_i, mean_c> (no scale), keeps its
// own block plus the min(top_k-1, b) best earlier ones (ties toward the
// lower block id), and never sees a later block.
//
// Accuracy: the pooled keys are split into three bf16 terms
// (mean = hi + mid + lo to about 24 bits) so the score GEMM runs on bf16
// matrix cores with fp32 accumulation and still carries fp32-level
// accuracy -- a single bf16 rounding of the mean (2^-9 relative) would flip
// selections whose top-k margin is far larger than the accepted tolerance.
// This is the bf16x3 splitting of Henry, Tang and Heinecke (ARITH 2019).
//
// Top-k: each lane owns one query row (lane pair l, l^32 split the blocks),
// packs every score into a 32-bit key that orders like the float and breaks
// ties toward the lower block id (the low idx_bits of the mantissa are
// replaced by (mask - c), costing 2^-(23-idx_bits) of relative precision),
// and keeps a sorted top-M list in registers with a max/min insertion chain.
#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

// ---------------------------------------------------------------------------
// Mean pool: one workgroup per (batch, kv head, block).
// ---------------------------------------------------------------------------
template <int D, bool F32IN>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
    constexpr int OCT = D / 8;            // 8-element column groups
    constexpr int NG = 256 / OCT;         // row groups
    __shared__ float red[NG * D];
    const int tid = threadIdx.x;
    const int list = blockIdx.x;          // (b*Hkv + g)*n + c
    const int bg = list / a.n, cblk = list % a.n;
    const int co = tid % OCT, rg = tid / OCT;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (rg < NG) {
        const size_t base = ((size_t)bg * a.N + (size_t)cblk * a.B) * D + co * 8;
        for (int j = rg; j < a.B; j += NG) {
            if constexpr (F32IN) {
                const float4* p = (const float4*)((const float*)a.k + base + (size_t)j * D);
                const float4 x0 = p[0], x1 = p[1];
                acc[0] += x0.x; acc[1] += x0.y; acc[2] += x0.z; acc[3] += x0.w;
                acc[4] += x1.x; acc[5] += x1.y; acc[6] += x1.z; acc[7] += x1.w;
            } else {
                const uint4 u = *(const uint4*)((const uint16_t*)a.k + base + (size_t)j * D);
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    acc[2 * t] += bf16_to_f32(w[t] & 0xffffu);
                    acc[2 * t + 1] += bf16_to_f32(w[t] >> 16);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) red[rg * D + co * 8 + t] = acc[t];
    }
    __syncthreads();
    if (tid < D) {
        float s = 0.f;
        for (int r = 0; r < NG; ++r) s += red[r * D + tid];
        const float mean = s / (float)a.B;
        const size_t o = (size_t)list * D + tid;
        if (a.kbar) a.kbar[o] = mean;
        if (a.kb3) {
            const __bf16 hi = (__bf16)mean;
            const float r1 = mean - (float)hi;
            const __bf16 mid = (__bf16)r1;
            const __bf16 lo = (__bf16)(r1 - (float)mid);
            a.kb3[o] = __builtin_bit_cast(uint16_t, hi);
            a.kb3[a.plane + o] = __builtin_bit_cast(uint16_t, mid);
            a.kb3[2 * a.plane + o] = __builtin_bit_cast(uint16_t, lo);
        }
    }
}

// ---------------------------------------------------------------------------
// Gate: one wave per 32 query rows of one head, 4 waves per workgroup.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float s, int cblk, uint32_t mask) {
    const uint32_t u = __float_as_uint(s);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (ord & ~mask) | (mask - (uint32_t)cblk);
}

template <int M>
__device__ __forceinline__ void insert_desc(uint32_t (&L)[M], uint32_t x) {
#pragma unroll
    for (int t = 0; t < M; ++t) {
        const uint32_t hi = max(L[t], x);
        x = min(L[t], x);
        L[t] = hi;
    }
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

// Candidate blocks are scored 32 at a time.  The three planes of those 32
// pooled keys go through LDS (double buffered, rows D + 8 elements apart so
// the 16-byte reads of 32 consecutive rows hit distinct banks); every wave
// of the workgroup reads them from there as the A operand of
// S^T = Kbar Q^T.
template <int D>
struct GateTile {
    static constexpr int RS = D + 8;                 // LDS row stride
    static constexpr int PLANE = 32 * RS;            // one plane of 32 rows
    static constexpr int CHUNKS = 3 * 32 * D / 8;    // 16-byte pieces per tile
    static constexpr int CPT = (CHUNKS + 255) / 256;
};

template <int D, int M, int QSPLIT>
__global__ __launch_bounds__(256) void gate_kernel(GateArgs a) {
    using GT = GateTile<D>;
    constexpr int DK = D / 16;
    __shared__ __align__(16) uint16_t lds[2][3 * GT::PLANE];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int BH = a.Bt * a.Hq;
    const int ntiles = (a.N + 127) / 128;
    const int bh = blockIdx.x % BH;
    const int tile = ntiles - 1 - (int)(blockIdx.x / BH);
    const int b = bh / a.Hq, h = bh % a.Hq, g = h / (a.Hq / a.Hkv);
    const int q0 = tile * 128 + __builtin_amdgcn_readfirstlane(wave) * 32;
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
    const int last = min(tile * 128 + 127, a.N - 1);
    const int ncand_wg = last / a.B;                           // candidates: blocks < own block
    const int ncand_wave = q0 < a.N ? min(q0 + 31, a.N - 1) / a.B : 0;
    const int ntc = (ncand_wg + 31) / 32;
    const uint32_t mask = (1u << a.idx_bits) - 1u;
    const uint16_t* kb = a.kb3 + (size_t)(b * a.Hkv + g) * a.n * D;

    // Staging of candidate tile mt: chunk x = (plane, row, 16-byte column).
    uint4 st[GT::CPT];
    auto load = [&](int mt) {
#pragma unroll
        for (int c = 0; c < GT::CPT; ++c) {
            const int x = min(tid + 256 * c, GT::CHUNKS - 1);
            const int pl = x / (32 * D / 8), r = (x / (D / 8)) % 32, cc = x % (D / 8);
            const int cblk = min(mt * 32 + r, a.n - 1);
            st[c] = *(const uint4*)(kb + pl * a.plane + (size_t)cblk * D + cc * 8);
        }
    };
    auto store = [&](uint16_t* dst) {
#pragma unroll
        for (int c = 0; c < GT::CPT; ++c) {
            const int x = min(tid + 256 * c, GT::CHUNKS - 1);
            const int pl = x / (32 * D / 8), r = (x / (D / 8)) % 32, cc = x % (D / 8);
            *(uint4*)(dst + pl * GT::PLANE + r * GT::RS + cc * 8) = st[c];
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
#pragma unroll
                for (int p = 0; p < 3; ++p) {
                    const bf16x8 av = *(const bf16x8*)(src + p * GT::PLANE + ks * 16);
                    acc = mfma32(av, qf[0][ks], acc);
                    if constexpr (QSPLIT == 2) {
                        if (p < 2) acc = mfma32(av, qf[1][ks], acc);
                    }
                }
            }
            // Insert the 16 scores of this lane; a score that does not beat
            // the lane's current M-th key cannot enter its list, and a wave
            // in which no lane has such a score skips the insertion.
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int cblk = mt * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
                const uint32_t key = cblk < row_blk ? order_key(acc[v], cblk, mask) : 0u;
                const bool in = key > L[M - 1];
                if (__any(in)) insert_desc<M>(L, in ? key : 0u);   // inserting 0 changes nothing
            }
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

    if (!row_ok || hh != 0) return;
    const int m = min(a.top_k - 1, row_blk);
    int ids[M];
#pragma unroll
    for (int t = 0; t < M; ++t) ids[t] = t < m ? (int)(mask - (L[t] & mask)) : 0x7fffffff;
    sort_asc<M>(ids);
    int32_t* out = a.sel + prow * a.top_k;
    for (int t = 0; t < a.top_k; ++t) {
        int val = -1;
        if (t < m) {
#pragma unroll
            for (int u = 0; u < M; ++u)
                if (u == t) val = ids[u];
        } else if (t == m) {
            val = row_blk;
        }
        out[t] = val;
    }
}

template <int D, bool F32IN>
static hipError_t pool_d(const PoolArgs& a, int lists, hipStream_t s) {
    hipLaunchKernelGGL((pool_kernel<D, F32IN>), dim3(lists), dim3(256), 0, s, a);
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

template <int D, int M, int QS>
static hipError_t gate_dm(const GateArgs& a, hipStream_t s) {
    const int ntiles = (a.N + 127) / 128;
    hipLaunchKernelGGL((gate_kernel<D, M, QS>), dim3(ntiles * a.Bt * a.Hq), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int D, int QS>
static hipError_t gate_d(const GateArgs& a, hipStream_t s) {
    const int need = a.top_k - 1;
    if (need <= 2) return gate_dm<D, 2, QS>(a, s);
    if (need <= 4) return gate_dm<D, 4, QS>(a, s);
    if (need <= 8) return gate_dm<D, 8, QS>(a, s);
    if (need <= 16) return gate_dm<D, 16, QS>(a, s);
    if (need <= 32) return gate_dm<D, 32, QS>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_gate(const GateArgs& a, int head_dim, int qsplit, hipStream_t s) {
    if (qsplit == 1) {
        if (head_dim == 64) return gate_d<64, 1>(a, s);
        if (head_dim == 80) return gate_d<80, 1>(a, s);
        if (head_dim == 128) return gate_d<128, 1>(a, s);
    } else {
        if (head_dim == 64) return gate_d<64, 2>(a, s);
        if (head_dim == 80) return gate_d<80, 2>(a, s);
        if (head_dim == 128) return gate_d<128, 2>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace sa
