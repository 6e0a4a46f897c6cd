// sa_token.hip -- token gate: single-head dot-product indexer and per-query
// top-k token selection.
//
// [Naive-N0.5-Flash page, "SWA와 DSA를 결합한 어텐션"]: a light indexer scores
// the whole history of each query and attention runs on the top 2,048
// tokens.  Reading taken here: score(i, j) = <idx_q_i, idx_k_j> with no scale,
// candidates j < i, keep the min(top_t, i) best, a tie going to the lower j;
// the selection is shared by every query head.
//
// Exact selection by radix select on a 48-bit key per candidate:
//   key = ord(score) << 16 | (0xFFFF - j)
// where ord maps fp32 to a uint32 with the same order.  The key order is
// (score descending, then j ascending), so "the k largest keys" is exactly
// the selection.  Passes 0-3 find the 32-bit ordered score T of the k-th key
// one byte at a time (per-row 256-bin histograms in LDS); rows where more
// candidates tie at T than slots remain run passes 4-5 over the index bits.
// Scores are recomputed on the matrix core in every pass (same instruction
// sequence, so bitwise the same values); they are never stored.
//
// Output: a keep mask in the layout of the attention kernel's registers.
// For the 32 query rows r0..r0+31 (row tile rt), the 64 keys kt*64 ..
// kt*64+63 (key tile kt) and lane L of the wave that owns those rows, word
// mask[(rt*NT64 + kt)*64 + L] has bit 16*sub + v set iff row r0 + L%32 keeps
// key kt*64 + 32*sub + 8*(v/4) + 4*(L/32) + v%4 -- the key held in register v
// of the sub-th 32-key half of the S^T tile.  The two halves are written as
// separate 16-bit halves of the word.
#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

constexpr int TOK_WAVES = 4;
constexpr int TOK_THREADS = 64 * TOK_WAVES;
constexpr uint32_t kTokAll = 1u;    // row keeps every candidate
constexpr uint32_t kTokNone = 2u;   // row keeps nothing
constexpr uint32_t kTokDone = 4u;   // threshold final
// Per-row 256-bin histograms in LDS, 257 words apart so that rows adding
// to the same bin hit different banks.
constexpr int HSTRIDE = 257;

__device__ __forceinline__ uint32_t ord32(float s) {
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 16-bit half of the mask word of (batch, row tile, 32-key tile kc, lane).
__device__ __forceinline__ size_t mask_half(int bt, int nt32, int nt64, int rt, int kc, int lane) {
    return ((((size_t)bt * nt32 + rt) * nt64 + (kc >> 1)) * 64 + lane) * 2 + (kc & 1);
}

// Indexer scores of one 32-key tile against the wave's 32 query rows:
// acc[v] = score(row r0 + lane%32, key kc*32 + 8*(v/4) + 4*(lane/32) + v%4).
template <int SPLIT>
__device__ __forceinline__ f32x16 index_scores(const TokArgs& a, int bt, int kc,
                                               const bf16x8 (&qf)[SPLIT][4], int lane) {
    const int col = lane & 31, hh = lane >> 5;
    const int key = min(kc * 32 + col, a.N - 1);
    const size_t off = ((size_t)bt * a.N + key) * 64 + 8 * hh;
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 k0 = as_bf16x8(*(const uint4*)(a.ik[0] + off + ks * 16));
        acc = mfma32(k0, qf[0][ks], acc);
        if constexpr (SPLIT == 2) {
            const bf16x8 k1 = as_bf16x8(*(const uint4*)(a.ik[1] + off + ks * 16));
            acc = mfma32(k0, qf[1][ks], acc);
            acc = mfma32(k1, qf[0][ks], acc);
        }
    }
    return acc;
}

// One pass over the candidates of a 32-row tile (4 waves split the key
// tiles).  pass 0..5: radix histogram step; pass 6: write the keep mask.
template <int SPLIT>
__global__ __launch_bounds__(TOK_THREADS) void token_select_kernel(TokArgs a, int pass) {
    __shared__ uint32_t hist[32 * HSTRIDE];
    __shared__ int s_skip;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hh = lane >> 5;
    const int nt = (a.N + 31) / 32;
    // Row tiles with the most candidates first (they run longest).
    const int rt = nt - 1 - (int)(blockIdx.x % nt), bt = blockIdx.x / nt;
    const int r0 = rt * 32;
    const int row = r0 + col;
    const bool row_ok = row < a.N;
    int4* state = a.state + (size_t)bt * a.N;

    // Row state: x = ordered-score prefix, y = index-key prefix, z = keys
    // still to take, w = flags.
    int4 stt = make_int4(0, 0, 0, 0);
    if (pass == 0) {
        const int k = row_ok ? min(a.top_t, row) : 0;
        uint32_t fl = 0;
        if (k == 0) fl = kTokNone | kTokDone;
        else if (k == row) fl = kTokAll | kTokDone;
        stt = make_int4(0, 0, k, (int)fl);
    } else if (row_ok) {
        stt = state[row];
    } else {
        stt = make_int4(0, 0, 0, (int)(kTokNone | kTokDone));
    }
    const uint32_t flags = (uint32_t)stt.w;
    const uint32_t pre32 = (uint32_t)stt.x, preidx = (uint32_t)stt.y;

    if (pass < 6) {
        if (tid == 0) s_skip = 1;
        __syncthreads();
        if (!(flags & kTokDone)) s_skip = 0;   // benign race: every writer stores 0
        for (int x = tid; x < 32 * HSTRIDE; x += TOK_THREADS) hist[x] = 0;
        __syncthreads();
        if (s_skip) {
            if (pass == 0 && tid < 32 && row_ok) state[row] = stt;
            return;
        }
    }

    bf16x8 qf[SPLIT][4];
#pragma unroll
    for (int p = 0; p < SPLIT; ++p)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (row_ok) u = *(const uint4*)(a.iq[p] + ((size_t)bt * a.N + row) * 64 + ks * 16 + 8 * hh);
            qf[p][ks] = as_bf16x8(u);
        }

    const bool active = !(flags & kTokDone);
    // Byte of the key examined in this pass and the prefix that must match.
    const int shift = pass < 4 ? 24 - 8 * pass : 8 - 8 * (pass - 4);
    for (int kc = wave; kc <= rt; kc += TOK_WAVES) {
        const f32x16 acc = index_scores<SPLIT>(a, bt, kc, qf, lane);
        const int rj = row - kc * 32 - 4 * hh;   // row - key = rj - cv
        if (pass < 6) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int cv = 8 * (v >> 2) + (v & 3);
                const uint32_t o = ord32(acc[v]);
                bool take = active && rj > cv;
                uint32_t digit;
                if (pass < 4) {
                    if (pass > 0) take = take && ((o ^ pre32) >> (shift + 8)) == 0;
                    digit = (o >> shift) & 0xffu;
                } else {
                    const uint32_t ik = 0xffffu - (uint32_t)(kc * 32 + 4 * hh + cv);
                    take = take && o == pre32;
                    if (pass == 5) take = take && ((ik ^ preidx) >> 8) == 0;
                    digit = (ik >> shift) & 0xffu;
                }
                if (take) atomicAdd(&hist[col * HSTRIDE + digit], 1u);
            }
        } else {
            // Keep mask: key >= threshold (all / none handled by the flags).
            uint32_t bits = 0;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int cv = 8 * (v >> 2) + (v & 3);
                const uint32_t o = ord32(acc[v]);
                const uint32_t ik = 0xffffu - (uint32_t)(kc * 32 + 4 * hh + cv);
                bool keep = row_ok && rj > cv && !(flags & kTokNone);
                if (!(flags & kTokAll)) keep = keep && (o > pre32 || (o == pre32 && ik >= preidx));
                bits |= (keep ? 1u : 0u) << v;
            }
            a.mask[mask_half(bt, nt, (a.N + 63) / 64, rt, kc, lane)] = (uint16_t)bits;
        }
    }
    if (pass == 6) return;
    __syncthreads();
    if (tid < 32 && row_ok) {
        if (active) {
            // Bin holding the k-th largest remaining key.
            uint32_t k = (uint32_t)stt.z, cum = 0;
            int b = 255;
            for (; b > 0; --b) {
                const uint32_t h = hist[tid * HSTRIDE + b];
                if (cum + h >= k) break;
                cum += h;
            }
            const uint32_t hb = hist[tid * HSTRIDE + b];
            k -= cum;
            uint32_t fl = flags;
            if (pass < 4) {
                stt.x = (int)(pre32 | ((uint32_t)b << shift));
                // After the last score byte: if every candidate tied at the
                // threshold is kept, the index bits need no selection.
                if (pass == 3 && hb == k) {
                    fl |= kTokDone;
                    stt.y = 0;
                }
            } else {
                stt.y = (int)(preidx | ((uint32_t)b << shift));
                if (pass == 5) fl |= kTokDone;
            }
            stt.z = (int)k;
            stt.w = (int)fl;
        }
        state[row] = stt;
    }
}

// Ascending token ids kept by each row, -1 padded, from the keep mask.
__global__ void token_list_kernel(TokArgs a, int32_t* out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int total = a.Bt * a.N;
    if (i >= total) return;
    const int bt = i / a.N, row = i % a.N;
    const int nt = (a.N + 31) / 32, nt64 = (a.N + 63) / 64, rt = row / 32, L = row % 32;
    int32_t* dst = out + (size_t)i * a.top_t;
    int n = 0;
    for (int kc = 0; kc <= rt && n < a.top_t; ++kc) {
        const uint32_t m0 = a.mask[mask_half(bt, nt, nt64, rt, kc, L)];        // lanes L
        const uint32_t m1 = a.mask[mask_half(bt, nt, nt64, rt, kc, L + 32)];   // and L+32
        for (int jl = 0; jl < 32 && n < a.top_t; ++jl) {
            const int v = 4 * (jl >> 3) + (jl & 3), h = (jl >> 2) & 1;
            if (((h ? m1 : m0) >> v) & 1u) dst[n++] = kc * 32 + jl;
        }
    }
    for (; n < a.top_t; ++n) dst[n] = -1;
}

hipError_t launch_token_select(const TokArgs& a, int split, hipStream_t s) {
    const int nt = (a.N + 31) / 32;
    const dim3 grid((unsigned)(nt * a.Bt));
    for (int pass = 0; pass <= 6; ++pass) {
        if (split == 2)
            hipLaunchKernelGGL(token_select_kernel<2>, grid, dim3(TOK_THREADS), 0, s, a, pass);
        else
            hipLaunchKernelGGL(token_select_kernel<1>, grid, dim3(TOK_THREADS), 0, s, a, pass);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_token_list(const TokArgs& a, int32_t* out, hipStream_t s) {
    const int total = a.Bt * a.N;
    hipLaunchKernelGGL(token_list_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a,
                       out);
    return hipGetLastError();
}

}  // namespace sa
