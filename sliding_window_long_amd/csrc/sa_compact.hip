// sa_compact.hip -- regroup query rows by the far block they kept.
//
// Steps 1-2 of the implementation on the MoBA summary page ("MoBA의 구현"):
// assign each query to the KV blocks it routes to, then reorder queries by
// block so each block is attended as one variable-length batch.  Here only
// the far blocks (entirely before the window span) are regrouped; the own
// block and the blocks overlapping the window span stay with the
// query-centric pass.
//
// count  : per (batch, kv head, block) list, number of (row, head) entries,
//          in total (one global atomic per non-empty bin of a row tile's LDS
//          histogram) and per row tile (the histogram itself)
// scan   : exclusive scan of the counts -> list offsets and each list's first
//          chunk (lists cut into chunks of rows_per_chunk entries)
// chunks : the chunk table (list and first entry of every chunk), a thread
//          per chunk
// scatter: write every entry (i*G + h_local)*kslots + slot into its list.
//          Fast form (forward): at the list's running cursor, in no fixed
//          order; each entry's result depends only on its own row and
//          block, so the attention's output is the same bit for bit.
//          Ordered form (backward, whose dK and dV sum over the lists):
//          tiles  -- per list, the first position of each row tile's
//                    entries (a running sum over the tiles in order);
//          scatter-- inside a tile, 64-row groups, heads, slots and lanes in
//                    order (lanes naming the same list ranked by a ballot),
//                    so the lists, and every sum over them, are the same on
//                    every call.
#include "sa_internal.hpp"

namespace sa {

constexpr int CT = 256;   // rows per workgroup tile

__global__ void fill_i32_kernel(int32_t* p, int32_t value, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = value;
}

hipError_t launch_fill_i32(int32_t* p, int32_t value, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p,
                       value, n);
    return hipGetLastError();
}

// Visit every far entry of query row i (all G heads of kv head g).
template <typename F>
__device__ __forceinline__ void for_far_entries(const CompactArgs& a, int b, int g, int i, F&& f) {
    const int G = a.Hq / a.Hkv;
    const int bi = i / a.B;
    for (int hl = 0; hl < G; ++hl) {
        const size_t prow = (size_t)(b * a.Hq + g * G + hl) * a.N + i;
        const int32_t* sr = a.sel + prow * a.top_k;
        for (int x = 0; x < a.top_k; ++x) {
            const int c = sr[x];
            // Ascending list: the far blocks come first.
            if (c < 0 || bi - c <= a.span) break;
            f(c, (i * G + hl) * a.kslots + x);
        }
    }
}

__global__ __launch_bounds__(CT) void compact_count_kernel(CompactArgs a) {
    extern __shared__ int32_t hist[];
    const int bg = blockIdx.y, b = bg / a.Hkv, g = bg % a.Hkv;
    for (int x = threadIdx.x; x < a.n; x += CT) hist[x] = 0;
    __syncthreads();
    const int i = blockIdx.x * CT + threadIdx.x;
    if (i < a.N) for_far_entries(a, b, g, i, [&](int c, int) { atomicAdd(&hist[c], 1); });
    __syncthreads();
    // The ordered scatter also needs every row tile's counts.
    int32_t* tb = a.ordered ? a.tile_base + ((size_t)bg * gridDim.x + blockIdx.x) * a.n : nullptr;
    for (int x = threadIdx.x; x < a.n; x += CT) {
        if (tb) tb[x] = hist[x];
        if (hist[x] > 0) atomicAdd(&a.count[bg * a.n + x], hist[x]);
    }
}

__global__ __launch_bounds__(1024) void compact_scan_kernel(CompactArgs a, int lists) {
    __shared__ int32_t s_cnt[1024];
    __shared__ int32_t s_nch[1024];
    __shared__ int32_t s_carry[2];
    const int tid = threadIdx.x;
    if (tid == 0) { s_carry[0] = 0; s_carry[1] = 0; }
    __syncthreads();
    const int R = a.rows_per_chunk;
    for (int base = 0; base < lists; base += 1024) {
        const int l = base + tid;
        const int cnt = l < lists ? a.count[l] : 0;
        const int nch = (cnt + R - 1) / R;
        s_cnt[tid] = cnt;
        s_nch[tid] = nch;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {   // inclusive Hillis-Steele scan
            const int vc = tid >= off ? s_cnt[tid - off] : 0;
            const int vn = tid >= off ? s_nch[tid - off] : 0;
            __syncthreads();
            s_cnt[tid] += vc;
            s_nch[tid] += vn;
            __syncthreads();
        }
        const int off_l = s_carry[0] + s_cnt[tid] - cnt;
        const int ch_l = s_carry[1] + s_nch[tid] - nch;
        if (l < lists) {
            a.list_off[l] = off_l;
            if (!a.ordered) a.cursor[l] = off_l;   // the fast scatter's running cursors
            a.list_ch[l] = ch_l;
        }
        __syncthreads();
        if (tid == 1023) {
            s_carry[0] += s_cnt[1023];
            s_carry[1] += s_nch[1023];
        }
        __syncthreads();
    }
    if (tid == 0) {
        a.list_off[lists] = s_carry[0];
        a.list_ch[lists] = s_carry[1];
        a.n_chunks[0] = min(s_carry[1], a.max_chunks);
    }
}

// Chunk table: thread per chunk q; its list l (list_ch[l] <= q <
// list_ch[l + 1], by bisection) and its first entry.
__global__ __launch_bounds__(256) void compact_chunks_kernel(CompactArgs a, int lists) {
    const int q = blockIdx.x * 256 + threadIdx.x;
    if (q >= a.n_chunks[0]) return;
    int lo = 0, hi = lists;   // list_ch[lo] <= q < list_ch[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.list_ch[mid] <= q) lo = mid;
        else hi = mid;
    }
    a.chunk_list[q] = lo;
    a.chunk_start[q] = a.list_off[lo] + (q - a.list_ch[lo]) * a.rows_per_chunk;
}

// Thread per list: each row tile's count becomes the tile's first position.
__global__ __launch_bounds__(256) void compact_tiles_kernel(CompactArgs a, int lists, int ntiles) {
    const int l = blockIdx.x * 256 + threadIdx.x;
    if (l >= lists) return;
    const int bg = l / a.n, c = l % a.n;
    int32_t* tb = a.tile_base + (size_t)bg * ntiles * a.n + c;
    int run = a.list_off[l];
    for (int t = 0; t < ntiles; ++t) {
        const int v = tb[(size_t)t * a.n];
        tb[(size_t)t * a.n] = run;
        run += v;
    }
}

__global__ __launch_bounds__(CT) void compact_scatter_kernel(CompactArgs a) {
    extern __shared__ int32_t sh[];
    int32_t* hist = sh;
    int32_t* base = sh + a.n;
    const int bg = blockIdx.y, b = bg / a.Hkv, g = bg % a.Hkv;
    for (int x = threadIdx.x; x < a.n; x += CT) hist[x] = 0;
    __syncthreads();
    const int i = blockIdx.x * CT + threadIdx.x;
    if (i < a.N) for_far_entries(a, b, g, i, [&](int c, int) { atomicAdd(&hist[c], 1); });
    __syncthreads();
    for (int x = threadIdx.x; x < a.n; x += CT) {
        if (hist[x] > 0) base[x] = atomicAdd(&a.cursor[bg * a.n + x], hist[x]);
        hist[x] = 0;
    }
    __syncthreads();
    if (i < a.N)
        for_far_entries(a, b, g, i, [&](int c, int ent) {
            const int pos = base[c] + atomicAdd(&hist[c], 1);
            a.entries[pos] = ent;
        });
}

// LDS writes of this wave's lanes are visible to its reads from here on.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Ordered scatter: NW waves per (row tile, batch x kv head), wave w taking
// the 64-row groups w, w + NW, ... of the tile.  With more than one wave,
// each first counts its groups' entries per list, and a prefix over the
// waves (in order) gives each wave its first position in every list.  LDS:
// per wave the running position of every list and one 64-row group's
// selections of one head.
template <int NW>
__global__ __launch_bounds__(64 * NW) void compact_scatter_ordered_kernel(CompactArgs a) {
    extern __shared__ int32_t sh[];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int K = a.top_k;
    int32_t* run = sh + w * a.n;
    int32_t* sel_st = sh + NW * a.n + w * 64 * K;
    const int tile = blockIdx.x, ntiles = gridDim.x;
    const int bg = blockIdx.y, b = bg / a.Hkv, g = bg % a.Hkv;
    const int G = a.Hq / a.Hkv;
    const int32_t* tb = a.tile_base + ((size_t)bg * ntiles + tile) * a.n;
    const int r_end = min(tile * CT + CT, a.N);
    // The far block of slot x for this lane's row, or -1 (and live = false
    // from the first slot that is not a far block on).
    auto far_id = [&](int x, int bi, bool& live) {
        int c = -1;
        if (live) {
            c = sel_st[lane * K + x];
            // Ascending list: the far blocks come first.
            if (c < 0 || bi - c <= a.span) {
                live = false;
                c = -1;
            }
        }
        return c;
    };
    auto stage = [&](int r0, int nr, int hl) {
        const int32_t* src = a.sel + ((size_t)(b * a.Hq + g * G + hl) * a.N + r0) * K;
        wave_lds_fence();   // this wave's reads of the previous group are done
        for (int x = lane; x < nr * K; x += 64) sel_st[x] = src[x];
        wave_lds_fence();
    };
    if constexpr (NW > 1) {
        for (int x = lane; x < a.n; x += 64) run[x] = 0;
        wave_lds_fence();
        for (int r0 = tile * CT + 64 * w; r0 < r_end; r0 += 64 * NW) {
            const int nr = min(64, a.N - r0), bi = (r0 + lane) / a.B;
            for (int hl = 0; hl < G; ++hl) {
                stage(r0, nr, hl);
                bool live = lane < nr;
                for (int x = 0; x < K && live; ++x) {
                    const int c = far_id(x, bi, live);
                    if (c >= 0) atomicAdd(&run[c], 1);   // integer counts: any order
                }
            }
        }
        __syncthreads();
        for (int c = tid; c < a.n; c += 64 * NW) {
            int p = tb[c];
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                const int t = sh[v * a.n + c];
                sh[v * a.n + c] = p;
                p += t;
            }
        }
        __syncthreads();
    } else {
        for (int x = lane; x < a.n; x += 64) run[x] = tb[x];
        wave_lds_fence();
    }
    const uint64_t below = (1ull << lane) - 1ull;
    for (int r0 = tile * CT + 64 * w; r0 < r_end; r0 += 64 * NW) {
        const int nr = min(64, a.N - r0);
        const int i = r0 + lane, bi = i / a.B;
        for (int hl = 0; hl < G; ++hl) {
            stage(r0, nr, hl);
            bool live = lane < nr;
            for (int x = 0; x < K; ++x) {
                const int c = far_id(x, bi, live);
                uint64_t pending = __ballot(c >= 0);
                if (pending == 0) break;   // no lane has a far block left
                while (pending) {
                    const int leader = __ffsll((unsigned long long)pending) - 1;
                    const int cl = __builtin_amdgcn_readlane(c, leader);
                    const uint64_t m = __ballot(c == cl);
                    // A wave's LDS operations execute in order: the reads of
                    // run[cl] above see it before the leader's update.
                    if (c == cl)
                        a.entries[run[cl] + __popcll(m & below)] = (i * G + hl) * a.kslots + x;
                    __builtin_amdgcn_wave_barrier();
                    if (lane == leader) run[cl] += __popcll(m);
                    __builtin_amdgcn_wave_barrier();
                    pending &= ~m;
                }
            }
        }
    }
}

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
    const int lists = a.Bt * a.Hkv * a.n;
    hipError_t e = launch_fill_i32(a.count, 0, (size_t)lists, s);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((a.N + CT - 1) / CT), (unsigned)(a.Bt * a.Hkv));
    hipLaunchKernelGGL(compact_count_kernel, grid, dim3(CT), a.n * sizeof(int32_t), s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(compact_scan_kernel, dim3(1), dim3(1024), 0, s, a, lists);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(compact_chunks_kernel, dim3((unsigned)((a.max_chunks + 255) / 256)), dim3(256),
                       0, s, a, lists);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (!a.ordered) {
        hipLaunchKernelGGL(compact_scatter_kernel, grid, dim3(CT), 2 * a.n * sizeof(int32_t), s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(compact_tiles_kernel, dim3((unsigned)((lists + 255) / 256)), dim3(256), 0, s, a,
                       lists, (int)grid.x);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // Four waves per tile while their LDS fits 64 KiB, else one.
    const size_t lds4 = (4 * (size_t)a.n + 4 * 64 * (size_t)a.top_k) * sizeof(int32_t);
    if (lds4 <= 65536)
        hipLaunchKernelGGL(compact_scatter_ordered_kernel<4>, grid, dim3(256), lds4, s, a);
    else
        hipLaunchKernelGGL(compact_scatter_ordered_kernel<1>, grid, dim3(64),
                           ((size_t)a.n + 64 * (size_t)a.top_k) * sizeof(int32_t), s, a);
    return hipGetLastError();
}

}  // namespace sa
