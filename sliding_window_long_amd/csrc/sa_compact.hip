// sa_compact.hip -- regroup query rows by the far block they kept.
//
// Steps 1-2 of the implementation on the MoBA summary page ("MoBA의 구현"):
// assign each query to the KV blocks it routes to, then reorder queries by
// block so each block is attended as one variable-length batch.  Here only
// the far blocks (entirely before the window span) are regrouped; the own
// block and the blocks overlapping the window span stay with the
// query-centric pass.
//
// count  : per (batch, kv head, block) list, number of (row, head) entries
//          (LDS histogram per row tile, one global atomic per non-empty bin)
// scan   : exclusive scan of the counts -> list offsets and each list's first
//          chunk (lists cut into chunks of rows_per_chunk entries)
// chunks : the chunk table (list and first entry of every chunk), a thread
//          per chunk
// scatter: write every entry (i*G + h_local)*kslots + slot at its list's
//          running cursor.  Order inside a list depends on atomic order, but
//          each entry's result depends only on its own row and block, so the
//          output of the attention is the same bit for bit.
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
    for (int x = threadIdx.x; x < a.n; x += CT)
        if (hist[x] > 0) atomicAdd(&a.count[bg * a.n + x], hist[x]);
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
            a.cursor[l] = off_l;
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
    hipLaunchKernelGGL(compact_scatter_kernel, grid, dim3(CT), 2 * a.n * sizeof(int32_t), s, a);
    return hipGetLastError();
}

}  // namespace sa
