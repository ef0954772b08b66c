// Shortlist construction: the union of the selected clusters' members, in
// ascending token id (DynaSpec abstract: the shortlist is the union of the
// selected clusters; summary page, "Problem Definition": the output is the
// shortlisted subset V_S).
//
// The vocabulary is cut into chunks of kBuildChunk = 4096 tokens.  A
// cluster index, built once per clustering from cluster_of, holds for every
// cluster c the number of its members in chunks 0..k-1 (index[k][c], k =
// 0..nchunks; index[nchunks][c] is the cluster size).  With it the offset of
// a (row, chunk) in the output is a sum over the row's selected clusters, so
// no counting pass over the vocabulary is needed:
//   rows (only when n > 1): one workgroup sums each row's selected cluster
//          sizes, scans them into row bases and sl_off, and raises the
//          capacity flag;
//   compact: one workgroup per (row, chunk) rebuilds the row's selected-
//          cluster bitmap in LDS, classifies its 4096 tokens with one read
//          of cluster_of, and writes them at row base + chunk offset + a
//          block-wide exclusive scan of per-thread counts -- ascending token
//          id without any sort.  For n = 1 the row base is sl_off[0] and
//          chunk 0 writes sl_off[1].  Optionally it also writes the row's
//          tile index for the batched head: per 32-token tile (two threads'
//          16 tokens) the tile's first shortlist position and membership
//          mask, which the compaction has in hand.
// All integer, hence bit-exact; no workgroup waits on another.
#include "common.h"
#include "kernels.h"

namespace ds {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kBuildChunk / kThreads;  // 16 consecutive tokens
constexpr int kMaxBitmapWords = DS_MAX_CLUSTERS / 32;

// bitmap of the row's selected clusters; returns after a barrier
__device__ __forceinline__ void load_bitmap(uint32_t *bm, int M, const int32_t *sel_row, int k,
                                            int32_t *err_flag)
{
    const int words = (M + 31) >> 5;
    for (int i = threadIdx.x; i < words; i += blockDim.x)
        bm[i] = 0;
    __syncthreads();
    if (k < 0 || k > M) {
        if (threadIdx.x == 0)
            raise_flag(err_flag, DS_EINVAL);
        k = k < 0 ? 0 : M;
    }
    for (int j = threadIdx.x; j < k; j += blockDim.x) {
        int c = sel_row[j];
        if (c < 0 || c >= M)
            raise_flag(err_flag, DS_EINVAL);
        else
            atomicOr(&bm[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
}

// selection mask of this thread's kPerThread consecutive tokens
__device__ __forceinline__ uint32_t token_mask(const uint32_t *bm, int M, int V,
                                               const int32_t *__restrict__ cluster_of, int64_t y0)
{
    uint32_t mask = 0;
    if (y0 + kPerThread <= V) {
        const int4 *p = reinterpret_cast<const int4 *>(cluster_of + y0);
#pragma unroll
        for (int q = 0; q < kPerThread / 4; ++q) {
            int4 c4 = p[q];
            int cs[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                int c = cs[e];
                if (c >= 0 && c < M && ((bm[c >> 5] >> (c & 31)) & 1u))
                    mask |= 1u << (q * 4 + e);
            }
        }
    } else {
        for (int e = 0; e < kPerThread; ++e) {
            int64_t y = y0 + e;
            if (y >= V)
                break;
            int c = cluster_of[y];
            if (c >= 0 && c < M && ((bm[c >> 5] >> (c & 31)) & 1u))
                mask |= 1u << e;
        }
    }
    return mask;
}

// sum over the row's selected (valid) clusters of index_row[c]
__device__ int64_t sum_selected(const int32_t *__restrict__ index_row, const int32_t *sel_row,
                                int k, int M, int64_t *sh)
{
    k = k < 0 ? 0 : (k > M ? M : k);
    int64_t v = 0;
    for (int j = threadIdx.x; j < k; j += blockDim.x) {
        int c = sel_row[j];
        if (c >= 0 && c < M)
            v += index_row[c];
    }
    int64_t tot;
    (void)block_excl_scan_i64(v, sh, &tot);
    return tot;
}

// ---------------------------------------------------------------- the index
__global__ __launch_bounds__(kThreads) void index_count_kernel(int M, int V,
                                                               const int32_t *__restrict__ cluster_of,
                                                               int32_t *__restrict__ index,
                                                               int32_t *err_flag)
{
    __shared__ int hist[DS_MAX_CLUSTERS];
    const int chunk = blockIdx.x;
    for (int c = threadIdx.x; c < M; c += blockDim.x)
        hist[c] = 0;
    __syncthreads();
    const int64_t y0 = (int64_t)chunk * kBuildChunk;
    for (int i = threadIdx.x; i < kBuildChunk; i += blockDim.x) {
        const int64_t y = y0 + i;
        if (y >= V)
            break;
        const int c = cluster_of[y];
        if (c < 0 || c >= M)
            raise_flag(err_flag, DS_EINVAL);
        else
            atomicAdd(&hist[c], 1);
    }
    __syncthreads();
    for (int c = threadIdx.x; c < M; c += blockDim.x) {
        index[(int64_t)(chunk + 1) * M + c] = hist[c];
        if (chunk == 0)
            index[c] = 0;
    }
}

__global__ __launch_bounds__(kThreads) void index_prefix_kernel(int M, int nchunks,
                                                                int32_t *__restrict__ index)
{
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= M)
        return;
    int32_t run = 0;
    for (int k = 1; k <= nchunks; ++k) {
        run += index[(int64_t)k * M + c];
        index[(int64_t)k * M + c] = run;
    }
}

// ---------------------------------------------------------------- the build
// n > 1: row totals from the index (one wave per row), scanned in tiles of
// 1024 rows into row bases and sl_off
__global__ __launch_bounds__(1024) void build_rows_kernel(int n, int M, int nchunks,
                                                          const int32_t *__restrict__ sel,
                                                          const int32_t *__restrict__ n_sel,
                                                          const int32_t *__restrict__ index,
                                                          int64_t capacity, int64_t *sl_off,
                                                          int32_t *err_flag, int64_t *row_base)
{
    __shared__ int64_t tot[1024];
    __shared__ int64_t sh[kWave + 1];
    const int32_t *sizes = index + (int64_t)nchunks * M;
    const int lane = lane_id(), wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int64_t carry = sl_off[0];
    for (int r0 = 0; r0 < n; r0 += 1024) {
        const int nr = min(1024, n - r0);
        for (int i = wave; i < nr; i += nw) {
            const int r = r0 + i;
            int k = n_sel[r];
            k = k < 0 ? 0 : (k > M ? M : k);
            int64_t v = 0;
            for (int j = lane; j < k; j += kWave) {
                const int c = sel[(int64_t)r * M + j];
                if (c >= 0 && c < M)
                    v += sizes[c];
            }
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1)
                v += __shfl_xor(v, o);
            if (lane == 0)
                tot[i] = v;
        }
        __syncthreads();
        const int64_t v = (int)threadIdx.x < nr ? tot[threadIdx.x] : 0;
        int64_t tile;
        const int64_t excl = block_excl_scan_i64(v, sh, &tile) + carry;
        if ((int)threadIdx.x < nr) {
            const int r = r0 + threadIdx.x;
            row_base[r] = excl;
            const int64_t end = excl + v;
            sl_off[r + 1] = end < capacity ? end : capacity;
            if (end > capacity)
                raise_flag(err_flag, DS_ECAPACITY);
        }
        carry += tile;
    }
}

__global__ __launch_bounds__(kThreads) void build_compact_kernel(
    int n, int M, int V, int nchunks, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ n_sel, const int32_t *__restrict__ cluster_of,
    const int32_t *__restrict__ index, int64_t capacity, int64_t *sl_off,
    int32_t *__restrict__ sl_ids, int32_t *err_flag, const int64_t *__restrict__ row_base,
    TileIx *__restrict__ tix)
{
    __shared__ uint32_t bm[kMaxBitmapWords];
    __shared__ int64_t sh[kWave + 1];
    const int chunk = blockIdx.x, row = blockIdx.y;
    const int32_t *sel_row = sel + (int64_t)row * M;
    const int k = n_sel[row];
    load_bitmap(bm, M, sel_row, k, chunk == 0 ? err_flag : nullptr);
    int64_t base;
    if (n == 1) {
        base = sl_off[0];
        if (chunk == 0) {  // the single row's end offset
            const int64_t tot = sum_selected(index + (int64_t)nchunks * M, sel_row, k, M, sh);
            if (threadIdx.x == 0) {
                const int64_t end = base + tot;
                sl_off[1] = end < capacity ? end : capacity;
                if (end > capacity)
                    raise_flag(err_flag, DS_ECAPACITY);
            }
        }
    } else {
        base = row_base[row];
    }
    const int64_t chunk_off = sum_selected(index + (int64_t)chunk * M, sel_row, k, M, sh);
    const int64_t y0 = (int64_t)chunk * kBuildChunk + threadIdx.x * kPerThread;
    uint32_t mask = y0 < V ? token_mask(bm, M, V, cluster_of, y0) : 0u;
    int64_t tot;
    const int64_t rel = block_excl_scan_i64(__popc(mask), sh, &tot) + chunk_off;
    int64_t pos = rel + base;
    static_assert(kPerThread == 16, "two threads per 32-token tile");
    if (tix) {  // block-uniform
        const uint32_t hi = (uint32_t)__shfl_down((int)mask, 1);  // the odd neighbour's 16 tokens
        const int nt = (V + 31) / 32;
        const int64_t t = y0 >> 5;
        if ((threadIdx.x & 1) == 0 && t < nt)
            tix[(int64_t)row * (nt + 1) + t] = TileIx{(int32_t)rel, mask | (hi << 16)};
    }
    while (mask) {
        int e = __ffs(mask) - 1;
        mask &= mask - 1;
        if (pos < capacity)
            sl_ids[pos] = (int32_t)(y0 + e);
        ++pos;
    }
}

}  // namespace

size_t index_bytes(int M, int V)
{
    const int64_t nchunks = ((int64_t)V + kBuildChunk - 1) / kBuildChunk;
    return (size_t)(nchunks + 1) * (size_t)M * sizeof(int32_t);
}

hipError_t index_launch(hipStream_t s, int M, int V, const int32_t *cluster_of, int32_t *index,
                        int32_t *err_flag)
{
    const int nchunks = (V + kBuildChunk - 1) / kBuildChunk;
    hipLaunchKernelGGL(index_count_kernel, dim3(nchunks), dim3(kThreads), 0, s, M, V, cluster_of,
                       index, err_flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(index_prefix_kernel, dim3((M + kThreads - 1) / kThreads), dim3(kThreads), 0,
                       s, M, nchunks, index);
    return hipGetLastError();
}

size_t build_ws_bytes(int n, int V)
{
    (void)V;
    return 256 + (size_t)n * sizeof(int64_t);
}

hipError_t build_launch(hipStream_t s, int n, int M, int V, const int32_t *sel,
                        const int32_t *n_sel, const int32_t *cluster_of, const int32_t *index,
                        int64_t capacity, int64_t *sl_off, int32_t *sl_ids, int32_t *err_flag,
                        void *ws, TileIx *tix)
{
    const int nchunks = (V + kBuildChunk - 1) / kBuildChunk;
    int64_t *row_base = reinterpret_cast<int64_t *>(reinterpret_cast<char *>(ws) + 256);
    hipError_t e;
    if (n > 1) {
        hipLaunchKernelGGL(build_rows_kernel, dim3(1), dim3(1024), 0, s, n, M, nchunks, sel, n_sel,
                           index, capacity, sl_off, err_flag, row_base);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(build_compact_kernel, dim3(nchunks, n), dim3(kThreads), 0, s, n, M, V,
                       nchunks, sel, n_sel, cluster_of, index, capacity, sl_off, sl_ids, err_flag,
                       (const int64_t *)row_base, tix);
    return hipGetLastError();
}

}  // namespace ds
