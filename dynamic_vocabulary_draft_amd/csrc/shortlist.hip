// Shortlist construction: the union of the selected clusters' members, in
// ascending token id (DynaSpec abstract: "the union of the top-selected
// clusters defines the drafter's shortlist"; summary page, "Problem
// Definition": the output is the shortlisted subset V_S).
//
// The vocabulary is cut into chunks of kBuildChunk tokens; one workgroup
// handles one (row, chunk).  Each workgroup rebuilds the row's selected-
// cluster bitmap in LDS (M bits), classifies its 4096 tokens with one read of
// cluster_of, and
//   pass 1 (count):   writes its selected-token count; the last workgroup to
//                     finish (ticket counter) scans all counts in row-major
//                     order into absolute chunk offsets and sl_off, raises
//                     the capacity flag, and re-arms the counter;
//   pass 2 (compact): writes its tokens at its chunk offset plus a block-wide
//                     exclusive scan of per-thread counts, so the output is
//                     in ascending token id without any sort.
// Both passes are integer-only, hence bit-exact.
#include "common.h"
#include "kernels.h"

namespace ds {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kBuildChunk / kThreads;  // 16 consecutive tokens
constexpr int kMaxBitmapWords = DS_MAX_CLUSTERS / 32;

struct BuildWs {
    unsigned int *ticket;  // one counter (zero when idle)
    int64_t *chunk;        // [n][nchunks]: counts, then absolute offsets
};

__device__ __forceinline__ BuildWs carve(void *ws)
{
    BuildWs w;
    w.ticket = reinterpret_cast<unsigned int *>(ws);
    w.chunk = reinterpret_cast<int64_t *>(reinterpret_cast<char *>(ws) + 256);
    return w;
}

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
                                               const int32_t *__restrict__ cluster_of, int64_t y0,
                                               int32_t *err_flag)
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
                bool bad = c < 0 || c >= M;
                if (bad)
                    raise_flag(err_flag, DS_EINVAL);
                else if ((bm[c >> 5] >> (c & 31)) & 1u)
                    mask |= 1u << (q * 4 + e);
            }
        }
    } else {
        for (int e = 0; e < kPerThread; ++e) {
            int64_t y = y0 + e;
            if (y >= V)
                break;
            int c = cluster_of[y];
            if (c < 0 || c >= M)
                raise_flag(err_flag, DS_EINVAL);
            else if ((bm[c >> 5] >> (c & 31)) & 1u)
                mask |= 1u << e;
        }
    }
    return mask;
}

__global__ __launch_bounds__(kThreads) void build_count_kernel(int n, int M, int V,
                                                               const int32_t *__restrict__ sel,
                                                               const int32_t *__restrict__ n_sel,
                                                               const int32_t *__restrict__ cluster_of,
                                                               int64_t capacity, int64_t *sl_off,
                                                               int32_t *err_flag, void *ws)
{
    __shared__ uint32_t bm[kMaxBitmapWords];
    __shared__ int64_t scan_sh[kWave + 1];
    __shared__ int s_count;
    __shared__ bool s_last;
    const int chunk = blockIdx.x, row = blockIdx.y, nchunks = gridDim.x;
    BuildWs w = carve(ws);
    if (threadIdx.x == 0)
        s_count = 0;
    load_bitmap(bm, M, sel + (int64_t)row * M, n_sel[row], err_flag);
    const int64_t y0 = (int64_t)chunk * kBuildChunk + threadIdx.x * kPerThread;
    uint32_t mask = y0 < V ? token_mask(bm, M, V, cluster_of, y0, err_flag) : 0u;
    atomicAdd(&s_count, __popc(mask));
    __syncthreads();
    if (threadIdx.x == 0) {
        w.chunk[(int64_t)row * nchunks + chunk] = s_count;
        __threadfence();
        unsigned int ticket = atomicAdd(w.ticket, 1u);
        s_last = ticket == (unsigned int)(gridDim.x * gridDim.y) - 1u;
    }
    __syncthreads();
    if (!s_last)
        return;
    // last workgroup: counts -> absolute chunk offsets, sl_off, capacity flag
    __threadfence();
    const int64_t total_chunks = (int64_t)n * nchunks;
    const int64_t base = sl_off[0];
    int64_t carry = base;
    for (int64_t b0 = 0; b0 < total_chunks; b0 += blockDim.x) {
        const int64_t i = b0 + threadIdx.x;
        int64_t v = i < total_chunks ? __hip_atomic_load(&w.chunk[i], __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT)
                                     : 0;
        int64_t tot;
        int64_t excl = block_excl_scan_i64(v, scan_sh, &tot) + carry;
        if (i < total_chunks) {
            w.chunk[i] = excl;
            if ((i % nchunks) == nchunks - 1) {  // end of a row
                int64_t end = excl + v;
                sl_off[i / nchunks + 1] = end < capacity ? end : capacity;
                if (end > capacity)
                    raise_flag(err_flag, DS_ECAPACITY);
            }
        }
        carry += tot;
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(w.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kThreads) void build_compact_kernel(int M, int V,
                                                                 const int32_t *__restrict__ sel,
                                                                 const int32_t *__restrict__ n_sel,
                                                                 const int32_t *__restrict__ cluster_of,
                                                                 int64_t capacity,
                                                                 int32_t *__restrict__ sl_ids,
                                                                 const void *ws)
{
    __shared__ uint32_t bm[kMaxBitmapWords];
    __shared__ int64_t scan_sh[kWave + 1];
    const int chunk = blockIdx.x, row = blockIdx.y, nchunks = gridDim.x;
    const int64_t *chunk_off = reinterpret_cast<const int64_t *>(reinterpret_cast<const char *>(ws) + 256);
    load_bitmap(bm, M, sel + (int64_t)row * M, n_sel[row], nullptr);
    const int64_t y0 = (int64_t)chunk * kBuildChunk + threadIdx.x * kPerThread;
    uint32_t mask = y0 < V ? token_mask(bm, M, V, cluster_of, y0, nullptr) : 0u;
    int64_t tot;
    int64_t pos = block_excl_scan_i64(__popc(mask), scan_sh, &tot) +
                  chunk_off[(int64_t)row * nchunks + chunk];
    while (mask) {
        int e = __ffs(mask) - 1;
        mask &= mask - 1;
        if (pos < capacity)
            sl_ids[pos] = (int32_t)(y0 + e);
        ++pos;
    }
}

}  // namespace

size_t build_ws_bytes(int n, int V)
{
    const int64_t nchunks = ((int64_t)V + kBuildChunk - 1) / kBuildChunk;
    return 256 + (size_t)n * (size_t)nchunks * sizeof(int64_t);
}

hipError_t build_launch(hipStream_t s, int n, int M, int V, const int32_t *sel,
                        const int32_t *n_sel, const int32_t *cluster_of, int64_t capacity,
                        int64_t *sl_off, int32_t *sl_ids, int32_t *err_flag, void *ws)
{
    const int nchunks = (V + kBuildChunk - 1) / kBuildChunk;
    dim3 grid(nchunks, n);
    hipLaunchKernelGGL(build_count_kernel, grid, dim3(kThreads), 0, s, n, M, V, sel, n_sel,
                       cluster_of, capacity, sl_off, err_flag, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(build_compact_kernel, grid, dim3(kThreads), 0, s, M, V, sel, n_sel,
                       cluster_of, capacity, sl_ids, (const void *)ws);
    return hipGetLastError();
}

}  // namespace ds
