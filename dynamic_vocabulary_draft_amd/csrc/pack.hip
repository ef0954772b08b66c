// Packed copy of a fixed shortlist's rows of W: out[i] = W[ids[i]].
//
// The static baselines the pages compare against draft from a fixed,
// frequency-ranked shortlist (DynaSpec abstract, on FR-Spec and VocabTrim;
// summary page, "Comparison to Prior Work" and "Evaluation Highlights": a
// static list of about 32K tokens).  A fixed list can be copied once into a
// contiguous slab, so its head is a dense GEMV over the slab with no gather;
// this kernel makes that slab.  A row whose id lies outside [0, V) is filled
// with NaN, so the slab's head gives NaN where the gathered head does.
//
// One wave per output row (grid-stride), 16-byte loads and stores: the copy
// reads and writes n * d * e bytes and is HBM-bound.
#include "common.h"
#include "kernels.h"

namespace ds {
namespace {

__global__ __launch_bounds__(256) void pack_rows_kernel(int V, int nch, const u32x4 *__restrict__ W,
                                                        int64_t n, const int32_t *__restrict__ ids,
                                                        u32x4 nan_fill, u32x4 *__restrict__ out)
{
    const int lane = lane_id();
    const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); row < n;
         row += nw) {
        const int32_t id = ids[row];
        const bool ok = id >= 0 && id < V;
        const u32x4 *src = W + (int64_t)(ok ? id : 0) * nch;
        u32x4 *dst = out + row * nch;
        for (int c = lane; c < nch; c += kWave)
            dst[c] = ok ? __builtin_nontemporal_load(src + c) : nan_fill;
    }
}

}  // namespace

hipError_t pack_launch(hipStream_t s, bool bf16, int V, int d, const void *W, int64_t n,
                       const int32_t *ids, void *out)
{
    if (n <= 0)
        return hipSuccess;
    const int nch = d * (bf16 ? 2 : 4) / 16;
    const uint32_t nanw = bf16 ? 0x7FC07FC0u : 0x7FC00000u;  // quiet NaN in every element
    int64_t blocks = (n + 3) / 4;
    const int64_t cap = 8LL * device_cu_count();
    if (blocks > cap)
        blocks = cap;
    hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, V, nch,
                       reinterpret_cast<const u32x4 *>(W), n, ids, u32x4{nanw, nanw, nanw, nanw},
                       reinterpret_cast<u32x4 *>(out));
    return hipGetLastError();
}

}  // namespace ds
