// Top-cluster selection under a position-aware budget (DynaSpec abstract:
// the union of the top-selected clusters is the shortlist; summary page,
// "Key Novelty" and "Key Hyperparameters": a budget k_c(t) that decays with
// the draft position).
//
// One workgroup per row.  The M (<= 4096) clusters are ranked in LDS with a
// bitonic sort over 64-bit keys (order-preserving score bits, inverted for
// descending order, above the cluster id), which realises the total order
// (score desc, id asc) exactly.  The budget cut is then one block-wide
// exclusive scan of the ranked sizes: with a token budget, a cluster is
// taken iff the tokens ranked before it fall short of the budget.
#include "common.h"
#include "kernels.h"

namespace ds {
namespace {

// monotone map fp32 -> uint32 (ascending), with -0.0 folded onto +0.0
__device__ __forceinline__ uint32_t ordered_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u)
        u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(1024) void select_kernel(int M, int P, const float *__restrict__ scores,
                                                      const int32_t *__restrict__ cluster_size,
                                                      int kind, const int32_t *__restrict__ budget,
                                                      int32_t *__restrict__ sel,
                                                      int32_t *__restrict__ n_sel,
                                                      int32_t *__restrict__ sl_len)
{
    extern __shared__ uint64_t keys[];  // P entries
    __shared__ int64_t scan_sh[kWave + 1];
    __shared__ int s_take;
    __shared__ unsigned long long s_total;
    const int row = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
    const float *s = scores + (int64_t)row * M;

    for (int i = tid; i < P; i += nt)
        keys[i] = i < M ? ((uint64_t)(~ordered_bits(s[i])) << 32) | (uint32_t)i : ~0ull;
    if (tid == 0) {
        s_take = 0;
        s_total = 0;
    }
    __syncthreads();

    // bitonic sort, ascending keys == (score desc, id asc)
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < (P >> 1); t += nt) {
                int i = 2 * stride * (t / stride) + (t % stride);
                int j = i + stride;
                bool asc = (i & size) == 0;
                uint64_t a = keys[i], b = keys[j];
                if ((a > b) == asc) {
                    keys[i] = b;
                    keys[j] = a;
                }
            }
            __syncthreads();
        }
    }

    const int32_t bud = budget[row];
    const int kclusters = bud < 1 ? 1 : (bud > M ? M : bud);
    const int64_t btokens = bud < 1 ? 1 : (int64_t)bud;
    int64_t carry = 0;
    for (int base = 0; base < M; base += nt) {  // uniform trip count
        const int j = base + tid;
        int64_t v = 0;
        if (j < M)
            v = cluster_size[(uint32_t)keys[j]];
        int64_t tot;
        int64_t excl = block_excl_scan_i64(v, scan_sh, &tot) + carry;
        bool take = j < M && (kind == DS_BUDGET_CLUSTERS ? j < kclusters : excl < btokens);
        if (take) {
            atomicAdd(&s_take, 1);
            atomicAdd(&s_total, (unsigned long long)v);
        }
        carry += tot;
    }
    __syncthreads();
    const int take = s_take;
    for (int j = tid; j < M; j += nt)
        sel[(int64_t)row * M + j] = j < take ? (int32_t)(uint32_t)keys[j] : -1;
    if (tid == 0) {
        n_sel[row] = take;
        sl_len[row] = (int32_t)s_total;
    }
}

}  // namespace

hipError_t select_launch(hipStream_t s, int n, int M, const float *scores,
                         const int32_t *cluster_size, int kind, const int32_t *budget,
                         int32_t *sel, int32_t *n_sel, int32_t *sl_len)
{
    int P = 1;
    while (P < M)
        P <<= 1;
    if (P < 2)
        P = 2;
    int threads = P / 2;
    if (threads < 64)
        threads = 64;
    if (threads > 1024)
        threads = 1024;
    hipLaunchKernelGGL(select_kernel, dim3(n), dim3(threads), P * sizeof(uint64_t), s, M, P,
                       scores, cluster_size, kind, budget, sel, n_sel, sl_len);
    return hipGetLastError();
}

}  // namespace ds
