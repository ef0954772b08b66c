// Top-cluster selection under a position-aware budget (DynaSpec abstract:
// the shortlist is the union of the best-scoring clusters; summary page,
// "Key Novelty" and "Key Hyperparameters": a budget k_c(t) that decays with
// the draft position).
//
// One workgroup per row.  The M (<= 4096) clusters are ranked with a bitonic
// sort over 64-bit keys (order-preserving score bits, inverted for
// descending order, above the cluster id), which realises the total order
// (score desc, id asc) exactly.  Keys live in registers (one to four per
// thread); compare-exchange partners closer than 64 positions are in the
// same wave and are fetched with lane shuffles, only the wider strides go
// through LDS with barriers.  The budget cut is one block-wide exclusive
// scan of the ranked sizes: with a token budget, a cluster is taken iff the
// tokens ranked before it fall short of the budget; the thread holding the
// last taken cluster writes the count and the total.
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

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m)
{
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo = __shfl_xor(lo, m);
    hi = __shfl_xor(hi, m);
    return ((uint64_t)hi << 32) | lo;
}

template <int KPT>
__global__ __launch_bounds__(1024) void select_kernel(int M, int P, const float *__restrict__ scores,
                                                      const int32_t *__restrict__ cluster_size,
                                                      int kind, const int32_t *__restrict__ budget,
                                                      int32_t *__restrict__ sel,
                                                      int32_t *__restrict__ n_sel,
                                                      int32_t *__restrict__ sl_len)
{
    extern __shared__ uint64_t keys[];  // P entries
    __shared__ int64_t scan_sh[kWave + 1];
    const int row = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
    const float *s = scores + (int64_t)row * M;

    uint64_t k[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int idx = tid + i * nt;
        k[i] = idx < M ? ((uint64_t)(~ordered_bits(s[idx])) << 32) | (uint32_t)idx : ~0ull;
    }
    // bitonic sort, ascending keys == (score desc, id asc)
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            uint64_t partner[KPT];
            if (stride >= kWave) {
#pragma unroll
                for (int i = 0; i < KPT; ++i)
                    keys[tid + i * nt] = k[i];
                __syncthreads();
#pragma unroll
                for (int i = 0; i < KPT; ++i)
                    partner[i] = keys[(tid + i * nt) ^ stride];
                __syncthreads();
            } else {
#pragma unroll
                for (int i = 0; i < KPT; ++i)
                    partner[i] = shfl_xor_u64(k[i], stride);
            }
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const int idx = tid + i * nt;
                const bool asc = (idx & size) == 0, lower = (idx & stride) == 0;
                const uint64_t lo = k[i] < partner[i] ? k[i] : partner[i];
                const uint64_t hi = k[i] < partner[i] ? partner[i] : k[i];
                k[i] = (lower == asc) ? lo : hi;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i)
        keys[tid + i * nt] = k[i];
    __syncthreads();

    const int32_t bud = budget[row];
    const int kclusters = bud < 1 ? 1 : (bud > M ? M : bud);
    const int64_t btokens = bud < 1 ? 1 : (int64_t)bud;
    __shared__ int s_take;
    __shared__ long long s_total;
    int64_t carry = 0;
    for (int base = 0; base < M; base += nt) {  // uniform trip count
        const int j = base + tid;
        const int64_t v = j < M ? cluster_size[(uint32_t)keys[j]] : 0;
        int64_t tot;
        const int64_t excl = block_excl_scan_i64(v, scan_sh, &tot) + carry;
        const bool take = j < M && (kind == DS_BUDGET_CLUSTERS ? j < kclusters : excl < btokens);
        const bool next = j + 1 < M &&
                          (kind == DS_BUDGET_CLUSTERS ? j + 1 < kclusters : excl + v < btokens);
        if (take && !next) {  // the last cluster of the taken prefix
            s_take = j + 1;
            s_total = excl + v;
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
    int P = kWave;
    while (P < M)
        P <<= 1;
    const int nt = P < 1024 ? P : 1024;
    const int kpt = P / nt;
    const size_t lds = (size_t)P * sizeof(uint64_t);
    if (kpt == 1)
        hipLaunchKernelGGL(select_kernel<1>, dim3(n), dim3(nt), lds, s, M, P, scores, cluster_size,
                           kind, budget, sel, n_sel, sl_len);
    else if (kpt == 2)
        hipLaunchKernelGGL(select_kernel<2>, dim3(n), dim3(nt), lds, s, M, P, scores, cluster_size,
                           kind, budget, sel, n_sel, sl_len);
    else
        hipLaunchKernelGGL(select_kernel<4>, dim3(n), dim3(nt), lds, s, M, P, scores, cluster_size,
                           kind, budget, sel, n_sel, sl_len);
    return hipGetLastError();
}

}  // namespace ds
