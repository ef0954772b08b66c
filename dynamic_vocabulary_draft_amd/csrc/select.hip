// Top-cluster selection under a position-aware budget (DynaSpec abstract:
// the shortlist is the union of the best-scoring clusters; summary page,
// "Key Novelty" and "Key Hyperparameters": a budget k_c(t) that decays with
// the draft position).
//
// One workgroup per row.  Every cluster gets a unique 64-bit key: the
// order-preserving bits of its score, inverted so that ascending keys are
// descending scores, above the cluster id; ascending keys are then exactly
// the order (score desc, id asc).  The selection is a prefix of that order
// ending at the first cluster where the running total reaches the target
// (the budget's token count with the cluster sizes as weights, or its
// cluster count with unit weights): with a token budget, a cluster is taken
// iff the tokens ranked before it fall short of the budget.  That last key
// is found without sorting, by a weighted radix search from the most
// significant bits: per pass a 4096-bin LDS histogram (12 bits) of the
// weights of the keys still in play, a block-wide scan for the bin where the
// running total reaches the target, and the next 12 bits within that bin,
// until one key is left (two passes for distinct scores).  Only the taken
// clusters are then ranked, each by counting the taken keys below its own
// (several threads per key), and written in that order.
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

constexpr int kSelThreads = 1024;
constexpr int kDigitBits = 12;
constexpr int kBins = 1 << kDigitBits;  // 4 bins per thread

// PART: the scores are the router's second-layer window partials
// wpart[w][row][idx] (nwin windows, window stride kRouterPassCols * M) added
// in window order plus the bias, exactly as the router's finish adds them;
// they are written to sc_out and selected from
template <int KPT, bool PART>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    int M, const float *__restrict__ scores, const float *__restrict__ wpart, int nwin,
    const uint16_t *__restrict__ b2, float *__restrict__ sc_out,
    const int32_t *__restrict__ cluster_size, int kind, const int32_t *__restrict__ budget,
    int32_t *__restrict__ sel, int32_t *__restrict__ n_sel, int32_t *__restrict__ sl_len)
{
    // weight histogram of one pass, then the taken keys
    __shared__ unsigned long long s_hw[kBins];
    __shared__ int s_hc[kBins];
    __shared__ int64_t scan_sh[kWave + 1];
    __shared__ int s_digit, s_cnt, s_ntake;
    __shared__ long long s_below;
    __shared__ unsigned long long s_kstar, s_tok;
    const int row = blockIdx.x, tid = threadIdx.x;
    const float *s = PART ? nullptr : scores + (int64_t)row * M;
    const bool tokens = kind != DS_BUDGET_CLUSTERS;
    uint64_t k[KPT];
    int64_t w[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int idx = tid + i * kSelThreads;
        const bool in = idx < M;
        float sc = 0.f;
        if (PART) {
            if (in) {
                const float *pp = wpart + (int64_t)row * M + idx;
                for (int w0 = 0; w0 < nwin; w0 += 8) {  // eight loads in flight
                    float v[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        v[j] = w0 + j < nwin ? pp[(int64_t)(w0 + j) * kRouterPassCols * M] : 0.f;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (w0 + j < nwin)
                            sc += v[j];
                }
                if (b2)
                    sc += __uint_as_float((uint32_t)b2[idx] << 16);
                sc_out[(int64_t)row * M + idx] = sc;
            }
        } else if (in) {
            sc = s[idx];
        }
        k[i] = in ? ((uint64_t)(~ordered_bits(sc)) << 32) | (uint32_t)idx : ~0ull;
        w[i] = in ? (tokens ? (int64_t)max(cluster_size[idx], 0) : 1) : 0;
    }
    const int32_t bud = budget[row];
    const int64_t target = tokens ? (bud < 1 ? 1 : (int64_t)bud) : (bud < 1 ? 1 : (bud > M ? M : bud));
    if (tid == 0) {
        s_ntake = 0;
        s_tok = 0;
    }

    uint64_t kstar = ~0ull;  // the last taken key (all of them when the target is out of reach)
    uint64_t prefix = 0;     // the key bits above `shift` fixed so far
    int64_t below = 0;       // weight of the keys below that prefix
    int shift = 64;
    for (;;) {
        const int bits = shift >= kDigitBits ? kDigitBits : shift;
        shift -= bits;
        const uint64_t dmask = ((uint64_t)1 << bits) - 1;
#pragma unroll
        for (int q = 0; q < kBins / kSelThreads; ++q) {
            s_hw[tid + q * kSelThreads] = 0;
            s_hc[tid + q * kSelThreads] = 0;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const bool cand = tid + i * kSelThreads < M &&
                              (shift + bits == 64 || (k[i] >> (shift + bits)) == prefix);
            if (cand) {
                const int d = (int)((k[i] >> shift) & dmask);
                if (w[i])
                    atomicAdd(&s_hw[d], (unsigned long long)w[i]);
                atomicAdd(&s_hc[d], 1);
            }
        }
        __syncthreads();
        // the first bin where below + (weights of the bins up to it) >= target
        constexpr int BPT = kBins / kSelThreads;
        int64_t bw[BPT], local = 0;
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            bw[q] = (int64_t)s_hw[tid * BPT + q];
            local += bw[q];
        }
        int64_t total;
        int64_t run = below + block_excl_scan_i64(local, scan_sh, &total);
        if (shift + bits == 64 && total < target)  // block-uniform: the whole order is taken
            break;
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            if (run < target && run + bw[q] >= target) {
                s_digit = tid * BPT + q;
                s_below = run;
                s_cnt = s_hc[tid * BPT + q];
            }
            run += bw[q];
        }
        __syncthreads();
        prefix = (prefix << bits) | (uint64_t)s_digit;
        below = s_below;
        if (s_cnt == 1 || shift == 0) {  // one key left in the bin: it is the cut
#pragma unroll
            for (int i = 0; i < KPT; ++i)
                if (tid + i * kSelThreads < M && (k[i] >> shift) == prefix)
                    s_kstar = k[i];
            __syncthreads();
            kstar = s_kstar;
            break;
        }
        __syncthreads();  // every thread has read the pass's result
    }

    // the taken keys (k <= kstar) into LDS, in any order; their count and
    // token total (integer sums: the same whatever the order)
    uint64_t *taken = reinterpret_cast<uint64_t *>(s_hw);
    static_assert(kBins >= kSelThreads * KPT, "room for every key");
    __syncthreads();  // the histogram is no longer read
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int idx = tid + i * kSelThreads;
        if (idx < M && k[i] <= kstar) {
            taken[atomicAdd(&s_ntake, 1)] = k[i];
            const int32_t sz = cluster_size[idx];
            if (sz > 0)
                atomicAdd(&s_tok, (unsigned long long)sz);
        }
    }
    __syncthreads();
    const int nt = s_ntake;
    int32_t *out = sel + (int64_t)row * M;
    // rank of each taken key = the number of smaller taken keys: P threads
    // per key (a power of two) each count a strided share, then add up
    int P = 1;
    while (P * 2 * nt <= kSelThreads && P < kWave)
        P *= 2;
    const int part = tid & (P - 1);
    for (int a0 = 0; a0 < nt; a0 += kSelThreads / P) {  // block-uniform trip count
        const int a = a0 + tid / P;
        const uint64_t ka = a < nt ? taken[a] : 0ull;
        int r = 0;
        if (a < nt)
            for (int j = part; j < nt; j += P)
                r += taken[j] < ka;
        for (int o = 1; o < P; o <<= 1)
            r += __shfl_xor(r, o);
        if (a < nt && part == 0)
            out[r] = (int32_t)(uint32_t)ka;
    }
    for (int j = nt + tid; j < M; j += kSelThreads)
        out[j] = -1;
    if (tid == 0) {
        n_sel[row] = nt;
        sl_len[row] = (int32_t)s_tok;
    }
}

}  // namespace

namespace {

template <bool PART>
hipError_t select_any(hipStream_t s, int n, int M, const float *scores, const float *part,
                      int nwin, const uint16_t *b2, float *sc_out, const int32_t *cluster_size,
                      int kind, const int32_t *budget, int32_t *sel, int32_t *n_sel,
                      int32_t *sl_len)
{
    const int kpt = (M + kSelThreads - 1) / kSelThreads;  // M <= 4096
    if (kpt == 1)
        hipLaunchKernelGGL((select_kernel<1, PART>), dim3(n), dim3(kSelThreads), 0, s, M, scores,
                           part, nwin, b2, sc_out, cluster_size, kind, budget, sel, n_sel, sl_len);
    else if (kpt == 2)
        hipLaunchKernelGGL((select_kernel<2, PART>), dim3(n), dim3(kSelThreads), 0, s, M, scores,
                           part, nwin, b2, sc_out, cluster_size, kind, budget, sel, n_sel, sl_len);
    else
        hipLaunchKernelGGL((select_kernel<4, PART>), dim3(n), dim3(kSelThreads), 0, s, M, scores,
                           part, nwin, b2, sc_out, cluster_size, kind, budget, sel, n_sel, sl_len);
    return hipGetLastError();
}

}  // namespace

hipError_t select_launch(hipStream_t s, int n, int M, const float *scores,
                         const int32_t *cluster_size, int kind, const int32_t *budget,
                         int32_t *sel, int32_t *n_sel, int32_t *sl_len)
{
    return select_any<false>(s, n, M, scores, nullptr, 0, nullptr, nullptr, cluster_size, kind,
                             budget, sel, n_sel, sl_len);
}

hipError_t select_partials_launch(hipStream_t s, int n, int M, const float *part, int nwin,
                                  const void *b2, float *scores, const int32_t *cluster_size,
                                  int kind, const int32_t *budget, int32_t *sel, int32_t *n_sel,
                                  int32_t *sl_len)
{
    return select_any<true>(s, n, M, nullptr, part, nwin, reinterpret_cast<const uint16_t *>(b2),
                            scores, cluster_size, kind, budget, sel, n_sel, sl_len);
}

}  // namespace ds
