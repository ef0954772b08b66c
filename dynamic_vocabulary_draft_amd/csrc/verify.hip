// Target side of the speculative step: full-vocabulary target distribution
// and rejection-sampling verification, which keeps the emitted tokens
// distributed exactly as the target (DynaSpec abstract: "the target model
// still verifies over the full vocabulary, preserving exactness"; summary
// page, "Pipeline Flow: Rejection Sampling Verification"; the accept /
// residual / bonus rules are textbook speculative sampling).
//
// softmax: one workgroup per row, three coalesced passes (fp32 max, fp64 sum
// of exp(l - max) with a fixed reduction order, fp32 write of the ratio).
//
// verify: one workgroup per sequence.  Wave 0 evaluates the T accept tests
// at once (lane t: binary search of the draft token in its ascending
// shortlist, exact fp64 product u*q against p) and finds the first
// rejection with a ballot.  The draw then scans all V tokens once through
// the block inverse CDF: for a rejection the weights are max(0, p - q),
// where q is scattered chunk by chunk into per-wave LDS from the shortlist
// (a table of chunk starts, built in one pass over the shortlist, says
// which entries fall in each 256-token chunk); otherwise the weights are
// the bonus position's p.
#include <float.h>

#include "cdf.h"
#include "common.h"
#include "kernels.h"

namespace ds {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxSub = 4096;  // 256-token chunks of V in the start table

struct ProbWeights {
    const float *p;
    int64_t V;
    __device__ void operator()(int64_t j0, double w[4]) const
    {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = j0 + k < V ? (double)p[j0 + k] : 0.0;
    }
};

struct ResidualWeights {
    const float *p;       // target probabilities of the rejected position
    const int32_t *S;     // its shortlist (ascending token ids)
    const float *q;       // draft probabilities aligned with S
    const int *start;     // LDS: first shortlist entry of every 256-token chunk
    float *qbuf;          // LDS: 256 floats per wave
    int64_t V;
    __device__ void operator()(int64_t j0, double w[4]) const
    {
        const int lane = lane_id();
        const int64_t base = j0 - lane * 4;
        const int sc = (int)(base >> 8);
        float *buf = qbuf + (threadIdx.x >> 6) * 256;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            buf[lane * 4 + k] = 0.f;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int e = start[sc] + lane; e < start[sc + 1]; e += kWave) {
            const int64_t off = (int64_t)S[e] - base;
            if (off >= 0 && off < 256)
                buf[off] = q[e];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t y = j0 + k;
            double r = y < V ? (double)p[y] - (double)buf[lane * 4 + k] : 0.0;
            w[k] = r > 0.0 ? r : 0.0;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
};

__global__ __launch_bounds__(kThreads) void softmax_kernel(int V, const float *__restrict__ logits,
                                                           float *__restrict__ p)
{
    __shared__ float shf[kThreads / kWave];
    __shared__ double shd[kThreads / kWave];
    const int64_t row = blockIdx.x;
    const float *l = logits + row * V;
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    float mx = -FLT_MAX;
    for (int y = threadIdx.x; y < V; y += blockDim.x)
        mx = fmaxf(mx, l[y]);
    mx = wave_max(mx);
    if (lane_id() == 0)
        shf[wave] = mx;
    __syncthreads();
    mx = shf[0];
    for (int i = 1; i < nw; ++i)
        mx = fmaxf(mx, shf[i]);
    const double dmx = (double)mx;
    double z = 0.0;
    for (int y = threadIdx.x; y < V; y += blockDim.x)
        z += exp((double)l[y] - dmx);
    z = wave_sum_f64(z);
    if (lane_id() == 0)
        shd[wave] = z;
    __syncthreads();
    double Z = shd[0];
    for (int i = 1; i < nw; ++i)
        Z += shd[i];
    for (int y = threadIdx.x; y < V; y += blockDim.x)
        p[row * V + y] = (float)(exp((double)l[y] - dmx) / Z);
}

__global__ __launch_bounds__(kThreads) void verify_kernel(int B, int T, int V,
                                                          const int32_t *__restrict__ draft,
                                                          const int64_t *__restrict__ sl_off,
                                                          const int32_t *__restrict__ sl_ids,
                                                          const float *__restrict__ q,
                                                          const float *__restrict__ p,
                                                          const float *__restrict__ u_acc,
                                                          const float *__restrict__ u_fin,
                                                          int32_t *__restrict__ n_acc,
                                                          int32_t *__restrict__ out)
{
    __shared__ double sh[kCdfShDoubles];
    __shared__ int start[kMaxSub + 1];
    __shared__ float qbuf[(kThreads / kWave) * 256];
    __shared__ int s_int[2];
    __shared__ int s_tstar;
    const int b = blockIdx.x, lane = lane_id(), wave = threadIdx.x >> 6;

    if (wave == 0) {
        bool reject = false;
        if (lane < T) {
            const int64_t row = (int64_t)lane * B + b;
            const int32_t x = draft[row];
            int64_t lo = sl_off[row], hi = sl_off[row + 1];
            while (lo < hi) {  // lower_bound of x in the ascending shortlist
                int64_t mid = (lo + hi) >> 1;
                if (sl_ids[mid] < x)
                    lo = mid + 1;
                else
                    hi = mid;
            }
            const bool found = lo < sl_off[row + 1] && sl_ids[lo] == x;
            const double qx = found ? (double)q[lo] : 0.0;
            const double px = (x >= 0 && x < V) ? (double)p[((int64_t)b * (T + 1) + lane) * V + x] : 0.0;
            reject = !((double)u_acc[row] * qx < px);
        }
        uint64_t bal = __ballot(reject);
        const int tstar = bal ? __ffsll((unsigned long long)bal) - 1 : T;
        if (lane == 0)
            s_tstar = tstar;
        for (int k = lane; k <= T; k += kWave)
            if (k != tstar)  // entry tstar is written once the draw is known
                out[(int64_t)b * (T + 1) + k] = k < tstar ? draft[(int64_t)k * B + b] : -1;
        if (lane == 0)
            n_acc[b] = tstar;
    }
    __syncthreads();
    const int tstar = s_tstar;
    const double uf = (double)u_fin[b];
    const float *pt = p + ((int64_t)b * (T + 1) + tstar) * V;
    int64_t pick;
    double total;
    if (tstar < T) {
        const int64_t row = (int64_t)tstar * B + b;
        const int64_t lo = sl_off[row], len = sl_off[row + 1] - lo;
        const int32_t *S = sl_ids + lo;
        const int nsub = (V + 255) >> 8;
        // start[c] = first shortlist entry with token id >= 256*c.  Every
        // entry is preset to len so the table stays within [0, len] even if
        // the shortlist is not ascending (invalid input).
        for (int c = threadIdx.x; c <= nsub; c += blockDim.x)
            start[c] = (int)len;
        __syncthreads();
        for (int64_t e = threadIdx.x; e < len; e += blockDim.x) {
            const int cy = S[e] >> 8;
            const int cp = e > 0 ? (S[e - 1] >> 8) : -1;
            for (int c = cp + 1 > 0 ? cp + 1 : 0; c <= cy && c <= nsub; ++c)
                start[c] = (int)e;
        }
        __syncthreads();
        ResidualWeights rw{pt, S, q + lo, start, qbuf, V};
        pick = block_inverse_cdf(rw, V, uf, sh, s_int, &total);
        if (!(total > 0.0)) {
            ProbWeights pw{pt, V};
            pick = block_inverse_cdf(pw, V, uf, sh, s_int, &total);
        }
    } else {
        ProbWeights pw{pt, V};
        pick = block_inverse_cdf(pw, V, uf, sh, s_int, &total);
    }
    if (threadIdx.x == 0)
        out[(int64_t)b * (T + 1) + tstar] = (int32_t)pick;
}

}  // namespace

hipError_t softmax_launch(hipStream_t s, int rows, int V, const float *logits, float *p)
{
    hipLaunchKernelGGL(softmax_kernel, dim3(rows), dim3(kThreads), 0, s, V, logits, p);
    return hipGetLastError();
}

hipError_t verify_launch(hipStream_t s, int B, int T, int V, const int32_t *draft,
                         const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                         const float *p, const float *u_acc, const float *u_fin, int32_t *n_acc,
                         int32_t *out)
{
    hipLaunchKernelGGL(verify_kernel, dim3(B), dim3(kThreads), 0, s, B, T, V, draft, sl_off,
                       sl_ids, q, p, u_acc, u_fin, n_acc, out);
    return hipGetLastError();
}

}  // namespace ds
