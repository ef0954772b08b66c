// Draft proposal from the shortlist distribution (DynaSpec abstract: the
// drafter proposes from its shortlist while the target verifies over the
// full vocabulary; summary page, "Pipeline Flow": gathered projection, then
// sampling).
//
// One workgroup per head row.  The shortlist logits are read three times
// from L2 (a row is at most a few hundred KB): a max pass (fp32 max is exact
// and order-independent), the fp64 inverse-CDF draw over
// exp((l_j - max) / T) (see cdf.h), and a pass that writes
// q_j = exp((l_j - max) / T) / Z.  Temperature 0 takes the argmax, ties to
// the lowest shortlist index.
#include <float.h>

#include "cdf.h"
#include "common.h"
#include "kernels.h"

namespace ds {
namespace {

constexpr int kThreads = 512;

struct ExpWeights {
    const float *l;
    int64_t len;
    double mx, tau;
    __device__ void operator()(int64_t j0, double w[4]) const
    {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t j = j0 + k;
            w[k] = j < len ? exp(((double)l[j] - mx) / tau) : 0.0;
        }
    }
};

__device__ float block_max(float v, float *sh)
{
    v = wave_max(v);
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if (lane_id() == 0)
        sh[wave] = v;
    __syncthreads();
    float r = sh[0];
    for (int i = 1; i < nw; ++i)
        r = fmaxf(r, sh[i]);
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kThreads) void sample_kernel(int m, const int64_t *__restrict__ sl_off,
                                                          const int32_t *__restrict__ sl_ids,
                                                          const float *__restrict__ logits,
                                                          float temperature,
                                                          const float *__restrict__ u,
                                                          int32_t *__restrict__ token,
                                                          float *__restrict__ q)
{
    __shared__ double sh[kCdfShDoubles];
    __shared__ float shf[kThreads / kWave];
    __shared__ int s_int[2];
    const int64_t row = blockIdx.x;
    const int g = (int)(row / m), i = (int)(row % m);
    const int64_t off = sl_off[g], len = sl_off[g + 1] - off;
    if (len <= 0) {
        if (threadIdx.x == 0)
            token[row] = -1;
        return;
    }
    const int64_t base = (int64_t)m * off + (int64_t)i * len;
    const float *l = logits + base;
    float *qr = q + base;

    float mx = -FLT_MAX;
    for (int64_t j = threadIdx.x; j < len; j += blockDim.x)
        mx = fmaxf(mx, l[j]);
    mx = block_max(mx, shf);

    if (temperature == 0.0f) {
        if (threadIdx.x == 0)
            s_int[0] = 0x7fffffff;
        __syncthreads();
        for (int64_t j = threadIdx.x; j < len; j += blockDim.x)
            if (l[j] == mx) {
                atomicMin(&s_int[0], (int)j);
                break;
            }
        __syncthreads();
        const int jstar = s_int[0] == 0x7fffffff ? 0 : s_int[0];
        for (int64_t j = threadIdx.x; j < len; j += blockDim.x)
            qr[j] = j == jstar ? 1.0f : 0.0f;
        if (threadIdx.x == 0)
            token[row] = sl_ids[off + jstar];
        return;
    }

    ExpWeights f{l, len, (double)mx, (double)temperature};
    double Z;
    int64_t pick = block_inverse_cdf(f, len, (double)u[row], sh, s_int, &Z);
    for (int64_t j = threadIdx.x; j < len; j += blockDim.x)
        qr[j] = (float)(exp(((double)l[j] - f.mx) / f.tau) / Z);
    if (threadIdx.x == 0)
        token[row] = sl_ids[off + (pick < 0 ? 0 : pick)];
}

}  // namespace

hipError_t sample_launch(hipStream_t s, int G, int m, const int64_t *sl_off,
                         const int32_t *sl_ids, const float *logits, float temperature,
                         const float *u, int32_t *token, float *q)
{
    const int64_t rows = (int64_t)G * m;
    hipLaunchKernelGGL(sample_kernel, dim3((unsigned)rows), dim3(kThreads), 0, s, m, sl_off,
                       sl_ids, logits, temperature, u, token, q);
    return hipGetLastError();
}

}  // namespace ds
