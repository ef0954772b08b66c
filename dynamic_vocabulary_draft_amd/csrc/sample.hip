// Draft proposal from the shortlist distribution (DynaSpec abstract: the
// drafter proposes from its shortlist while the target verifies over the
// full vocabulary; summary page, "Pipeline Flow": gathered projection, then
// sampling), and the full-vocabulary target softmax (same normalisation on
// dense rows).
//
// Both run as the two chunked launches of dist.h, one 256-thread workgroup
// per 1024-element chunk of a row, so a 29K-entry shortlist is spread over
// 29 workgroups instead of one:
//   stats: chunk max m_c (fp32, exact), its first index, and the chunk sum
//          of exp((l - m_c) / T) in a fixed association;
//   final: row max M from the chunk maxima, chunk sums rescaled to M, their
//          prefixes and the row total rebuilt identically by every
//          workgroup; q (or p) = exp((l - M) / T) / total written as fp32;
//          the workgroup owning the threshold u * total walks its chunk.
// Temperature 0 is the argmax (ties to the lowest index) with one-hot q.
#include <float.h>

#include "common.h"
#include "dist.h"
#include "kernels.h"

namespace ds {
namespace {

constexpr int kMaxRowChunks = 1024;  // rows up to 2^20 entries

// Row r of the ragged shortlist layout: group g = r / m, head row i = r % m.
struct Ragged {
    const int64_t *sl_off;
    int m;
    __device__ void locate(int64_t row, int64_t *in_off, int64_t *len, int64_t *ids_off) const
    {
        const int64_t g = row / m, i = row % m;
        const int64_t off = sl_off[g];
        *len = sl_off[g + 1] - off;
        *in_off = (int64_t)m * off + i * (*len);
        *ids_off = off;
    }
};

// Row r of a dense [rows][V] array.
struct Dense {
    int64_t V;
    __device__ void locate(int64_t row, int64_t *in_off, int64_t *len, int64_t *ids_off) const
    {
        *len = V;
        *in_off = row * V;
        *ids_off = 0;
    }
};

__device__ __forceinline__ void load4(const float *__restrict__ l, int64_t j0, int64_t len,
                                      float v[4])
{
#pragma unroll
    for (int k = 0; k < 4; ++k)
        v[k] = j0 + k < len ? l[j0 + k] : -FLT_MAX;
}

// row max from the chunk maxima (order-independent), into every thread
__device__ float row_max(const float *__restrict__ cmax, int nch, float *sh)
{
    float m = -FLT_MAX;
    for (int c = threadIdx.x; c < nch; c += blockDim.x)
        m = fmaxf(m, cmax[c]);
    m = wave_max(m);
    if (lane_id() == 0)
        sh[threadIdx.x >> 6] = m;
    __syncthreads();
    float r = sh[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w)
        r = fmaxf(r, sh[w]);
    return r;
}

// chunk max m_c, first index of it, and the chunk sum of exp((l - m_c)/T)
template <class L>
__global__ __launch_bounds__(kChunkThreads) void norm_stats_kernel(L layout,
                                                                   const float *__restrict__ in,
                                                                   double tau, int64_t nchmax,
                                                                   void *ws, int64_t rows)
{
    __shared__ float s_max[4];
    __shared__ int s_idx[4];
    __shared__ double s_wt[4];
    const int64_t row = blockIdx.y, c = blockIdx.x;
    int64_t off, len, ids_off;
    layout.locate(row, &off, &len, &ids_off);
    if (c * kChunk >= len)
        return;
    ChunkWs w = chunk_ws(ws, rows, nchmax);
    const int64_t j0 = c * kChunk + (threadIdx.x >> 6) * 256 + lane_id() * 4;
    float v[4];
    load4(in + off, j0, len, v);
    block_chunk_max(v, j0, s_max, s_idx, &w.cmax[row * nchmax + c], &w.cidx[row * nchmax + c]);
    if (tau == 0.0)
        return;
    float mc = s_max[0];  // block_chunk_max ends after a barrier
    for (int i = 1; i < 4; ++i)
        mc = fmaxf(mc, s_max[i]);
    double wt[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        wt[k] = j0 + k < len ? exp(((double)v[k] - (double)mc) / tau) : 0.0;
    double incl;
    double tot = wave_chunk_sum(wt, &incl);
    if (lane_id() == 0)
        s_wt[threadIdx.x >> 6] = tot;
    __syncthreads();
    if (threadIdx.x == 0)
        w.csum[row * nchmax + c] = ((s_wt[0] + s_wt[1]) + s_wt[2]) + s_wt[3];
}

// chunk sums rescaled to the row max: csum_c * exp((m_c - M)/T), into LDS
__device__ void rescaled_sums(const float *__restrict__ cmax, const double *__restrict__ csum,
                              int nch, double mx, double tau, double *S)
{
    for (int c = threadIdx.x; c < nch; c += blockDim.x)
        S[c] = csum[c] * exp(((double)cmax[c] - mx) / tau);
    __syncthreads();
}

// PICK: draw a token with u (sampler); otherwise only normalise (softmax).
template <class L, bool PICK>
__global__ __launch_bounds__(kChunkThreads) void norm_final_kernel(
    L layout, const float *__restrict__ in, double tau, int64_t nchmax, const void *ws,
    int64_t rows, const int32_t *__restrict__ sl_ids, const float *__restrict__ u,
    int32_t *__restrict__ token, float *__restrict__ out)
{
    __shared__ double P[kMaxRowChunks], S[kMaxRowChunks], S2[kMaxRowChunks];
    __shared__ double s_wt[4];
    __shared__ double s_total;
    __shared__ float s_f[4];
    __shared__ int s_owner, s_fallback;
    __shared__ int64_t s_pick[2];
    const int64_t row = blockIdx.y, c = blockIdx.x;
    int64_t off, len, ids_off;
    layout.locate(row, &off, &len, &ids_off);
    if (PICK && c == 0 && len <= 0 && threadIdx.x == 0)
        token[row] = -1;
    if (c * kChunk >= len)
        return;
    ChunkWs w = chunk_ws(const_cast<void *>(ws), rows, nchmax);
    const int nch = (int)min(chunks_for(len), nchmax);  // rows beyond max_len: in bounds
    const float *cmax = w.cmax + row * nchmax;
    const double *csum = w.csum + row * nchmax;
    const float mxf = row_max(cmax, nch, s_f);
    const int64_t j0 = c * kChunk + (threadIdx.x >> 6) * 256 + lane_id() * 4;

    if (tau == 0.0) {  // argmax: the first chunk holding the max has its index
        if ((threadIdx.x >> 6) == 0) {
            int ca = nch - 1;
            for (int b = 0; b < nch; b += kWave) {
                const uint64_t bal = __ballot(b + lane_id() < nch && cmax[b + lane_id()] == mxf);
                if (bal) {
                    ca = b + __ffsll((unsigned long long)bal) - 1;
                    break;
                }
            }
            if (lane_id() == 0) {
                s_owner = ca;
                s_fallback = w.cidx[row * nchmax + ca];
            }
        }
        __syncthreads();
        const int64_t jstar = s_fallback;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (j0 + k < len)
                out[off + j0 + k] = j0 + k == jstar ? 1.0f : 0.0f;
        if (PICK && c == s_owner && threadIdx.x == 0)
            token[row] = sl_ids[ids_off + jstar];
        return;
    }

    const double mx = (double)mxf;
    rescaled_sums(cmax, csum, nch, mx, tau, S2);
    const double Z = row_prefix(S2, nch, P, S, &s_total);
    double wt[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        wt[k] = j0 + k < len ? exp(((double)in[off + j0 + k] - mx) / tau) : 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (j0 + k < len)
            out[off + j0 + k] = (float)(wt[k] / Z);
    if (!PICK)
        return;
    const double thr = (double)u[row] * Z;
    owner_chunk(P, S, nch, thr, &s_owner, &s_fallback);
    if (c != s_owner)
        return;
    double incl;
    double tot = wave_chunk_sum(wt, &incl);
    if (lane_id() == 0)
        s_wt[threadIdx.x >> 6] = tot;
    __syncthreads();
    int64_t pick = chunk_walk(wt, j0, s_wt, incl, P[c], thr, s_fallback != 0, s_pick);
    if (threadIdx.x == 0)
        token[row] = sl_ids[ids_off + (pick < 0 ? 0 : pick)];
}

template <class L, bool PICK>
hipError_t launch_norm(hipStream_t s, L layout, int64_t rows, int64_t max_len, const float *in,
                       double tau, void *ws, const int32_t *sl_ids, const float *u,
                       int32_t *token, float *out)
{
    const int64_t nchmax = chunks_for(max_len > 0 ? max_len : 1);
    dim3 grid((unsigned)nchmax, (unsigned)rows);
    hipLaunchKernelGGL((norm_stats_kernel<L>), grid, dim3(kChunkThreads), 0, s, layout, in, tau,
                       nchmax, ws, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((norm_final_kernel<L, PICK>), grid, dim3(kChunkThreads), 0, s, layout, in,
                       tau, nchmax, (const void *)ws, rows, sl_ids, u, token, out);
    return hipGetLastError();
}

}  // namespace

size_t sample_ws_bytes(int64_t rows, int64_t max_len)
{
    return chunk_ws_bytes(rows, chunks_for(max_len > 0 ? max_len : 1));
}

hipError_t sample_launch(hipStream_t s, int G, int m, const int64_t *sl_off,
                         const int32_t *sl_ids, const float *logits, float temperature,
                         const float *u, int32_t *token, float *q, int64_t max_len, void *ws)
{
    Ragged layout{sl_off, m};
    return launch_norm<Ragged, true>(s, layout, (int64_t)G * m, max_len, logits,
                                     (double)temperature, ws, sl_ids, u, token, q);
}

size_t softmax_ws_bytes(int64_t rows, int64_t V) { return chunk_ws_bytes(rows, chunks_for(V)); }

hipError_t softmax_launch(hipStream_t s, int rows, int V, const float *logits, float *p, void *ws)
{
    Dense layout{V};
    return launch_norm<Dense, false>(s, layout, rows, V, logits, 1.0, ws, nullptr, nullptr,
                                     nullptr, p);
}

}  // namespace ds
