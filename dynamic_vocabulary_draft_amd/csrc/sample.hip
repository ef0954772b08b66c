// Draft proposal from the shortlist distribution (DynaSpec abstract: the
// drafter proposes from its shortlist while the target verifies over the
// full vocabulary; summary page, "Pipeline Flow": gathered projection, then
// sampling), and the full-vocabulary target softmax (same normalisation on
// dense rows).
//
// The sampler runs as the two chunked launches of dist.h over 1024-element
// chunks, one 256-thread workgroup per chunk when the launch is small (a
// 29K-entry shortlist is spread over 29 workgroups instead of one), several
// consecutive chunks per workgroup when it is large:
//   stats: chunk max m_c (fp32, exact), its first index, and the chunk sum
//          of exp((l - m_c) / T) in a fixed association;
//   final: row max M from the chunk maxima, chunk sums rescaled to M, their
//          prefixes and the row total rebuilt identically by every
//          workgroup; q (or p) = exp((l - M) / T) * (1 / total) written as
//          fp32 (within one fp32 ulp of the quotient);
//          the workgroup owning the threshold u * total walks its chunk.
// Temperature 0 is the argmax (ties to the lowest index) with one-hot q.
// The target softmax draws nothing, so it needs no prefix sums: two launches
// over 4096-element segments, the first writing each segment's max and sum
// of exp(l - max), the second rebuilding the row max and total in every
// wave and writing p.
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

// chunk max m_c, first index of it, and the chunk sum of exp((l - m_c)/T);
// a workgroup handles R consecutive chunks of a row: all loads issued first,
// then each step done for the R chunks side by side, so the workgroup waits
// at two barriers in all rather than three per chunk.  Per chunk the
// reductions are those of block_chunk_max and wave_chunk_sum (the same
// values and summation order as one chunk at a time).
template <class L, int R>
__global__ __launch_bounds__(kChunkThreads) void norm_stats_kernel(L layout,
                                                                   const float *__restrict__ in,
                                                                   double tau, int64_t nchmax,
                                                                   void *ws, int64_t rows)
{
    constexpr int NW = kChunkThreads / kWave;
    __shared__ float s_max[R][NW];
    __shared__ int s_idx[R][NW];
    __shared__ double s_wt[R][NW];
    __shared__ double s_exp2[64];
    const int64_t row = blockIdx.y, c0 = (int64_t)blockIdx.x * R;
    int64_t off, len, ids_off;
    layout.locate(row, &off, &len, &ids_off);
    if (c0 * kChunk >= len)
        return;
    ChunkWs w = chunk_ws(ws, rows, nchmax);
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t jl = wave * 256 + lane * 4;  // lane's offset in a chunk
    float v[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
        load4(in + off, (c0 + r) * kChunk + jl, len, v[r]);
    fill_exp2_table(s_exp2);  // ordered before its use by the first barrier
    // chunks c0 .. c0+nr-1 hold entries (block-uniform)
    const int nr = (int)min((int64_t)R, min(nchmax, (len + kChunk - 1) / kChunk) - c0);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r >= nr)
            break;
        float m = v[r][0];
        int idx = 0;
#pragma unroll
        for (int k = 1; k < 4; ++k)
            if (v[r][k] > m) {
                m = v[r][k];
                idx = k;
            }
        const float wm = wave_max(m);
        const uint64_t bal = __ballot(m == wm);
        const int first = __shfl((int)((c0 + r) * kChunk + jl + idx),
                                 __ffsll((unsigned long long)bal) - 1);
        if (lane == 0) {
            s_max[r][wave] = wm;
            s_idx[r][wave] = first;
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < nr) {  // thread r: chunk c0 + r, the first wave's index on ties
        const int r = (int)threadIdx.x;
        float bm = s_max[r][0];
        int bi = s_idx[r][0];
        for (int q = 1; q < NW; ++q)
            if (s_max[r][q] > bm) {
                bm = s_max[r][q];
                bi = s_idx[r][q];
            }
        w.cmax[row * nchmax + c0 + r] = bm;
        w.cidx[row * nchmax + c0 + r] = bi;
    }
    if (tau == 0.0)
        return;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r >= nr)
            break;
        float mc = s_max[r][0];
        for (int q = 1; q < NW; ++q)
            mc = fmaxf(mc, s_max[r][q]);
        const int64_t j0 = (c0 + r) * kChunk + jl;
        double wt[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            wt[k] = j0 + k < len ? exp_tab(over_tau((double)v[r][k] - (double)mc, tau), s_exp2)
                                 : 0.0;
        double incl;
        const double tot = wave_chunk_sum(wt, &incl);
        if (lane == 0)
            s_wt[r][wave] = tot;
    }
    __syncthreads();
    if ((int)threadIdx.x < nr) {
        const int r = (int)threadIdx.x;
        w.csum[row * nchmax + c0 + r] = ((s_wt[r][0] + s_wt[r][1]) + s_wt[r][2]) + s_wt[r][3];
    }
}

// chunk sums rescaled to the row max: csum_c * exp((m_c - M)/T), into LDS
__device__ void rescaled_sums(const float *__restrict__ cmax, const double *__restrict__ csum,
                              int nch, double mx, double tau, const double *tab, double *S)
{
    for (int c = threadIdx.x; c < nch; c += blockDim.x)
        S[c] = csum[c] * exp_tab(over_tau((double)cmax[c] - mx, tau), tab);
    __syncthreads();
}

// PICK: draw a token with u (sampler); otherwise only normalise (softmax).
// A workgroup handles R consecutive chunks of a row: the row statistics are
// rebuilt once for all of them, after the chunks' loads have been issued.
template <class L, bool PICK, int R>
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
    __shared__ double s_exp2[64];
    const int64_t row = blockIdx.y, c0 = (int64_t)blockIdx.x * R;
    int64_t off, len, ids_off;
    layout.locate(row, &off, &len, &ids_off);
    if (PICK && c0 == 0 && len <= 0 && threadIdx.x == 0)
        token[row] = -1;
    if (c0 * kChunk >= len)
        return;
    ChunkWs w = chunk_ws(const_cast<void *>(ws), rows, nchmax);
    const int nch = (int)min(chunks_for(len), nchmax);  // rows beyond max_len: in bounds
    const int64_t jl = (threadIdx.x >> 6) * 256 + lane_id() * 4;
    float v[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
        load4(in + off, (c0 + r) * kChunk + jl, (c0 + r) < nch ? len : 0, v[r]);
    const float *cmax = w.cmax + row * nchmax;
    const double *csum = w.csum + row * nchmax;
    fill_exp2_table(s_exp2);  // ordered before its use by the barrier in row_max
    const float mxf = row_max(cmax, nch, s_f);

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
        for (int r = 0; r < R; ++r) {
            const int64_t j0 = (c0 + r) * kChunk + jl;
            if (c0 + r >= nch)
                break;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (j0 + k < len)
                    out[off + j0 + k] = j0 + k == jstar ? 1.0f : 0.0f;
        }
        if (PICK && s_owner >= c0 && s_owner < c0 + R && threadIdx.x == 0)
            token[row] = sl_ids[ids_off + jstar];
        return;
    }

    const double mx = (double)mxf;
    rescaled_sums(cmax, csum, nch, mx, tau, s_exp2, S2);
    const double Z = row_prefix(S2, nch, P, S, &s_total);
    const double rZ = 1.0 / Z;  // q = w * (1/Z): within one fp32 ulp of w / Z
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t j0 = (c0 + r) * kChunk + jl;
        if (c0 + r >= nch)
            break;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (j0 + k < len)
                out[off + j0 + k] = q_elem(v[r][k], mxf, rZ, tau, s_exp2);
    }
    if (!PICK)
        return;
    const double thr = (double)u[row] * Z;
    owner_chunk(P, S, nch, thr, &s_owner, &s_fallback);
    const int64_t c = s_owner;
    if (c < c0 || c >= c0 + R)
        return;
    // the owner chunk's weights again (same operations, same values)
    const int64_t j0 = c * kChunk + jl;
    double wt[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (c0 + r == c) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                wt[k] = j0 + k < len ? draft_w(v[r][k], mx, tau, s_exp2) : 0.0;
        }
    double incl;
    double tot = wave_chunk_sum(wt, &incl);
    if (lane_id() == 0)
        s_wt[threadIdx.x >> 6] = tot;
    __syncthreads();
    int64_t pick = chunk_walk(wt, j0, s_wt, incl, P[c], thr, s_fallback != 0, s_pick);
    if (threadIdx.x == 0)
        token[row] = sl_ids[ids_off + (pick < 0 ? 0 : pick)];
}

// The draw without q (tau > 0): one workgroup per row rebuilds the row's
// statistics exactly as norm_final_kernel does, stores (M, 1 / Z), and walks
// the chunk holding u * Z with the same weights, so the token is the one
// norm_final_kernel draws and q_elem of the logits gives its q bit for bit.
template <class L>
__global__ __launch_bounds__(kChunkThreads) void norm_pick_kernel(
    L layout, const float *__restrict__ in, double tau, int64_t nchmax, const void *ws,
    int64_t rows, const int32_t *__restrict__ sl_ids, const float *__restrict__ u,
    int32_t *__restrict__ token, QStats *__restrict__ qs)
{
    __shared__ double P[kMaxRowChunks], S[kMaxRowChunks], S2[kMaxRowChunks];
    __shared__ double s_wt[4];
    __shared__ double s_total;
    __shared__ float s_f[4];
    __shared__ int s_owner, s_fallback;
    __shared__ int64_t s_pick[2];
    __shared__ double s_exp2[64];
    const int64_t row = blockIdx.x;
    int64_t off, len, ids_off;
    layout.locate(row, &off, &len, &ids_off);
    if (len <= 0) {
        if (threadIdx.x == 0) {
            token[row] = -1;
            qs[row] = QStats{0.0f, 0, 0.0};
        }
        return;
    }
    ChunkWs w = chunk_ws(const_cast<void *>(ws), rows, nchmax);
    const int nch = (int)min(chunks_for(len), nchmax);  // rows beyond max_len: in bounds
    const float *cmax = w.cmax + row * nchmax;
    const double *csum = w.csum + row * nchmax;
    fill_exp2_table(s_exp2);  // ordered before its use by the barrier in row_max
    const float mxf = row_max(cmax, nch, s_f);
    const double mx = (double)mxf;
    rescaled_sums(cmax, csum, nch, mx, tau, s_exp2, S2);
    const double Z = row_prefix(S2, nch, P, S, &s_total);
    const double rZ = 1.0 / Z;
    if (threadIdx.x == 0)
        qs[row] = QStats{mxf, 0, rZ};
    const double thr = (double)u[row] * Z;
    owner_chunk(P, S, nch, thr, &s_owner, &s_fallback);
    const int64_t c = s_owner;
    if (c < 0)
        return;  // as in norm_final_kernel: no chunk with mass
    const int64_t j0 = c * kChunk + (threadIdx.x >> 6) * 256 + lane_id() * 4;
    float v[4];
    load4(in + off, j0, len, v);
    double wt[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        wt[k] = j0 + k < len ? draft_w(v[k], mx, tau, s_exp2) : 0.0;
    double incl;
    const double tot = wave_chunk_sum(wt, &incl);
    if (lane_id() == 0)
        s_wt[threadIdx.x >> 6] = tot;
    __syncthreads();
    const int64_t pick = chunk_walk(wt, j0, s_wt, incl, P[c], thr, s_fallback != 0, s_pick);
    if (threadIdx.x == 0)
        token[row] = sl_ids[ids_off + (pick < 0 ? 0 : pick)];
}

template <class L, bool PICK, int R>
hipError_t launch_norm_r(hipStream_t s, L layout, int64_t rows, int64_t nchmax, const float *in,
                         double tau, void *ws, const int32_t *sl_ids, const float *u,
                         int32_t *token, float *out)
{
    dim3 grid((unsigned)((nchmax + R - 1) / R), (unsigned)rows);
    hipLaunchKernelGGL((norm_stats_kernel<L, R>), grid, dim3(kChunkThreads), 0, s, layout, in, tau,
                       nchmax, ws, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((norm_final_kernel<L, PICK, R>), grid, dim3(kChunkThreads), 0, s, layout,
                       in, tau, nchmax, (const void *)ws, rows, sl_ids, u, token, out);
    return hipGetLastError();
}

// Chunks per workgroup: one by default (a short shortlist still spreads
// over many workgroups); two for launches of 256 rows or more (the 512 rows
// of 8 trees x 64 nodes: tree step 0.590 -> 0.582 ms; the same at 32 rows
// cost 16 us per step); four for long rows in large launches, where every
// workgroup would otherwise rebuild the statistics of hundreds of chunks.
template <class L, bool PICK>
hipError_t launch_norm(hipStream_t s, L layout, int64_t rows, int64_t max_len, const float *in,
                       double tau, void *ws, const int32_t *sl_ids, const float *u,
                       int32_t *token, float *out)
{
    const int64_t nchmax = chunks_for(max_len > 0 ? max_len : 1);
    if (rows >= 256 && nchmax >= 16)  // many rows (tree nodes): two chunks per workgroup
        return launch_norm_r<L, PICK, 2>(s, layout, rows, nchmax, in, tau, ws, sl_ids, u, token,
                                         out);
    if (nchmax >= 64 && rows * nchmax / 4 >= 2048)
        return launch_norm_r<L, PICK, 4>(s, layout, rows, nchmax, in, tau, ws, sl_ids, u, token,
                                         out);
    return launch_norm_r<L, PICK, 1>(s, layout, rows, nchmax, in, tau, ws, sl_ids, u, token, out);
}

// ------------------------------------------------------------ target softmax
// Segment statistics (segment_stats in dist.h), one workgroup per segment.
__global__ __launch_bounds__(kChunkThreads) void softmax_stats_kernel(int64_t V,
                                                                      const float *__restrict__ in,
                                                                      double *__restrict__ ssum,
                                                                      float *__restrict__ smax)
{
    const int64_t row = blockIdx.y, nseg = gridDim.x;
    segment_stats(V, in + row * V, blockIdx.x, &ssum[row * nseg + blockIdx.x],
                  &smax[row * nseg + blockIdx.x]);
}

// p = exp(l - M) * (1 / Z), M the row max, Z = sum over segments of
// ssum_s * exp(smax_s - M); every wave rebuilds M and Z in the same order,
// so all workgroups of a row use the same values.
__global__ __launch_bounds__(kChunkThreads) void softmax_final_kernel(
    int64_t V, const float *__restrict__ in, const double *__restrict__ ssum,
    const float *__restrict__ smax, float *__restrict__ p)
{
    __shared__ double s_exp2[64];
    const int64_t row = blockIdx.y, nseg = gridDim.x;
    const int64_t j0 = (int64_t)blockIdx.x * kSeg + (threadIdx.x >> 6) * 256 + lane_id() * 4;
    float v[4][4];
    load_seg(in + row * V, j0, V, v);
    fill_exp2_table(s_exp2);
    __syncthreads();  // the table
    float M;
    double rZ;
    row_norm(smax + row * nseg, ssum + row * nseg, nseg, s_exp2, &M, &rZ);
    float *pr = p + row * V;
    const bool vec = (reinterpret_cast<uintptr_t>(pr) & 15) == 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t j = j0 + i * kChunk;
        float o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            o[k] = p_elem(v[i][k], M, rZ, s_exp2);
        if (vec && j + 3 < V) {
            *reinterpret_cast<float4 *>(pr + j) = make_float4(o[0], o[1], o[2], o[3]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (j + k < V)
                    pr[j + k] = o[k];
        }
    }
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

hipError_t sample_stats_launch(hipStream_t s, int G, int m, const int64_t *sl_off,
                               const int32_t *sl_ids, const float *logits, float temperature,
                               const float *u, int32_t *token, QStats *qs, int64_t max_len,
                               void *ws)
{
    Ragged layout{sl_off, m};
    const int64_t rows = (int64_t)G * m;
    const int64_t nchmax = chunks_for(max_len > 0 ? max_len : 1);
    const double tau = (double)temperature;
    // the chunk statistics as in launch_norm (their values do not depend on
    // the chunks per workgroup)
    const int R = rows >= 256 && nchmax >= 16 ? 2 : (nchmax >= 64 && rows * nchmax / 4 >= 2048 ? 4 : 1);
    const dim3 grid((unsigned)((nchmax + R - 1) / R), (unsigned)rows);
    if (R == 2)
        hipLaunchKernelGGL((norm_stats_kernel<Ragged, 2>), grid, dim3(kChunkThreads), 0, s, layout,
                           logits, tau, nchmax, ws, rows);
    else if (R == 4)
        hipLaunchKernelGGL((norm_stats_kernel<Ragged, 4>), grid, dim3(kChunkThreads), 0, s, layout,
                           logits, tau, nchmax, ws, rows);
    else
        hipLaunchKernelGGL((norm_stats_kernel<Ragged, 1>), grid, dim3(kChunkThreads), 0, s, layout,
                           logits, tau, nchmax, ws, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((norm_pick_kernel<Ragged>), dim3((unsigned)rows), dim3(kChunkThreads), 0, s,
                       layout, logits, tau, nchmax, (const void *)ws, rows, sl_ids, u, token, qs);
    return hipGetLastError();
}

static int64_t segments_for(int64_t V) { return (V + kSeg - 1) / kSeg; }

// [rows][nseg] segment sums (fp64), then [rows][nseg] segment maxima (fp32)
size_t softmax_ws_bytes(int64_t rows, int64_t V)
{
    return (size_t)rows * (size_t)segments_for(V) * 12 + 256;
}

int64_t softmax_segments(int64_t V) { return segments_for(V); }

hipError_t softmax_stats_launch(hipStream_t s, int rows, int V, const float *logits, void *ws)
{
    const int64_t nseg = segments_for(V);
    double *ssum = reinterpret_cast<double *>(ws);
    float *smax = reinterpret_cast<float *>(ssum + (size_t)rows * nseg);
    const dim3 grid((unsigned)nseg, (unsigned)rows);
    hipLaunchKernelGGL(softmax_stats_kernel, grid, dim3(kChunkThreads), 0, s, (int64_t)V, logits,
                       ssum, smax);
    return hipGetLastError();
}

hipError_t softmax_launch(hipStream_t s, int rows, int V, const float *logits, float *p, void *ws)
{
    const int64_t nseg = segments_for(V);
    double *ssum = reinterpret_cast<double *>(ws);
    float *smax = reinterpret_cast<float *>(ssum + (size_t)rows * nseg);
    hipError_t e = softmax_stats_launch(s, rows, V, logits, ws);
    if (e != hipSuccess)
        return e;
    const dim3 grid((unsigned)nseg, (unsigned)rows);
    hipLaunchKernelGGL(softmax_final_kernel, grid, dim3(kChunkThreads), 0, s, (int64_t)V, logits,
                       (const double *)ssum, (const float *)smax, p);
    return hipGetLastError();
}

}  // namespace ds
