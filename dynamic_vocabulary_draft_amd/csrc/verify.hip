// Rejection-sampling verification over the full vocabulary, which keeps the
// emitted tokens distributed exactly as the target (DynaSpec abstract: the
// target checks every draft against its whole vocabulary, so the output is
// exact; summary page, "Pipeline Flow: Rejection Sampling Verification"; the
// accept / residual / bonus rules are textbook speculative sampling).
//
// Two launches, one workgroup per (1024-token chunk of V, sequence):
//   sum:    the workgroup's four waves run the T accept tests (the draft
//           token is found in its ascending shortlist with a three-round
//           wave search; the exact fp64 test u*q < p) and take the first
//           rejected position t*; for a rejection the chunk's residual
//           weights max(0, p - q) (q of the shortlist entries inside the
//           chunk scattered into LDS) and the plain p weights are summed;
//           after T acceptances the bonus position's p is summed;
//   final:  every workgroup rebuilds the same prefixes and total (the
//           residual, or p when the residual has no mass); the owner of the
//           threshold u_fin * total walks its chunk and writes the drawn
//           token; chunk 0 writes the accepted tokens, -1 padding and n_acc.
#include <float.h>

#include "common.h"
#include "dist.h"
#include "kernels.h"

namespace ds {
namespace {

constexpr int kMaxVChunks = 1024;  // V up to 2^20
constexpr int kMaxRows = 65;       // T + 1 <= 65

struct VerifyWs {
    ChunkWs ch;
    int32_t *tstar;  // [B]: first rejected position (T if none)
};

__host__ __device__ inline VerifyWs verify_ws(void *ws, int B, int64_t nchV)
{
    VerifyWs w;
    w.ch = chunk_ws(ws, B, nchV);
    w.tstar = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(ws) + chunk_ws_bytes(B, nchV));
    return w;
}

// The target rows of sequence b: probabilities p [B][T+1][V], or (LOGITS)
// target logits of that shape with each row's softmax normaliser rebuilt
// from the softmax's segment statistics, p taken where it is read
// (p_elem: the same bits as the softmax's output).
template <bool LOGITS>
struct Target {
    const float *x;
    int64_t V;
    int T;
    const float *M;    // LDS [T+1] (LOGITS)
    const double *rZ;  // LDS [T+1] (LOGITS)
    const double *tab; // LDS exp table (LOGITS)
    __device__ const float *row(int b, int t) const { return x + ((int64_t)b * (T + 1) + t) * V; }
    __device__ float at(const float *r, int t, int64_t y) const
    {
        return LOGITS ? p_elem(r[y], M[t], rZ[t], tab) : r[y];
    }
};

// LOGITS: every row's normaliser of sequence b into LDS (wave w: rows w,
// w + 4, ...) and the exp table; returns after a barrier
template <bool LOGITS>
__device__ __forceinline__ void target_norms(int b, int T, const float *__restrict__ smax,
                                             const double *__restrict__ ssum, int64_t nseg,
                                             float *sM, double *srZ, double *tab)
{
    if (!LOGITS)
        return;
    fill_exp2_table(tab);
    __syncthreads();
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    for (int t = wave; t <= T; t += nw) {
        const int64_t r = (int64_t)b * (T + 1) + t;
        float M;
        double rZ;
        row_norm(smax + r * nseg, ssum + r * nseg, nseg, tab, &M, &rZ);
        if (lane_id() == 0) {
            sM[t] = M;
            srZ[t] = rZ;
        }
    }
    __syncthreads();
}

// The T accept tests of sequence b, split over the workgroup's waves; returns
// (to every thread) the first rejected position, T if all are accepted.
template <bool LOGITS>
__device__ int first_rejection(int B, int T, int V, int b, const int32_t *__restrict__ draft,
                               const int64_t *__restrict__ sl_off,
                               const int32_t *__restrict__ sl_ids, const float *__restrict__ q,
                               const Target<LOGITS> &tg, const float *__restrict__ u_acc,
                               int *s_rej)
{
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if (threadIdx.x == 0)
        *s_rej = T;
    __syncthreads();
    for (int t = wave; t < T; t += nw) {
        const int64_t row = (int64_t)t * B + b;
        const int32_t x = draft[row];
        const int64_t lo = sl_off[row], len = sl_off[row + 1] - lo;
        const int64_t j = wave_lower_bound(sl_ids + lo, len, x);
        const bool found = j < len && sl_ids[lo + j] == x;
        const double qx = found ? (double)q[lo + j] : 0.0;
        const double px = (x >= 0 && x < V) ? (double)tg.at(tg.row(b, t), t, x) : 0.0;
        if (lane_id() == 0 && !((double)u_acc[row] * qx < px))
            atomicMin(s_rej, t);
    }
    __syncthreads();
    return *s_rej;
}

// The chunk's q values (shortlist entries with token ids in [base, base+1024))
// scattered into a dense LDS array; returns after a barrier.
__device__ void scatter_q(const int32_t *__restrict__ S, const float *__restrict__ qrow,
                          int64_t len, int64_t base, float *qd, int64_t *s_rng)
{
    for (int i = threadIdx.x; i < kChunk; i += blockDim.x)
        qd[i] = 0.0f;
    if ((threadIdx.x >> 6) == 0) {
        const int64_t a = wave_lower_bound(S, len, (int32_t)base);
        const int64_t e = wave_lower_bound(S, len, (int32_t)min(base + kChunk, (int64_t)INT32_MAX));
        if (lane_id() == 0) {
            s_rng[0] = a;
            s_rng[1] = e;
        }
    }
    __syncthreads();
    for (int64_t k = s_rng[0] + threadIdx.x; k < s_rng[1]; k += blockDim.x) {
        const int64_t o = (int64_t)S[k] - base;
        if (o >= 0 && o < kChunk)
            qd[o] = qrow[k];
    }
    __syncthreads();
}

// weights of this lane's four tokens: family 0 = residual (or bonus p),
// family 1 = plain p of the rejected position
template <bool LOGITS>
__device__ __forceinline__ void lane_weights(const Target<LOGITS> &tg, const float *__restrict__ pt,
                                             int t, int64_t y0, int V, const float *qd,
                                             int64_t local0, bool resid, double w0[4],
                                             double w1[4])
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t y = y0 + k;
        const double pv = y < V ? (double)tg.at(pt, t, y) : 0.0;
        w1[k] = pv;
        if (resid) {
            const double r = y < V ? pv - (double)qd[local0 + k] : 0.0;
            w0[k] = r > 0.0 ? r : 0.0;
        } else {
            w0[k] = pv;
        }
    }
}

template <bool LOGITS>
__global__ __launch_bounds__(kChunkThreads) void verify_sum_kernel(
    int B, int T, int V, const int32_t *__restrict__ draft, const int64_t *__restrict__ sl_off,
    const int32_t *__restrict__ sl_ids, const float *__restrict__ q, const float *__restrict__ p,
    const float *__restrict__ smax, const double *__restrict__ ssum, int64_t nseg,
    const float *__restrict__ u_acc, int64_t nchV, void *ws)
{
    __shared__ float qd[kChunk];
    __shared__ int64_t s_rng[2];
    __shared__ double s_w0[4], s_w1[4];
    __shared__ int s_rej;
    __shared__ float sM[LOGITS ? kMaxRows : 1];
    __shared__ double srZ[LOGITS ? kMaxRows : 1], tab[LOGITS ? 64 : 1];
    const int b = blockIdx.y;
    const int64_t c = blockIdx.x;
    VerifyWs w = verify_ws(ws, B, nchV);
    target_norms<LOGITS>(b, T, smax, ssum, nseg, sM, srZ, tab);
    const Target<LOGITS> tg{p, (int64_t)V, T, sM, srZ, tab};
    const int tstar =
        first_rejection<LOGITS>(B, T, V, b, draft, sl_off, sl_ids, q, tg, u_acc, &s_rej);
    if (c == 0 && threadIdx.x == 0)
        w.tstar[b] = tstar;
    const float *pt = tg.row(b, tstar);
    const bool resid = tstar < T;
    const int64_t base = c * kChunk;
    if (resid) {
        const int64_t row = (int64_t)tstar * B + b;
        const int64_t lo = sl_off[row];
        scatter_q(sl_ids + lo, q + lo, sl_off[row + 1] - lo, base, qd, s_rng);
    }
    const int64_t local0 = (threadIdx.x >> 6) * 256 + lane_id() * 4;
    double w0[4], w1[4];
    lane_weights<LOGITS>(tg, pt, tstar, base + local0, V, qd, local0, resid, w0, w1);
    double i0, i1;
    double t0 = wave_chunk_sum(w0, &i0), t1 = wave_chunk_sum(w1, &i1);
    if (lane_id() == 0) {
        s_w0[threadIdx.x >> 6] = t0;
        s_w1[threadIdx.x >> 6] = t1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        w.ch.csum[(int64_t)b * nchV + c] = ((s_w0[0] + s_w0[1]) + s_w0[2]) + s_w0[3];
        w.ch.csum2[(int64_t)b * nchV + c] = ((s_w1[0] + s_w1[1]) + s_w1[2]) + s_w1[3];
    }
}

template <bool LOGITS>
__global__ __launch_bounds__(kChunkThreads) void verify_final_kernel(
    int B, int T, int V, const int32_t *__restrict__ draft, const int64_t *__restrict__ sl_off,
    const int32_t *__restrict__ sl_ids, const float *__restrict__ q, const float *__restrict__ p,
    const float *__restrict__ smax, const double *__restrict__ ssum, int64_t nseg,
    const float *__restrict__ u_fin, int64_t nchV, const void *ws, int32_t *__restrict__ n_acc,
    int32_t *__restrict__ out)
{
    __shared__ double P[kMaxVChunks], S[kMaxVChunks];
    __shared__ float qd[kChunk];
    __shared__ int64_t s_rng[2];
    __shared__ double s_wt[4];
    __shared__ double s_total;
    __shared__ int s_owner, s_fallback;
    __shared__ int64_t s_pick[2];
    __shared__ float sM[LOGITS ? kMaxRows : 1];
    __shared__ double srZ[LOGITS ? kMaxRows : 1], tab[LOGITS ? 64 : 1];
    const int b = blockIdx.y;
    const int64_t c = blockIdx.x;
    VerifyWs w = verify_ws(const_cast<void *>(ws), B, nchV);
    const int tstar = w.tstar[b];
    const int nch = (int)nchV;
    const double *cs0 = w.ch.csum + (int64_t)b * nchV;
    const double *cs1 = w.ch.csum2 + (int64_t)b * nchV;
    const bool resid = tstar < T;
    double Z = row_prefix(cs0, nch, P, S, &s_total);
    bool use_p = false;
    if (resid && !(Z > 0.0)) {  // residual without mass: draw from p_t itself
        use_p = true;
        __syncthreads();
        Z = row_prefix(cs1, nch, P, S, &s_total);
    }
    const double thr = (double)u_fin[b] * Z;
    owner_chunk(P, S, nch, thr, &s_owner, &s_fallback);
    int32_t *ob = out + (int64_t)b * (T + 1);
    if (c == 0) {
        for (int k = threadIdx.x; k <= T; k += blockDim.x)
            if (k != tstar || s_owner < 0)
                ob[k] = k < tstar ? draft[(int64_t)k * B + b] : -1;
        if (threadIdx.x == 0)
            n_acc[b] = tstar;
    }
    if (c != s_owner)
        return;
    target_norms<LOGITS>(b, T, smax, ssum, nseg, sM, srZ, tab);
    const Target<LOGITS> tg{p, (int64_t)V, T, sM, srZ, tab};
    const float *pt = tg.row(b, tstar);
    const int64_t base = c * kChunk;
    if (resid && !use_p) {
        const int64_t row = (int64_t)tstar * B + b;
        const int64_t lo = sl_off[row];
        scatter_q(sl_ids + lo, q + lo, sl_off[row + 1] - lo, base, qd, s_rng);
    }
    const int64_t local0 = (threadIdx.x >> 6) * 256 + lane_id() * 4;
    double w0[4], w1[4];
    lane_weights<LOGITS>(tg, pt, tstar, base + local0, V, qd, local0, resid && !use_p, w0, w1);
    double incl;
    double tot = wave_chunk_sum(w0, &incl);
    if (lane_id() == 0)
        s_wt[threadIdx.x >> 6] = tot;
    __syncthreads();
    const int64_t pick = chunk_walk(w0, base + local0, s_wt, incl, P[c], thr, s_fallback != 0,
                                    s_pick);
    if (threadIdx.x == 0)
        ob[tstar] = (int32_t)pick;
}

template <bool LOGITS>
hipError_t verify_kernels(hipStream_t s, int B, int T, int V, const int32_t *draft,
                          const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                          const float *x, const float *smax, const double *ssum, int64_t nseg,
                          const float *u_acc, const float *u_fin, int32_t *n_acc, int32_t *out,
                          void *ws)
{
    const int64_t nchV = chunks_for(V);
    dim3 grid((unsigned)nchV, (unsigned)B);
    hipLaunchKernelGGL(verify_sum_kernel<LOGITS>, grid, dim3(kChunkThreads), 0, s, B, T, V, draft,
                       sl_off, sl_ids, q, x, smax, ssum, nseg, u_acc, nchV, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(verify_final_kernel<LOGITS>, grid, dim3(kChunkThreads), 0, s, B, T, V,
                       draft, sl_off, sl_ids, q, x, smax, ssum, nseg, u_fin, nchV,
                       (const void *)ws, n_acc, out);
    return hipGetLastError();
}

}  // namespace

size_t verify_ws_bytes(int B, int T, int V)
{
    (void)T;
    return chunk_ws_bytes(B, chunks_for(V)) + (size_t)B * sizeof(int32_t) + 256;
}

hipError_t verify_launch(hipStream_t s, int B, int T, int V, const int32_t *draft,
                         const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                         const float *p, const float *u_acc, const float *u_fin, int32_t *n_acc,
                         int32_t *out, void *ws)
{
    return verify_kernels<false>(s, B, T, V, draft, sl_off, sl_ids, q, p, nullptr, nullptr, 0,
                                 u_acc, u_fin, n_acc, out, ws);
}

// the verification workspace, then the softmax statistics of the B*(T+1) rows
size_t verify_logits_ws_bytes(int B, int T, int V)
{
    return (verify_ws_bytes(B, T, V) + 255) / 256 * 256 +
           softmax_ws_bytes((int64_t)B * (T + 1), V);
}

hipError_t verify_logits_launch(hipStream_t s, int B, int T, int V, const int32_t *draft,
                                const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                                const float *logits, const float *u_acc, const float *u_fin,
                                int32_t *n_acc, int32_t *out, void *ws)
{
    const int rows = B * (T + 1);
    char *sws = reinterpret_cast<char *>(ws) + (verify_ws_bytes(B, T, V) + 255) / 256 * 256;
    hipError_t e = softmax_stats_launch(s, rows, V, logits, sws);
    if (e != hipSuccess)
        return e;
    const int64_t nseg = softmax_segments(V);
    const double *ssum = reinterpret_cast<const double *>(sws);
    const float *smax = reinterpret_cast<const float *>(ssum + (size_t)rows * nseg);
    return verify_kernels<true>(s, B, T, V, draft, sl_off, sl_ids, q, logits, smax, ssum, nseg,
                                u_acc, u_fin, n_acc, out, ws);
}

}  // namespace ds
