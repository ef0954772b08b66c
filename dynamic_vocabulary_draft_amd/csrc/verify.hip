// Rejection-sampling verification over the full vocabulary, which keeps the
// emitted tokens distributed exactly as the target (DynaSpec abstract: the
// target checks every draft against its whole vocabulary, so the output is
// exact; summary page, "Pipeline Flow: Rejection Sampling Verification"; the
// accept / residual / bonus rules are textbook speculative sampling).
//
// Three launches (four from logits, the first being the target softmax's
// segment statistics):
//   prep:   one workgroup per sequence, one wave per position: the draft
//           token x is found in its ascending shortlist with a three-round
//           wave search, and the exact fp64 test u*q < p decides; t* = the
//           first rejected position (from logits, the target rows'
//           normalisers are rebuilt first);
//   sum:    one wave per (chunk, sequence): the chunk's residual weights
//           max(0, p - q) after a rejection (the chunk's shortlist entries,
//           found with one two-key wave search, scattered into the wave's
//           LDS array), the bonus position's p after T acceptances, summed;
//   final:  one workgroup per sequence: the chunk prefixes and total, the
//           chunk owning the threshold u_fin * total, the walk of that
//           chunk, the drawn token, the accepted tokens, -1 padding and
//           n_acc.  A residual without mass draws from p_t itself: that
//           workgroup then sums p_t's chunks first (a degenerate case).
#include <float.h>

#include "common.h"
#include "dist.h"
#include "kernels.h"

namespace ds {
namespace {

constexpr int kMaxVChunks = 1024;  // V up to 2^20
constexpr int kMaxRows = 65;       // T + 1 <= 65
constexpr int kPrepThreads = 1024;  // one wave per position, 16 at a time

struct VerifyWs {
    double *csum;    // [B][nchV]: chunk sums of the drawn distribution
    int32_t *tstar;  // [B]: first rejected position (T if none)
    float *rowM;     // [B] (logits): normaliser of row t* ...
    double *rowZ;    // [B] ... and its 1 / Z
};

__host__ __device__ inline size_t align256(size_t n) { return (n + 255) / 256 * 256; }

__host__ __device__ inline size_t verify_ws_layout(int B, int64_t nchV, size_t off[4])
{
    size_t o = 0;
    off[0] = o;
    o += align256((size_t)B * (size_t)nchV * 8);
    off[1] = o;
    o += align256((size_t)B * 4);
    off[2] = o;
    o += align256((size_t)B * 4);
    off[3] = o;
    return o + (size_t)B * 8;
}

__host__ __device__ inline VerifyWs verify_ws(void *ws, int B, int64_t nchV)
{
    size_t off[4];
    verify_ws_layout(B, nchV, off);
    char *p = reinterpret_cast<char *>(ws);
    VerifyWs w;
    w.csum = reinterpret_cast<double *>(p + off[0]);
    w.tstar = reinterpret_cast<int32_t *>(p + off[1]);
    w.rowM = reinterpret_cast<float *>(p + off[2]);
    w.rowZ = reinterpret_cast<double *>(p + off[3]);
    return w;
}

// One target row and (logits) its normaliser: p = p_elem(logit, M, rZ), the
// same bits as the target softmax writes
template <bool LOGITS>
struct RowP {
    const float *r;
    float M;
    double rZ;
    const double *tab;
};

// One workgroup per sequence: (logits) every target row's normaliser, the T
// accept tests (wave t: position t, t + 16, ...) and t*.
// QL: q is recomputed from the draft logits (q points to them) and each
// draft row's statistics qs (temperature qtau), bit for bit the sampler's q.
template <bool LOGITS, bool QL>
__global__ __launch_bounds__(kPrepThreads) void verify_prep_kernel(
    int B, int T, int V, const int32_t *__restrict__ draft, const int64_t *__restrict__ sl_off,
    const int32_t *__restrict__ sl_ids, const float *__restrict__ q, const float *__restrict__ p,
    const float *__restrict__ smax, const double *__restrict__ ssum, int64_t nseg,
    const float *__restrict__ u_acc, int64_t nchV, void *ws, const QStats *__restrict__ qs,
    double qtau)
{
    __shared__ int s_rej;
    __shared__ float sM[LOGITS ? kMaxRows : 1];
    __shared__ double srZ[LOGITS ? kMaxRows : 1], tab[LOGITS || QL ? 64 : 1];
    const int b = blockIdx.x, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    VerifyWs w = verify_ws(ws, B, nchV);
    if (threadIdx.x == 0)
        s_rej = T;
    if (QL && !LOGITS)
        fill_exp2_table(tab);  // ordered by the barrier below
    if (LOGITS) {
        fill_exp2_table(tab);
        __syncthreads();
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
    }
    __syncthreads();
    for (int t = wave; t < T; t += nw) {
        const int64_t row = (int64_t)t * B + b;
        const int32_t x = draft[row];
        const int64_t lo = sl_off[row], len = sl_off[row + 1] - lo;
        const bool xin = x >= 0 && x < V;
        // the target value at x, loaded before the search
        const float px_raw = xin ? p[((int64_t)b * (T + 1) + t) * V + x] : 0.f;
        const int64_t j = wave_lower_bound(sl_ids + lo, len, x);
        const bool found = j < len && sl_ids[lo + j] == x;
        double qx = 0.0;
        if (found)
            qx = QL ? (double)q_elem(q[lo + j], qs[row].M, qs[row].rZ, qtau, tab)
                    : (double)q[lo + j];
        double px = 0.0;
        if (xin)
            px = LOGITS ? (double)p_elem(px_raw, sM[t], srZ[t], tab) : (double)px_raw;
        if (lane_id() == 0 && !((double)u_acc[row] * qx < px))
            atomicMin(&s_rej, t);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int tstar = s_rej;
        w.tstar[b] = tstar;
        if (LOGITS) {
            w.rowM[b] = sM[tstar];
            w.rowZ[b] = srZ[tstar];
        }
    }
}

// this lane's four raw target values (p, or logits) of tokens y0 .. y0+3
__device__ __forceinline__ void lane_raw(const float *__restrict__ r, int64_t y0, int V,
                                         float x[4])
{
#pragma unroll
    for (int k = 0; k < 4; ++k)
        x[k] = y0 + k < V ? r[y0 + k] : 0.f;
}

// weights of this lane's four tokens from their raw values: the residual
// max(0, p - q) (resid), else p
template <bool LOGITS>
__device__ __forceinline__ void lane_weights(const RowP<LOGITS> &rp, const float x[4], int64_t y0,
                                             int V, const float *qd, int64_t local0, bool resid,
                                             double w[4])
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t y = y0 + k;
        const double pv =
            y < V ? (double)(LOGITS ? p_elem(x[k], rp.M, rp.rZ, rp.tab) : x[k]) : 0.0;
        if (resid) {
            const double r = y < V ? pv - (double)qd[local0 + k] : 0.0;
            w[k] = r > 0.0 ? r : 0.0;
        } else {
            w[k] = pv;
        }
    }
}

// The chunk's entries [a, e) of the rejected row's shortlist (ids in
// [base, base + 1024)) scattered into the dense array qd by `nt` threads
// with index i; the caller zeroes qd first and orders the writes before the
// reads.
// qf maps a stored value to q (identity, or q_elem of a draft logit).
template <class QF>
__device__ __forceinline__ void scatter_q(const int32_t *__restrict__ S,
                                          const float *__restrict__ qrow, int64_t a, int64_t e,
                                          int64_t base, float *qd, int i, int nt, QF qf)
{
    for (int64_t k = a + i; k < e; k += nt) {
        const int64_t o = (int64_t)S[k] - base;
        if (o >= 0 && o < kChunk)
            qd[o] = qf(qrow[k]);
    }
}


// the chunk's entries [a, e) of an ascending shortlist S of length len:
// ids in [base, base + 1024), by one wave
__device__ __forceinline__ void chunk_range(const int32_t *__restrict__ S, int64_t len,
                                            int64_t base, int64_t *a, int64_t *e)
{
    wave_lower_bound2(S, len, (int32_t)base, (int32_t)min(base + kChunk, (int64_t)INT32_MAX), a,
                      e);
}

// One wave's sum over chunk c (1024 tokens from base) of the weights: four
// 256-token parts, each summed as in the final walk (four-term lane sums,
// the wave's inclusive scan), then the parts in order.  x: the raw values.
template <bool LOGITS>
__device__ __forceinline__ double wave_chunk_total(const RowP<LOGITS> &rp, const float x[4][4],
                                                   int64_t base, int V, const float *qd,
                                                   bool resid)
{
    const int lane = lane_id();
    double t = 0.0;
#pragma unroll
    for (int part = 0; part < 4; ++part) {
        const int64_t local0 = part * 256 + lane * 4;
        double w[4], incl;
        lane_weights<LOGITS>(rp, x[part], base + local0, V, qd, local0, resid, w);
        const double s = wave_chunk_sum(w, &incl);
        t = part == 0 ? s : t + s;
    }
    return t;
}

// Chunk sums: wave w of workgroup x takes chunk 4x + w of sequence blockIdx.y.
template <bool LOGITS, bool QL>
__global__ __launch_bounds__(kChunkThreads) void verify_sum_kernel(
    int B, int T, int V, const int64_t *__restrict__ sl_off, const int32_t *__restrict__ sl_ids,
    const float *__restrict__ q, const float *__restrict__ p, int64_t nchV, void *ws,
    const QStats *__restrict__ qs, double qtau)
{
    __shared__ float qd_all[4][kChunk];
    __shared__ double tab[LOGITS || QL ? 64 : 1];
    const int b = blockIdx.y, wave = threadIdx.x >> 6, lane = lane_id();
    VerifyWs w = verify_ws(ws, B, nchV);
    if (LOGITS || QL) {
        fill_exp2_table(tab);
        __syncthreads();
    }
    const int64_t c = (int64_t)blockIdx.x * 4 + wave;
    if (c >= nchV)
        return;  // no barrier follows
    const int tstar = w.tstar[b];
    const bool resid = tstar < T;
    const RowP<LOGITS> rp{p + ((int64_t)b * (T + 1) + tstar) * V, LOGITS ? w.rowM[b] : 0.f,
                          LOGITS ? w.rowZ[b] : 0.0, tab};
    const int64_t base = c * kChunk;
    float *qd = qd_all[wave];
    float x[4][4];  // loaded before the scatter so that both are in flight
#pragma unroll
    for (int part = 0; part < 4; ++part)
        lane_raw(rp.r, base + part * 256 + lane * 4, V, x[part]);
    if (resid) {
        const int64_t row = (int64_t)tstar * B + b;
        const int64_t lo = sl_off[row], len = sl_off[row + 1] - lo;
        int64_t a, e;
        chunk_range(sl_ids + lo, len, base, &a, &e);
        for (int k = lane; k < kChunk; k += kWave)
            qd[k] = 0.0f;
        scatter_q(sl_ids + lo, q + lo, a, e, base, qd, lane, kWave, q_row<QL>(qs, row, qtau, tab));
    }
    // one wave's LDS operations complete in order: the scatter is visible
    const double t = wave_chunk_total<LOGITS>(rp, x, base, V, qd, resid);
    if (lane == 0)
        w.csum[(int64_t)b * nchV + c] = t;
}

template <bool LOGITS, bool QL>
__global__ __launch_bounds__(kChunkThreads) void verify_final_kernel(
    int B, int T, int V, const int32_t *__restrict__ draft, const int64_t *__restrict__ sl_off,
    const int32_t *__restrict__ sl_ids, const float *__restrict__ q, const float *__restrict__ p,
    const float *__restrict__ u_fin, int64_t nchV, const void *ws, int32_t *__restrict__ n_acc,
    int32_t *__restrict__ out, const QStats *__restrict__ qs, double qtau)
{
    __shared__ double P[kMaxVChunks], S[kMaxVChunks];
    __shared__ float qd[kChunk];
    __shared__ double s_wt[4];
    __shared__ double s_total;
    __shared__ int s_owner, s_fallback;
    __shared__ int64_t s_pick[2];
    __shared__ double tab[LOGITS || QL ? 64 : 1];
    const int b = blockIdx.x, wave = threadIdx.x >> 6, lane = lane_id();
    VerifyWs w = verify_ws(const_cast<void *>(ws), B, nchV);
    if (LOGITS || QL)
        fill_exp2_table(tab);  // ordered by the barrier in row_prefix
    const int tstar = w.tstar[b];
    const int nch = (int)nchV;
    const bool resid = tstar < T;
    const RowP<LOGITS> rp{p + ((int64_t)b * (T + 1) + tstar) * V, LOGITS ? w.rowM[b] : 0.f,
                          LOGITS ? w.rowZ[b] : 0.0, tab};
    double Z = row_prefix(w.csum + (int64_t)b * nchV, nch, P, S, &s_total);
    bool use_p = false;
    if (resid && !(Z > 0.0)) {
        // the residual has no mass: draw from p_t itself, whose chunk sums
        // (the same association as the sum launch) this workgroup takes now
        use_p = true;
        for (int c = wave; c < nch; c += 4) {
            float x[4][4];
#pragma unroll
            for (int part = 0; part < 4; ++part)
                lane_raw(rp.r, (int64_t)c * kChunk + part * 256 + lane * 4, V, x[part]);
            const double t = wave_chunk_total<LOGITS>(rp, x, (int64_t)c * kChunk, V, qd, false);
            if (lane == 0)
                S[c] = t;
        }
        __syncthreads();
        Z = row_prefix(S, nch, P, S, &s_total);
    }
    const double thr = (double)u_fin[b] * Z;
    owner_chunk(P, S, nch, thr, &s_owner, &s_fallback);
    int32_t *ob = out + (int64_t)b * (T + 1);
    const int owner = s_owner;
    for (int k = threadIdx.x; k <= T; k += blockDim.x)
        if (k != tstar || owner < 0)
            ob[k] = k < tstar ? draft[(int64_t)k * B + b] : -1;
    if (threadIdx.x == 0)
        n_acc[b] = tstar;
    if (owner < 0)
        return;
    const int64_t c = owner, base = c * kChunk;
    const int64_t local0 = wave * 256 + lane * 4;
    float x[4];
    lane_raw(rp.r, base + local0, V, x);
    const bool rq = resid && !use_p;
    if (rq) {
        const int64_t row = (int64_t)tstar * B + b;
        const int64_t lo = sl_off[row], len = sl_off[row + 1] - lo;
        __shared__ int64_t s_rng[2];
        if (wave == 0) {
            int64_t a, e;
            chunk_range(sl_ids + lo, len, base, &a, &e);
            if (lane == 0)
                s_rng[0] = a, s_rng[1] = e;
        }
        for (int k = threadIdx.x; k < kChunk; k += blockDim.x)
            qd[k] = 0.0f;
        __syncthreads();
        scatter_q(sl_ids + lo, q + lo, s_rng[0], s_rng[1], base, qd, threadIdx.x, blockDim.x,
                  q_row<QL>(qs, row, qtau, tab));
        __syncthreads();
    }
    double w0[4];
    lane_weights<LOGITS>(rp, x, base + local0, V, qd, local0, rq, w0);
    double incl;
    const double tot = wave_chunk_sum(w0, &incl);
    if (lane == 0)
        s_wt[wave] = tot;
    __syncthreads();
    const int64_t pick = chunk_walk(w0, base + local0, s_wt, incl, P[c], thr, s_fallback != 0,
                                    s_pick);
    if (threadIdx.x == 0)
        ob[tstar] = (int32_t)pick;
}

template <bool LOGITS, bool QL = false>
hipError_t verify_kernels(hipStream_t s, int B, int T, int V, const int32_t *draft,
                          const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                          const float *x, float *smax, double *ssum, int64_t nseg,
                          const float *u_acc, const float *u_fin, int32_t *n_acc, int32_t *out,
                          void *ws, const QStats *qs = nullptr, double qtau = 1.0)
{
    const int64_t nchV = chunks_for(V);
    hipError_t e;
    if (LOGITS && (e = softmax_stats_launch(s, B * (T + 1), V, x, ssum)) != hipSuccess)
        return e;
    hipLaunchKernelGGL((verify_prep_kernel<LOGITS, QL>), dim3((unsigned)B), dim3(kPrepThreads), 0,
                       s, B, T, V, draft, sl_off, sl_ids, q, x, (const float *)smax,
                       (const double *)ssum, nseg, u_acc, nchV, ws, qs, qtau);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL((verify_sum_kernel<LOGITS, QL>),
                       dim3((unsigned)((nchV + 3) / 4), (unsigned)B), dim3(kChunkThreads), 0, s, B,
                       T, V, sl_off, sl_ids, q, x, nchV, ws, qs, qtau);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL((verify_final_kernel<LOGITS, QL>), dim3((unsigned)B), dim3(kChunkThreads),
                       0, s, B, T, V, draft, sl_off, sl_ids, q, x, u_fin, nchV, (const void *)ws,
                       n_acc, out, qs, qtau);
    return hipGetLastError();
}

}  // namespace

size_t verify_ws_bytes(int B, int T, int V)
{
    (void)T;
    size_t off[4];
    return verify_ws_layout(B, chunks_for(V), off) + 256;
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
    return align256(verify_ws_bytes(B, T, V)) + softmax_ws_bytes((int64_t)B * (T + 1), V);
}

hipError_t verify_logits_launch(hipStream_t s, int B, int T, int V, const int32_t *draft,
                                const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                                const float *logits, const float *u_acc, const float *u_fin,
                                int32_t *n_acc, int32_t *out, void *ws)
{
    const int rows = B * (T + 1);
    char *sws = reinterpret_cast<char *>(ws) + align256(verify_ws_bytes(B, T, V));
    // the statistics layout of the target softmax: [rows][nseg] sums, then maxima
    const int64_t nseg = softmax_segments(V);
    double *ssum = reinterpret_cast<double *>(sws);
    float *smax = reinterpret_cast<float *>(ssum + (size_t)rows * nseg);
    return verify_kernels<true>(s, B, T, V, draft, sl_off, sl_ids, q, logits, smax, ssum, nseg,
                                u_acc, u_fin, n_acc, out, ws);
}

hipError_t verify_logits_qstats_launch(hipStream_t s, int B, int T, int V, const int32_t *draft,
                                       const int64_t *sl_off, const int32_t *sl_ids,
                                       const float *draft_logits, const QStats *qs,
                                       float temperature, const float *logits,
                                       const float *u_acc, const float *u_fin, int32_t *n_acc,
                                       int32_t *out, void *ws)
{
    const int rows = B * (T + 1);
    char *sws = reinterpret_cast<char *>(ws) + align256(verify_ws_bytes(B, T, V));
    const int64_t nseg = softmax_segments(V);
    double *ssum = reinterpret_cast<double *>(sws);
    float *smax = reinterpret_cast<float *>(ssum + (size_t)rows * nseg);
    return verify_kernels<true, true>(s, B, T, V, draft, sl_off, sl_ids, draft_logits, logits,
                                      smax, ssum, nseg, u_acc, u_fin, n_acc, out, ws, qs,
                                      (double)temperature);
}

}  // namespace ds
