// Rejection-sampling verification over the full vocabulary, which keeps the
// emitted tokens distributed exactly as the target (DynaSpec abstract: the
// target checks every draft against its whole vocabulary, so the output is
// exact; summary page, "Pipeline Flow: Rejection Sampling Verification"; the
// accept / residual / bonus rules are textbook speculative sampling).
//
// Three launches:
//   prep:   one workgroup per sequence: its waves run the T accept
//           tests (the draft token is found in its ascending shortlist with
//           a three-round wave search; the exact fp64 test u*q < p) and take
//           the first rejected position t*; after a rejection one pass over
//           the rejected row's shortlist records where each 1024-token chunk
//           of V starts in it;
//   sum:    one wave per (chunk, sequence): for a rejection the chunk's
//           residual weights max(0, p - q) (q of the chunk's shortlist
//           entries scattered into the wave's LDS array) and the plain p
//           weights are summed; after T acceptances the bonus position's p;
//   final:  one workgroup per sequence: the chunk prefixes and total (the
//           residual, or p when the residual has no mass), the chunk owning
//           the threshold u_fin * total, the walk of that chunk, the drawn
//           token, the accepted tokens, -1 padding and n_acc.
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
    int32_t *cbeg;   // [B][nchV+1]: first entry of chunk c in the rejected row's shortlist
    float *rowM;     // [B] (logits): normaliser of row t* ...
    double *rowZ;    // [B] ... and its 1 / Z
};

__host__ __device__ inline size_t verify_ws_layout(int B, int64_t nchV, size_t off[4])
{
    size_t o = (chunk_ws_bytes(B, nchV) + 255) / 256 * 256;
    off[0] = o;                                           // tstar
    o += ((size_t)B * 4 + 255) / 256 * 256;
    off[1] = o;                                           // cbeg
    o += ((size_t)B * (size_t)(nchV + 1) * 4 + 255) / 256 * 256;
    off[2] = o;                                           // rowM
    o += ((size_t)B * 4 + 255) / 256 * 256;
    off[3] = o;                                           // rowZ
    return o + (size_t)B * 8;
}

__host__ __device__ inline VerifyWs verify_ws(void *ws, int B, int64_t nchV)
{
    size_t off[4];
    verify_ws_layout(B, nchV, off);
    char *p = reinterpret_cast<char *>(ws);
    VerifyWs w;
    w.ch = chunk_ws(ws, B, nchV);
    w.tstar = reinterpret_cast<int32_t *>(p + off[0]);
    w.cbeg = reinterpret_cast<int32_t *>(p + off[1]);
    w.rowM = reinterpret_cast<float *>(p + off[2]);
    w.rowZ = reinterpret_cast<double *>(p + off[3]);
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

// One target row and (LOGITS) its normaliser
template <bool LOGITS>
struct RowP {
    const float *r;
    float M;
    double rZ;
    const double *tab;
};

// LOGITS: every row's normaliser of sequence b into LDS (wave w: rows w,
// w + 4, ...); the exp table must be filled and visible.  Returns after a
// barrier.
template <bool LOGITS>
__device__ __forceinline__ void target_norms(int b, int T, const float *__restrict__ smax,
                                             const double *__restrict__ ssum, int64_t nseg,
                                             float *sM, double *srZ, const double *tab)
{
    if (!LOGITS)
        return;
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

// Per-sequence preparation, one workgroup per sequence: the accept tests,
// t*, the normaliser of row t* (logits) and, after a rejection, where each
// 1024-token chunk of V starts in the rejected row's ascending shortlist
// (cbeg[c] = first entry with id >= 1024 c, len if none; found in one pass:
// entry k starts every chunk c with ids[k-1] < 1024 c <= ids[k]).
constexpr int kPrepThreads = 1024;
constexpr int kPrepPer = 16;  // shortlist entries per thread and pass

template <bool LOGITS>
__global__ __launch_bounds__(kPrepThreads) void verify_prep_kernel(
    int B, int T, int V, const int32_t *__restrict__ draft, const int64_t *__restrict__ sl_off,
    const int32_t *__restrict__ sl_ids, const float *__restrict__ q, const float *__restrict__ p,
    const float *__restrict__ smax, const double *__restrict__ ssum, int64_t nseg,
    const float *__restrict__ u_acc, int64_t nchV, void *ws)
{
    __shared__ int s_rej;
    __shared__ float sM[LOGITS ? kMaxRows : 1];
    __shared__ double srZ[LOGITS ? kMaxRows : 1], tab[LOGITS ? 64 : 1];
    const int b = blockIdx.x;
    VerifyWs w = verify_ws(ws, B, nchV);
    if (LOGITS) {
        fill_exp2_table(tab);
        __syncthreads();
    }
    target_norms<LOGITS>(b, T, smax, ssum, nseg, sM, srZ, tab);
    const Target<LOGITS> tg{p, (int64_t)V, T, sM, srZ, tab};
    const int tstar =
        first_rejection<LOGITS>(B, T, V, b, draft, sl_off, sl_ids, q, tg, u_acc, &s_rej);
    if (threadIdx.x == 0) {
        w.tstar[b] = tstar;
        if (LOGITS) {
            w.rowM[b] = sM[tstar];
            w.rowZ[b] = srZ[tstar];
        }
    }
    if (tstar == T)
        return;
    const int64_t row = (int64_t)tstar * B + b;
    const int64_t lo = sl_off[row], len = sl_off[row + 1] - lo;
    const int32_t *S = sl_ids + lo;
    int32_t *cb = w.cbeg + (int64_t)b * (nchV + 1);
    // each thread takes kPrepPer consecutive entries (and the one before),
    // all loaded before any is used: a pass covers 16K entries
    for (int64_t k0 = (int64_t)threadIdx.x * kPrepPer; k0 <= len;
         k0 += (int64_t)blockDim.x * kPrepPer) {
        int32_t v[kPrepPer + 1];  // v[i] = S[k0 - 1 + i]
#pragma unroll
        for (int i = 0; i <= kPrepPer; ++i) {
            const int64_t k = k0 - 1 + i;
            v[i] = (k >= 0 && k < len) ? S[k] : 0;
        }
#pragma unroll
        for (int i = 1; i <= kPrepPer; ++i) {
            const int64_t k = k0 - 1 + i;  // entry k starts chunks c_lo .. c_hi
            if (k > len)
                break;
            const int64_t prev = k > 0 ? (int64_t)v[i - 1] : -1;
            const int64_t c_lo = prev < 0 ? 0 : prev / kChunk + 1;
            const int64_t c_hi =
                k < len ? (v[i] < 0 ? -1 : min((int64_t)v[i] / kChunk, nchV)) : nchV;
            for (int64_t c = c_lo; c <= c_hi; ++c)
                cb[c] = (int32_t)k;
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

// weights of this lane's four tokens from their raw values: family 0 =
// residual (or bonus p), family 1 = plain p of the rejected position
template <bool LOGITS>
__device__ __forceinline__ void lane_weights(const RowP<LOGITS> &rp, const float x[4], int64_t y0,
                                             int V, const float *qd, int64_t local0, bool resid,
                                             double w0[4], double w1[4])
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t y = y0 + k;
        const double pv =
            y < V ? (double)(LOGITS ? p_elem(x[k], rp.M, rp.rZ, rp.tab) : x[k]) : 0.0;
        w1[k] = pv;
        if (resid) {
            const double r = y < V ? pv - (double)qd[local0 + k] : 0.0;
            w0[k] = r > 0.0 ? r : 0.0;
        } else {
            w0[k] = pv;
        }
    }
}

// The chunk's entries [a, e) of the rejected row's shortlist (ids in
// [base, base + 1024)) scattered into the dense array qd (zeroed first) by
// `nt` threads with index i; the caller orders the writes before the reads.
__device__ __forceinline__ void scatter_q(const int32_t *__restrict__ S,
                                          const float *__restrict__ qrow, int64_t a, int64_t e,
                                          int64_t base, float *qd, int i, int nt, bool zero)
{
    if (zero)
        for (int k = i; k < kChunk; k += nt)
            qd[k] = 0.0f;
    for (int64_t k = a + i; k < e; k += nt) {
        const int64_t o = (int64_t)S[k] - base;
        if (o >= 0 && o < kChunk)
            qd[o] = qrow[k];
    }
}

// the chunk's entry range [a, e), clamped to the row (cbeg comes from the
// shortlist itself; the clamp keeps a malformed list in bounds)
__device__ __forceinline__ void chunk_range(const int32_t *cb, int64_t c, int64_t len, int64_t *a,
                                            int64_t *e)
{
    int64_t x = cb[c], y = cb[c + 1];
    x = x < 0 ? 0 : (x > len ? len : x);
    y = y < x ? x : (y > len ? len : y);
    *a = x;
    *e = y;
}

// Chunk sums: wave w of workgroup x takes chunk 4x + w of sequence blockIdx.y
// (its 1024 tokens as four 256-token parts, each summed as in the final
// walk: four-term lane sums, the wave's inclusive scan, then the parts in
// order).  The q values of the chunk go through the wave's own LDS array.
template <bool LOGITS>
__global__ __launch_bounds__(kChunkThreads) void verify_sum_kernel(
    int B, int T, int V, const int64_t *__restrict__ sl_off, const int32_t *__restrict__ sl_ids,
    const float *__restrict__ q, const float *__restrict__ p, int64_t nchV, void *ws)
{
    __shared__ float qd_all[4][kChunk];
    __shared__ double tab[LOGITS ? 64 : 1];
    const int b = blockIdx.y, wave = threadIdx.x >> 6, lane = lane_id();
    VerifyWs w = verify_ws(ws, B, nchV);
    if (LOGITS) {
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
        chunk_range(w.cbeg + (int64_t)b * (nchV + 1), c, len, &a, &e);
        scatter_q(sl_ids + lo, q + lo, a, e, base, qd, lane, kWave, true);
    }
    // one wave's LDS operations complete in order: the scatter is visible
    double t0 = 0.0, t1 = 0.0;
#pragma unroll
    for (int part = 0; part < 4; ++part) {
        const int64_t local0 = part * 256 + lane * 4;
        double w0[4], w1[4], i0, i1;
        lane_weights<LOGITS>(rp, x[part], base + local0, V, qd, local0, resid, w0, w1);
        const double s0 = wave_chunk_sum(w0, &i0), s1 = wave_chunk_sum(w1, &i1);
        t0 = part == 0 ? s0 : t0 + s0;
        t1 = part == 0 ? s1 : t1 + s1;
    }
    if (lane == 0) {
        w.ch.csum[(int64_t)b * nchV + c] = t0;
        w.ch.csum2[(int64_t)b * nchV + c] = t1;
    }
}

// One workgroup per sequence: the prefix over the chunk sums (the residual,
// or p when the residual has no mass), the chunk owning u_fin * total, the
// walk of that chunk, and the outputs.
template <bool LOGITS>
__global__ __launch_bounds__(kChunkThreads) void verify_final_kernel(
    int B, int T, int V, const int32_t *__restrict__ draft, const int64_t *__restrict__ sl_off,
    const int32_t *__restrict__ sl_ids, const float *__restrict__ q, const float *__restrict__ p,
    const float *__restrict__ u_fin, int64_t nchV, const void *ws, int32_t *__restrict__ n_acc,
    int32_t *__restrict__ out)
{
    __shared__ double P[kMaxVChunks], S[kMaxVChunks];
    __shared__ float qd[kChunk];
    __shared__ double s_wt[4];
    __shared__ double s_total;
    __shared__ int s_owner, s_fallback;
    __shared__ int64_t s_pick[2];
    __shared__ double tab[LOGITS ? 64 : 1];
    const int b = blockIdx.x;
    VerifyWs w = verify_ws(const_cast<void *>(ws), B, nchV);
    if (LOGITS)
        fill_exp2_table(tab);  // ordered by the barriers below
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
    const int owner = s_owner;
    for (int k = threadIdx.x; k <= T; k += blockDim.x)
        if (k != tstar || owner < 0)
            ob[k] = k < tstar ? draft[(int64_t)k * B + b] : -1;
    if (threadIdx.x == 0)
        n_acc[b] = tstar;
    if (owner < 0)
        return;
    const RowP<LOGITS> rp{p + ((int64_t)b * (T + 1) + tstar) * V, LOGITS ? w.rowM[b] : 0.f,
                          LOGITS ? w.rowZ[b] : 0.0, tab};
    const int64_t c = owner, base = c * kChunk;
    const int64_t local0 = (threadIdx.x >> 6) * 256 + lane_id() * 4;
    float x[4];
    lane_raw(rp.r, base + local0, V, x);
    if (resid && !use_p) {
        const int64_t row = (int64_t)tstar * B + b;
        const int64_t lo = sl_off[row], len = sl_off[row + 1] - lo;
        int64_t a, e;
        chunk_range(w.cbeg + (int64_t)b * (nchV + 1), c, len, &a, &e);
        for (int k = threadIdx.x; k < kChunk; k += blockDim.x)
            qd[k] = 0.0f;
        __syncthreads();
        scatter_q(sl_ids + lo, q + lo, a, e, base, qd, threadIdx.x, blockDim.x, false);
        __syncthreads();
    }
    double w0[4], w1[4];
    lane_weights<LOGITS>(rp, x, base + local0, V, qd, local0, resid && !use_p, w0, w1);
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
    hipLaunchKernelGGL(verify_prep_kernel<LOGITS>, dim3((unsigned)B), dim3(kPrepThreads), 0, s,
                       B, T, V, draft, sl_off, sl_ids, q, x, smax, ssum, nseg, u_acc, nchV, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(verify_sum_kernel<LOGITS>, dim3((unsigned)((nchV + 3) / 4), (unsigned)B),
                       dim3(kChunkThreads), 0, s, B, T, V, sl_off, sl_ids, q, x, nchV, ws);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(verify_final_kernel<LOGITS>, dim3((unsigned)B), dim3(kChunkThreads), 0, s,
                       B, T, V, draft, sl_off, sl_ids, q, x, u_fin, nchV, (const void *)ws, n_acc,
                       out);
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
