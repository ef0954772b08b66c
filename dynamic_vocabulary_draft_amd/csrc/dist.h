// Chunked normalisation and inverse-CDF draws over long rows, shared by the
// shortlist sampler, the target softmax and the verifier.  Not method
// arithmetic of its own: this is how "normalise non-negative weights, then
// take the first index whose running sum exceeds u * total" is spread over
// many workgroups on gfx950 without any cross-workgroup wait.
//
// A row is cut into chunks of kChunk = 1024 elements; one 256-thread
// workgroup owns a chunk, wave w its w-th 256-element sub-chunk, lane l its
// four consecutive elements 4l..4l+3 (coalesced 16-byte accesses).  Two
// launches, each with one workgroup per (chunk, row):
//   1. chunk statistics: the chunk max m_c (and the first index holding
//      it) and the chunk sum of the weights taken relative to m_c, in a
//      fixed association (lane sums of four, wave inclusive scan, the four
//      wave totals in order);
//   2. every workgroup rebuilds the same row max M, the chunk sums rescaled
//      to M (s_c * exp(m_c - M)), their prefix sums and the total (one
//      wave, fixed order), writes its normalised chunk, and the one
//      workgroup whose chunk holds the threshold walks it with weights
//      taken relative to M.
// The running sum at an element is: chunk prefix + earlier waves' totals +
// earlier lanes' inclusive scan + this lane's partial sum.  If rounding
// leaves no element past the threshold in that chunk, its last element with
// non-zero mass is taken; if no chunk reaches the threshold, the last
// element with non-zero mass of the row.  All sums have fixed association,
// so results are reproducible bit for bit.
#pragma once

#include <float.h>

#include "common.h"
#include "kernels.h"

namespace ds {

constexpr int kChunk = 1024;
constexpr int kChunkThreads = 256;

// exp(x) in fp64 by Tang's table-driven method (ACM TOMS 15(2), 1989):
// x = (64n + j) ln2/64 + r with |r| <= ln2/128 (ln2/64 split in two parts,
// so r is exact to ~1e-19), exp(x) = 2^n * 2^(j/64) * e^r, and e^r - 1 from
// its Taylor series through r^5 (the next term is below 4e-17).  About 16
// instructions against some 75 for the library routine; relative error at
// most 2 fp64 ulp for x > -708 (below that the result is subnormal and its
// absolute error under one subnormal ulp).  x below -1000 (-inf included)
// gives exactly 0, NaN stays NaN.  Every caller passes x <= 0 (a value minus
// a maximum), so there is no upper clamp: x above ~709 overflows to inf as
// exp does, up to x ~ 2e7.  tab[j] = 2^(j/64), filled by fill_exp2_table.
__device__ __forceinline__ double exp_tab(double x, const double *tab)
{
    constexpr double kInvL = 0x1.71547652b82fep+6;   // 64 / ln 2
    constexpr double kL1 = 0x1.62e42fefa39efp-7;     // ln 2 / 64, leading part
    constexpr double kL2 = 0x1.abc9e3b39803fp-62;    // ln 2 / 64 - kL1
    x = x < -1000.0 ? -1000.0 : x;
    const double kf = rint(x * kInvL);
    double r = fma(-kf, kL1, x);
    r = fma(-kf, kL2, r);
    const int k = (int)kf;
    const double t = tab[k & 63];
    double q = fma(r, 1.0 / 120, 1.0 / 24);
    q = fma(q, r, 1.0 / 6);
    q = fma(q, r, 0.5);
    const double pm1 = fma(q, r * r, r);  // e^r - 1
    return ldexp(fma(t, pm1, t), k >> 6);
}

// tab[j] = 2^(j/64) in LDS, by the first wave; visible after the caller's
// next barrier
__device__ __forceinline__ void fill_exp2_table(double *tab)
{
    if (threadIdx.x < 64)
        tab[threadIdx.x] = exp2((double)threadIdx.x / 64.0);
}

// The target softmax's row normaliser, rebuilt from its per-segment
// statistics (segment maxima smax and sums of exp(l - smax), nseg of each):
// M = the row max, rZ = 1 / sum_s ssum_s exp(smax_s - M), by one whole wave
// in a fixed association (every lane gets the values).  Any kernel that
// rebuilds it from the same statistics gets the same bits, so p_elem below
// reproduces the softmax's output exactly.
__device__ __forceinline__ void row_norm(const float *__restrict__ sm, const double *__restrict__ ss,
                                         int64_t nseg, const double *tab, float *M, double *rZ)
{
    float m = -INFINITY;
    for (int64_t c = lane_id(); c < nseg; c += kWave)
        m = fmaxf(m, sm[c]);
    m = wave_max(m);
    double z = 0.0;
    for (int64_t c = lane_id(); c < nseg; c += kWave)
        z += ss[c] * exp_tab((double)sm[c] - (double)m, tab);
    z = wave_sum_f64(z);
    *M = m;
    *rZ = 1.0 / z;  // p = w * (1/Z): within one fp32 ulp of w / Z
}

// p for logit l of a row with normaliser (M, rZ)
__device__ __forceinline__ float p_elem(float l, float M, double rZ, const double *tab)
{
    return (float)(exp_tab((double)l - (double)M, tab) * rZ);
}

// (x) / T; T = 1 (the usual case, and always for the target) skips the
// fp64 division, which leaves the value unchanged
__device__ __forceinline__ double over_tau(double x, double tau) { return tau == 1.0 ? x : x / tau; }

// a draft row's weight of logit l relative to its max M, exp((l - M) / T)
__device__ __forceinline__ double draft_w(float l, double M, double tau, const double *tab)
{
    return exp_tab(over_tau((double)l - M, tau), tab);
}
// q for draft logit l of a row with statistics (M, rZ): the sampler's q
__device__ __forceinline__ float q_elem(float l, float M, double rZ, double tau, const double *tab)
{
    return (float)(draft_w(l, (double)M, tau, tab) * rZ);
}

// q of one draft row from its stored values: the values themselves, or
// (QL) draft logits turned into q with the row's statistics
template <bool QL>
struct QRow {
    float M;
    double rZ, tau;
    const double *tab;
    __device__ __forceinline__ float operator()(float x) const
    {
        return QL ? q_elem(x, M, rZ, tau, tab) : x;
    }
};
template <bool QL>
__device__ __forceinline__ QRow<QL> q_row(const QStats *qs, int64_t row, double qtau,
                                          const double *tab)
{
    return QL ? QRow<QL>{qs[row].M, qs[row].rZ, qtau, tab} : QRow<QL>{0.f, 0.0, 0.0, tab};
}

// this lane's four consecutive elements (-FLT_MAX past the row end); one
// 16-byte load when the row base is 16-byte aligned (j0 is a multiple of 4)
__device__ __forceinline__ void load4(const float *__restrict__ l, int64_t j0, int64_t len,
                                      float v[4])
{
    const bool vec = (reinterpret_cast<uintptr_t>(l) & 15) == 0;
    if (vec && j0 + 3 < len) {
        const float4 q = *reinterpret_cast<const float4 *>(l + j0);
        v[0] = q.x, v[1] = q.y, v[2] = q.z, v[3] = q.w;
        return;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
        v[k] = j0 + k < len ? l[j0 + k] : -FLT_MAX;
}

// Target softmax segments: kSeg elements per 256-thread workgroup; lane l
// of wave w holds elements 1024 i + 256 w + 4 l + k (i, k < 4) of it.
constexpr int kSeg = 4 * kChunk;

__device__ __forceinline__ void load_seg(const float *__restrict__ lr, int64_t j0, int64_t V,
                                         float v[4][4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        load4(lr, j0 + i * kChunk, V, v[i]);
}

// Statistics of segment `seg` of one row of V logits, by the whole
// (256-thread) workgroup: its max (fp32, exact) and the sum of exp(l - max)
// over it in fp64, in a fixed association (each lane's 16 terms in order,
// the wave butterfly, the four wave sums in order); -inf logits weigh 0.
// Thread 0 writes *sum_out and *max_out.
__device__ __forceinline__ void segment_stats(int64_t V, const float *__restrict__ row,
                                              int64_t seg, double *sum_out, float *max_out)
{
    __shared__ float s_m[4];
    __shared__ double s_s[4];
    __shared__ double s_exp2[64];
    const int64_t j0 = seg * kSeg + (threadIdx.x >> 6) * 256 + lane_id() * 4;
    float v[4][4];
    load_seg(row, j0, V, v);
    fill_exp2_table(s_exp2);
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k)
            m = fmaxf(m, v[i][k]);  // -FLT_MAX past V
    m = wave_max(m);
    if (lane_id() == 0)
        s_m[threadIdx.x >> 6] = m;
    __syncthreads();  // also orders the table
    const float mseg = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // computed for every element and selected (no branch per
            // element); adding an exact 0 leaves the sum unchanged
            const float x = v[i][k];
            const double e = exp_tab((double)x - (double)mseg, s_exp2);
            acc += (j0 + i * kChunk + k < V && x != -INFINITY) ? e : 0.0;
        }
    acc = wave_sum_f64(acc);
    if (lane_id() == 0)
        s_s[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        *sum_out = ((s_s[0] + s_s[1]) + s_s[2]) + s_s[3];
        *max_out = mseg;
    }
}

// chunk statistics kept in a caller workspace: [rows][nchmax] of each
struct ChunkWs {
    float *cmax;
    int *cidx;
    double *csum;
    double *csum2;  // second weight family (verify: plain p for the fallback)
};

__host__ __device__ inline size_t chunk_ws_bytes(int64_t rows, int64_t nchmax)
{
    return (size_t)rows * (size_t)nchmax * (8 + 8 + 4 + 4) + 256;
}

__host__ __device__ inline int64_t chunks_for(int64_t len) { return (len + kChunk - 1) / kChunk; }

__host__ __device__ inline ChunkWs chunk_ws(void *ws, int64_t rows, int64_t nchmax)
{
    ChunkWs w;
    char *p = reinterpret_cast<char *>(ws);
    const size_t n = (size_t)rows * (size_t)nchmax;
    w.csum = reinterpret_cast<double *>(p);
    w.csum2 = reinterpret_cast<double *>(p + n * 8);
    w.cmax = reinterpret_cast<float *>(p + n * 16);
    w.cidx = reinterpret_cast<int *>(p + n * 20);
    return w;
}

// Block (256 threads) max over a chunk and the first index attaining it.
// `v[k]` is this lane's element 4l+k of wave w's sub-chunk (-inf if absent).
__device__ inline void block_chunk_max(const float v[4], int64_t j0_lane, float *s_max, int *s_idx,
                                       float *out_max, int *out_idx)
{
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    float m = v[0];
    int idx = 0;
#pragma unroll
    for (int k = 1; k < 4; ++k)
        if (v[k] > m) {
            m = v[k];
            idx = k;
        }
    float wm = wave_max(m);
    uint64_t bal = __ballot(m == wm);
    int L = __ffsll((unsigned long long)bal) - 1;
    int first = __shfl((int)(j0_lane + idx), L);
    if (lane == 0) {
        s_max[wave] = wm;
        s_idx[wave] = first;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float bm = s_max[0];
        int bi = s_idx[0];
        for (int w = 1; w < (int)(blockDim.x >> 6); ++w)
            if (s_max[w] > bm) {
                bm = s_max[w];
                bi = s_idx[w];
            }
        *out_max = bm;
        *out_idx = bi;
    }
}

// Sum of four fp64 weights per lane over the wave: returns the wave total;
// *incl gets this lane's inclusive prefix (lane order).
__device__ __forceinline__ double wave_chunk_sum(const double w[4], double *incl)
{
    double lv = ((w[0] + w[1]) + w[2]) + w[3];
    *incl = wave_incl_scan_f64(lv);
    return __shfl(*incl, kWave - 1);
}

// Row-wide chunk prefix sums (exclusive) into P[0..nch), the chunk sums into
// S[0..nch) (both LDS) and the row total, computed by wave 0 in a fixed
// order; call from all threads (barrier inside).
__device__ inline double row_prefix(const double *__restrict__ csum, int nch, double *P, double *S,
                                    double *s_total)
{
    if ((threadIdx.x >> 6) == 0) {
        const int lane = lane_id();
        double carry = 0.0;
        for (int b = 0; b < nch; b += kWave) {
            const int c = b + lane;
            double v = c < nch ? csum[c] : 0.0;
            double incl = wave_incl_scan_f64(v);
            double ex = __shfl_up(incl, 1);
            if (lane == 0)
                ex = 0.0;
            if (c < nch) {
                P[c] = carry + ex;
                S[c] = v;
            }
            carry += __shfl(incl, kWave - 1);
        }
        if (lane == 0)
            *s_total = carry;
    }
    __syncthreads();
    return *s_total;
}

// Which chunk owns the draw: the first with prefix + sum > thr; else (no
// crossing) the last chunk with non-zero mass, flagged as a fallback (-1 if
// none).  P and S in LDS; evaluated by wave 0 with ballots, 64 chunks per
// step; the result goes to *s_owner / *s_fb after a barrier.
__device__ inline void owner_chunk(const double *P, const double *S, int nch, double thr,
                                   int *s_owner, int *s_fb)
{
    if ((threadIdx.x >> 6) == 0) {
        const int lane = lane_id();
        int owner = -1, fb = 0;
        for (int b = 0; b < nch; b += kWave) {
            const int c = b + lane;
            const uint64_t bal = __ballot(c < nch && P[c] + S[c] > thr);
            if (bal) {
                owner = b + __ffsll((unsigned long long)bal) - 1;
                break;
            }
        }
        if (owner < 0) {
            fb = 1;
            for (int b = ((nch - 1) / kWave) * kWave; b >= 0; b -= kWave) {
                const int c = b + lane;
                const uint64_t bal = __ballot(c < nch && S[c] > 0.0);
                if (bal) {
                    owner = b + 63 - __clzll((long long)bal);
                    break;
                }
            }
        }
        if (lane == 0) {
            *s_owner = owner;
            *s_fb = fb;
        }
    }
    __syncthreads();
}

// Walk of the owning chunk by its workgroup.  w[4] are this lane's weights
// (elements j0_lane..j0_lane+3), wtot[wave] the four wave totals of the
// chunk (in LDS), Pc the chunk prefix.  Returns (to every thread) the
// element index picked: first with non-zero mass whose running sum exceeds
// thr, else (fallback or rounding) the last element with non-zero mass.
__device__ inline int64_t chunk_walk(const double w[4], int64_t j0_lane, const double *wtot,
                                     double incl, double Pc, double thr, bool fallback,
                                     int64_t *s_pick)
{
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    unsigned long long *sp = reinterpret_cast<unsigned long long *>(s_pick);
    if (threadIdx.x == 0)
        sp[0] = ~0ull, sp[1] = 0ull;  // first pick; last positive index + 1
    __syncthreads();
    double run = Pc;
    for (int k = 0; k < wave; ++k)
        run += wtot[k];
    double prev = __shfl_up(incl, 1);
    if (lane == 0)
        prev = 0.0;
    double pk = 0.0;
    int64_t first = INT64_MAX, last = -1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        pk += w[k];
        if (w[k] > 0.0) {
            last = j0_lane + k;
            if (first == INT64_MAX && !fallback && run + (prev + pk) > thr)
                first = j0_lane + k;
        }
    }
    // elements ascend with the lane: the wave's first pick is the lowest
    // lane's, its last positive index the highest lane's; one LDS atomic per
    // wave (same-address atomics from every lane serialise)
    const uint64_t bf = __ballot(first != INT64_MAX), bl = __ballot(last >= 0);
    if (bf) {
        const int64_t f = __shfl(first, __ffsll((unsigned long long)bf) - 1);
        if (lane == 0)
            atomicMin(&sp[0], (unsigned long long)f);
    }
    if (bl) {
        const int64_t l = __shfl(last, 63 - __clzll((long long)bl));
        if (lane == 0)
            atomicMax(&sp[1], (unsigned long long)(l + 1));
    }
    __syncthreads();
    return sp[0] != ~0ull ? (int64_t)sp[0] : (int64_t)sp[1] - 1;
}

// First index a in [0, len] with S[a] >= x for an ascending int32 array,
// found by a whole wave in three dependent loads for len <= 64^3 (each
// round samples 64 evenly spaced entries and keeps one gap).  For an array
// that is not ascending the result is still within [0, len].
__device__ inline int64_t wave_lower_bound(const int32_t *__restrict__ S, int64_t len, int32_t x)
{
    const int lane = lane_id();
    int64_t lo = 0, hi = len;
    while (hi - lo > kWave) {
        const int64_t step = (hi - lo + kWave - 1) / kWave;
        const int64_t idx = lo + (int64_t)lane * step;
        const bool lt = idx < hi && S[idx] < x;
        const int k = __popcll(__ballot(lt));
        const int64_t nlo = k > 0 ? lo + (int64_t)(k - 1) * step + 1 : lo;
        const int64_t nhi = min(hi, lo + (int64_t)k * step);
        lo = nlo;
        hi = nhi;
    }
    const int64_t idx = lo + lane;
    const bool lt = idx < hi && S[idx] < x;
    return lo + __popcll(__ballot(lt));
}

// wave_lower_bound for two keys x0 <= x1 at once (the loads of both
// searches of a round are issued together): *r0, *r1 as two calls would give.
__device__ inline void wave_lower_bound2(const int32_t *__restrict__ S, int64_t len, int32_t x0,
                                         int32_t x1, int64_t *r0, int64_t *r1)
{
    const int lane = lane_id();
    int64_t lo0 = 0, hi0 = len, lo1 = 0, hi1 = len;
    while (hi0 - lo0 > kWave || hi1 - lo1 > kWave) {
        const bool a0 = hi0 - lo0 > kWave, a1 = hi1 - lo1 > kWave;  // wave-uniform
        const int64_t st0 = (hi0 - lo0 + kWave - 1) / kWave, st1 = (hi1 - lo1 + kWave - 1) / kWave;
        const int64_t i0 = lo0 + (int64_t)lane * st0, i1 = lo1 + (int64_t)lane * st1;
        const bool in0 = a0 && i0 < hi0, in1 = a1 && i1 < hi1;
        const int32_t v0 = in0 ? S[i0] : 0, v1 = in1 ? S[i1] : 0;
        if (a0) {
            const int k = __popcll(__ballot(in0 && v0 < x0));
            const int64_t nlo = k > 0 ? lo0 + (int64_t)(k - 1) * st0 + 1 : lo0;
            hi0 = min(hi0, lo0 + (int64_t)k * st0);
            lo0 = nlo;
        }
        if (a1) {
            const int k = __popcll(__ballot(in1 && v1 < x1));
            const int64_t nlo = k > 0 ? lo1 + (int64_t)(k - 1) * st1 + 1 : lo1;
            hi1 = min(hi1, lo1 + (int64_t)k * st1);
            lo1 = nlo;
        }
    }
    const int64_t i0 = lo0 + lane, i1 = lo1 + lane;
    const bool in0 = i0 < hi0, in1 = i1 < hi1;
    const int32_t v0 = in0 ? S[i0] : 0, v1 = in1 ? S[i1] : 0;
    *r0 = lo0 + __popcll(__ballot(in0 && v0 < x0));
    *r1 = lo1 + __popcll(__ballot(in1 && v1 < x1));
}

}  // namespace ds
