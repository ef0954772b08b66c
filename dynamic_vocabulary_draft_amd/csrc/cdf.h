// Block-wide inverse-CDF draw over non-negative fp64 weights w[0..n), shared
// by the shortlist sampler and the verifier.  Not method arithmetic of its
// own: it is how the "first index whose running sum exceeds u * total"
// rule is evaluated by one workgroup on gfx950.
//
// Layout: the index range is cut into chunks of `span` = 256*per elements
// (per >= 1 keeps the chunk count within kCdfMaxChunks); a whole wave owns a
// chunk, lane l taking elements 4l..4l+3 of each 256-element sub-chunk, so
// every weight load is coalesced.  Pass 1 sums each chunk (lane sums, wave
// inclusive scan, sub-chunks in order); the chunk sums are scanned in LDS;
// the first chunk whose prefix + sum exceeds the threshold is then walked by
// wave 0 only, which recomputes its weights and finds the first element with
// non-zero mass whose running sum (chunk prefix + lane prefix + in-lane
// prefix) exceeds u*total.  If rounding leaves no such element, the last
// element with non-zero mass is taken.  Every sum has a fixed association,
// so the draw is reproducible bit for bit.
//
// The weight functor F is called by a full wave with a wave-uniform
// sub-chunk and must fill this lane's four weights (0 past the end):
//     __device__ void operator()(int64_t j0_of_this_lane, double w[4]) const;
// It may use wave-level LDS scratch but no block barrier.
#pragma once

#include "common.h"

namespace ds {

constexpr int kCdfMaxChunks = 2048;
// doubles of LDS the caller reserves for block_inverse_cdf
constexpr int kCdfShDoubles = 2 * kCdfMaxChunks + kWave + 1;

template <class F>
__device__ int64_t block_inverse_cdf(const F &f, int64_t n, double u, double *sh, int *s_int,
                                     double *total_out)
{
    double *P = sh, *S = sh + kCdfMaxChunks, *scan_sh = sh + 2 * kCdfMaxChunks;
    const int lane = lane_id(), wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int tid = threadIdx.x, nt = blockDim.x;
    const int64_t nsub = (n + 255) / 256;
    const int64_t per = (nsub + kCdfMaxChunks - 1) / kCdfMaxChunks > 0
                            ? (nsub + kCdfMaxChunks - 1) / kCdfMaxChunks
                            : 1;
    const int64_t span = per * 256;
    const int nch = (int)((n + span - 1) / span);

    // pass 1: chunk sums
    for (int c = wave; c < nch; c += nw) {
        double acc = 0.0;
        for (int64_t sidx = 0; sidx < per; ++sidx) {
            const int64_t j0 = (int64_t)c * span + sidx * 256;
            if (j0 >= n)
                break;
            double w[4];
            f(j0 + lane * 4, w);
            double lv = ((w[0] + w[1]) + w[2]) + w[3];
            double incl = wave_incl_scan_f64(lv);
            acc += __shfl(incl, kWave - 1);
        }
        if (lane == 0)
            S[c] = acc;
    }
    if (tid == 0)
        s_int[0] = nch;
    __syncthreads();

    // exclusive scan of the chunk sums: thread t owns a contiguous run
    const int per_t = (nch + nt - 1) / nt;
    const int c0 = min(nch, tid * per_t), c1 = min(nch, c0 + per_t);
    double loc = 0.0;
    for (int c = c0; c < c1; ++c)
        loc += S[c];
    double total;
    double ex = block_excl_scan_f64(loc, scan_sh, &total);
    for (int c = c0; c < c1; ++c) {
        P[c] = ex;
        ex += S[c];
    }
    __syncthreads();
    const double thr = u * total;
    for (int c = c0; c < c1; ++c)
        if (P[c] + S[c] > thr) {
            atomicMin(&s_int[0], c);
            break;
        }
    __syncthreads();

    if (wave == 0) {
        int64_t pick = -1;
        for (int c = s_int[0]; c < nch && pick < 0; ++c) {
            double run = P[c];
            for (int64_t sidx = 0; sidx < per; ++sidx) {
                const int64_t j0 = (int64_t)c * span + sidx * 256;
                if (j0 >= n)
                    break;
                double w[4];
                f(j0 + lane * 4, w);
                double lv = ((w[0] + w[1]) + w[2]) + w[3];
                double incl = wave_incl_scan_f64(lv);
                double prev = __shfl_up(incl, 1);
                if (lane == 0)
                    prev = 0.0;
                int kk = -1;
                double pk = 0.0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    pk += w[k];
                    if (kk < 0 && w[k] > 0.0 && run + (prev + pk) > thr)
                        kk = k;
                }
                uint64_t bal = __ballot(kk >= 0);
                if (bal) {
                    int L = __ffsll((unsigned long long)bal) - 1;
                    pick = j0 + L * 4 + __shfl(kk, L);
                    break;
                }
                run += __shfl(incl, kWave - 1);
            }
        }
        if (pick < 0) {  // rounding left no crossing: the last element with mass
            for (int c = nch - 1; c >= 0 && pick < 0; --c) {
                if (!(S[c] > 0.0))
                    continue;
                for (int64_t sidx = per - 1; sidx >= 0; --sidx) {
                    const int64_t j0 = (int64_t)c * span + sidx * 256;
                    if (j0 >= n)
                        continue;
                    double w[4];
                    f(j0 + lane * 4, w);
                    int kk = -1;
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (w[k] > 0.0)
                            kk = k;
                    uint64_t bal = __ballot(kk >= 0);
                    if (bal) {
                        int L = 63 - __clzll((long long)bal);
                        pick = j0 + L * 4 + __shfl(kk, L);
                        break;
                    }
                }
            }
        }
        if (lane == 0)
            s_int[1] = (int)pick;
    }
    __syncthreads();
    *total_out = total;
    return s_int[1];
}

}  // namespace ds
