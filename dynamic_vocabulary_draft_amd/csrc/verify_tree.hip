// Tree verification by multi-step speculative sampling (SpecInfer:
// "Accelerating Generative Large Language Model Serving with Tree-based
// Speculative Inference and Verification", cited by the DySpec page; the
// DynaSpec pages draft trees in the tree-shaped workload but verify only
// chains).  From the root, the children of the current node u are tried in
// index order against a running residual r that starts as the target p_u:
// child c (token x drawn from its own proposal q_c) is accepted iff
// u_acc * q_c(x) < r(x); after a rejection r <- max(0, r - q_c) / sum.  An
// accepted child becomes the current node; otherwise one token is drawn
// from r and the sequence stops.
//
// The walk is sequential per sequence, so one 1024-thread workgroup owns a
// sequence.  The residual is kept unnormalised: r = R / P with R = p_u off
// the shortlist (a proposal has no mass there, so those entries only
// rescale) and R_S in a workspace on the shortlist, P the current
// normaliser.  A rejection updates R_S <- max(0, R_S - P q_c) and P <-
// (off-shortlist mass of p_u) + sum R_S, so the long V-wide row is read
// once per node that sees a rejection (for its off-shortlist mass, per
// 1024-token chunk) and never rescaled.  The first test at a node compares
// fp32 values exactly in fp64 (u * q < p); every later test and the final
// draw differ from a sequential fp64 evaluation by rounding order only.
//
// Two launches:
//   bits: one workgroup per (32768 tokens, sequence) writes the shortlist's
//         membership bitmap (bit y set iff token y is in the shortlist), so
//         the position of a token in the ascending shortlist is the chunk's
//         first shortlist index plus a popcount;
//   walk: one workgroup per sequence: chunk ranges of the shortlist, every
//         drafted node's shortlist position, u * q and target value at its
//         parent (in LDS, all tests at a node's first child need nothing
//         else), then the walk and the final inverse-CDF draw over V.
#include <limits.h>

#include "common.h"
#include "dist.h"
#include "kernels.h"

namespace ds {
namespace {

constexpr int kTreeThreads = 1024;
constexpr int kTreeWaves = kTreeThreads / kWave;
constexpr int kTreeMaxNodes = DS_MAX_TREE_NODES;
constexpr int kTreeMaxChunks = (1 << 20) / kChunk;  // V <= 2^20
constexpr int kBitsTokens = 32768;                  // tokens per bitmap workgroup
constexpr int kWordsPerChunk = kChunk / 32;

__host__ __device__ inline int tree_chunks(int V) { return (V + kChunk - 1) / kChunk; }

__host__ __device__ inline size_t tree_R_bytes(int B, int64_t max_len)
{
    return ((size_t)B * (size_t)max_len * 8 + 255) / 256 * 256;
}

__global__ __launch_bounds__(256) void tree_bits_kernel(int V, int64_t max_len,
                                                         const int64_t *__restrict__ sl_off,
                                                         const int32_t *__restrict__ sl_ids,
                                                         uint32_t *__restrict__ bits)
{
    __shared__ uint32_t sw[kBitsTokens / 32];
    __shared__ int64_t s_rng[2];
    const int b = blockIdx.y;
    const int64_t nwords = (int64_t)tree_chunks(V) * kWordsPerChunk;
    const int64_t t0 = (int64_t)blockIdx.x * kBitsTokens;  // < V by the grid
    const int64_t t1 = min(t0 + kBitsTokens, (int64_t)V);
    const int64_t off = sl_off[b];
    int64_t len = sl_off[b + 1] - off;
    if (len < 0 || len > max_len)
        len = 0;  // the walk reports such a sequence
    for (int i = threadIdx.x; i < kBitsTokens / 32; i += blockDim.x)
        sw[i] = 0u;
    if (threadIdx.x < kWave) {
        const int64_t a = wave_lower_bound(sl_ids + off, len, (int32_t)t0);
        const int64_t e = wave_lower_bound(sl_ids + off, len, (int32_t)t1);
        if (lane_id() == 0) {
            s_rng[0] = a;
            s_rng[1] = e;
        }
    }
    __syncthreads();
    for (int64_t j = s_rng[0] + threadIdx.x; j < s_rng[1]; j += blockDim.x) {
        const int32_t y = sl_ids[off + j];
        if (y >= t0 && y < t1)
            atomicOr(&sw[(y - t0) >> 5], 1u << (y & 31));
    }
    __syncthreads();
    uint32_t *ob = bits + (int64_t)b * nwords + t0 / 32;
    for (int i = threadIdx.x; i < kBitsTokens / 32 && t0 / 32 + i < nwords; i += blockDim.x)
        ob[i] = sw[i];
}

__device__ __forceinline__ int wave_sum_int(int v)
{
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1)
        v += __shfl_xor(v, o);
    return v;
}

// Block sum with a fixed association (lane 0's wave sum, then the wave sums
// in order); every thread gets the same value.
__device__ double block_sum_f64(double v, double *sh)
{
    const double w = wave_sum_f64(v);
    if (lane_id() == 0)
        sh[threadIdx.x >> 6] = w;
    __syncthreads();
    double t = 0.0;
    for (int k = 0; k < kTreeWaves; ++k)
        t += sh[k];
    __syncthreads();
    return t;
}

// Position of token x in the ascending shortlist (-1 if absent), from the
// chunk's first shortlist index cb and the bitmap words of x's chunk; called
// by a whole wave.
__device__ __forceinline__ int shortlist_pos(const uint32_t *__restrict__ bits_b, const int *cb,
                                             int V, int32_t x)
{
    if (x < 0 || x >= V)
        return -1;
    const int lane = lane_id();
    const int ch = x >> 10, o = x & (kChunk - 1), wi = o >> 5;
    const uint32_t mw = lane < kWordsPerChunk ? bits_b[(int64_t)ch * kWordsPerChunk + lane] : 0u;
    const uint32_t below = lane < wi ? mw : (lane == wi ? mw & ((1u << (o & 31)) - 1u) : 0u);
    const int cnt = wave_sum_int(__popc(below));
    const uint32_t word = __shfl(mw, wi);
    return ((word >> (o & 31)) & 1u) ? cb[ch] + cnt : -1;
}

// Target mass of row pu off the shortlist, per 1024-token chunk into s_off;
// returns the row's total (chunk order).  Wave w takes chunks w, w+16, ...,
// two at a time; lane l its tokens 64k + l of the chunk (coalesced loads).
__device__ double off_sums(const float *__restrict__ pu, const uint32_t *__restrict__ bits_b,
                           int V, int nch, double *s_off, double *sh)
{
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    for (int c0 = wave; c0 < nch; c0 += 2 * kTreeWaves) {
        float pv[2][16];
        uint32_t mw[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = c0 + h * kTreeWaves;
            const int64_t base = (int64_t)c * kChunk;
            mw[h] = (c < nch && lane < kWordsPerChunk) ? bits_b[(int64_t)c * kWordsPerChunk + lane]
                                                       : 0u;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int64_t y = base + k * kWave + lane;
                pv[h][k] = (c < nch && y < V) ? pu[y] : 0.0f;
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            double acc = 0.0;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const uint32_t w = __shfl(mw[h], 2 * k + (lane >> 5));
                if (!((w >> (lane & 31)) & 1u))
                    acc += (double)pv[h][k];
            }
            acc = wave_sum_f64(acc);
            const int c = c0 + h * kTreeWaves;
            if (lane == 0 && c < nch)
                s_off[c] = acc;
        }
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
        double carry = 0.0;
        for (int c0 = 0; c0 < nch; c0 += kWave)
            carry += wave_sum_f64(c0 + lane < nch ? s_off[c0 + lane] : 0.0);
        if (lane == 0)
            sh[kWave] = carry;
    }
    __syncthreads();
    const double t = sh[kWave];
    __syncthreads();
    return t;
}

// R <- max(0, R - P q_c) on the shortlist (R read as p_u at the shortlist
// ids when fresh); returns sum R.
__device__ double residual_update(const float *__restrict__ pu, const int32_t *__restrict__ S,
                                  const float *__restrict__ qc, int len, int V, bool fresh,
                                  double P, double *__restrict__ R, double *sh)
{
    constexpr int U = 4;
    double acc = 0.0;
    for (int j0 = threadIdx.x; j0 < len; j0 += kTreeThreads * U) {
        double r[U];
        float qv[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int j = j0 + k * kTreeThreads;
            qv[k] = j < len ? qc[j] : 0.0f;
            if (fresh) {
                const int32_t y = j < len ? S[j] : -1;
                r[k] = (y >= 0 && y < V) ? (double)pu[y] : 0.0;
            } else {
                r[k] = j < len ? R[j] : 0.0;
            }
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int j = j0 + k * kTreeThreads;
            const double t = P * (double)qv[k];
            const double nr = r[k] > t ? r[k] - t : 0.0;
            if (j < len) {
                R[j] = nr;
                acc += nr;
            }
        }
    }
    return block_sum_f64(acc, sh);
}

__global__ __launch_bounds__(kTreeThreads) void verify_tree_kernel(
    int m, int V, int64_t max_len, const int32_t *__restrict__ parent,
    const int32_t *__restrict__ token, const int64_t *__restrict__ sl_off,
    const int32_t *__restrict__ sl_ids, const float *__restrict__ q, const float *__restrict__ p,
    const float *__restrict__ u_acc, const float *__restrict__ u_fin,
    const uint32_t *__restrict__ bits, double *__restrict__ Rws, int32_t *__restrict__ n_acc,
    int32_t *__restrict__ out, int32_t *__restrict__ path)
{
    __shared__ int s_par[kTreeMaxNodes], s_pos[kTreeMaxNodes], s_tok[kTreeMaxNodes];
    __shared__ double s_lhs[kTreeMaxNodes], s_px[kTreeMaxNodes];
    __shared__ int s_cb[kTreeMaxChunks + 2];
    __shared__ double s_off[kTreeMaxChunks], s_tot[kTreeMaxChunks], s_pre[kTreeMaxChunks];
    __shared__ double sh[kWave + 1];
    __shared__ uint32_t s_mw[kWordsPerChunk];
    __shared__ int s_mpre[kWordsPerChunk];
    __shared__ int s_int[4];

    const int b = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int nch = tree_chunks(V);
    const int64_t nwords = (int64_t)nch * kWordsPerChunk;
    const uint32_t *bits_b = bits + (int64_t)b * nwords;
    double *R = Rws + (int64_t)b * max_len;
    const int64_t off = sl_off[b];
    const int64_t len64 = sl_off[b + 1] - off;
    int32_t *ob = out + (int64_t)b * (m + 1), *pb = path + (int64_t)b * m;
    for (int i = tid; i <= m; i += kTreeThreads) {
        ob[i] = -1;
        if (i < m)
            pb[i] = -1;
    }
    if (len64 < 0 || len64 > max_len) {
        if (tid == 0)
            n_acc[b] = -1;
        return;
    }
    const int len = (int)len64;
    const int32_t *S = sl_ids + off;

    // shortlist range of every chunk: s_cb[c] = #{ids < 1024 c}, c = 0..nch
    for (int i = tid; i < nch + 2; i += kTreeThreads)
        s_cb[i] = 0;
    __syncthreads();
    for (int j = tid; j < len; j += kTreeThreads) {
        const int32_t y = S[j];
        const int k = y < 0 ? 0 : (y >= nch * kChunk ? nch + 1 : (y >> 10) + 1);
        atomicAdd(&s_cb[k], 1);
    }
    __syncthreads();
    if (wave == 0) {
        int carry = 0;
        for (int c0 = 0; c0 <= nch; c0 += kWave) {
            const int c = c0 + lane;
            int v = c <= nch ? s_cb[c] : 0;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const int t = __shfl_up(v, o);
                if (lane >= o)
                    v += t;
            }
            if (c <= nch)
                s_cb[c] = carry + v;
            carry += __shfl(v, kWave - 1);
        }
    }
    __syncthreads();

    // per drafted node i (index i-1): parent, token, shortlist position,
    // u * q_i(x) (exact in fp64) and the target at its parent p_par(x)
    for (int i = wave + 1; i <= m; i += kTreeWaves) {
        const int64_t e = (int64_t)b * m + i - 1;
        const int32_t x = token[e];
        const int par = parent[e];
        const int pos = shortlist_pos(bits_b, s_cb, V, x);
        if (lane == 0) {
            const float *qi = q + (int64_t)m * off + (int64_t)(i - 1) * len;
            const double qx = pos >= 0 ? (double)qi[pos] : 0.0;
            const bool valid = x >= 0 && x < V;
            const bool linked = par >= 0 && par < i;
            s_par[i - 1] = linked ? par : -1;
            s_tok[i - 1] = x;
            s_pos[i - 1] = pos;
            s_lhs[i - 1] = (double)u_acc[e] * qx;
            s_px[i - 1] = (valid && linked) ? (double)p[((int64_t)b * (m + 1) + par) * V + x] : 0.0;
        }
    }
    __syncthreads();

    int u = 0, n = 0;
    for (int visit = 0; visit <= m; ++visit) {  // u increases on every acceptance
        const float *pu = p + ((int64_t)b * (m + 1) + u) * V;
        bool fresh = true, have_off = false;
        double P = 1.0, Poff = 0.0;
        int acc = -1;
        for (int c = u + 1; c <= m; ++c) {
            if (s_par[c - 1] != u)
                continue;
            const int pos = s_pos[c - 1];
            // R and the LDS tables were written before a barrier; every
            // thread takes the same decision
            const double rx = fresh ? s_px[c - 1] : (pos >= 0 ? R[pos] : s_px[c - 1]) / P;
            if (s_lhs[c - 1] < rx) {
                acc = c;
                break;
            }
            if (!have_off) {  // (its barriers also order this test's reads of R)
                Poff = off_sums(pu, bits_b, V, nch, s_off, sh);
                have_off = true;
            } else {
                __syncthreads();  // every thread has read R for this test
            }
            const float *qc = q + (int64_t)m * off + (int64_t)(c - 1) * len;
            const double sr = residual_update(pu, S, qc, len, V, fresh, P, R, sh);
            const double Pn = Poff + sr;
            if (Pn > 0.0) {
                P = Pn;
                fresh = false;
            } else {  // the residual has no mass: back to p_u
                P = 1.0;
                fresh = true;
            }
        }
        if (acc >= 0) {
            if (tid == 0) {
                ob[n] = s_tok[acc - 1];
                pb[n] = acc;
            }
            ++n;
            u = acc;
            continue;
        }

        // final draw from r over all V (inverse CDF, chunk by chunk)
        if (!have_off)
            Poff = off_sums(pu, bits_b, V, nch, s_off, sh);
        for (int c = wave; c < nch; c += kTreeWaves) {
            const int lo = s_cb[c], hi = s_cb[c + 1];
            double a = 0.0;
            for (int j = lo + lane; j < hi; j += kWave) {
                if (fresh) {
                    const int32_t y = S[j];
                    a += (y >= 0 && y < V) ? (double)pu[y] : 0.0;
                } else {
                    a += R[j];
                }
            }
            a = wave_sum_f64(a);
            if (lane == 0)
                s_tot[c] = s_off[c] + a;
        }
        __syncthreads();
        const double total = row_prefix(s_tot, nch, s_pre, s_tot, &sh[kWave]);
        const double thr = (double)u_fin[b] * total;
        owner_chunk(s_pre, s_tot, nch, thr, &s_int[0], &s_int[1]);
        const int owner = s_int[0];
        const bool fb = s_int[1] != 0;
        int32_t pick = -1;
        if (owner >= 0) {
            if (wave == 0) {
                const uint32_t mw =
                    lane < kWordsPerChunk ? bits_b[(int64_t)owner * kWordsPerChunk + lane] : 0u;
                int v = __popc(mw), incl = v;
#pragma unroll
                for (int o = 1; o < kWave; o <<= 1) {
                    const int t = __shfl_up(incl, o);
                    if (lane >= o)
                        incl += t;
                }
                if (lane < kWordsPerChunk) {
                    s_mw[lane] = mw;
                    s_mpre[lane] = incl - v;
                }
            }
            if (tid == 0) {
                s_int[2] = INT_MAX;  // first index past the threshold
                s_int[3] = -1;       // last index with mass
            }
            __syncthreads();
            const int o = tid;
            const int64_t y = (int64_t)owner * kChunk + o;
            double w = 0.0;
            if (y < V) {
                const uint32_t word = s_mw[o >> 5];
                if (!fresh && ((word >> (o & 31)) & 1u))
                    w = R[s_cb[owner] + s_mpre[o >> 5] + __popc(word & ((1u << (o & 31)) - 1u))];
                else
                    w = (double)pu[y];
            }
            double tot;
            const double ex = block_excl_scan_f64(w, sh, &tot);
            if (w > 0.0) {
                if (!fb && s_pre[owner] + (ex + w) > thr)
                    atomicMin(&s_int[2], o);
                atomicMax(&s_int[3], o);
            }
            __syncthreads();
            const int first = s_int[2], last = s_int[3];
            if (first != INT_MAX)
                pick = owner * kChunk + first;
            else if (last >= 0)
                pick = owner * kChunk + last;
        }
        if (tid == 0)
            ob[n] = pick;
        break;
    }
    if (tid == 0)
        n_acc[b] = n;
}

}  // namespace

size_t verify_tree_ws_bytes(int B, int m, int V, int64_t max_len)
{
    (void)m;
    return tree_R_bytes(B, max_len) + (size_t)B * tree_chunks(V) * kWordsPerChunk * 4 + 256;
}

hipError_t verify_tree_launch(hipStream_t s, int B, int m, int V, const int32_t *parent,
                              const int32_t *token, const int64_t *sl_off, const int32_t *sl_ids,
                              const float *q, const float *p, const float *u_acc,
                              const float *u_fin, int64_t max_len, int32_t *n_acc, int32_t *out,
                              int32_t *path, void *ws, hipEvent_t t0, hipEvent_t t1)
{
    double *R = reinterpret_cast<double *>(ws);
    uint32_t *bits = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(ws) +
                                                  tree_R_bytes(B, max_len));
    const int nch = tree_chunks(V);
    const int bx = (nch * kChunk + kBitsTokens - 1) / kBitsTokens;
    hipError_t e = launch_timed(tree_bits_kernel, dim3((unsigned)bx, (unsigned)B), dim3(256), s,
                                t0, nullptr, V, max_len, sl_off, sl_ids, bits);
    if (e != hipSuccess)
        return e;
    return launch_timed(verify_tree_kernel, dim3((unsigned)B), dim3(kTreeThreads), s, nullptr,
                        t1, m, V, max_len, parent, token, sl_off, sl_ids, q, p, u_acc, u_fin,
                        (const uint32_t *)bits, R, n_acc, out, path);
}

}  // namespace ds
