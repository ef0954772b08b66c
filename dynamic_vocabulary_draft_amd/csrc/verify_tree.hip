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
// The walk is sequential per sequence, so one 512-thread workgroup owns a
// sequence, and every phase is a flat stream that keeps many loads in
// flight from that one compute unit.  The residual is kept unnormalised:
// r = R / P with R = p_u off the shortlist (a proposal has no mass there, so
// those entries only rescale) and R_S in a workspace on the shortlist, P the
// current normaliser.  A rejection updates R_S <- max(0, R_S - P q_c) and
// P <- (off-shortlist mass of p_u) + sum R_S, so the long V-wide row is read
// once per node that sees a rejection or ends the walk, never rescaled.
// The first test at a node compares fp32 values exactly in fp64
// (u * q < p); every later test and the final draw differ from a sequential
// fp64 evaluation by rounding order only.
//
// The chain at a node does not depend on how the walk reached it, and every
// walk starts at the root, so the root's chain is precomputed on many
// compute units (when the root has one or two children): after a rejection
// of its first child the residual is max(0, p_0 - q_c1) on the shortlist,
// after the second max(0, R_1 - P_1 q_c2).  Per 4096-token chunk, one pass
// totals the mass off the shortlist, p_0 on it and R_1; a second pass, which
// rebuilds P_1 from those totals in chunk order, totals R_2.  The walk then
// tests the root's children from these normalisers and, when both are
// rejected, finds the chunk holding the threshold from the chunk totals and
// draws inside that chunk alone.  Below the root the walk is sequential.
//
// Four launches:
//   bits: one workgroup per (32768 tokens, sequence) writes the shortlist's
//         membership bitmap (bit y set iff token y is listed) and, per
//         32-token word, the number of listed tokens before it, so the
//         position of a listed token in the ascending shortlist is
//         rank[word] + a popcount;
//   root1, root2: the root's chunk totals (one workgroup per chunk and
//         sequence);
//   walk: one workgroup per sequence: every drafted node's shortlist
//         position, u * q and target value at its parent go to LDS (a
//         node's first test then needs no memory access), then the walk.
//         The vocabulary is cut into eight slices, one per wave: at a
//         node's first rejection one pass over p_u totals each slice's mass
//         off and on the shortlist; each rejection streams R_S, q_c (and,
//         the first time, p_u at the listed ids); the final draw adds R_S
//         over each slice's listed range, picks the slice holding the
//         threshold, scans one segment of that slice per thread and walks
//         the one segment that holds it.
#include <limits.h>

#include "common.h"
#include "dist.h"
#include "kernels.h"

namespace ds {
namespace {

constexpr int kTreeThreads = 512;
constexpr int kTreeWaves = kTreeThreads / kWave;
constexpr int kTreeMaxNodes = DS_MAX_TREE_NODES;
constexpr int kBitsTokens = 32768;  // tokens per bitmap workgroup
constexpr int kBitsThreads = 256;

// bitmap words per sequence: whole bitmap workgroups
__host__ __device__ inline int64_t tree_words(int V)
{
    return ((int64_t)V + kBitsTokens - 1) / kBitsTokens * (kBitsTokens / 32);
}

__host__ __device__ inline size_t tree_R_bytes(int B, int64_t max_len)
{
    return ((size_t)B * (size_t)max_len * 8 + 255) / 256 * 256;
}

__host__ __device__ inline size_t tree_bits_bytes(int B, int V)
{
    return ((size_t)B * (size_t)tree_words(V) * 4 + 255) / 256 * 256;
}

// A target row: p itself, or (LOGITS) target logits with the row's softmax
// normaliser (M, rZ) rebuilt from the softmax's segment statistics, each
// value taken as p_elem (the bits the target softmax writes).  tab: the exp
// table in LDS (LOGITS).
template <bool LOGITS>
struct TRow {
    float M;
    double rZ;
    const double *tab;
    __device__ __forceinline__ float operator()(float x) const
    {
        return LOGITS ? p_elem(x, M, rZ, tab) : x;
    }
};

// Row normalisers of the B*(m+1) target rows, one wave per row
__global__ __launch_bounds__(256) void tree_norms_kernel(int rows, int64_t nseg,
                                                         const float *__restrict__ smax,
                                                         const double *__restrict__ ssum,
                                                         float *__restrict__ nM,
                                                         double *__restrict__ nZ)
{
    __shared__ double tab[64];
    fill_exp2_table(tab);
    __syncthreads();
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows)
        return;
    float M;
    double rZ;
    row_norm(smax + (int64_t)r * nseg, ssum + (int64_t)r * nseg, nseg, tab, &M, &rZ);
    if (lane_id() == 0) {
        nM[r] = M;
        nZ[r] = rZ;
    }
}

__global__ __launch_bounds__(kBitsThreads) void tree_bits_kernel(
    int V, int64_t max_len, const int64_t *__restrict__ sl_off, const int32_t *__restrict__ sl_ids,
    uint32_t *__restrict__ bits, uint32_t *__restrict__ rank)
{
    __shared__ uint32_t sw[kBitsTokens / 32];
    __shared__ int64_t s_rng[2];
    __shared__ int64_t s_scan[kWave + 1];
    const int b = blockIdx.y, tid = threadIdx.x;
    const int64_t nw = tree_words(V);
    const int64_t t0 = (int64_t)blockIdx.x * kBitsTokens;  // < V by the grid
    const int64_t t1 = min(t0 + kBitsTokens, (int64_t)V);
    const int64_t off = sl_off[b];
    int64_t len = sl_off[b + 1] - off;
    if (len < 0 || len > max_len)
        len = 0;  // the walk reports such a sequence
    const int32_t *S = sl_ids + off;
    for (int i = tid; i < kBitsTokens / 32; i += kBitsThreads)
        sw[i] = 0u;
    if (tid < 2 * kWave) {  // wave 0: first entry >= t0, wave 1: first entry >= t1
        const int64_t r = wave_lower_bound(S, len, (int32_t)(tid < kWave ? t0 : t1));
        if (lane_id() == 0)
            s_rng[tid >> 6] = r;
    }
    __syncthreads();
    const int64_t a = s_rng[0], e = s_rng[1];
    constexpr int U = 8;
    for (int64_t j0 = a + tid; j0 < e; j0 += (int64_t)kBitsThreads * U) {
        int32_t y[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t j = j0 + (int64_t)k * kBitsThreads;
            y[k] = j < e ? S[j] : -1;
        }
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (y[k] >= t0 && y[k] < t1)
                atomicOr(&sw[(y[k] - t0) >> 5], 1u << (y[k] & 31));
    }
    __syncthreads();
    // thread t owns words 4t .. 4t+3 of the block
    uint32_t w[4];
    int64_t cnt = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        w[k] = sw[4 * tid + k];
        cnt += __popc(w[k]);
    }
    int64_t tot;
    int64_t run = a + block_excl_scan_i64(cnt, s_scan, &tot);
    uint32_t *ob = bits + (int64_t)b * nw, *orank = rank + (int64_t)b * nw;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t gw = t0 / 32 + 4 * tid + k;
        if (gw < nw) {
            ob[gw] = w[k];
            orank[gw] = (uint32_t)run;
        }
        run += __popc(w[k]);
    }
}

// Every thread gets the block sum of one double per thread, in a fixed
// association (lane 0's wave butterfly, then the wave sums in order).
__device__ __forceinline__ double block_sum_f64(double v, double *sh)
{
    const double w = wave_sum_f64(v);
    if (lane_id() == 0)
        sh[threadIdx.x >> 6] = w;
    __syncthreads();
    double t = 0.0;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k)
        t += sh[k];
    __syncthreads();
    return t;
}

// four consecutive target values from y0 (y0 % 4 == 0); zero at or beyond
// lim (<= V).  The loads are unconditional (clamped addresses), so no
// branch separates them from the loads issued around them.
template <bool LOGITS>
__device__ __forceinline__ void load4(const float *__restrict__ pu, int64_t y0, int64_t lim, int V,
                                      bool vec, const TRow<LOGITS> &tv, float v[4])
{
    if (vec) {  // V % 4 == 0 and pu 16-byte aligned: one dwordx4 load
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 t = reinterpret_cast<const f32x4 *>(pu)[min(y0, (int64_t)V - 4) >> 2];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = y0 + e < lim ? tv(t[e]) : 0.f;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float t = pu[min(y0 + e, (int64_t)V - 1)];
            v[e] = y0 + e < lim ? tv(t) : 0.0f;
        }
    }
}

// The vocabulary is split into kTreeWaves slices of SC tokens (SC a multiple
// of 32), slice w = [w SC, (w+1) SC) clipped to V.
struct Slices {
    int64_t SC;
    __device__ int64_t lo(int w, int V) const { return min((int64_t)w * SC, (int64_t)V); }
    __device__ int64_t hi(int w, int V) const { return min((int64_t)(w + 1) * SC, (int64_t)V); }
};

// Listed tokens below token a (a a multiple of 32, or V).
__device__ __forceinline__ int rank_at(const uint32_t *__restrict__ rank_b, int64_t a, int V,
                                       int rank_end)
{
    return a >= V ? rank_end : (int)rank_b[a >> 5];
}

// One pass over row pu: wave w streams its slice (lane l the tokens
// lo + 4(l + 64 i) .. +3, eight float4 loads in flight per lane) and totals
// into s_wsum[w] the target mass off the shortlist (OFF) or all of it.
// Branch-free fp64 accumulation: on one compute unit the conversions and
// adds cost as much as the loads.
template <bool OFF, bool LOGITS>
__device__ __forceinline__ void slice_pass(const float *__restrict__ pu,
                                           const uint32_t *__restrict__ bits_b, int V, Slices sl,
                                           bool vec, const TRow<LOGITS> &tv, double *s_wsum)
{
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t a = sl.lo(wave, V), e = sl.hi(wave, V);
    constexpr int U = 8;
    double acc = 0.0;
    for (int64_t y00 = a + 4 * lane; y00 < e; y00 += 4 * kWave * U) {
        float v[U][4];
        uint32_t wd[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t y0 = y00 + 4 * kWave * k;
            load4(pu, y0, e, V, vec, tv, v[k]);
            if (OFF)
                wd[k] = bits_b[min(y0, (int64_t)V - 1) >> 5];
        }
        const int sh0 = (lane & 7) << 2;  // y0 & 31 (slices start at multiples of 32)
#pragma unroll
        for (int k = 0; k < U; ++k)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const double x = (double)v[k][c];
                acc += (OFF && ((wd[k] >> (sh0 + c)) & 1u)) ? 0.0 : x;
            }
    }
    acc = wave_sum_f64(acc);
    if (lane == 0)
        s_wsum[wave] = acc;
}

// R <- max(0, R - P q_c) over the shortlist (R read as p_u at the listed
// ids when fresh; ids outside [0, V) carry no mass); returns sum R.
template <bool LOGITS, class QF>
__device__ __forceinline__ double residual_update(const float *__restrict__ pu,
                                                  const int32_t *__restrict__ S,
                                                  const float *__restrict__ qc, int len, int V,
                                                  bool fresh, double P, double *__restrict__ R,
                                                  const TRow<LOGITS> &tv, double *sh, QF qf)
{
    constexpr int U = 16;
    double acc = 0.0;
    for (int j0 = threadIdx.x; j0 < len; j0 += kTreeThreads * U) {
        double r[U];
        float qv[U];
        // unconditional loads at clamped indices (j0 < len), masked after
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int j = min(j0 + k * kTreeThreads, len - 1);
            qv[k] = qc[j];  // turned into q below
            if (fresh) {
                const int32_t y = S[j];
                const bool ok = y >= 0 && y < V;
                const float t = pu[ok ? y : 0];
                r[k] = ok ? (double)tv(t) : 0.0;
            } else {
                r[k] = R[j];
            }
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int j = j0 + k * kTreeThreads;
            const double t = P * (double)qf(qv[k]);
            const double nr = r[k] > t ? r[k] - t : 0.0;
            if (j < len) {
                R[j] = nr;
                acc += nr;
            }
        }
    }
    return block_sum_f64(acc, sh);
}

// Weights of the four tokens y0 .. y0+3 (zero at or beyond lim) in the
// final draw: the target off the shortlist, R on it (p_u everywhere when
// fresh).
template <bool LOGITS>
__device__ __forceinline__ void draw_weights(const float *__restrict__ pu,
                                             const uint32_t *__restrict__ bits_b,
                                             const uint32_t *__restrict__ rank_b,
                                             const double *__restrict__ R, int len, int64_t y0,
                                             int64_t lim, int V, bool vec, bool fresh,
                                             const TRow<LOGITS> &tv, double w[4])
{
    float v[4];
    load4(pu, y0, lim, V, vec, tv, v);
    if (fresh) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            w[c] = (double)v[c];
        return;
    }
    const int64_t wi = min(y0, (int64_t)V - 1) >> 5;
    const uint32_t wd = bits_b[wi];
    const int rk = (int)rank_b[wi];
    const int sh0 = (int)(y0 & 31);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int bit = sh0 + c;
        const bool in = y0 + c < lim && ((wd >> bit) & 1u);
        w[c] = in ? R[max(0, min(len - 1, rk + (int)__popc(wd & ((1u << bit) - 1u))))]
                   : (double)v[c];
    }
}

// ---------------------------------------------------------------- root
constexpr int kRootChunk = 4096;    // tokens per chunk of the root's passes
constexpr int kRootThreads = 256;   // 16 tokens per thread
constexpr int kRootMaxKids = 2;     // children handled by the precomputed chain

__host__ __device__ inline int64_t root_chunks(int V) { return ((int64_t)V + kRootChunk - 1) / kRootChunk; }

// per (sequence, chunk): mass off the shortlist, p_0 on it, sum R_1, sum R_2
struct RootPart {
    double off, sp, s1, s2;
};

__host__ __device__ inline size_t root_part_bytes(int B, int V)
{
    return ((size_t)B * (size_t)root_chunks(V) * sizeof(RootPart) + 255) / 256 * 256;
}

// residual update max(0, r - P q) without contraction into an fma (the
// walk recomputes it and must get the same bits)
__device__ __forceinline__ double resid(double r, double P, float q)
{
    const double t = __dmul_rn(P, (double)q);
    return r > t ? __dsub_rn(r, t) : 0.0;
}

// the root's first two children (node numbers, in increasing order) and the
// number of its children (capped at kRootMaxKids + 1); all threads
__device__ void root_kids(const int32_t *__restrict__ parent_b, int m, int *s3, int *c1, int *c2,
                          int *k)
{
    if (threadIdx.x == 0) {
        s3[0] = INT_MAX;
        s3[1] = INT_MAX;
        s3[2] = 0;
    }
    __syncthreads();
    for (int i = threadIdx.x + 1; i <= m; i += blockDim.x)
        if (parent_b[i - 1] == 0) {
            atomicMin(&s3[0], i);
            atomicAdd(&s3[2], 1);
        }
    __syncthreads();
    const int a = s3[0];
    for (int i = threadIdx.x + 1; i <= m; i += blockDim.x)
        if (parent_b[i - 1] == 0 && i > a)
            atomicMin(&s3[1], i);
    __syncthreads();
    *c1 = a;
    *c2 = s3[1];
    *k = min(s3[2], kRootMaxKids + 1);
    __syncthreads();
}

// The shortlist entries with ids in [base, base + kRootChunk): membership
// bits (from the sequence's bitmap) and the proposals q1 (and q2) of the
// root's children at those ids, scattered into LDS (the entries are
// positions rank[base/32] .. of the ascending shortlist); returns after a
// barrier.
template <bool QL>
__device__ void root_scatter(const uint32_t *__restrict__ bits_b, const uint32_t *__restrict__ rank_b,
                             int V, int len, int64_t base, const float *__restrict__ q1,
                             const float *__restrict__ q2, uint32_t *mem, float *q1d, float *q2d,
                             QRow<QL> f1, QRow<QL> f2)
{
    const int64_t nw = tree_words(V);
    const int64_t w0 = base >> 5;
    for (int i = threadIdx.x; i < kRootChunk / 32; i += blockDim.x) {
        const uint32_t wd = w0 + i < nw ? bits_b[w0 + i] : 0u;
        mem[i] = wd;
    }
    __syncthreads();
    // thread t handles words t, t + blockDim.x, ...: the first listed
    // position of word i is rank[w0 + i]
    for (int i = threadIdx.x; i < kRootChunk / 32; i += blockDim.x) {
        uint32_t wd = mem[i];
        if (!wd)
            continue;
        int j = (int)rank_b[w0 + i];
        while (wd) {
            const int bit = __ffs(wd) - 1;
            wd &= wd - 1u;
            if (j < len) {
                const int o = 32 * i + bit;
                q1d[o] = f1(q1[j]);
                if (q2)
                    q2d[o] = f2(q2[j]);
            }
            ++j;
        }
    }
    __syncthreads();
}

// the chunk totals of sequence b into LDS (all threads load in parallel)
__device__ __forceinline__ void root_parts_lds(const RootPart *__restrict__ pp, int nch, RootPart *lds)
{
    for (int c = threadIdx.x; c < nch; c += blockDim.x)
        lds[c] = pp[c];
    __syncthreads();
}

// P_1 (and the fresh flag: the residual had no mass, back to p_0), the
// same sums in every kernel that needs them: chunk order, one thread's
// sequence of adds
__device__ __forceinline__ void root_p1(const RootPart *__restrict__ part, int nch, double *Poff,
                                        double *P1, bool *fresh1)
{
    double off = 0.0, s1 = 0.0;
    for (int c = 0; c < nch; ++c) {
        off += part[c].off;
        s1 += part[c].s1;
    }
    const double pn = off + s1;
    *Poff = off;
    *fresh1 = !(pn > 0.0);
    *P1 = *fresh1 ? 1.0 : pn;
}

// the on-shortlist weight after the root's chain: R_1 (one child) or R_2
__device__ __forceinline__ double root_R(double pv, float q1v, float q2v, int k, bool fresh1,
                                         double P1)
{
    const double r1 = fresh1 ? pv : resid(pv, 1.0, q1v);
    return k == 1 ? r1 : resid(r1, P1, q2v);
}

// PASS 1: off, sp, s1 per chunk; PASS 2: s2 per chunk (two children only)
constexpr int kRootMaxChunks = 256;  // V <= 2^20

// QL: q is recomputed from the draft logits (q points to them) and the
// draft rows' statistics qs (row b * m + node), bit for bit the sampler's q
template <int PASS, bool LOGITS, bool QL>
__global__ __launch_bounds__(kRootThreads) void root_pass_kernel(
    int m, int V, int64_t max_len, const int32_t *__restrict__ parent,
    const int64_t *__restrict__ sl_off, const float *__restrict__ q,
    const float *__restrict__ p, const float *__restrict__ nM, const double *__restrict__ nZ,
    const uint32_t *__restrict__ bits, const uint32_t *__restrict__ rank,
    RootPart *__restrict__ part, const QStats *__restrict__ qs, double qtau)
{
    __shared__ double tab[LOGITS || QL ? 64 : 1];
    if (LOGITS || QL)
        fill_exp2_table(tab);  // ordered by the barriers in root_kids
    __shared__ uint32_t mem[kRootChunk / 32];
    __shared__ float q1d[kRootChunk], q2d[PASS == 2 ? kRootChunk : 1];
    __shared__ RootPart s_part[PASS == 2 ? kRootMaxChunks : 1];
    __shared__ int s3[3];
    __shared__ double sh[kWave + 1];
    const int b = blockIdx.y, nch = (int)gridDim.x;
    const int64_t base = (int64_t)blockIdx.x * kRootChunk;
    const int64_t off = sl_off[b], len64 = sl_off[b + 1] - off;
    if (len64 < 0 || len64 > max_len)
        return;  // the walk reports such a sequence
    const int len = (int)len64;
    int c1, c2, k;
    root_kids(parent + (int64_t)b * m, m, s3, &c1, &c2, &k);
    if (k < 1 || k > kRootMaxKids || (PASS == 2 && k != 2))
        return;  // block-uniform; the walk takes the sequential path
    RootPart *pb = part + (int64_t)b * nch;
    double Poff = 0.0, P1 = 1.0;
    bool fresh1 = true;
    if (PASS == 2) {
        root_parts_lds(pb, nch, s_part);
        root_p1(s_part, nch, &Poff, &P1, &fresh1);
    }
    const float *qrow = q + (int64_t)m * off;
    const int64_t nw = tree_words(V);
    root_scatter<QL>(bits + (int64_t)b * nw, rank + (int64_t)b * nw, V, len, base,
                     qrow + (int64_t)(c1 - 1) * len,
                     PASS == 2 ? qrow + (int64_t)(c2 - 1) * len : nullptr, mem, q1d, q2d,
                     q_row<QL>(qs, (int64_t)b * m + c1 - 1, qtau, tab),
                     q_row<QL>(qs, (int64_t)b * m + (PASS == 2 ? c2 : c1) - 1, qtau, tab));
    const float *pu = p + (int64_t)b * (m + 1) * V;
    const int64_t r0 = (int64_t)b * (m + 1);
    const TRow<LOGITS> tv{LOGITS ? nM[r0] : 0.f, LOGITS ? nZ[r0] : 0.0, tab};
    double a0 = 0.0, a1 = 0.0, a2 = 0.0;
#pragma unroll
    for (int kk = 0; kk < kRootChunk / (4 * kRootThreads); ++kk) {
        const int o0 = 4 * threadIdx.x + 4 * kRootThreads * kk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int o = o0 + e;
            const int64_t y = base + o;
            const double pv = y < V ? (double)tv(pu[y]) : 0.0;
            const bool in = y < V && ((mem[o >> 5] >> (o & 31)) & 1u);
            if (PASS == 1) {
                a0 += in ? 0.0 : pv;
                a1 += in ? pv : 0.0;
                a2 += in ? resid(pv, 1.0, q1d[o]) : 0.0;
            } else {
                a2 += in ? root_R(pv, q1d[o], q2d[o], 2, fresh1, P1) : 0.0;
            }
        }
    }
    if (PASS == 1) {
        a0 = block_sum_f64(a0, sh);
        a1 = block_sum_f64(a1, sh);
    }
    a2 = block_sum_f64(a2, sh);
    if (threadIdx.x == 0) {
        if (PASS == 1) {
            pb[blockIdx.x].off = a0;
            pb[blockIdx.x].sp = a1;
            pb[blockIdx.x].s1 = a2;
        } else {
            pb[blockIdx.x].s2 = a2;
        }
    }
}

template <bool LOGITS, bool QL>
__global__ __launch_bounds__(kTreeThreads) void verify_tree_kernel(
    int m, int V, int64_t max_len, bool vec, const int32_t *__restrict__ parent,
    const int32_t *__restrict__ token, const int64_t *__restrict__ sl_off,
    const int32_t *__restrict__ sl_ids, const float *__restrict__ q, const float *__restrict__ p,
    const float *__restrict__ nM, const double *__restrict__ nZ,
    const float *__restrict__ u_acc, const float *__restrict__ u_fin,
    const uint32_t *__restrict__ bits, const uint32_t *__restrict__ rank,
    const RootPart *__restrict__ rpart, double *__restrict__ Rws, int32_t *__restrict__ n_acc,
    int32_t *__restrict__ out, int32_t *__restrict__ path, const QStats *__restrict__ qs,
    double qtau)
{
    __shared__ int s_par[kTreeMaxNodes], s_pos[kTreeMaxNodes], s_tok[kTreeMaxNodes];
    __shared__ double s_lhs[kTreeMaxNodes], s_px[kTreeMaxNodes];
    __shared__ double s_woff[kTreeWaves], s_wt[kTreeWaves], s_w2[kTreeWaves];
    __shared__ double sh[kWave + 1];
    __shared__ int s_int[4];
    __shared__ uint32_t s_mem[kRootChunk / 32];
    __shared__ float s_q1[kRootChunk], s_q2[kRootChunk];
    __shared__ RootPart s_part[kRootMaxChunks];
    __shared__ double tab[LOGITS || QL ? 64 : 1];

    const int b = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    if (LOGITS || QL) {
        fill_exp2_table(tab);
        __syncthreads();
    }
    // draft row of node i (1-based): its q conversion
    auto qrow_f = [&](int i) { return q_row<QL>(qs, (int64_t)b * m + i - 1, qtau, tab); };
    // target row u of this sequence and its value conversion
    auto trow = [&](int u) {
        const int64_t r = (int64_t)b * (m + 1) + u;
        return TRow<LOGITS>{LOGITS ? nM[r] : 0.f, LOGITS ? nZ[r] : 0.0, tab};
    };
    const int64_t nw = tree_words(V);
    const uint32_t *bits_b = bits + (int64_t)b * nw, *rank_b = rank + (int64_t)b * nw;
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
    // listed ids in [0, V)
    const int rank_end = min(len, (int)rank_b[nw - 1] + (int)__popc(bits_b[nw - 1]));
    const Slices sl{((int64_t)V + 32 * kTreeWaves - 1) / (32 * kTreeWaves) * 32};

    // drafted node i (index i-1): parent, token, shortlist position,
    // u * q_i(x) (exact in fp64) and the target at its parent
    for (int i = tid + 1; i <= m; i += kTreeThreads) {
        const int64_t e = (int64_t)b * m + i - 1;
        const int32_t x = token[e];
        const int par = parent[e];
        const float ua = u_acc[e];
        const bool valid = x >= 0 && x < V;
        const bool linked = par >= 0 && par < i;
        int pos = -1;
        if (valid) {
            const uint32_t w = bits_b[x >> 5];
            if ((w >> (x & 31)) & 1u)
                pos = min(len - 1, (int)rank_b[x >> 5] + (int)__popc(w & ((1u << (x & 31)) - 1u)));
        }
        const double qx =
            pos >= 0 ? (double)qrow_f(i)(q[(int64_t)m * off + (int64_t)(i - 1) * len + pos]) : 0.0;
        s_par[i - 1] = linked ? par : -1;
        s_tok[i - 1] = x;
        s_pos[i - 1] = pos;
        s_lhs[i - 1] = (double)ua * qx;
        s_px[i - 1] = (valid && linked)
                          ? (double)trow(par)(p[((int64_t)b * (m + 1) + par) * V + x])
                          : 0.0;
    }
    __syncthreads();

    int u = 0, n = 0;
    // the root's chain from its precomputed chunk totals (one or two
    // children); an accepted child continues the walk below
    int c1, c2, kr;
    root_kids(parent + (int64_t)b * m, m, s_int, &c1, &c2, &kr);
    if (kr >= 1 && kr <= kRootMaxKids) {  // block-uniform
        const int nch = (int)root_chunks(V);
        root_parts_lds(rpart + (int64_t)b * nch, nch, s_part);
        const RootPart *pp = s_part;
        const float *qrow = q + (int64_t)m * off;
        int acc = -1;
        bool ffin = true;  // the final draw is from p_0 itself
        double Poff = 0.0, P1 = 1.0;
        bool fresh1 = true;
        if (s_lhs[c1 - 1] < s_px[c1 - 1]) {
            acc = c1;
        } else {
            root_p1(pp, nch, &Poff, &P1, &fresh1);
            ffin = fresh1;
            if (kr == 2) {
                const int pos = s_pos[c2 - 1];
                double rx = s_px[c2 - 1];
                if (!fresh1)
                    rx = (pos >= 0 ? resid(s_px[c2 - 1], 1.0,
                                           qrow_f(c1)(qrow[(int64_t)(c1 - 1) * len + pos]))
                                   : s_px[c2 - 1]) / P1;
                if (s_lhs[c2 - 1] < rx) {
                    acc = c2;
                } else {
                    double s2 = 0.0;
                    for (int c = 0; c < nch; ++c)
                        s2 += pp[c].s2;
                    ffin = !(Poff + s2 > 0.0);
                }
            }
        }
        if (acc >= 0) {
            if (tid == 0) {
                ob[0] = s_tok[acc - 1];
                pb[0] = acc;
            }
            n = 1;
            u = acc;
        } else {
            // chunk totals of the final weights, the chunk holding u_fin *
            // total (else the last chunk with mass), then that chunk's tokens
            double pre = 0.0, tot = 0.0;
            for (int c = 0; c < nch; ++c)
                tot += pp[c].off + (ffin ? pp[c].sp : (kr == 1 ? pp[c].s1 : pp[c].s2));
            const double thr = (double)u_fin[b] * tot;
            int owner = -1, lastc = -1;
            double run = 0.0;
            for (int c = 0; c < nch; ++c) {
                const double t = pp[c].off + (ffin ? pp[c].sp : (kr == 1 ? pp[c].s1 : pp[c].s2));
                if (owner < 0 && run + t > thr) {
                    owner = c;
                    pre = run;
                }
                if (t > 0.0)
                    lastc = c;
                run += t;
            }
            const bool fb = owner < 0;
            if (fb)
                owner = lastc;
            int32_t pick = -1;
            if (owner >= 0) {
                const int64_t cb = (int64_t)owner * kRootChunk;
                root_scatter<QL>(bits_b, rank_b, V, len, cb, qrow + (int64_t)(c1 - 1) * len,
                                 kr == 2 ? qrow + (int64_t)(c2 - 1) * len : nullptr, s_mem, s_q1,
                                 s_q2, qrow_f(c1), qrow_f(kr == 2 ? c2 : c1));
                const float *pu = p + (int64_t)b * (m + 1) * V;
                const TRow<LOGITS> tv0 = trow(0);
                constexpr int TPT = kRootChunk / kTreeThreads;  // 8 consecutive tokens
                double w[TPT], mine = 0.0;
#pragma unroll
                for (int e = 0; e < TPT; ++e) {
                    const int o = TPT * tid + e;
                    const int64_t y = cb + o;
                    const double pv = y < V ? (double)tv0(pu[y]) : 0.0;
                    const bool in = y < V && ((s_mem[o >> 5] >> (o & 31)) & 1u);
                    w[e] = (!ffin && in) ? root_R(pv, s_q1[o], kr == 2 ? s_q2[o] : 0.f, kr, fresh1, P1)
                                         : pv;
                    mine += w[e];
                }
                double tot2;
                double part = pre + block_excl_scan_f64(mine, sh, &tot2);
                if (tid == 0) {
                    s_int[0] = INT_MAX;
                    s_int[1] = -1;
                }
                __syncthreads();
                int found = INT_MAX, last = -1;
#pragma unroll
                for (int e = 0; e < TPT; ++e) {
                    part += w[e];
                    if (w[e] > 0.0) {
                        last = (int)(cb + TPT * tid + e);
                        if (found == INT_MAX && !fb && part > thr)
                            found = last;
                    }
                }
                if (found != INT_MAX)
                    atomicMin(&s_int[0], found);
                if (last >= 0)
                    atomicMax(&s_int[1], last);
                __syncthreads();
                pick = s_int[0] != INT_MAX ? s_int[0] : s_int[1];
            }
            if (tid == 0) {
                ob[0] = pick;
                n_acc[b] = 0;
            }
            return;
        }
    }
    for (int visit = 0; visit <= m; ++visit) {  // u increases on every acceptance
        const float *pu = p + ((int64_t)b * (m + 1) + u) * V;
        const TRow<LOGITS> tv = trow(u);
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
            if (!have_off) {
                slice_pass<true>(pu, bits_b, V, sl, vec, tv, s_woff);
                __syncthreads();  // (also orders this test's reads of R)
                Poff = 0.0;
#pragma unroll
                for (int w = 0; w < kTreeWaves; ++w)
                    Poff += s_woff[w];
                have_off = true;
            } else {
                __syncthreads();  // every thread has read R for this test
            }
            const float *qc = q + (int64_t)m * off + (int64_t)(c - 1) * len;
            const double sr = residual_update(pu, S, qc, len, V, fresh, P, R, tv, sh, qrow_f(c));
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

        // final draw from r over all V (inverse CDF): slice totals, the
        // owning slice, the owning thread's segment of it, its token
        if (fresh) {  // r is p_u: slice totals of the row
            slice_pass<false>(pu, bits_b, V, sl, vec, tv, s_wt);
        } else {  // wave w adds R over the listed ids of its slice
            const int j0 = rank_at(rank_b, sl.lo(wave, V), V, rank_end);
            const int j1 = rank_at(rank_b, sl.hi(wave, V), V, rank_end);
            double a = 0.0;
            constexpr int U = 16;
            for (int jj = j0 + lane; jj < j1; jj += kWave * U) {
                double r[U];
#pragma unroll
                for (int k = 0; k < U; ++k)
                    r[k] = R[min(jj + k * kWave, j1 - 1)];
#pragma unroll
                for (int k = 0; k < U; ++k)
                    if (jj + k * kWave < j1)
                        a += r[k];
            }
            a = wave_sum_f64(a);
            if (lane == 0)
                s_wt[wave] = s_woff[wave] + a;
        }
        __syncthreads();
        // slice prefix (fixed order), threshold, owner (first slice whose
        // prefix passes the threshold; else the last slice with mass)
        double pre[kTreeWaves + 1];
        pre[0] = 0.0;
#pragma unroll
        for (int w = 0; w < kTreeWaves; ++w)
            pre[w + 1] = pre[w] + s_wt[w];
        const double thr = (double)u_fin[b] * pre[kTreeWaves];
        int owner = -1;
        bool fb = false;
#pragma unroll
        for (int w = kTreeWaves - 1; w >= 0; --w)
            if (pre[w + 1] > thr)
                owner = w;
        if (owner < 0) {
            fb = true;
#pragma unroll
            for (int w = 0; w < kTreeWaves; ++w)
                if (s_wt[w] > 0.0)
                    owner = w;
        }
        int32_t pick = -1;
        if (owner >= 0) {
            // The owning slice in rows of 256 tokens (lane l: tokens 4l ..
            // 4l+3 of a row); wave w takes RW consecutive rows.  Pass 1: the
            // wave totals; pass 2: the wave holding the threshold scans its
            // rows in order.
            const int64_t a = sl.lo(owner, V), e = sl.hi(owner, V);
            const int nrows = (int)((e - a + 4 * kWave - 1) / (4 * kWave));
            const int RW = (nrows + kTreeWaves - 1) / kTreeWaves;
            const int r0 = min(nrows, wave * RW), r1 = min(nrows, r0 + RW);
            constexpr int G = 8;  // rows in flight per wave
            double mine = 0.0;
            for (int g = r0; g < r1; g += G) {
                double w[G][4];
#pragma unroll
                for (int k = 0; k < G; ++k) {
                    const int64_t y0 = a + (int64_t)(g + k) * 4 * kWave + 4 * lane;
                    draw_weights(pu, bits_b, rank_b, R, len, y0, g + k < r1 ? e : 0, V, vec,
                                 fresh, tv, w[k]);
                }
#pragma unroll
                for (int k = 0; k < G; ++k)
                    mine += ((w[k][0] + w[k][1]) + w[k][2]) + w[k][3];
            }
            mine = wave_sum_f64(mine);
            if (lane == 0)
                s_w2[wave] = mine;
            __syncthreads();
            double run = pre[owner];
            int ow = -1;
            for (int w = 0; w < kTreeWaves; ++w) {  // first wave past the threshold
                if (ow < 0 && !fb && run + s_w2[w] > thr)
                    ow = w;
                if (ow < 0)
                    run += s_w2[w];
            }
            if (tid == 0) {
                s_int[0] = -1;  // the pick
                s_int[1] = -1;  // last token with mass in the slice
            }
            __syncthreads();
            if (ow < 0) {  // rounding or fallback: the last token with mass
                int64_t last = -1;
                for (int g = r0; g < r1; g += G) {
                    double w[G][4];
#pragma unroll
                    for (int k = 0; k < G; ++k) {
                        const int64_t y0 = a + (int64_t)(g + k) * 4 * kWave + 4 * lane;
                        draw_weights(pu, bits_b, rank_b, R, len, y0, g + k < r1 ? e : 0, V, vec,
                                     fresh, tv, w[k]);
                    }
#pragma unroll
                    for (int k = 0; k < G; ++k)
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            if (w[k][c] > 0.0)
                                last = a + (int64_t)(g + k) * 4 * kWave + 4 * lane + c;
                }
                if (last >= 0)
                    atomicMax(&s_int[1], (int)last);
            } else if (wave == ow) {
                const int rw0 = min(nrows, ow * RW), rw1 = min(nrows, rw0 + RW);
                int64_t last = -1;
                for (int r = rw0; r < rw1; ++r) {
                    const int64_t y0 = a + (int64_t)r * 4 * kWave + 4 * lane;
                    double w[4];
                    draw_weights(pu, bits_b, rank_b, R, len, y0, e, V, vec, fresh, tv, w);
                    const double lsum = ((w[0] + w[1]) + w[2]) + w[3];
                    const double incl = wave_incl_scan_f64(lsum);
                    double part = run + (incl - lsum);
                    int found = -1;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        part += w[c];
                        if (w[c] > 0.0) {
                            last = y0 + c;
                            if (found < 0 && part > thr)
                                found = c;
                        }
                    }
                    const uint64_t hit = __ballot(found >= 0);
                    if (hit) {  // wave-uniform
                        if (lane == __ffsll((unsigned long long)hit) - 1)
                            s_int[0] = (int)(y0 + found);
                        break;
                    }
                    run += __shfl(incl, kWave - 1);
                }
                if (last >= 0)
                    atomicMax(&s_int[1], (int)last);
            }
            __syncthreads();
            pick = s_int[0] >= 0 ? s_int[0] : s_int[1];
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
    return tree_R_bytes(B, max_len) + 2 * tree_bits_bytes(B, V) + root_part_bytes(B, V) + 256;
}

namespace {

template <bool LOGITS, bool QL = false>
hipError_t tree_kernels(hipStream_t s, int B, int m, int V, const int32_t *parent,
                        const int32_t *token, const int64_t *sl_off, const int32_t *sl_ids,
                        const float *q, const float *x, const float *nM, const double *nZ,
                        const float *u_acc, const float *u_fin, int64_t max_len, int32_t *n_acc,
                        int32_t *out, int32_t *path, void *ws, hipEvent_t t0, hipEvent_t t1,
                        const QStats *qs = nullptr, double qtau = 1.0)
{
    char *base = reinterpret_cast<char *>(ws);
    double *R = reinterpret_cast<double *>(base);
    uint32_t *bits = reinterpret_cast<uint32_t *>(base + tree_R_bytes(B, max_len));
    uint32_t *rank = reinterpret_cast<uint32_t *>(base + tree_R_bytes(B, max_len) +
                                                  tree_bits_bytes(B, V));
    RootPart *rpart = reinterpret_cast<RootPart *>(base + tree_R_bytes(B, max_len) +
                                                   2 * tree_bits_bytes(B, V));
    const int bx = (V + kBitsTokens - 1) / kBitsTokens;
    const bool vec = V % 4 == 0 && (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
    hipError_t e = launch_timed(tree_bits_kernel, dim3((unsigned)bx, (unsigned)B),
                                dim3(kBitsThreads), s, t0, nullptr, V, max_len, sl_off, sl_ids,
                                bits, rank);
    if (e != hipSuccess)
        return e;
    const dim3 rgrid((unsigned)root_chunks(V), (unsigned)B);
    hipLaunchKernelGGL((root_pass_kernel<1, LOGITS, QL>), rgrid, dim3(kRootThreads), 0, s, m, V,
                       max_len, parent, sl_off, q, x, nM, nZ, (const uint32_t *)bits,
                       (const uint32_t *)rank, rpart, qs, qtau);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL((root_pass_kernel<2, LOGITS, QL>), rgrid, dim3(kRootThreads), 0, s, m, V,
                       max_len, parent, sl_off, q, x, nM, nZ, (const uint32_t *)bits,
                       (const uint32_t *)rank, rpart, qs, qtau);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    return launch_timed(verify_tree_kernel<LOGITS, QL>, dim3((unsigned)B), dim3(kTreeThreads), s,
                        nullptr, t1, m, V, max_len, vec, parent, token, sl_off, sl_ids, q, x, nM,
                        nZ, u_acc, u_fin, (const uint32_t *)bits, (const uint32_t *)rank,
                        (const RootPart *)rpart, R, n_acc, out, path, qs, qtau);
}

}  // namespace

hipError_t verify_tree_launch(hipStream_t s, int B, int m, int V, const int32_t *parent,
                              const int32_t *token, const int64_t *sl_off, const int32_t *sl_ids,
                              const float *q, const float *p, const float *u_acc,
                              const float *u_fin, int64_t max_len, int32_t *n_acc, int32_t *out,
                              int32_t *path, void *ws, hipEvent_t t0, hipEvent_t t1)
{
    return tree_kernels<false>(s, B, m, V, parent, token, sl_off, sl_ids, q, p, nullptr, nullptr,
                               u_acc, u_fin, max_len, n_acc, out, path, ws, t0, t1);
}

// the tree workspace, the row normalisers, then the softmax statistics
size_t verify_tree_logits_ws_bytes(int B, int m, int V, int64_t max_len)
{
    const size_t rows = (size_t)B * (m + 1);
    return (verify_tree_ws_bytes(B, m, V, max_len) + 255) / 256 * 256 + rows * 8 +
           (rows * 4 + 255) / 256 * 256 + softmax_ws_bytes((int64_t)rows, V);
}

// QL: q from the draft logits (q points to them) and the rows' statistics qs
template <bool QL>
static hipError_t tree_logits_kernels(hipStream_t s, int B, int m, int V, const int32_t *parent,
                               const int32_t *token, const int64_t *sl_off,
                               const int32_t *sl_ids, const float *q, const float *logits,
                               const float *u_acc, const float *u_fin, int64_t max_len,
                               int32_t *n_acc, int32_t *out, int32_t *path, void *ws,
                               hipEvent_t t0, hipEvent_t t1, const QStats *qs, double qtau)
{
    const int rows = B * (m + 1);
    char *b = reinterpret_cast<char *>(ws) + (verify_tree_ws_bytes(B, m, V, max_len) + 255) /
                                                 256 * 256;
    double *nZ = reinterpret_cast<double *>(b);
    float *nM = reinterpret_cast<float *>(b + (size_t)rows * 8);
    char *sws = b + (size_t)rows * 8 + ((size_t)rows * 4 + 255) / 256 * 256;
    hipError_t e = softmax_stats_launch(s, rows, V, logits, sws);
    if (e != hipSuccess)
        return e;
    const int64_t nseg = softmax_segments(V);
    const double *ssum = reinterpret_cast<const double *>(sws);
    const float *smax = reinterpret_cast<const float *>(ssum + (size_t)rows * nseg);
    hipLaunchKernelGGL(tree_norms_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
                       rows, nseg, smax, ssum, nM, nZ);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    return tree_kernels<true, QL>(s, B, m, V, parent, token, sl_off, sl_ids, q, logits, nM, nZ,
                                  u_acc, u_fin, max_len, n_acc, out, path, ws, t0, t1, qs, qtau);
}

hipError_t verify_tree_logits_launch(hipStream_t s, int B, int m, int V, const int32_t *parent,
                                     const int32_t *token, const int64_t *sl_off,
                                     const int32_t *sl_ids, const float *q, const float *logits,
                                     const float *u_acc, const float *u_fin, int64_t max_len,
                                     int32_t *n_acc, int32_t *out, int32_t *path, void *ws,
                                     hipEvent_t t0, hipEvent_t t1)
{
    return tree_logits_kernels<false>(s, B, m, V, parent, token, sl_off, sl_ids, q, logits, u_acc,
                                      u_fin, max_len, n_acc, out, path, ws, t0, t1, nullptr, 1.0);
}

hipError_t verify_tree_logits_qstats_launch(hipStream_t s, int B, int m, int V,
                                            const int32_t *parent, const int32_t *token,
                                            const int64_t *sl_off, const int32_t *sl_ids,
                                            const float *draft_logits, const QStats *qs,
                                            float temperature, const float *logits,
                                            const float *u_acc, const float *u_fin,
                                            int64_t max_len, int32_t *n_acc, int32_t *out,
                                            int32_t *path, void *ws, hipEvent_t t0, hipEvent_t t1)
{
    return tree_logits_kernels<true>(s, B, m, V, parent, token, sl_off, sl_ids, draft_logits,
                                     logits, u_acc, u_fin, max_len, n_acc, out, path, ws, t0, t1,
                                     qs, (double)temperature);
}

}  // namespace ds
