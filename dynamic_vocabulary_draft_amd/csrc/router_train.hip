// Router training (DynaSpec summary page, "Modeling": the router is trained
// by supervised multi-label classification, binary cross entropy over the
// clusters, a cluster's label being positive when it holds a token from the
// top-L of the full drafter; the trainable part is the 2-layer MLP).
//
// Labels: one workgroup per training row selects the row's top-L tokens of
// the full drafter's logits (logit descending, token id ascending) on
// order-preserving 32-bit keys, then marks the clusters of the selected
// tokens.  Two reads of the row: the first bounds the L-th largest key from
// below by the L-th largest of the threads' maxima, the second gathers the
// few keys at or above that bound into LDS, where each is ranked exactly.
// Where the bound admits more than the LDS holds (heavy ties) or L exceeds
// the thread count, a four-pass radix select (per-wave LDS histograms of one
// byte per pass) finds the L-th key instead; ties at it are resolved by id
// with a block scan, which only runs when the tie is split.
//
// Training step (fp32 parameters, fp32 arithmetic): a 64 x 64-tile GEMM
// kernel (256 threads, 4 x 4 outputs per thread, 16-deep k slices staged in
// LDS, every output summed in ascending k order; the products with a long k
// and a small output -- the two forward ones, the gradient through act' and
// dW2 -- split k in up to sixteen chunks and add the chunks in order) with a
// fused epilogue per product:
//   a = h W1^T + b1, z = act(a)        (epilogue keeps a and z)
//   s = z W2^T + b2                    (then g_s = (sigmoid(s) - y)/(n M) and
//                                       the loss, summed in fp64 in a fixed order)
//   g_a = (g_s W2) * act'(a)           (before W2 moves)
//   dW2 = g_s^T z, W2 -= lr dW2;  dW1 = g_a^T h, W1 -= lr dW1
//   db2, db1: column sums of g_s and g_a, then the bias steps.
// These products are small (inner sizes n, r or d up to a few thousand) and
// run on the vector ALUs; the dense logits that feed the labels come from
// the gathered head with the whole vocabulary as the shortlist.
#include <limits.h>

#include "common.h"
#include "kernels.h"

namespace ds {
namespace {

// ------------------------------------------------------------------ labels
constexpr int kLabThreads = 1024;
constexpr int kLabWaves = kLabThreads / kWave;
constexpr int kLabCap = 2048;  // candidates ranked in LDS
static_assert(kLabCap >= kLabThreads, "the threads' maxima share the candidate buffer");
constexpr int kLabU = 16;      // elements loaded per thread and round (all in flight)

// larger float -> larger key; -0 and +0 are one value, as in a float compare
__device__ __forceinline__ uint32_t order_key(float x)
{
    const uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Calls f(y, key(y), valid) for the row's elements y, kLabU per thread and
// round, with every lane of a wave calling in step (f may use wave votes).
// VEC (row start 16-byte aligned): 16-byte loads of four elements, then the
// last V % 4 elements one per thread.
template <bool VEC, class F>
__device__ __forceinline__ void for_row_keys(const float *__restrict__ lg, int V, int tid,
                                             int lane, F f)
{
    if constexpr (VEC) {
        constexpr int U4 = kLabU / 4;
        const int nv = V >> 2;  // whole 4-element pieces
        const float4 *l4 = reinterpret_cast<const float4 *>(lg);
        for (int c0 = tid; c0 - lane < nv; c0 += kLabThreads * U4) {  // wave-uniform bound
            float4 v[U4];
#pragma unroll
            for (int u = 0; u < U4; ++u)
                v[u] = l4[min(c0 + u * kLabThreads, nv - 1)];  // nv >= 1 inside the loop
#pragma unroll
            for (int u = 0; u < U4; ++u) {
                const int c = c0 + u * kLabThreads;
                const bool ok = c < nv;
                f(4 * c + 0, order_key(v[u].x), ok);
                f(4 * c + 1, order_key(v[u].y), ok);
                f(4 * c + 2, order_key(v[u].z), ok);
                f(4 * c + 3, order_key(v[u].w), ok);
            }
        }
        const int y = 4 * nv + tid;  // the tail, fewer than four
        const bool ok = y < V;
        const uint32_t kt = order_key(lg[ok ? y : 0]);  // V >= 1
        f(y, ok ? kt : 0u, ok);
    } else {
        for (int y0 = tid; y0 - lane < V; y0 += kLabThreads * kLabU) {  // wave-uniform bound
            uint32_t k[kLabU];
#pragma unroll
            for (int u = 0; u < kLabU; ++u)
                k[u] = order_key(lg[min(y0 + u * kLabThreads, V - 1)]);
#pragma unroll
            for (int u = 0; u < kLabU; ++u)
                f(y0 + u * kLabThreads, k[u], y0 + u * kLabThreads < V);
        }
    }
}

template <bool VEC>
__global__ __launch_bounds__(kLabThreads) void topl_labels_kernel(int V, int M, int L,
                                                                 const float *__restrict__ logits,
                                                                 int64_t ldl,
                                                                 const int32_t *__restrict__ cluster_of,
                                                                 uint8_t *__restrict__ labels)
{
    __shared__ uint32_t hist[kLabWaves][256];
    __shared__ uint32_t s_tot[256];
    __shared__ uint8_t s_lab[DS_MAX_CLUSTERS];
    __shared__ uint32_t s_sel[4];  // prefix, need (rank within the equal keys), equal count
    __shared__ int s_wsum[kLabWaves];
    __shared__ uint64_t s_cand[kLabCap];
    __shared__ uint32_t s_cnt, s_t0;
    const int row = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const float *lg = logits + (int64_t)row * ldl;
    for (int c = tid; c < M; c += kLabThreads)
        s_lab[c] = 0;
    const int Lc = min(L, V);
    bool fast = false;
    if (Lc > 0 && Lc <= kLabThreads) {
        // Pass 1: each thread's largest key over its elements.  The Lc-th
        // largest of these maxima, T0, belongs to Lc distinct elements, so the
        // Lc-th largest key of the row is >= T0 and every element that can be
        // selected (ties at the cut included) has a key >= T0.
        uint32_t mx = 0;
        for_row_keys<VEC>(lg, V, tid, lane, [&](int, uint32_t k, bool ok) {
            if (ok)
                mx = max(mx, k);
        });
        s_cand[tid] = ((uint64_t)mx << 32) | (uint32_t)~(uint32_t)tid;  // distinct: ties by thread
        if (tid == 0)
            s_cnt = 0u;
        __syncthreads();
        {
            const uint64_t mine = s_cand[tid];
            int rank = 0;
#pragma unroll 16
            for (int j = 0; j < kLabThreads; ++j)  // broadcast reads, many in flight
                rank += s_cand[j] > mine ? 1 : 0;
            if (rank == Lc - 1)
                s_t0 = mx;
        }
        __syncthreads();
        const uint32_t T0 = s_t0;
        // Pass 2: the candidates (key >= T0) into LDS as (key, ~id): a larger
        // value ranks first, which is logit descending, then id ascending.
        for_row_keys<VEC>(lg, V, tid, lane, [&](int y, uint32_t k, bool ok) {
            const bool c = ok && k >= T0;
            const uint64_t bal = __ballot(c);
            if (bal != 0ull) {  // uniform over the wave
                uint32_t base = 0u;
                if (lane == 0)
                    base = atomicAdd(&s_cnt, (uint32_t)__popcll(bal));
                base = (uint32_t)__shfl((int)base, 0);
                const uint32_t pos = base + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
                if (c && pos < (uint32_t)kLabCap)
                    s_cand[pos] = ((uint64_t)k << 32) | (uint32_t)~(uint32_t)y;
            }
        });
        __syncthreads();
        const uint32_t C = s_cnt;
        if (C <= (uint32_t)kLabCap) {
            // a candidate is selected iff fewer than Lc candidates rank above it
            fast = true;
            for (uint32_t i = tid; i < C; i += kLabThreads) {
                const uint64_t v = s_cand[i];
                int rank = 0;
#pragma unroll 8
                for (uint32_t j = 0; j < C; ++j)
                    rank += s_cand[j] > v ? 1 : 0;
                if (rank < Lc) {
                    const int32_t c = cluster_of[(int)~(uint32_t)v];
                    if (c >= 0 && c < M)
                        s_lab[c] = 1;
                }
            }
        }
    }
    if (Lc > 0 && !fast) {
        // more than kLabCap candidates (heavy ties) or Lc above the thread
        // count: radix select of the Lc-th largest key, one byte per pass
        uint32_t prefix = 0, mask = 0, need = (uint32_t)Lc;
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            for (int i = tid; i < kLabWaves * 256; i += kLabThreads)
                (&hist[0][0])[i] = 0u;
            __syncthreads();
            constexpr int U = 8;
            for (int y0 = tid; y0 < V; y0 += kLabThreads * U) {
                uint32_t k[U];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    k[u] = order_key(lg[min(y0 + u * kLabThreads, V - 1)]);
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (y0 + u * kLabThreads < V && (k[u] & mask) == prefix)
                        atomicAdd(&hist[wave][(k[u] >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid < 256) {
                uint32_t t = 0;
#pragma unroll
                for (int w = 0; w < kLabWaves; ++w)
                    t += hist[w][tid];
                s_tot[tid] = t;
            }
            __syncthreads();
            if (tid == 0) {  // the digit holding the need-th largest key
                uint32_t cum = 0;
                int digit = 0;
                for (int b = 255; b >= 0; --b) {
                    if (cum + s_tot[b] >= need) {
                        digit = b;
                        break;
                    }
                    cum += s_tot[b];
                }
                s_sel[0] = prefix | ((uint32_t)digit << shift);
                s_sel[1] = need - cum;
                s_sel[2] = s_tot[digit];
            }
            __syncthreads();
            prefix = s_sel[0];
            need = s_sel[1];
            mask |= 0xFFu << shift;
        }
        const uint32_t K = prefix, n_eq = s_sel[2];
        // every key above K is taken; of the n_eq keys equal to K the first
        // `need` by token id
        if (need >= n_eq) {
            for (int y = tid; y < V; y += kLabThreads)
                if (order_key(lg[y]) >= K) {
                    const int32_t c = cluster_of[y];
                    if (c >= 0 && c < M)
                        s_lab[c] = 1;
                }
        } else {
            int carry = 0;  // equal keys at ids below this chunk
            for (int y0 = 0; y0 < V; y0 += kLabThreads) {
                const int y = y0 + tid;
                const uint32_t k = y < V ? order_key(lg[y]) : 0u;
                const bool eq = y < V && k == K;
                const uint64_t bal = __ballot(eq);
                const int below = __popcll(bal & ((1ull << lane) - 1ull));
                if (lane == 0)
                    s_wsum[wave] = __popcll(bal);
                __syncthreads();
                int before = carry;
                for (int w = 0; w < wave; ++w)
                    before += s_wsum[w];
                int tot = 0;
                for (int w = 0; w < kLabWaves; ++w)
                    tot += s_wsum[w];
                if (y < V && (k > K || (eq && (uint32_t)(before + below) < need))) {
                    const int32_t c = cluster_of[y];
                    if (c >= 0 && c < M)
                        s_lab[c] = 1;
                }
                carry += tot;
                __syncthreads();
            }
        }
    }
    __syncthreads();
    uint8_t *out = labels + (int64_t)row * M;
    for (int c = tid; c < M; c += kLabThreads)
        out[c] = s_lab[c];
}

// -------------------------------------------------------------- fp32 GEMM
constexpr int kGT = 64;   // output tile edge
constexpr int kGK = 16;   // k slice

// element of an fp32 array, or of bf16 bits widened exactly
__device__ __forceinline__ float ld_f(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_f(const uint16_t *p, int64_t i) { return bf16_lo((uint32_t)p[i]); }

// C[m][n] = sum_k A(m, k) B(k, n) with A(m, k) = A[m*sam + k*sak] and
// B(k, n) = B[k*sbk + n*sbn]; the epilogue consumes each C entry.
// Split K: blockIdx.z takes k in [z*kchunk, min((z+1)*kchunk, K)) and, with
// more than one split, writes its partial tile to part[z][Mr][Nc] instead of
// calling the epilogue (a second kernel adds the splits in z order).
template <class TA, class TB, class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(int Mr, int Nc, int K, const TA *__restrict__ A,
                                                       int64_t sam, int64_t sak,
                                                       const TB *__restrict__ B, int64_t sbk,
                                                       int64_t sbn, Epi epi, int kchunk,
                                                       float *__restrict__ part)
{
    __shared__ float As[kGK][kGT + 4];
    __shared__ float Bs[kGK][kGT + 4];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * kGT, n0 = blockIdx.x * kGT;
    const int kb = blockIdx.z * kchunk, ke = min(K, kb + kchunk);
    float acc[4][4] = {};
    for (int k0 = kb; k0 < ke; k0 += kGK) {
        // 64 x 16 of A and 16 x 64 of B, four elements of each per thread
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = tid + 256 * u;
            const int am = e >> 4, ak = e & 15;        // A: m-major pieces
            const int bk = e >> 6, bn = e & 63;        // B: n-major pieces
            const int gm = m0 + am, gk = k0 + ak;
            As[ak][am] = (gm < Mr && gk < ke) ? ld_f(A, gm * sam + gk * sak) : 0.0f;
            const int gk2 = k0 + bk, gn = n0 + bn;
            Bs[bk][bn] = (gk2 < ke && gn < Nc) ? ld_f(B, gk2 * sbk + gn * sbn) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kGK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = As[kk][ty * 4 + i];
                b[i] = Bs[kk][tx * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
            if (m < Mr && n < Nc) {
                if (gridDim.z > 1)
                    part[((int64_t)blockIdx.z * Mr + m) * Nc + n] = acc[i][j];
                else
                    epi(m, n, acc[i][j]);
            }
        }
}

// the split-K partials added in split order, then the epilogue
template <class Epi>
__global__ __launch_bounds__(256) void splitk_sum_kernel(int Mr, int Nc, int splits,
                                                         const float *__restrict__ part, Epi epi)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)Mr * Nc)
        return;
    float t = part[e];
    for (int z = 1; z < splits; ++z)
        t += part[(int64_t)z * Mr * Nc + e];
    epi((int)(e / Nc), (int)(e % Nc), t);
}

__device__ __forceinline__ float sigmoidf_(float x)
{
    if (x >= 0.0f)
        return 1.0f / (1.0f + expf(-x));
    const float e = expf(x);
    return e / (1.0f + e);
}

__device__ __forceinline__ float act_f(int act, float x)
{
    return act == DS_RELU ? fmaxf(x, 0.0f) : x * sigmoidf_(x);
}

__device__ __forceinline__ float act_grad_f(int act, float x)
{
    if (act == DS_RELU)
        return x > 0.0f ? 1.0f : 0.0f;
    const float s = sigmoidf_(x);
    return s * (1.0f + x * (1.0f - s));
}

struct EpiFwd1 {  // a = acc + b1, z = act(a)
    const float *b1;
    float *a, *z;
    int r, act;
    __device__ void operator()(int i, int j, float v) const
    {
        v += b1[j];
        a[(int64_t)i * r + j] = v;
        z[(int64_t)i * r + j] = act_f(act, v);
    }
};

struct EpiFwd2 {  // s = acc + b2
    const float *b2;
    float *s;
    int M;
    __device__ void operator()(int i, int c, float v) const { s[(int64_t)i * M + c] = v + b2[c]; }
};

struct EpiGa {  // g_a = acc * act'(a)
    const float *a;
    float *ga;
    int r, act;
    __device__ void operator()(int i, int j, float v) const
    {
        ga[(int64_t)i * r + j] = v * act_grad_f(act, a[(int64_t)i * r + j]);
    }
};

struct EpiStep {  // grad = acc, param -= lr * grad
    float *grad, *param;
    float lr;
    int ld;
    __device__ void operator()(int m, int n, float v) const
    {
        const int64_t e = (int64_t)m * ld + n;
        grad[e] = v;
        param[e] -= lr * v;
    }
};

// g_s = (sigmoid(s) - y) / (n M) in place; per-block fp64 loss partials of
// softplus(s) - y s (a fixed association: each thread's terms in order, then
// a wave sum, then the block's waves in order)
constexpr int kBceThreads = 256;
__global__ __launch_bounds__(kBceThreads) void bce_kernel(int64_t total, float inv,
                                                           const uint8_t *__restrict__ y,
                                                           float *__restrict__ s,
                                                           double *__restrict__ part)
{
    __shared__ double sw[kBceThreads / kWave];
    double acc = 0.0;
    const int64_t stride = (int64_t)gridDim.x * kBceThreads;
    for (int64_t e = (int64_t)blockIdx.x * kBceThreads + threadIdx.x; e < total; e += stride) {
        const float v = s[e];
        const double yv = y[e] ? 1.0 : 0.0;
        const double dv = (double)v;
        acc += (dv > 0.0 ? dv : 0.0) + log1p(exp(-fabs(dv))) - yv * dv;
        s[e] = (sigmoidf_(v) - (float)yv) * inv;
    }
    acc = wave_sum_f64(acc);
    if (lane_id() == 0)
        sw[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int w = 0; w < kBceThreads / kWave; ++w)
            t += sw[w];
        part[blockIdx.x] = t;
    }
}

// the kBceBlocks partials: one per thread, a wave sum each, the wave sums
// added in wave order
__global__ __launch_bounds__(kBceThreads) void loss_final_kernel(double inv,
                                                                 const double *__restrict__ part,
                                                                 double *__restrict__ loss)
{
    __shared__ double sw[kBceThreads / kWave];
    const double t = wave_sum_f64(part[threadIdx.x]);
    if (lane_id() == 0)
        sw[threadIdx.x >> 6] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
        double u = 0.0;
        for (int w = 0; w < kBceThreads / kWave; ++w)
            u += sw[w];
        *loss = u * inv;
    }
}

// column sums of X [rows][cols], written as the gradient; the bias steps
// by -lr times it.  A workgroup owns 64 columns; thread (q, c) sums the rows
// q, q + 16, q + 32, ... of column c, and the 16 partials are added in q
// order (a fixed association).
constexpr int kColQ = 16;
__global__ __launch_bounds__(64 * kColQ) void colsum_step_kernel(int rows, int cols,
                                                                 const float *__restrict__ X,
                                                                 float *__restrict__ grad,
                                                                 float *__restrict__ bias, float lr)
{
    __shared__ float part[kColQ][64];
    const int cl = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + cl;
    float t = 0.0f;
    if (c < cols)
        for (int i = q; i < rows; i += kColQ)
            t += X[(int64_t)i * cols + c];
    part[q][cl] = t;
    __syncthreads();
    if (q == 0 && c < cols) {
        float s = part[0][cl];
        for (int k = 1; k < kColQ; ++k)
            s += part[k][cl];
        grad[c] = s;
        bias[c] -= lr * s;
    }
}

constexpr int kBceBlocks = 256;

// split-K ways of the products with a long K and a small output (second
// layer and the gradient through act': K = r or M)
constexpr int kSplitK = 8;
constexpr int kSplitL1 = 16;  // first layer: K = d
constexpr int kSplitW2 = 4;   // dW2: K = n, a 1024 x 1024 output at the Llama shape

struct TrainWs {
    float *a, *z, *s, *ga, *kpart;
    double *part;
};

inline size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// floats of split-K partials: the largest of the split products
inline size_t kpart_floats(int n, int r, int M)
{
    const size_t a = (size_t)kSplitL1 * n * r, b = (size_t)kSplitK * n * (r > M ? r : M),
                 c = (size_t)kSplitW2 * M * r;
    return a > b ? (a > c ? a : c) : (b > c ? b : c);
}

TrainWs train_ws(void *ws, int n, int r, int M)
{
    char *p = reinterpret_cast<char *>(ws);
    TrainWs w;
    const size_t nr = al256((size_t)n * r * 4), nm = al256((size_t)n * M * 4);
    w.a = reinterpret_cast<float *>(p);
    w.z = reinterpret_cast<float *>(p + nr);
    w.ga = reinterpret_cast<float *>(p + 2 * nr);
    w.s = reinterpret_cast<float *>(p + 3 * nr);
    w.part = reinterpret_cast<double *>(p + 3 * nr + nm);
    w.kpart = reinterpret_cast<float *>(p + 3 * nr + nm + al256((size_t)kBceBlocks * 8));
    return w;
}

// splits > 1 needs part >= splits * Mr * Nc floats
template <class TA, class TB, class Epi>
hipError_t gemm(hipStream_t s, int Mr, int Nc, int K, const TA *A, int64_t sam, int64_t sak,
                const TB *B, int64_t sbk, int64_t sbn, Epi epi, int splits = 1,
                float *part = nullptr)
{
    const int kchunk = ((K + splits - 1) / splits + kGK - 1) / kGK * kGK;
    splits = (K + kchunk - 1) / kchunk;
    dim3 grid((unsigned)((Nc + kGT - 1) / kGT), (unsigned)((Mr + kGT - 1) / kGT), (unsigned)splits);
    hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, Epi>), grid, dim3(256), 0, s, Mr, Nc, K, A, sam,
                       sak, B, sbk, sbn, epi, kchunk, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1)
        return e;
    const int64_t total = (int64_t)Mr * Nc;
    hipLaunchKernelGGL((splitk_sum_kernel<Epi>), dim3((unsigned)((total + 255) / 256)), dim3(256),
                       0, s, Mr, Nc, splits, (const float *)part, epi);
    return hipGetLastError();
}

}  // namespace

hipError_t topl_labels_launch(hipStream_t s, int n, int V, int M, int L, const float *logits,
                              int64_t ldl, const int32_t *cluster_of, uint8_t *labels)
{
    // 16-byte loads where every row starts on a 16-byte boundary
    const bool vec = (reinterpret_cast<uintptr_t>(logits) & 15) == 0 && ldl % 4 == 0;
    hipLaunchKernelGGL(vec ? topl_labels_kernel<true> : topl_labels_kernel<false>,
                       dim3((unsigned)n), dim3(kLabThreads), 0, s, V, M, L,
                       logits, ldl, cluster_of, labels);
    return hipGetLastError();
}

size_t router_train_ws_bytes(int n, int r, int M)
{
    return 3 * al256((size_t)n * r * 4) + al256((size_t)n * M * 4) +
           al256((size_t)kBceBlocks * 8) + al256(kpart_floats(n, r, M) * 4) + 256;
}

hipError_t router_train_launch(hipStream_t s, int n, int d, int r, int M, int act, bool h_bf16,
                               const void *h, int64_t ldh, const uint8_t *labels, float lr,
                               float *W1, float *b1, float *W2, float *b2, float *dW1,
                               float *db1, float *dW2, float *db2, double *loss, void *ws)
{
    TrainWs w = train_ws(ws, n, r, M);
    hipError_t e;
    // a = h W1^T + b1, z = act(a): A = h [n][d], B(k, j) = W1[j][k]
    if (h_bf16)
        e = gemm(s, n, r, d, reinterpret_cast<const uint16_t *>(h), ldh, (int64_t)1, W1,
                 (int64_t)1, (int64_t)d, EpiFwd1{b1, w.a, w.z, r, act}, kSplitL1, w.kpart);
    else
        e = gemm(s, n, r, d, reinterpret_cast<const float *>(h), ldh, (int64_t)1, W1,
                 (int64_t)1, (int64_t)d, EpiFwd1{b1, w.a, w.z, r, act}, kSplitL1, w.kpart);
    if (e != hipSuccess)
        return e;
    // s = z W2^T + b2
    if ((e = gemm(s, n, M, r, (const float *)w.z, (int64_t)r, (int64_t)1, W2, (int64_t)1,
                  (int64_t)r, EpiFwd2{b2, w.s, M}, kSplitK, w.kpart)) != hipSuccess)
        return e;
    const int64_t total = (int64_t)n * M;
    const double inv = 1.0 / ((double)n * (double)M);
    hipLaunchKernelGGL(bce_kernel, dim3(kBceBlocks), dim3(kBceThreads), 0, s, total, (float)inv,
                       labels, w.s, w.part);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    static_assert(kBceBlocks == kBceThreads, "one loss partial per thread");
    hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(kBceThreads), 0, s, inv,
                       (const double *)w.part, loss);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    // g_a = (g_s W2) * act'(a), with W2 before its step
    if ((e = gemm(s, n, r, M, (const float *)w.s, (int64_t)M, (int64_t)1, W2, (int64_t)r,
                  (int64_t)1, EpiGa{w.a, w.ga, r, act}, kSplitK, w.kpart)) != hipSuccess)
        return e;
    // dW2[c][j] = sum_i g_s[i][c] z[i][j]
    if ((e = gemm(s, M, r, n, (const float *)w.s, (int64_t)1, (int64_t)M, w.z, (int64_t)r,
                  (int64_t)1, EpiStep{dW2, W2, lr, r}, kSplitW2, w.kpart)) != hipSuccess)
        return e;
    // dW1[j][k] = sum_i g_a[i][j] h[i][k]
    if (h_bf16)
        e = gemm(s, r, d, n, (const float *)w.ga, (int64_t)1, (int64_t)r,
                 reinterpret_cast<const uint16_t *>(h), ldh, (int64_t)1, EpiStep{dW1, W1, lr, d});
    else
        e = gemm(s, r, d, n, (const float *)w.ga, (int64_t)1, (int64_t)r,
                 reinterpret_cast<const float *>(h), ldh, (int64_t)1, EpiStep{dW1, W1, lr, d});
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(colsum_step_kernel, dim3((unsigned)((M + 63) / 64)), dim3(64 * kColQ), 0, s,
                       n, M, (const float *)w.s, db2, b2, lr);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(colsum_step_kernel, dim3((unsigned)((r + 63) / 64)), dim3(64 * kColQ), 0, s,
                       n, r, (const float *)w.ga, db1, b1, lr);
    return hipGetLastError();
}

}  // namespace ds
