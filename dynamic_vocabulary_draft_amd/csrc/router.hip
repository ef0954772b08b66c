// Router / meta-classifier: a two-layer MLP that scores every vocabulary
// cluster from the draft hidden state (DynaSpec summary page, "System
// Modules: Router" and "Key Hyperparameters": 2-layer MLP; "Problem
// Definition": input H_{t-1}).
//
// For a few inputs both layers are matrix-vector products against weights
// that are read once from HBM (8 MB + 2 MB bf16 for the Llama-shaped
// router), so each is a GEMV: a wave owns one weight row and up to 8 input
// rows, holds
// the whole weight row in registers (16-byte loads per lane, 1 KB per wave
// per load instruction, all issued at once), and reduces each partial sum
// across the wave with a fixed DPP order.  Bias and activation are fused
// into the epilogue; the hidden activations z stay fp32.  Weight rows are
// limited to 8192 elements (KC <= 16 chunks of 8 per lane).  A batch of
// 8 or more bf16 inputs runs the first layer on the matrix cores instead
// (head_mfma.hip), with the same fp32 accumulation of exact bf16 products.
#include "common.h"
#include "kernels.h"

namespace ds {
namespace {

template <bool BF16>
struct Chunk8;  // 8 consecutive elements = one 16-byte (bf16) or two (fp32) loads

template <>
struct Chunk8<true> {
    u32x4 v;
    __device__ __forceinline__ void load(const void *base, int64_t elem)
    {
        v = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(base) + elem);
    }
    __device__ __forceinline__ void unpack(float f[8]) const
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16_lo(v[i]);
            f[2 * i + 1] = bf16_hi(v[i]);
        }
    }
};

template <>
struct Chunk8<false> {
    float4 a, b;
    __device__ __forceinline__ void load(const void *base, int64_t elem)
    {
        const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + elem);
        a = p[0];
        b = p[1];
    }
    __device__ __forceinline__ void unpack(float f[8]) const
    {
        f[0] = a.x, f[1] = a.y, f[2] = a.z, f[3] = a.w;
        f[4] = b.x, f[5] = b.y, f[6] = b.z, f[7] = b.w;
    }
};

__device__ __forceinline__ float load_scalar(const void *p, int idx, bool bf16)
{
    if (bf16)
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(p)[idx] << 16);
    return reinterpret_cast<const float *>(p)[idx];
}

// Y[row][o] = act(sum_k A[o][k] X[row][k] + bias[o]) for o < R, row < n.
// One wave per weight row o; lane l owns the 8-element chunks l, l+64, ...
// (KC of them).  Every weight chunk is loaded before any arithmetic, so a
// wave keeps a whole row (8 KB at d = 4096 bf16) in flight; the XB input
// rows are then read chunk by chunk (L1/L2-resident, shared by all waves).
template <bool A_BF16, bool X_BF16, int KC, int XB>
__global__ __launch_bounds__(256) void gemv_rows_kernel(int n, int K, int R, const void *__restrict__ A,
                                                        const void *__restrict__ bias,
                                                        const void *__restrict__ X, int64_t ldx,
                                                        int act, float *__restrict__ Y, int64_t ldy)
{
    const int lane = lane_id();
    const int o = uniform(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
    const int x0 = uniform(blockIdx.y * XB);
    if (o >= R)
        return;
    const int nch = K >> 3;
    Chunk8<A_BF16> a[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        const int c = lane + k * kWave;
        if (c < nch)
            a[k].load(A, (int64_t)o * K + c * 8);
    }
    float acc[XB];
#pragma unroll
    for (int x = 0; x < XB; ++x)
        acc[x] = 0.f;
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        const int c = lane + k * kWave;
        if (c >= nch)
            break;
        float av[8];
        if constexpr (!(A_BF16 && X_BF16))
            a[k].unpack(av);
#pragma unroll
        for (int x = 0; x < XB; ++x) {
            if (x0 + x >= n)
                break;
            Chunk8<X_BF16> xc;
            xc.load(X, (int64_t)(x0 + x) * ldx + c * 8);
            if constexpr (A_BF16 && X_BF16) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[x] = dot2_bf16(a[k].v[e], xc.v[e], acc[x]);
            } else {
                float xv[8];
                xc.unpack(xv);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[x] = fmaf(av[e], xv[e], acc[x]);
            }
        }
    }
    const float bv = bias ? load_scalar(bias, o, A_BF16) : 0.f;
#pragma unroll
    for (int x = 0; x < XB; ++x) {
        float s = wave_sum(acc[x]);
        if (x0 + x < n && lane == 0) {
            s += bv;
            if (act == DS_RELU + 1)       // layer-1 ReLU
                s = fmaxf(s, 0.f);
            else if (act == DS_SILU + 1)  // layer-1 SiLU
                s = s / (1.f + expf(-s));
            Y[(int64_t)(x0 + x) * ldy + o] = s;
        }
    }
}

template <bool A_BF16, bool X_BF16, int KC>
hipError_t launch_kc(hipStream_t s, int n, int K, int R, const void *A, const void *bias,
                     const void *X, int64_t ldx, int act, float *Y, int64_t ldy)
{
    dim3 block(256);
    if (n == 1) {
        hipLaunchKernelGGL((gemv_rows_kernel<A_BF16, X_BF16, KC, 1>), dim3((R + 3) / 4, 1), block,
                           0, s, n, K, R, A, bias, X, ldx, act, Y, ldy);
    } else if (n <= 4) {
        hipLaunchKernelGGL((gemv_rows_kernel<A_BF16, X_BF16, KC, 4>), dim3((R + 3) / 4, 1), block,
                           0, s, n, K, R, A, bias, X, ldx, act, Y, ldy);
    } else {
        hipLaunchKernelGGL((gemv_rows_kernel<A_BF16, X_BF16, KC, 8>),
                           dim3((R + 3) / 4, (n + 7) / 8), block, 0, s, n, K, R, A, bias, X, ldx,
                           act, Y, ldy);
    }
    return hipGetLastError();
}

template <bool A_BF16, bool X_BF16>
hipError_t launch_gemv(hipStream_t s, int n, int K, int R, const void *A, const void *bias,
                       const void *X, int64_t ldx, int act, float *Y, int64_t ldy)
{
    const int kc = ((K >> 3) + kWave - 1) / kWave;
    if (kc <= 1)
        return launch_kc<A_BF16, X_BF16, 1>(s, n, K, R, A, bias, X, ldx, act, Y, ldy);
    if (kc <= 2)
        return launch_kc<A_BF16, X_BF16, 2>(s, n, K, R, A, bias, X, ldx, act, Y, ldy);
    if (kc <= 4)
        return launch_kc<A_BF16, X_BF16, 4>(s, n, K, R, A, bias, X, ldx, act, Y, ldy);
    if (kc <= 8)
        return launch_kc<A_BF16, X_BF16, 8>(s, n, K, R, A, bias, X, ldx, act, Y, ldy);
    return launch_kc<A_BF16, X_BF16, 16>(s, n, K, R, A, bias, X, ldx, act, Y, ldy);
}

}  // namespace

size_t router_ws_bytes(int n, int r)
{
    const size_t zb = ((size_t)n * (size_t)r * sizeof(float) + 255) / 256 * 256;
    return zb + (n >= kRouterMfmaMin ? router_l1_ws_bytes(r) : 0);
}

hipError_t router_launch(hipStream_t s, bool bf16, int n, int d, int r, int M, int act,
                         const void *h, int64_t ldh, const void *W1, const void *b1,
                         const void *W2, const void *b2, float *scores, float *z)
{
    hipError_t e;
    float *part = reinterpret_cast<float *>(
        reinterpret_cast<char *>(z) + ((size_t)n * (size_t)r * sizeof(float) + 255) / 256 * 256);
    // layer 1: z = act(W1 h + b1).  A batch of bf16 inputs is a dense
    // contraction: matrix cores, split over k (the GEMV below re-reads each
    // weight row once per 8 inputs); else the GEMV with act encoded as
    // act + 1 (0 = identity)
    if (bf16 && n >= kRouterMfmaMin) {
        e = router_l1_mfma_launch(s, n, d, r, act, h, ldh, W1, b1, z, part);
    } else {
        e = bf16 ? launch_gemv<true, true>(s, n, d, r, W1, b1, h, ldh, act + 1, z, r)
                 : launch_gemv<false, false>(s, n, d, r, W1, b1, h, ldh, act + 1, z, r);
    }
    if (e != hipSuccess)
        return e;
    // layer 2: scores = W2 z + b2 (z is fp32).  A batch re-reads every W2
    // row once per 8 inputs in the GEMV, and reads z once per W2 row: on
    // the matrix cores (z split exactly into bf16 pieces) instead
    if (bf16 && n >= kRouterMfmaMin && router_l2_mfma_applies(r, M))
        return router_l2_mfma_launch(s, n, r, M, z, W2, b2, scores, part);
    return bf16 ? launch_gemv<true, false>(s, n, r, M, W2, b2, z, r, 0, scores, M)
                : launch_gemv<false, false>(s, n, r, M, W2, b2, z, r, 0, scores, M);
}

// the partials are read beside the batched head: only when they are small
// (measured: 2 MB at 32 inputs, M = 1024 saved 10 us per step; 8 MB at 64
// inputs, M = 2048 slowed the head beside them and cost 7 us)
constexpr size_t kSplitMaxBytes = (size_t)2 << 20;

bool router_split_applies(bool bf16, int n, int r, int M)
{
    const int nwin = router_l2_windows(r, M);
    return bf16 && n >= kRouterMfmaMin && n <= kRouterPassCols && nwin > 0 &&
           (size_t)nwin * (size_t)n * (size_t)M * sizeof(float) <= kSplitMaxBytes;
}

hipError_t router_launch_split(hipStream_t s, int n, int d, int r, int M, int act, const void *h,
                               int64_t ldh, const void *W1, const void *b1, const void *W2,
                               float *z, float *part2)
{
    if (!router_split_applies(true, n, r, M))
        return hipErrorInvalidValue;
    float *part = reinterpret_cast<float *>(
        reinterpret_cast<char *>(z) + ((size_t)n * (size_t)r * sizeof(float) + 255) / 256 * 256);
    hipError_t e = router_l1_mfma_launch(s, n, d, r, act, h, ldh, W1, b1, z, part);
    if (e != hipSuccess)
        return e;
    return router_l2_mfma_partials(s, n, r, M, z, W2, part2);
}

}  // namespace ds
