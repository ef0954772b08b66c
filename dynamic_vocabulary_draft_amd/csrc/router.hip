// Router / meta-classifier: a two-layer MLP that scores every vocabulary
// cluster from the draft hidden state (DynaSpec summary page, "System
// Modules: Router" and "Key Hyperparameters": 2-layer MLP; "Problem
// Definition": input H_{t-1}).
//
// Both layers are small-n matrix-vector products against weights that are
// read once from HBM (8 MB + 2 MB bf16 for the Llama-shaped router), so
// each is a tiled GEMV: a wave owns NR weight rows and XB input rows, walks
// the reduction dimension in 16-byte chunks per lane (coalesced 1 KB per
// wave per load), and reduces its NR*XB partial sums across the wave with a
// fixed DPP order.  Bias and activation are fused into the epilogue; the
// hidden activations z stay fp32.
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
template <bool A_BF16, bool X_BF16, int NR, int XB>
__global__ __launch_bounds__(256) void gemv_tile_kernel(int n, int K, int R, const void *__restrict__ A,
                                                        const void *__restrict__ bias,
                                                        const void *__restrict__ X, int64_t ldx,
                                                        int act, float *__restrict__ Y, int64_t ldy)
{
    const int lane = lane_id();
    const int wave = uniform(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
    const int o0 = wave * NR;
    const int x0 = uniform(blockIdx.y * XB);
    if (o0 >= R)
        return;
    const int nr = min(NR, R - o0), nx = min(XB, n - x0);
    const int nch = K >> 3;
    float acc[NR][XB];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int x = 0; x < XB; ++x)
            acc[r][x] = 0.f;

    for (int c = lane; c < nch; c += kWave) {
        float a[NR][8];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            Chunk8<A_BF16> ch;
            if (r < nr) {
                ch.load(A, (int64_t)(o0 + r) * K + c * 8);
                ch.unpack(a[r]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    a[r][e] = 0.f;
            }
        }
#pragma unroll
        for (int x = 0; x < XB; ++x) {
            if (x < nx) {
                Chunk8<X_BF16> ch;
                ch.load(X, (int64_t)(x0 + x) * ldx + c * 8);
                float xv[8];
                ch.unpack(xv);
#pragma unroll
                for (int r = 0; r < NR; ++r)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[r][x] = fmaf(a[r][e], xv[e], acc[r][x]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int x = 0; x < XB; ++x) {
            float s = wave_sum(acc[r][x]);
            if (r < nr && x < nx && lane == ((r * XB + x) & (kWave - 1))) {
                if (bias)
                    s += load_scalar(bias, o0 + r, A_BF16);
                if (act == DS_RELU + 1)       // layer-1 ReLU
                    s = fmaxf(s, 0.f);
                else if (act == DS_SILU + 1)  // layer-1 SiLU
                    s = s / (1.f + expf(-s));
                Y[(int64_t)(x0 + x) * ldy + o0 + r] = s;
            }
        }
    }
}

template <bool A_BF16, bool X_BF16>
hipError_t launch_gemv(hipStream_t s, int n, int K, int R, const void *A, const void *bias,
                       const void *X, int64_t ldx, int act, float *Y, int64_t ldy)
{
    constexpr int NR = 2, XB = 4;
    const int waves = (R + NR - 1) / NR;
    dim3 grid((waves + 3) / 4, (n + XB - 1) / XB);
    hipLaunchKernelGGL((gemv_tile_kernel<A_BF16, X_BF16, NR, XB>), grid, dim3(256), 0, s, n, K, R,
                       A, bias, X, ldx, act, Y, ldy);
    return hipGetLastError();
}

}  // namespace

hipError_t router_launch(hipStream_t s, bool bf16, int n, int d, int r, int M, int act,
                         const void *h, int64_t ldh, const void *W1, const void *b1,
                         const void *W2, const void *b2, float *scores, float *z)
{
    hipError_t e;
    // layer 1: z = act(W1 h + b1), act encoded as act + 1 (0 = identity)
    e = bf16 ? launch_gemv<true, true>(s, n, d, r, W1, b1, h, ldh, act + 1, z, r)
             : launch_gemv<false, false>(s, n, d, r, W1, b1, h, ldh, act + 1, z, r);
    if (e != hipSuccess)
        return e;
    // layer 2: scores = W2 z + b2 (z is fp32)
    return bf16 ? launch_gemv<true, false>(s, n, r, M, W2, b2, z, r, 0, scores, M)
                : launch_gemv<false, false>(s, n, r, M, W2, b2, z, r, 0, scores, M);
}

}  // namespace ds
