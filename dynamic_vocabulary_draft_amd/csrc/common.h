// Shared device helpers for the gfx950 (CDNA4, wave64) kernels of the
// shortlisted draft head.  Nothing here is method arithmetic: loads, wave and
// block reductions with a fixed association (so results are bit-reproducible
// run to run), and launch-error plumbing.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dynaspec.h"

namespace ds {

constexpr int kWave = 64;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// wave-uniform value -> scalar register
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64(int64_t v)
{
    uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// bf16 pair packed in a dword -> the two fp32 values (exact widening)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// fp32 += a.lo*b.lo + a.hi*b.hi on packed bf16 pairs (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), acc, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes with a fixed association: pairs, quads, octets and
// rows of 16 through DPP, then the four row sums in lane order.  Every lane
// receives the result.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f32<0x141>(v);  // row_half_mirror
    v += dpp_f32<0x140>(v);  // row_mirror
    float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return ((r0 + r1) + r2) + r3;
}

// A double moved across lanes by DPP (both halves with the same control);
// lanes whose source is outside the row, or whose row is not in ROWS, get 0.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROWS, 0xF,
                                                             false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL,
                                                             ROWS, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double readlane_f64(double v, int l)
{
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Sum over the 64 lanes in a fixed association (as wave_sum), every lane
// receiving the same value.
__device__ __forceinline__ double wave_sum_f64(double v)
{
    v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f64<0x141>(v);  // row_half_mirror
    v += dpp_f64<0x140>(v);  // row_mirror
    return ((readlane_f64(v, 0) + readlane_f64(v, 16)) + readlane_f64(v, 32)) + readlane_f64(v, 48);
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    v = fmaxf(v, dpp_f32<0x140>(v));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Inclusive scan over the wave in lane order, fixed association: within each
// row of 16 lanes by shifts of 1, 2, 4, 8 (Hillis-Steele), then the row
// totals carried across rows (row 0's into row 1, row 2's into row 3, then
// rows 0-1's into rows 2 and 3).
__device__ __forceinline__ double wave_incl_scan_f64(double v)
{
    v += dpp_f64<0x111>(v);       // row_shr:1
    v += dpp_f64<0x112>(v);       // row_shr:2
    v += dpp_f64<0x114>(v);       // row_shr:4
    v += dpp_f64<0x118>(v);       // row_shr:8
    v += dpp_f64<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_f64<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

__device__ __forceinline__ int64_t wave_incl_scan_i64(int64_t v)
{
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int64_t t = __shfl_up(v, o);
        if (lane >= o)
            v += t;
    }
    return v;
}

// Block-wide exclusive scan of doubles (blockDim.x = 64 * nwaves, nwaves <=
// 64).  Returns this thread's exclusive prefix; *total gets the block sum.
// `sh` must hold at least 64 doubles.  Contains barriers: call from all threads.
__device__ __forceinline__ double block_excl_scan_f64(double v, double *sh, double *total)
{
    const int lane = lane_id(), wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    double incl = wave_incl_scan_f64(v);
    if (lane == kWave - 1)
        sh[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        double w = lane < nw ? sh[lane] : 0.0;
        double wi = wave_incl_scan_f64(w);
        if (lane < nw)
            sh[lane] = wi - w;  // exclusive prefix of wave totals
        if (lane == nw - 1)
            sh[kWave] = wi;
    }
    __syncthreads();
    double r = sh[wave] + (incl - v);
    *total = sh[kWave];
    __syncthreads();
    return r;
}

__device__ __forceinline__ int64_t block_excl_scan_i64(int64_t v, int64_t *sh, int64_t *total)
{
    const int lane = lane_id(), wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int64_t incl = wave_incl_scan_i64(v);
    if (lane == kWave - 1)
        sh[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int64_t w = lane < nw ? sh[lane] : 0;
        int64_t wi = wave_incl_scan_i64(w);
        if (lane < nw)
            sh[lane] = wi - w;
        if (lane == nw - 1)
            sh[kWave] = wi;
    }
    __syncthreads();
    int64_t r = sh[wave] + (incl - v);
    *total = sh[kWave];
    __syncthreads();
    return r;
}

// Raise a device-side error code; the largest code wins (deterministic).
__device__ __forceinline__ void raise_flag(int32_t *flag, int32_t code)
{
    if (flag)
        atomicMax(flag, code);
}

// Host-side: compute units of the current device (cached per device id; the
// first call on a device queries the runtime).
int device_cu_count();

// Host-side: launch `kernel`; non-null t0 / t1 are timing events stamped at
// the kernel's own start / end (the dispatch's begin and end timestamps,
// not the host-enqueue order), for measuring a kernel inside a sequence.
template <typename K, typename... Args>
inline hipError_t launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t t0,
                               hipEvent_t t1, Args... args)
{
    if (t0 || t1)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, t0, t1, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
    return hipGetLastError();
}

}  // namespace ds

// Host-side: turn a launch error into a status.
#define DS_LAUNCH_CHECK()                                  \
    do {                                                   \
        if (hipGetLastError() != hipSuccess)               \
            return DS_EHIP;                                \
    } while (0)
