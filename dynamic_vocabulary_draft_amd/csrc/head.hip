// Gathered LM head: draft logits only for the shortlisted rows of W
// (DynaSpec summary page, "System Modules: Gathered LM Head" and "Novel
// Architectural Elements": index selection fused with the matrix product,
// no gathered copy of W; "Comparison to Prior Work": O(|V_S| d) instead of
// O(|V| d)).
//
// GEMV regime (few head rows per shortlist).  The work is the flattened list
// of shortlist entries J in [sl_off[0], sl_off[G]); a wave owns RPW
// consecutive entries.  For each it reads the token id, then streams that
// token's whole W row with 16-byte loads per lane (64 lanes x 16 B = 1 KB
// contiguous per load instruction, KC instructions per row), all RPW rows
// issued before any arithmetic so that RPW*d*e bytes per wave are in
// flight; the grid is capped at two workgroups per compute unit and strides
// over the entries.  The hidden vector of the entry's group is held in registers in
// the same lane layout and reloaded only when the group changes.  Products
// use v_dot2_f32_bf16 (bf16 pairs, fp32 accumulation); the lane partials are
// reduced with a fixed DPP order, so the result is reproducible bit for bit.
// The kernel is HBM-bound: per entry it moves d*e bytes of W, 4 bytes of id
// and 4*m bytes of logits.
#include "common.h"
#include "kernels.h"

namespace ds {
namespace {

template <bool BF16>
__device__ __forceinline__ float dot_chunk(const u32x4 &w, const u32x4 &x, float acc)
{
    if constexpr (BF16) {
        acc = dot2_bf16(w[0], x[0], acc);
        acc = dot2_bf16(w[1], x[1], acc);
        acc = dot2_bf16(w[2], x[2], acc);
        acc = dot2_bf16(w[3], x[3], acc);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = fmaf(__uint_as_float(w[e]), __uint_as_float(x[e]), acc);
    }
    return acc;
}

// group g with sl_off[g] <= J < sl_off[g+1] (the last such g when empty
// groups share an offset); wave-uniform result.
__device__ __forceinline__ int group_of(const int64_t *__restrict__ sl_off, int G, int64_t J)
{
    const int lane = lane_id();
    int count = 0;
    for (int b = 0; b <= G; b += kWave) {
        int idx = b + lane;
        bool le = idx <= G && sl_off[idx] <= J;
        uint64_t bal = __ballot(le);
        count += __popcll(bal);
        if (bal != ~0ull)
            break;
    }
    return uniform(count - 1);
}

template <bool BF16, int KC, int RPW>
__global__ __launch_bounds__(256) void head_gemv_kernel(int V, int nch, const u32x4 *__restrict__ W,
                                                        int G, int m, const u32x4 *__restrict__ h,
                                                        int64_t ldh_g_ch,
                                                        const int64_t *__restrict__ sl_off,
                                                        const int32_t *__restrict__ sl_ids,
                                                        float *__restrict__ logits)
{
    const int lane = lane_id();
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t beg = sl_off[0], end = sl_off[G];
    int g = -1, hi = -1;
    int64_t g_lo = 0, g_hi = -1, len = 0;
    u32x4 x[KC];
    // grid-stride over blocks of RPW entries: correct for any grid size
    for (int64_t J0 = uniform64(beg + gw * RPW); J0 < end; J0 += nwaves * RPW) {
        const int nr = (int)min((int64_t)RPW, end - J0);

        // token ids of this wave's entries (lane r holds entry r)
        int id_lane = lane < nr ? sl_ids[J0 + lane] : 0;
        int ids[RPW];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            ids[r] = __builtin_amdgcn_readlane(id_lane, r);
            if (ids[r] < 0 || ids[r] >= V)
                ids[r] = -1;
        }

        // issue every W load first
        u32x4 w[RPW][KC];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const u32x4 *row = W + (int64_t)(ids[r] < 0 ? 0 : ids[r]) * nch;
#pragma unroll
            for (int k = 0; k < KC; ++k) {
                const int c = lane + k * kWave;
                if (r < nr && (KC * kWave == nch || c < nch))
                    w[r][k] = __builtin_nontemporal_load(row + c);
                else
                    w[r][k] = u32x4{0u, 0u, 0u, 0u};
            }
        }

#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            if (r >= nr)
                break;
            const int64_t J = J0 + r;
            if (J >= g_hi || J < g_lo) {  // entered a new group
                g = group_of(sl_off, G, J);
                g_lo = sl_off[g];
                g_hi = sl_off[g + 1];
                len = g_hi - g_lo;
                hi = -1;
            }
            const int64_t obase = (int64_t)m * g_lo + (J - g_lo);
            for (int i = 0; i < m; ++i) {
                if (i != hi) {
                    const u32x4 *hr = h + (int64_t)g * ldh_g_ch + (int64_t)i * nch;
#pragma unroll
                    for (int k = 0; k < KC; ++k) {
                        const int c = lane + k * kWave;
                        x[k] = (KC * kWave == nch || c < nch) ? hr[c] : u32x4{0u, 0u, 0u, 0u};
                    }
                    hi = i;
                }
                float acc = 0.f;
#pragma unroll
                for (int k = 0; k < KC; ++k)
                    acc = dot_chunk<BF16>(w[r][k], x[k], acc);
                float s = wave_sum(acc);
                if (lane == 0)
                    logits[obase + (int64_t)i * len] = ids[r] < 0 ? __builtin_nanf("") : s;
            }
        }
    }
}

template <bool BF16, int KC>
hipError_t launch_kc(hipStream_t s, int V, int nch, const void *W, int G, int m, const void *h,
                     int64_t ldh_g_ch, const int64_t *sl_off, const int32_t *sl_ids,
                     int64_t max_rows, float *logits, hipEvent_t t0, hipEvent_t t1)
{
    constexpr int RPW = (KC >= 8) ? 2 : 4;
    const int64_t waves = (max_rows + RPW - 1) / RPW;
    int64_t blocks = (waves + 3) / 4;
    if (blocks <= 0)
        return hipSuccess;
    // At most kBlocksPerCU resident workgroups per compute unit: enough
    // bytes in flight to saturate HBM, while half of each CU's wave slots
    // stay free so kernels on other streams (the router of the next draft
    // position) start at once instead of queueing behind thousands of
    // pending head workgroups.  The grid-stride loop covers the rest.
    constexpr int kBlocksPerCU = 2;
    const int64_t cap = (int64_t)kBlocksPerCU * device_cu_count();
    if (blocks > cap)
        blocks = cap;
    return launch_timed(head_gemv_kernel<BF16, KC, RPW>, dim3((unsigned)blocks), dim3(256), s, t0,
                        t1, V, nch, reinterpret_cast<const u32x4 *>(W), G, m,
                        reinterpret_cast<const u32x4 *>(h), ldh_g_ch, sl_off, sl_ids, logits);
}

template <bool BF16>
hipError_t launch_dtype(hipStream_t s, int V, int d, const void *W, int G, int m, const void *h,
                        int64_t ldh_g, const int64_t *sl_off, const int32_t *sl_ids,
                        int64_t max_rows, float *logits, hipEvent_t t0, hipEvent_t t1)
{
    const int e = BF16 ? 2 : 4;
    const int nch = d * e / 16;                 // 16-byte chunks per row
    const int64_t ldh_g_ch = ldh_g * e / 16;    // group stride in chunks
    const int kc = (nch + kWave - 1) / kWave;
    if (kc <= 1)
        return launch_kc<BF16, 1>(s, V, nch, W, G, m, h, ldh_g_ch, sl_off, sl_ids, max_rows, logits, t0, t1);
    if (kc <= 2)
        return launch_kc<BF16, 2>(s, V, nch, W, G, m, h, ldh_g_ch, sl_off, sl_ids, max_rows, logits, t0, t1);
    if (kc <= 4)
        return launch_kc<BF16, 4>(s, V, nch, W, G, m, h, ldh_g_ch, sl_off, sl_ids, max_rows, logits, t0, t1);
    if (kc <= 8)
        return launch_kc<BF16, 8>(s, V, nch, W, G, m, h, ldh_g_ch, sl_off, sl_ids, max_rows, logits, t0, t1);
    return launch_kc<BF16, 16>(s, V, nch, W, G, m, h, ldh_g_ch, sl_off, sl_ids, max_rows, logits, t0, t1);
}

}  // namespace

hipError_t head_launch(hipStream_t s, bool bf16, int V, int d, const void *W, int G, int m,
                       const void *h, int64_t ldh_g, const int64_t *sl_off,
                       const int32_t *sl_ids, int64_t max_rows, float *logits, void *ws,
                       hipEvent_t t0, hipEvent_t t1)
{
    if (head_mfma_applies(bf16, V, d, G, m))
        return head_mfma_launch(s, V, d, W, G, m, h, ldh_g, sl_off, sl_ids, max_rows, logits, ws,
                                t0, t1);
    return bf16 ? launch_dtype<true>(s, V, d, W, G, m, h, ldh_g, sl_off, sl_ids, max_rows, logits,
                                     t0, t1)
                : launch_dtype<false>(s, V, d, W, G, m, h, ldh_g, sl_off, sl_ids, max_rows,
                                      logits, t0, t1);
}

}  // namespace ds
