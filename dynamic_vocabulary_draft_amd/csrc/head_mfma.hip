// Gathered LM head, matrix-core regimes (DynaSpec summary page, "System
// Modules: Gathered LM Head" and "Novel Architectural Elements": the
// projection restricted to the shortlist rows, fused with the index
// selection; "Comparison to Prior Work": O(|V_S| d)).
//
// Both kernels use v_mfma_f32_32x32x16_bf16 (bf16 inputs, fp32
// accumulation).  A wave owns 32 rows of W; per 64-element slice of the
// hidden dimension it reads the rows' 128-byte lines whole and passes them
// through a small per-wave LDS buffer into MFMA order, where lane l holds
// 64 contiguous bytes of row l%32 (lanes l and l+32 the two halves) for four
// MFMA steps; the same permutation of the reduction index is applied to the
// B operand, so the products are exact and only the summation order differs
// from a plain dot product.  The B operand (hidden vectors) is staged in LDS
// per phase of several slices and shared by the workgroup's waves (4 or 8).
//
// union (batched drafting: many shortlists, one head row each): the union
//   of B shortlists covers nearly all of V already at B = 32, so instead of
//   streaming every group's rows (B times the bytes) the kernel walks W in
//   128- or 256-token tiles in token-id order (a persistent grid, the same
//   number of tiles per workgroup), reads each row once, multiplies it
//   with all G hidden vectors (columns of the MFMA), and writes only the
//   (row, group) pairs on that group's shortlist.  It reads, per group and
//   32-token tile, where the tile's entries start in the group's shortlist
//   (shortlists are ascending) and which of the tile's 32 tokens they are:
//   inside the draft chain the build writes this index, a standalone call
//   builds it in a pre-pass over the shortlists.
// gathered (tree drafting: m head rows share one shortlist): a gathered
//   GEMM per group, rows = shortlist entries (gathered W rows), columns =
//   the m head rows; a persistent grid strides over one list of every
//   group's tiles, ordered by tile index, so groups of unequal length share
//   the compute units and walk their shortlists side by side.
#include "common.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace ds {
namespace {

// B operand (hidden vectors) for one phase of KP hidden elements, staged in
// LDS as [NB*32][KP + 8] bf16 (rows past nrows and elements past d are zero).
// Each of the NT threads moves stage_n<NT>() 16-byte pieces: all loads of a
// phase are issued one slice group before the phase starts, into registers.
template <int NB>
constexpr int phase_len() { return 512 / NB; }
constexpr int kPhaseRot = 7;  // phase rotation per tile (coprime to 8, 15 and 16 phases)
template <int NB>
constexpr int lds_row() { return phase_len<NB>() + 8; }
template <int NT>
constexpr int stage_n() { return 32 * 512 / 8 / NT; }  // pieces per thread per phase

template <int NB, int NT, class Src>
__device__ __forceinline__ void load_phase(u32x4 v[stage_n<NT>()], int k0, int d, int nrows,
                                           Src src)
{
    constexpr int KP = phase_len<NB>();
#pragma unroll
    for (int i = 0; i < stage_n<NT>(); ++i) {
        const int p = threadIdx.x + NT * i;
        const int r = min(p / (KP / 8), nrows - 1), k = min(k0 + (p % (KP / 8)) * 8, d - 8);
        v[i] = *reinterpret_cast<const u32x4 *>(src(r) + k);
    }
}

template <int NB, int NT>
__device__ __forceinline__ void store_phase(uint16_t *lds, const u32x4 v[stage_n<NT>()], int k0,
                                            int d, int nrows)
{
    constexpr int KP = phase_len<NB>(), LR = lds_row<NB>();
#pragma unroll
    for (int i = 0; i < stage_n<NT>(); ++i) {
        const int p = threadIdx.x + NT * i;
        const int r = p / (KP / 8), kk = (p % (KP / 8)) * 8;
        const bool ok = r < nrows && k0 + kk < d;
        *reinterpret_cast<u32x4 *>(lds + r * LR + kk) = ok ? v[i] : u32x4{0u, 0u, 0u, 0u};
    }
}

// MFMA over one 64-wide slice (hidden offset kabs, column koff of the staged
// phase): the slice's loads go through the wave's LDS slice into MFMA order
// (lane l: row l%32, pieces 4*(l/32) .. +3); a slice reaching past d zeroes
// this lane's pieces at k >= d.  One wave's LDS operations execute in order,
// so the wave's slice buffer needs no barrier.
// With NP > 1 the slice multiplies NP staged B buffers, pstride elements
// apart, into the same accumulators (one pass of A through the slice buffer).
// LR: row stride of the staged B rows.
template <int NB, int NP = 1, int LR = lds_row<NB>()>
__device__ __forceinline__ void slice_mma(const u32x4 ld[4], uint16_t *aw, const uint16_t *lds,
                                          int koff, int kabs, int d, f32x16 acc[NB],
                                          int pstride = 0)
{
    const int lane = lane_id();
    const int wr = lane >> 3, wp = lane & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4 *>(aw + (wr + 8 * i) * kKs + ((wp ^ akey(wr + 8 * i)) << 3)) = ld[i];
    const int rr = lane & 31, hh = lane >> 5;
    u32x4 a[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        a[s] = *reinterpret_cast<const u32x4 *>(aw + rr * kKs + (((4 * hh + s) ^ akey(rr)) << 3));
    if (kabs + kKs > d) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            if (kabs + 32 * hh + 8 * s >= d)
                a[s] = u32x4{0u, 0u, 0u, 0u};
    }
    const int kb = koff + 32 * hh;
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const uint16_t *brow = lds + p * pstride + (nb * 32 + rr) * LR + kb;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32x4 b = *reinterpret_cast<const u32x4 *>(brow + 8 * s);
                acc[nb] = mfma(a[s], b, acc[nb]);
            }
        }
}

// acc[nb] = (this wave's 32 W rows) x (NB*32 staged B rows)^T over all d.
// W streams through a register ring of four 64-wide slices (16 KB per wave
// in flight); a phase (phase_len<NB>() hidden elements of B) is staged in
// LDS between two barriers, its loads issued one slice group earlier so the
// switch waits for them and not for the W ring.
// The phases are visited from phase rot % nph on, wrapping around (when d
// fills every phase): rows read at the same moment by different workgroups
// then sit at different column offsets, which spreads consecutive rows (8 KB
// apart) over the memory channels -- without it, consecutive rows read 128
// bytes at a time stream at 4.8 TB/s instead of 5.7.  Only the order of the
// hidden-dimension sums changes, the same for every call.  The union head
// rotates by tile; the gathered head's rows are scattered over the table
// already and start at phase 0.
// The ring's refill after the last group has no slice left to load: `tail`
// >= 0 is the slice index it loads instead, one whose byte offset lies past
// the buffer's range (the loads return zero without touching memory);
// tail < 0 reloads the slices after the last (the next row's first bytes).
constexpr int kTailOob = 1 << 24;  // slice offset 2^31 bytes, past any range < 2^31
template <int NB, int NT, int AUX, class Src>
__device__ __forceinline__ void rows_times_b(rsrc_t w, const uint32_t voff[4], int d,
                                             uint16_t *lds, uint16_t *aw, int nrows, Src src,
                                             f32x16 acc[NB], int rot, int tail)
{
    constexpr int KP = phase_len<NB>(), NS = KP / kKs, GP = NS / 4;  // groups of 4 slices
    const int nsl = (d + kKs - 1) / kKs, nph = (d + KP - 1) / KP;
    const int ph0 = nsl == nph * NS ? rot % nph : 0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        acc[nb] = f32x16{};
    u32x4 hv[stage_n<NT>()];
    load_phase<NB, NT>(hv, ph0 * KP, d, nrows, src);
    __builtin_amdgcn_sched_barrier(0);  // B loads first, as in the loop
    u32x4 r0[4], r1[4], r2[4], r3[4];
    load_a<AUX>(w, voff, (ph0 * NS + 0) * kKs, r0);
    load_a<AUX>(w, voff, (ph0 * NS + 1) * kKs, r1);
    load_a<AUX>(w, voff, (ph0 * NS + 2) * kKs, r2);
    load_a<AUX>(w, voff, (ph0 * NS + 3) * kKs, r3);
    for (int j = 0; j < nph; ++j) {
        const int ph = j + ph0 < nph ? j + ph0 : j + ph0 - nph;
        const int phn = j + 1 + ph0 < nph ? j + 1 + ph0 : j + 1 + ph0 - nph;  // next phase
        __syncthreads();  // every wave is done with the previous phase
        store_phase<NB, NT>(lds, hv, ph * KP, d, nrows);
        __syncthreads();
#pragma unroll
        for (int gi = 0; gi < GP; ++gi) {
            const int ks = ph * NS + 4 * gi;  // first slice of this group
            if (ks >= nsl)
                break;  // only in the last phase
            // first slice of the next group: the next in this phase, else the
            // next phase's first (after the last group: `tail`, whose data
            // goes unused)
            const bool fin = j + 1 == nph && (gi == GP - 1 || ks + 4 >= nsl);
            const int kn = fin && tail >= 0 ? tail
                                            : ((gi < GP - 1 || j + 1 == nph) ? ks + 4 : phn * NS);
            if (gi == GP - 1) {
                load_phase<NB, NT>(hv, phn * KP, d, nrows, src);
                // keep these loads ahead of the ring reloads below: the switch
                // then waits for them alone (loads complete in issue order)
                __builtin_amdgcn_sched_barrier(0);
            }
            slice_mma<NB>(r0, aw, lds, (4 * gi + 0) * kKs, (ks + 0) * kKs, d, acc);
            load_a<AUX>(w, voff, (kn + 0) * kKs, r0);
            slice_mma<NB>(r1, aw, lds, (4 * gi + 1) * kKs, (ks + 1) * kKs, d, acc);
            load_a<AUX>(w, voff, (kn + 1) * kKs, r1);
            slice_mma<NB>(r2, aw, lds, (4 * gi + 2) * kKs, (ks + 2) * kKs, d, acc);
            load_a<AUX>(w, voff, (kn + 2) * kKs, r2);
            slice_mma<NB>(r3, aw, lds, (4 * gi + 3) * kKs, (ks + 3) * kKs, d, acc);
            load_a<AUX>(w, voff, (kn + 3) * kKs, r3);
        }
    }
}

// LDS of the matrix-core heads: the B phase buffer, then the waves' A slices;
// after the K loop the union epilogue reuses the front as its run buffer
template <int NB, int WV>
constexpr int lds_bytes()
{
    return NB * 32 * lds_row<NB>() * 2 + WV * kASlice * 2;
}

// ------------------------------------------------------------------ union
// Tile index (TileIx) of the shortlists, built here from the shortlists
// themselves: shortlists are ascending, so a tile's entries are contiguous
// and the first of them builds the tile's mask from at most 32 following
// entries.  Written only for non-empty groups.  Entries with ids outside
// [0, V) get their NaN logit here.

// OR over the 64 lanes (DPP within rows, then the four row results)
__device__ __forceinline__ uint32_t wave_or(uint32_t v)
{
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);
    return (uint32_t)(__builtin_amdgcn_readlane((int)v, 0) | __builtin_amdgcn_readlane((int)v, 16) |
                      __builtin_amdgcn_readlane((int)v, 32) | __builtin_amdgcn_readlane((int)v, 48));
}

constexpr int kIxLdsGroups = 4095;  // group offsets staged in LDS up to this G

__global__ __launch_bounds__(256) void union_index_kernel(int G, int nt, int V,
                                                          const int64_t *__restrict__ sl_off,
                                                          const int32_t *__restrict__ sl_ids,
                                                          TileIx *__restrict__ tix,
                                                          float *__restrict__ logits)
{
    __shared__ int64_t s_off[kIxLdsGroups + 1];
    const int lane = lane_id();
    const bool lds_off = G <= kIxLdsGroups;
    if (lds_off) {
        for (int i = threadIdx.x; i <= G; i += blockDim.x)
            s_off[i] = sl_off[i];
        __syncthreads();
    }
    const int64_t *off = lds_off ? s_off : sl_off;
    const int64_t beg = off[0], end = off[G];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    // the loop runs the same number of times in every lane of a wave (the
    // mask below combines lanes), so lanes past the end carry an empty key
    for (int64_t J0 = beg + (int64_t)blockIdx.x * blockDim.x + (threadIdx.x & ~(kWave - 1));
         J0 < end; J0 += stride) {
        const int64_t J = J0 + lane;
        const bool in = J < end;
        int g = 0;
        int64_t gbeg = 0, j = 0, len = 0, tc = -1, tp = -1;
        int32_t yJ = -1;
        auto tile = [nt](int32_t y) { return y < 0 ? -1 : min((int64_t)(y >> 5), (int64_t)nt); };
        if (in) {
            int lo = 0, hi = G;  // group: last g with sl_off[g] <= J
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (off[mid] <= J)
                    lo = mid;
                else
                    hi = mid;
            }
            g = lo;
            gbeg = off[g];
            j = J - gbeg;
            len = off[g + 1] - gbeg;
            yJ = sl_ids[J];
            if (yJ < 0 || yJ >= V)
                logits[J] = __builtin_nanf("");
            tc = tile(yJ);
            tp = j > 0 ? tile(sl_ids[J - 1]) : -1;
        }
        // mask of tile tc: OR over the following lanes with the same (group,
        // tile) key -- a contiguous run of lanes, as the shortlist ascends
        const int64_t key = in && tc >= 0 ? (int64_t)g * (nt + 1) + tc : -1 - lane;
        uint32_t m = (in && yJ >= 0 && yJ < V) ? 1u << (yJ & 31) : 0u;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const uint32_t mo = __shfl_down(m, o);
            const int64_t ko = __shfl_down(key, o);
            if (lane + o < kWave && ko == key)
                m |= mo;
        }
        const int64_t last_key = __shfl(key, kWave - 1);  // all lanes, before any branch
        // The run of the last lane's key may continue past this wave (at
        // most 31 more entries of one tile): lanes 0..31 take the next 32
        // entries; the leading ones in the same group and tile add their
        // bits, one OR over the wave.
        uint32_t mx = 0u;
        if (last_key >= 0) {  // wave-uniform
            const int64_t gl = last_key / (nt + 1), tl = last_key % (nt + 1);
            const int64_t gend = off[gl + 1];
            const int64_t JX = J0 + kWave + lane;
            const bool ld = lane < 32 && JX < gend;
            const int32_t yx = ld ? sl_ids[JX] : -1;
            const bool same = ld && tile(yx) == tl;
            const uint64_t bc = __ballot(same);
            const int run = __ffsll((unsigned long long)~bc) - 1;  // leading lanes in the run
            mx = wave_or(lane < run && yx < V ? 1u << (yx & 31) : 0u);
        }
        if (!in)
            continue;
        TileIx *row = tix + (int64_t)g * (nt + 1);
        for (int64_t t = tp + 1; t < tc; ++t)  // tiles without entries
            row[t] = TileIx{(int32_t)j, 0u};
        if (tc > tp) {  // first entry of tile tc
            if (last_key == key)
                m |= mx;
            row[tc] = TileIx{(int32_t)j, m};
        }
        if (j == len - 1)
            for (int64_t t = (tc < 0 ? 0 : tc + 1); t <= nt; ++t)
                row[t] = TileIx{(int32_t)len, 0u};
    }
}

// Union tiles are walked back to back by each workgroup of a persistent
// grid.  A tile's W ring (its first four slices) is issued ahead, by the
// previous tile's last slice group in place of refills that would have no
// slice left to load: the next tile's first W bytes are in flight while
// this tile's epilogue runs, and no tile starts its K loop on a cold ring.
template <int NB, int NT>
struct Ring {
    u32x4 hv[stage_n<NT>()];
    u32x4 r0[4], r1[4], r2[4], r3[4];
};

// the phase the walk of union tile `tile` starts at (rotation by tile)
__device__ __forceinline__ int union_ph0(int tile, int d, int KP)
{
    const int nsl = (d + kKs - 1) / kKs, nph = (d + KP - 1) / KP;
    return nsl == nph * (KP / kKs) ? (tile * kPhaseRot) % nph : 0;
}

// W rows y0 .. y0+tile_rows-1 of a union tile (rows past V read zero; never
// written)
template <int WV>
__device__ __forceinline__ rsrc_t union_rsrc(const uint16_t *W, int V, int d, int tile)
{
    const int64_t y0 = (int64_t)tile * tile_rows<WV>();
    const int64_t rows = min((int64_t)tile_rows<WV>(), (int64_t)V - y0);
    return make_rsrc(W + y0 * d, (uint32_t)(rows * d * 2));
}

// the first B phase (hidden vectors, from L2) and the first four W slices
template <int NB, int NT, class Src>
__device__ __forceinline__ void ring_prime(Ring<NB, NT> &rg, rsrc_t w, const uint32_t voff[4],
                                           int d, int nrows, Src src, int ph0)
{
    constexpr int KP = phase_len<NB>(), NS = KP / kKs;
    load_phase<NB, NT>(rg.hv, ph0 * KP, d, nrows, src);
    __builtin_amdgcn_sched_barrier(0);  // B loads first, as in the loop
    load_a<kNonTemporal>(w, voff, (ph0 * NS + 0) * kKs, rg.r0);
    load_a<kNonTemporal>(w, voff, (ph0 * NS + 1) * kKs, rg.r1);
    load_a<kNonTemporal>(w, voff, (ph0 * NS + 2) * kKs, rg.r2);
    load_a<kNonTemporal>(w, voff, (ph0 * NS + 3) * kKs, rg.r3);
}

// rows_times_b for a primed ring; the last group's refills load the next
// tile's first slices (wn, ph0n) when has_next, else nothing (a slice past
// the buffer range); after the loop, the next tile's first B phase.
template <int NB, int NT, class Src>
__device__ __forceinline__ void union_rows_times_b(Ring<NB, NT> &rg, rsrc_t w, rsrc_t wn,
                                                   const uint32_t voff[4], int d, uint16_t *lds,
                                                   uint16_t *aw, int nrows, Src src,
                                                   f32x16 acc[NB], int ph0, int ph0n,
                                                   bool has_next)
{
    constexpr int KP = phase_len<NB>(), NS = KP / kKs, GP = NS / 4;
    const int nsl = (d + kKs - 1) / kKs, nph = (d + KP - 1) / KP;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        acc[nb] = f32x16{};
    for (int j = 0; j < nph; ++j) {
        const int ph = j + ph0 < nph ? j + ph0 : j + ph0 - nph;
        const int phn = j + 1 + ph0 < nph ? j + 1 + ph0 : j + 1 + ph0 - nph;
        __syncthreads();  // every wave is done with the previous phase (or tile)
        store_phase<NB, NT>(lds, rg.hv, ph * KP, d, nrows);
        __syncthreads();
#pragma unroll
        for (int gi = 0; gi < GP; ++gi) {
            const int ks = ph * NS + 4 * gi;
            if (ks >= nsl)
                break;  // only in the last phase
            const bool fin = j + 1 == nph && (gi == GP - 1 || ks + 4 >= nsl);
            const int kn = fin ? (has_next ? ph0n * NS : kTailOob)
                               : (gi < GP - 1 ? ks + 4 : phn * NS);
            const rsrc_t wr = fin && has_next ? wn : w;
            if (gi == GP - 1 && j + 1 < nph) {
                load_phase<NB, NT>(rg.hv, phn * KP, d, nrows, src);
                __builtin_amdgcn_sched_barrier(0);
            }
            slice_mma<NB>(rg.r0, aw, lds, (4 * gi + 0) * kKs, (ks + 0) * kKs, d, acc);
            load_a<kNonTemporal>(wr, voff, (kn + 0) * kKs, rg.r0);
            slice_mma<NB>(rg.r1, aw, lds, (4 * gi + 1) * kKs, (ks + 1) * kKs, d, acc);
            load_a<kNonTemporal>(wr, voff, (kn + 1) * kKs, rg.r1);
            slice_mma<NB>(rg.r2, aw, lds, (4 * gi + 2) * kKs, (ks + 2) * kKs, d, acc);
            load_a<kNonTemporal>(wr, voff, (kn + 2) * kKs, rg.r2);
            slice_mma<NB>(rg.r3, aw, lds, (4 * gi + 3) * kKs, (ks + 3) * kKs, d, acc);
            load_a<kNonTemporal>(wr, voff, (kn + 3) * kKs, rg.r3);
        }
    }
    if (has_next)
        load_phase<NB, NT>(rg.hv, ph0n * KP, d, nrows, src);
}

// does any shortlist of the column pass touch union tile `tile`?  (every
// thread; barriers inside)
template <int WV>
__device__ __forceinline__ bool union_tile_any(int G, int g0, int ng,
                                               const int64_t *__restrict__ sl_off,
                                               const TileIx *__restrict__ tix, int nt, int tile,
                                               int *s_any)
{
    const int64_t y0 = (int64_t)tile * tile_rows<WV>();
    __syncthreads();  // the previous reader of *s_any is done
    if (threadIdx.x == 0)
        *s_any = 0;
    __syncthreads();
    for (int q = threadIdx.x; q < ng * WV; q += blockDim.x) {
        const int g = g0 + q / WV, t = (int)(y0 >> 5) + q % WV;
        if (t < nt && sl_off[g + 1] > sl_off[g] && tix[(int64_t)g * (nt + 1) + t].mask != 0u)
            *s_any = 1;
    }
    __syncthreads();
    return *s_any != 0;
}

// one 32*WV-row tile of W (tile index `tile`, ring primed) against the
// column pass; primes the ring for `next` when has_next
template <int NB, int WV>
__device__ __forceinline__ void union_tile(int V, int d, const uint16_t *__restrict__ W, int G,
                                           int g0, const uint16_t *__restrict__ h, int64_t ldh_g,
                                           const int64_t *__restrict__ sl_off,
                                           const TileIx *__restrict__ tix, int nt,
                                           float *__restrict__ logits, int tile, int next,
                                           bool has_next, Ring<NB, 64 * WV> &rg,
                                           uint16_t *lds_all)
{
    constexpr int kTileRows = tile_rows<WV>();
    uint16_t *lds = lds_all, *lds_a = lds_all + NB * 32 * lds_row<NB>();
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int ng = min(NB * 32, G - g0);  // groups of this column pass
    const int64_t y0 = (int64_t)tile * kTileRows;
    const int t32 = (int)(y0 >> 5) + wave;  // this wave's 32-token tile

    // where this lane's groups put the tile's logits, fetched before the
    // K loop (lane l, column block nb: group g0 + 32*nb + l%32); wave 0
    // records where each group's run for the block's WV tiles begins
    __shared__ int64_t s_dst[NB * 32];
    __shared__ int32_t s_s0[NB * 32], s_cnt[NB * 32];
    int64_t o_off[NB];
    TileIx o_ix[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int gl = nb * 32 + (lane & 31);
        o_off[nb] = 0;
        o_ix[nb] = TileIx{0, 0u};
        if (gl < ng && t32 < nt) {
            const int g = g0 + gl;
            const int64_t off = sl_off[g], len = sl_off[g + 1] - off;
            if (len > 0) {
                o_off[nb] = off;
                o_ix[nb] = tix[(int64_t)g * (nt + 1) + t32];
                const int64_t a0 = o_ix[nb].start;  // entries a0 .. a0+popc(mask)-1 < len
                if (a0 < 0 || a0 + __popc(o_ix[nb].mask) > len)
                    o_ix[nb].mask = 0u;
            }
        }
        if (wave == 0 && lane < 32) {
            s_dst[gl] = o_off[nb] + o_ix[nb].start;
            s_s0[gl] = o_ix[nb].start;
            s_cnt[gl] = 0;
        }
    }

    uint32_t voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        voff[i] = (uint32_t)((32 * wave + (lane >> 3) + 8 * i) * d * 2 + 16 * (lane & 7));
    f32x16 acc[NB];
    auto hsrc = [&](int r) { return h + (int64_t)(g0 + r) * ldh_g; };
    // the ranges are at most 256 rows x 16 KB: the tail slice reads nothing
    union_rows_times_b<NB, 64 * WV>(rg, union_rsrc<WV>(W, V, d, tile),
                                    union_rsrc<WV>(W, V, d, has_next ? next : tile), voff, d, lds,
                                    lds_a + wave * kASlice, ng, hsrc, acc,
                                    union_ph0(tile, d, phase_len<NB>()),
                                    union_ph0(next, d, phase_len<NB>()), has_next);

    // epilogue: the (row, group) pairs on the group's shortlist.  A group's
    // entries for the block's WV tiles are one contiguous run of its logits;
    // the values are gathered per group in LDS (the phase and A buffers,
    // free after the K loop) and each run is written with coalesced stores.
    float *res = reinterpret_cast<float *>(lds_all);  // [NB*32][kTileRows]
    static_assert(lds_bytes<NB, WV>() >= NB * 32 * kTileRows * (int)sizeof(float),
                  "LDS run buffer");
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int gl = nb * 32 + (lane & 31);
        uint32_t mask = o_ix[nb].mask;
        const int base = o_ix[nb].start - s_s0[gl];  // entries of earlier tiles of the block
        if (base < 0 || base + __popc(mask) > kTileRows)
            mask = 0u;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int mrow = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if ((mask >> mrow) & 1u)
                res[gl * kTileRows + base + __popc(mask & ((1u << mrow) - 1u))] = acc[nb][r];
        }
        if (mask != 0u && lane < 32)
            atomicMax(&s_cnt[gl], base + __popc(mask));
    }
    __syncthreads();
    for (int q = threadIdx.x; q < ng * kTileRows; q += blockDim.x) {
        const int gl = q / kTileRows, k = q % kTileRows;
        if (k < s_cnt[gl])
            logits[s_dst[gl] + k] = res[q];
    }
}

template <int NB, int WV>
__global__ __launch_bounds__(64 * WV) void head_union_kernel(int V, int d, const uint16_t *__restrict__ W,
                                                         int G, int g0, const uint16_t *__restrict__ h,
                                                         int64_t ldh_g, const int64_t *__restrict__ sl_off,
                                                         const TileIx *__restrict__ tix, int nt,
                                                         float *__restrict__ logits, int ntiles)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds_all[lds_bytes<NB, WV>() / 2];
    __shared__ int s_any;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int ng = min(NB * 32, G - g0);
    uint32_t voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        voff[i] = (uint32_t)((32 * wave + (lane >> 3) + 8 * i) * d * 2 + 16 * (lane & 7));
    Ring<NB, 64 * WV> rg;
    int tile = blockIdx.x;
    if (tile >= ntiles)
        return;
    // tiles no shortlist touches are skipped (and never primed).  CROSS:
    // the ring for the next tile is primed by this one (measured: the
    // 64-group Gemma-shaped head 348 -> 344 us; the 32-group Llama-shaped
    // head, 4-wave tiles with less register room, 179 -> 181 us without
    // its B phase primed, so it primes per tile)
    constexpr bool CROSS = NB == 2;
    auto hsrc = [&](int r) { return h + (int64_t)(g0 + r) * ldh_g; };
    if constexpr (!CROSS) {  // each tile primes its own ring
        for (; tile < ntiles; tile += gridDim.x)
            if (union_tile_any<WV>(G, g0, ng, sl_off, tix, nt, tile, &s_any)) {
                ring_prime<NB, 64 * WV>(rg, union_rsrc<WV>(W, V, d, tile), voff, d, ng, hsrc,
                                        union_ph0(tile, d, phase_len<NB>()));
                union_tile<NB, WV>(V, d, W, G, g0, h, ldh_g, sl_off, tix, nt, logits, tile, tile,
                                   false, rg, lds_all);
                __syncthreads();  // the tile's epilogue is done with the shared buffers
            }
        return;
    }
    bool any = union_tile_any<WV>(G, g0, ng, sl_off, tix, nt, tile, &s_any);
    if (any)
        ring_prime<NB, 64 * WV>(rg, union_rsrc<WV>(W, V, d, tile), voff, d, ng, hsrc,
                                union_ph0(tile, d, phase_len<NB>()));
    while (tile < ntiles) {
        const int next = tile + (int)gridDim.x;
        const bool any_next =
            next < ntiles && union_tile_any<WV>(G, g0, ng, sl_off, tix, nt, next, &s_any);
        if (any) {
            union_tile<NB, WV>(V, d, W, G, g0, h, ldh_g, sl_off, tix, nt, logits, tile, next,
                               any_next, rg, lds_all);
            __syncthreads();  // the tile's epilogue is done with the shared buffers
        } else if (any_next) {
            ring_prime<NB, 64 * WV>(rg, union_rsrc<WV>(W, V, d, next), voff, d, ng, hsrc,
                                    union_ph0(next, d, phase_len<NB>()));
        }
        tile = next;
        any = any_next;
    }
}

// --------------------------------------------------------------- gathered
// one 32*WV-entry tile of group g's shortlist against head rows n0..n0+mm-1
template <int NB, int WV>
__device__ __forceinline__ void gathered_tile(rsrc_t w, int V, int d, int m, int n0, int mm,
                                              const uint16_t *__restrict__ h, int64_t ldh_g,
                                              const int64_t *__restrict__ sl_off,
                                              const int32_t *__restrict__ sl_ids,
                                              float *__restrict__ logits, uint16_t *lds,
                                              uint16_t *lds_a, int g, int64_t tile)
{
    constexpr int kTileRows = tile_rows<WV>();
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t off = sl_off[g], len = sl_off[g + 1] - off;
    const uint16_t *hg = h + (int64_t)g * ldh_g + (int64_t)n0 * d;
    auto hsrc = [&](int r) { return hg + (int64_t)r * d; };
    const int64_t e = tile * kTileRows + 32 * wave + (lane & 31);
    const bool evalid = e < len;
    int32_t id = evalid ? sl_ids[off + e] : 0;
    const bool valid = evalid && id >= 0 && id < V;  // else row 0, result not used
    const int yrow = valid ? id : 0;
    uint32_t voff[4];  // load i of lane l reads the row of the wave's entry l/8 + 8i
#pragma unroll
    for (int i = 0; i < 4; ++i)
        voff[i] = (uint32_t)__shfl(yrow, (lane >> 3) + 8 * i) * (uint32_t)d * 2u +
                  16u * (lane & 7);
    f32x16 acc[NB];
    // the range is all of W: the tail slice reads nothing when offsets below
    // 2^31 cover it (voff + 2^31 stays below 2^32)
    const int tail = (int64_t)V * d * 2 <= (1ll << 31) ? kTailOob : -1;
    rows_times_b<NB, 64 * WV, kCached>(w, voff, d, lds, lds_a + wave * kASlice, mm, hsrc, acc, 0,
                                       tail);
    // epilogue: column = head row (node), row = shortlist entry; the entry
    // of accumulator row i was loaded by lanes i and i + 32
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int nl = nb * 32 + (lane & 31);
        float *out = logits + (int64_t)m * off + (int64_t)(n0 + nl) * len;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int64_t ent = tile * kTileRows + 32 * wave + i;
            const bool ok = __shfl(valid ? 1 : 0, i) != 0;
            if (nl < mm && ent < len)
                out[ent] = ok ? acc[nb][r] : __builtin_nanf("");
        }
    }
}

// The tiles of all groups form one list that the persistent grid strides
// over.  Shortlists of one launch differ in length (a token budget
// overshoots by up to one cluster: 24.6K to 51K entries on the Qwen-shaped
// 8-tree workload), so a fixed number of workgroups per group would leave
// the longest group's workgroups running alone.
//   up to kTreeMixGroups groups and kTreeMergeTiles tiles: merged by token
//     id (the tiles of all groups ordered by the id of their first entry,
//     ties to the lower group; each shortlist ascends, so this merges G
//     sorted lists), the list cut into 8 slices of consecutive tiles, and
//     slice x walked by the workgroups of XCD x.  Groups' shortlists
//     overlap (the 8-tree workload's rows sit on 2.0 shortlists on average):
//     a row that several groups share falls in one slice, and the tiles
//     that read it run at about the same time on one XCD, so it is fetched
//     from HBM once and then read from that XCD's L2.  Every workgroup
//     rebuilds the order in LDS (each tile's rank: its index in its group
//     plus binary searches in the other groups' first ids).
//   else up to kTreeMixGroups groups: tile-index-major (tile t of every
//     group that has one, in group order, then tile t+1): the groups walk
//     their shortlists side by side.  Every workgroup rebuilds in LDS the
//     tile counts and C(t) = the number of tiles before index t.
//   up to kTreeLdsGroups groups: group-major (tile t of group g is entry
//     tpre[g] + t, tpre = exclusive prefix of the tile counts, in LDS).
//   above: each group keeps tiles_stride workgroups of its own.
// Measured on the 8-tree workload (mean over four input instances): a fixed
// share of workgroups per group 436 us, group-major 424 us, tile-index-major
// 373 us (338 us later); merged with XCD slices 301 us and 1.17 GB fetched
// per launch against 1.93 GB (the same merged order dealt round-robin over
// the XCDs: 349 us, 2.02 GB).
constexpr int kTreeMixGroups = 64;
constexpr int kTreeMixTiles = 4096;  // tile indices covered by C in LDS
constexpr int kTreeLdsGroups = 4096;
constexpr int kTreeMergeTiles = 4096;  // tiles of all groups in the merged order

template <int NB, int WV>
__global__ __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(2))) void head_gathered_kernel(int V, int d, const uint16_t *__restrict__ W,
                                                            int G, int m, int n0,
                                                            const uint16_t *__restrict__ h,
                                                            int64_t ldh_g,
                                                            const int64_t *__restrict__ sl_off,
                                                            const int32_t *__restrict__ sl_ids,
                                                            int tiles_stride,
                                                            float *__restrict__ logits)
{
    constexpr int kTileRows = tile_rows<WV>();
    constexpr int NT = 64 * WV;
    __shared__ __attribute__((aligned(16))) uint16_t lds_all[lds_bytes<NB, WV>() / 2];
    __shared__ int32_t s_tpre[kTreeLdsGroups + 1 > kTreeMixTiles + 1 + kTreeMixGroups
                                  ? kTreeLdsGroups + 1
                                  : kTreeMixTiles + 1 + kTreeMixGroups];
    __shared__ int64_t s_scan[kWave + 1];
    uint16_t *lds = lds_all, *lds_a = lds_all + NB * 32 * lds_row<NB>();
    const int mm = min(m - n0, NB * 32);  // head rows n0 .. n0+mm-1 in this pass
    const rsrc_t w = make_rsrc(W, (uint32_t)((int64_t)V * d * 2));  // V*d*2 < 4 GiB
    if (G <= kTreeMixGroups) {  // block-uniform: the merged order when it applies
        __shared__ int32_t s_mpre[kTreeMixGroups + 1];  // exclusive prefix of tile counts
        __shared__ int32_t s_f[kTreeMergeTiles];        // first token id of every tile
        if (threadIdx.x == 0) {
            int32_t run = 0;
            for (int g = 0; g < G; ++g) {
                s_mpre[g] = run;
                const int64_t len = sl_off[g + 1] - sl_off[g];
                const int64_t c = len > 0 ? (len + kTileRows - 1) / kTileRows : 0;
                run = (int32_t)min((int64_t)run + c, (int64_t)kTreeMergeTiles + 1);
            }
            s_mpre[G] = run;
        }
        __syncthreads();
        const int total = s_mpre[G];
        if (total <= kTreeMergeTiles) {
            auto group_of = [&](int i) {  // group of tile i: last g with s_mpre[g] <= i
                int lo = 0, hi = G;
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (s_mpre[mid] <= i)
                        lo = mid;
                    else
                        hi = mid;
                }
                return lo;
            };
            for (int i = threadIdx.x; i < total; i += NT) {
                const int g = group_of(i);
                s_f[i] = sl_ids[sl_off[g] + (int64_t)(i - s_mpre[g]) * kTileRows];
            }
            __syncthreads();
            // the merge needs each group's first ids strictly increasing (a
            // shortlist in ascending token order); else the tile-index order
            int bad = 0;
            for (int i = threadIdx.x; i < total; i += NT) {
                const int g = group_of(i);
                bad |= i > s_mpre[g] && s_f[i - 1] >= s_f[i];
            }
            if (!__syncthreads_or(bad)) {
                // rank of tile (g, t): t plus, for every other group h, its
                // tiles with a smaller first id (ties: lower group first)
                int32_t *s_ord = s_tpre;
                for (int i = threadIdx.x; i < total; i += NT) {
                    const int g = group_of(i);
                    const int32_t f = s_f[i];
                    int rank = i - s_mpre[g];
                    for (int hg = 0; hg < G; ++hg) {
                        if (hg == g)
                            continue;
                        int lo = s_mpre[hg], hi = s_mpre[hg + 1];
                        while (lo < hi) {
                            const int mid = (lo + hi) >> 1;
                            const int32_t fm = s_f[mid];
                            if (fm < f || (hg < g && fm == f))
                                lo = mid + 1;
                            else
                                hi = mid;
                        }
                        rank += lo - s_mpre[hg];
                    }
                    s_ord[rank] = i;
                }
                __syncthreads();
                // XCD x (blocks b with b % 8 == x, dealt round-robin) walks
                // slice x of the merged list: the groups' tiles over one
                // eighth of the token ids, so a row that several groups
                // share is fetched once into that XCD's L2
                const int b = blockIdx.x, nb = gridDim.x;
                int64_t k0 = b, k1 = total, ks = nb;
                if (nb % 8 == 0) {
                    const int x = b % 8;
                    k0 = (int64_t)x * total / 8 + b / 8;
                    k1 = (int64_t)(x + 1) * total / 8;
                    ks = nb / 8;
                }
                for (int64_t k = k0; k < k1; k += ks) {
                    const int i = s_ord[k], g = group_of(i);
                    gathered_tile<NB, WV>(w, V, d, m, n0, mm, h, ldh_g, sl_off, sl_ids, logits,
                                          lds, lds_a, g, i - s_mpre[g]);
                }
                return;
            }
        }
    }
    if (G <= kTreeMixGroups) {  // block-uniform; s_tpre holds C(t), then the tile counts
        int32_t *s_cnt = s_tpre + kTreeMixTiles + 1;
        __shared__ int s_tmax;
        if (threadIdx.x == 0)
            s_tmax = 0;
        __syncthreads();
        for (int g = threadIdx.x; g < G; g += NT) {
            const int64_t len = sl_off[g + 1] - sl_off[g];
            const int64_t c = len > 0 ? (len + kTileRows - 1) / kTileRows : 0;
            s_cnt[g] = (int32_t)min(c, (int64_t)kTreeMixTiles);
            atomicMax(&s_tmax, s_cnt[g]);
        }
        __syncthreads();
        const int tmax = s_tmax;  // tiles of the longest group (capped: see below)
        constexpr int PER = (kTreeMixTiles + NT) / NT;  // tile indices per thread
        int64_t sum = 0;
        int32_t act[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int t = threadIdx.x * PER + i;
            int a = 0;
            if (t < tmax)
                for (int g = 0; g < G; ++g)
                    a += s_cnt[g] > t;
            act[i] = a;
            sum += a;
        }
        int64_t total;
        int64_t run = block_excl_scan_i64(sum, s_scan, &total);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int t = threadIdx.x * PER + i;
            if (t <= tmax)
                s_tpre[t] = (int32_t)run;
            run += act[i];
        }
        __syncthreads();
        for (int64_t gt = blockIdx.x; gt < total; gt += gridDim.x) {
            int lo = 0, hi = tmax;  // tile index: last t with C(t) <= gt
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_tpre[mid] <= gt)
                    lo = mid;
                else
                    hi = mid;
            }
            int r = (int)(gt - s_tpre[lo]), g = 0;  // the r-th group with a tile lo
            for (;; ++g)
                if (s_cnt[g] > lo && r-- == 0)
                    break;
            gathered_tile<NB, WV>(w, V, d, m, n0, mm, h, ldh_g, sl_off, sl_ids, logits, lds, lds_a,
                                  g, lo);
        }
        // groups longer than kTreeMixTiles tiles: the rest of their tiles,
        // one group at a time (only for shortlists of over a million entries)
        for (int g = 0; g < G; ++g) {
            const int64_t len = sl_off[g + 1] - sl_off[g];
            for (int64_t tile = kTreeMixTiles + blockIdx.x; tile * kTileRows < len;
                 tile += gridDim.x)
                gathered_tile<NB, WV>(w, V, d, m, n0, mm, h, ldh_g, sl_off, sl_ids, logits, lds,
                                      lds_a, g, tile);
        }
        return;
    }
    if (G <= kTreeLdsGroups) {  // block-uniform
        constexpr int PER = (kTreeLdsGroups + NT) / NT;  // groups per thread (G + 1 slots)
        int64_t cnt[PER], sum = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int g = threadIdx.x * PER + i;
            const int64_t len = g < G ? sl_off[g + 1] - sl_off[g] : 0;
            cnt[i] = len > 0 ? (len + kTileRows - 1) / kTileRows : 0;
            sum += cnt[i];
        }
        int64_t total;
        int64_t run = block_excl_scan_i64(sum, s_scan, &total);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int g = threadIdx.x * PER + i;
            if (g <= G)
                s_tpre[g] = (int32_t)run;
            run += cnt[i];
        }
        __syncthreads();
        for (int64_t gt = blockIdx.x; gt < total; gt += gridDim.x) {
            int lo = 0, hi = G;  // group: last g with s_tpre[g] <= gt
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_tpre[mid] <= gt)
                    lo = mid;
                else
                    hi = mid;
            }
            gathered_tile<NB, WV>(w, V, d, m, n0, mm, h, ldh_g, sl_off, sl_ids, logits, lds, lds_a,
                                  lo, gt - s_tpre[lo]);
        }
        return;
    }
    const int g = blockIdx.x % G;  // neighbouring workgroups: same tile, other groups
    const int64_t len = sl_off[g + 1] - sl_off[g];
    for (int64_t tile = blockIdx.x / G; tile * kTileRows < len; tile += tiles_stride)
        gathered_tile<NB, WV>(w, V, d, m, n0, mm, h, ldh_g, sl_off, sl_ids, logits, lds, lds_a, g,
                              tile);
}

// ------------------------------------------------------- router, layer 1
// The router's first layer for a batch of n >= 8 bf16 inputs is a dense
// n x r x d contraction (32 x 1024 x 4096 at the Llama shape: 8 MB of
// weights, 268 MFLOP): split over k into windows of kRouterWin elements so
// that about a hundred workgroups stream the weights at once.  A workgroup
// takes 128 weight rows (4 waves x 32) of one window and up to 64 inputs
// (columns): every W load of the window is issued at once, the inputs'
// window is staged in LDS, and the slices go through the waves' LDS slices
// into MFMA order as in the heads.  part[w][c][i] holds window w's sum for
// input c0 + c of the current column pass and weight row i;
// router_l1_finish adds the windows in order.  Passes run in stream order
// and reuse part.
constexpr int kRouterWin = 256;  // k-window (4 slices)
constexpr int kRouterCols = kRouterPassCols;  // inputs per column pass
constexpr int kRouterMaxWin = 8192 / kRouterWin;  // d <= 8192

// part[c][row0 + i] = this workgroup's sums for input c and weight row i
// (i < rows, c < ncols).  Register q of lane l holds weight row 8*(q/4) +
// 4*(l/32) + q%4 of the wave's 32 and input (l%32) + 32*nb; the tile passes
// through the wave's share of `buf` (NB*32 x 33 floats) so that each input's
// 32 rows go out as one 128-byte store.
template <int NB>
__device__ __forceinline__ void store_part(const f32x16 acc[NB], float *buf, float *part, int ld,
                                           int row0, int rows, int ncols)
{
    constexpr int LB = 33;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    float *wb = buf + wave * NB * 32 * LB;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 16; ++q)
            wb[(nb * 32 + (lane & 31)) * LB + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)] =
                acc[nb][q];
    // one wave's LDS operations complete in order: no barrier before reading
    const int i = lane & 31, row = 32 * wave + i;
#pragma unroll
    for (int cc = 0; cc < NB * 16; ++cc) {
        const int c = 2 * cc + (lane >> 5);
        if (c < ncols && row < rows)
            part[(int64_t)c * ld + row0 + row] = wb[c * LB + i];
    }
}

template <int NB>
__global__ __launch_bounds__(256) void router_l1_kernel(int n, int d, int r,
                                                        const uint16_t *__restrict__ W1,
                                                        const uint16_t *__restrict__ h,
                                                        int64_t ldh, int c0,
                                                        float *__restrict__ part)
{
    static_assert(phase_len<NB>() >= kRouterWin, "the window is one staged phase");
    __shared__ __attribute__((aligned(16))) uint16_t lds[NB * 32 * lds_row<NB>()];
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[4 * kASlice];
    static_assert(sizeof(lds) >= 4 * NB * 32 * 33 * sizeof(float), "partial tile buffer");
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int row0 = blockIdx.x * 128, win = blockIdx.y;
    const int k0 = win * kRouterWin, klen = min(kRouterWin, d - k0);
    const int rows = min(128, r - row0), ncols = min(kRouterCols, n - c0);
    const int nsl = (klen + kKs - 1) / kKs;
    // rows past the tile read zero (the range ends with the last row's window)
    const rsrc_t w = make_rsrc(W1 + (int64_t)row0 * d + k0,
                               (uint32_t)((rows - 1) * d * 2 + klen * 2));
    uint32_t voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        voff[i] = (uint32_t)((32 * wave + (lane >> 3) + 8 * i) * d * 2 + 16 * (lane & 7));
    u32x4 ld[4][4];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
        if (sl < nsl)
            load_a<kNonTemporal>(w, voff, sl * kKs, ld[sl]);
    const uint16_t *hb = h + (int64_t)c0 * ldh + k0;
    auto hsrc = [&](int c) { return hb + (int64_t)c * ldh; };
    u32x4 hv[stage_n<256>()];
    load_phase<NB, 256>(hv, 0, klen, ncols, hsrc);
    store_phase<NB, 256>(lds, hv, 0, klen, ncols);
    __syncthreads();
    f32x16 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        acc[nb] = f32x16{};
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
        if (sl < nsl)
            slice_mma<NB>(ld[sl], lds_a + wave * kASlice, lds, sl * kKs, sl * kKs, klen, acc);
    __syncthreads();  // every wave is done with the staged inputs
    store_part<NB>(acc, reinterpret_cast<float *>(lds), part + (int64_t)win * kRouterCols * r, r,
                   row0, rows, ncols);
}

// z[c0 + c][i] = act(sum over windows w in order of part[w][c][i] + b1[i])
__global__ __launch_bounds__(256) void router_l1_finish(int r, int nwin, int c0, int ncols,
                                                        const float *__restrict__ part,
                                                        const uint16_t *__restrict__ b1, int act,
                                                        float *__restrict__ z)
{
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= (int64_t)ncols * r)
        return;
    // windows in order; eight loads in flight at a time
    float s = 0.f;
    for (int w0 = 0; w0 < nwin; w0 += 8) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = w0 + i < nwin ? part[(int64_t)(w0 + i) * kRouterCols * r + q] : 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (w0 + i < nwin)
                s += v[i];
    }
    if (b1)
        s += __uint_as_float((uint32_t)b1[q % r] << 16);
    if (act == DS_RELU)
        s = fmaxf(s, 0.f);
    else if (act == DS_SILU)
        s = s / (1.f + expf(-s));
    z[(int64_t)c0 * r + q] = s;
}

// ------------------------------------------------------- router, layer 2
// scores = W2 z + b2 for the same batches, z fp32.  Each z value splits
// exactly into three bf16 pieces: hi = bf16(z), mid = bf16(z - hi), lo =
// z - hi - mid (both differences are exact in fp32 and lo has at most 8
// significant bits), so W2 z = W2 hi + W2 mid + W2 lo is a bf16 contraction
// with exact products, accumulated in fp32 as in the first layer.  A
// workgroup takes 128 rows of W2 and one k-window of NSW slices, stages the
// three pieces of the window for up to 64 inputs in LDS and multiplies each
// W2 slice with all three; part[w][c][o] as in the first layer, summed by
// router_l1_finish (no activation).
__device__ __forceinline__ uint32_t bf16_rne_bits(float x)
{
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // finite x
}

__device__ __forceinline__ void split3(float z, uint32_t &hi, uint32_t &mid, uint32_t &lo)
{
    hi = bf16_rne_bits(z);
    const float r1 = z - __uint_as_float(hi << 16);
    mid = bf16_rne_bits(r1);
    const float r2 = r1 - __uint_as_float(mid << 16);
    lo = bf16_rne_bits(r2);  // exact: r2 has at most 8 significant bits
}

template <int NB, int NSW>
__global__ __launch_bounds__(256) void router_l2_kernel(int n, int r, int M,
                                                        const uint16_t *__restrict__ W2,
                                                        const float *__restrict__ z, int c0,
                                                        float *__restrict__ part)
{
    constexpr int KW = NSW * kKs, LR = KW + 8, PS = NB * 32 * LR;  // piece stride
    constexpr int LDS_U16 = 3 * PS > 4 * NB * 32 * 33 * 2 ? 3 * PS : 4 * NB * 32 * 33 * 2;
    __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_U16];
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[4 * kASlice];
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int row0 = blockIdx.x * 128, win = blockIdx.y;
    const int k0 = win * KW, klen = min(KW, r - k0);
    const int rows = min(128, M - row0), ncols = min(kRouterCols, n - c0);
    const rsrc_t w = make_rsrc(W2 + (int64_t)row0 * r + k0,
                               (uint32_t)((rows - 1) * r * 2 + klen * 2));
    uint32_t voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        voff[i] = (uint32_t)((32 * wave + (lane >> 3) + 8 * i) * r * 2 + 16 * (lane & 7));
    u32x4 ld[NSW][4];
#pragma unroll
    for (int sl = 0; sl < NSW; ++sl)
        load_a<kNonTemporal>(w, voff, sl * kKs, ld[sl]);
    // the window's inputs, 4 values per thread and step (r % 8 == 0: whole
    // float4s); columns past ncols and k past klen stage zeros
    constexpr int Q = KW / 4;  // float4s per input row
#pragma unroll
    for (int it = 0; it < NB * 32 * Q / 256; ++it) {
        const int p = threadIdx.x + 256 * it;
        const int c = p / Q, kk = (p % Q) * 4;
        float4 v = {0.f, 0.f, 0.f, 0.f};
        if (c < ncols && kk < klen)
            v = *reinterpret_cast<const float4 *>(z + (int64_t)(c0 + c) * r + k0 + kk);
        uint32_t h0, m0, l0, h1, m1, l1, h2, m2, l2, h3, m3, l3;
        split3(v.x, h0, m0, l0);
        split3(v.y, h1, m1, l1);
        split3(v.z, h2, m2, l2);
        split3(v.w, h3, m3, l3);
        uint16_t *dst = lds + c * LR + kk;
        *reinterpret_cast<uint2 *>(dst) = uint2{h0 | (h1 << 16), h2 | (h3 << 16)};
        *reinterpret_cast<uint2 *>(dst + PS) = uint2{m0 | (m1 << 16), m2 | (m3 << 16)};
        *reinterpret_cast<uint2 *>(dst + 2 * PS) = uint2{l0 | (l1 << 16), l2 | (l3 << 16)};
    }
    __syncthreads();
    f32x16 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        acc[nb] = f32x16{};
#pragma unroll
    for (int sl = 0; sl < NSW; ++sl)
        slice_mma<NB, 3, LR>(ld[sl], lds_a + wave * kASlice, lds, sl * kKs, sl * kKs, klen, acc,
                             PS);
    __syncthreads();
    store_part<NB>(acc, reinterpret_cast<float *>(lds), part + (int64_t)win * kRouterCols * M, M,
                   row0, rows, ncols);
}

}  // namespace

size_t tile_index_bytes(int G, int V)
{
    const int64_t nt = ((int64_t)V + 31) / 32;
    return (size_t)G * (size_t)(nt + 1) * sizeof(TileIx);
}

size_t head_ws_bytes(int G, int m, int V)
{
    if (G < kUnionMinGroups || m != 1)
        return 0;
    return tile_index_bytes(G, V) + 256;
}

bool head_mfma_applies(bool bf16, int V, int d, int G, int m)
{
    if (!bf16)
        return false;
    if (m == 1)
        return G >= kUnionMinGroups;
    // gathered rows are addressed by 32-bit byte offsets into the whole of W
    return m >= kGatheredMinRows && (int64_t)V * d * 2 + 4096 <= (int64_t)UINT32_MAX;
}

namespace {

// Persistent grid over ntiles tiles with at most `slots` workgroups resident:
// every workgroup takes the same number of tiles (give or take one), so no
// partial round of workgroups trails the launch (32 groups, Llama shape:
// 1002 tiles on 501 workgroups, 186.5 us against 204.7 us with one
// workgroup per tile).
inline int balanced_grid(int ntiles, int slots)
{
    if (slots < 1)
        slots = 1;
    const int per = (ntiles + slots - 1) / slots;
    return (ntiles + per - 1) / per;
}

// Column passes of up to 64 groups.  Passes over 33..64 groups run 256-row
// tiles (8 waves; measured 444 vs 471 us at 64 groups on the Gemma shape),
// passes over up to 32 groups 128-row tiles, two workgroups per compute unit
// (208 vs 274 us at 32 groups on the Llama shape).
hipError_t union_passes(hipStream_t s, int V, int d, const uint16_t *Wb, int G, const uint16_t *hb,
                        int64_t ldh_g, const int64_t *sl_off, const TileIx *tix, int nt,
                        float *logits, hipEvent_t t0, hipEvent_t t1)
{
    const int cus = device_cu_count();
    for (int g0 = 0; g0 < G; g0 += 64) {
        hipEvent_t start = g0 == 0 ? t0 : nullptr, stop = g0 + 64 >= G ? t1 : nullptr;
        hipError_t e;
        if (G - g0 > 32) {
            const int nti = (V + tile_rows<8>() - 1) / tile_rows<8>();
            e = launch_timed(head_union_kernel<2, 8>, dim3(balanced_grid(nti, cus)), dim3(512), s,
                             start, stop, V, d, Wb, G, g0, hb, ldh_g, sl_off, tix, nt, logits,
                             nti);
        } else {
            const int nti = (V + tile_rows<4>() - 1) / tile_rows<4>();
            e = launch_timed(head_union_kernel<1, 4>, dim3(balanced_grid(nti, 2 * cus)), dim3(256),
                             s, start, stop, V, d, Wb, G, g0, hb, ldh_g, sl_off, tix, nt, logits,
                             nti);
        }
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// gathered: persistent grid (one 8-wave or two 4-wave workgroups per compute
// unit) over the tiles of all groups
template <int WV>
hipError_t gathered_passes(hipStream_t s, int V, int d, const uint16_t *Wb, int G, int m,
                           const uint16_t *hb, int64_t ldh_g, const int64_t *sl_off,
                           const int32_t *sl_ids, int64_t max_rows, float *logits, hipEvent_t t0,
                           hipEvent_t t1)
{
    const int64_t slots = (8 / WV) * (int64_t)device_cu_count();
    int64_t per_group = (max_rows + tile_rows<WV>() - 1) / tile_rows<WV>();
    int64_t blocks;
    if (G <= kTreeMixGroups) {  // the merged list: every compute unit (XCD slices when a multiple of 8)
        blocks = slots;
        per_group = 1;  // unused
    } else if (G <= kTreeLdsGroups) {  // one list of all groups' tiles: at most this many
        blocks = per_group + G;
        if (blocks > slots)
            blocks = slots;
        per_group = 1;  // unused
    } else {
        const int64_t want = (slots + G - 1) / G;
        if (per_group > want)
            per_group = want;
        if (per_group < 1)
            per_group = 1;
        blocks = per_group * G;
    }
    const int ts = (int)per_group;
    for (int n0 = 0; n0 < m; n0 += 64) {  // passes of up to 64 head rows
        hipEvent_t start = n0 == 0 ? t0 : nullptr, stop = n0 + 64 >= m ? t1 : nullptr;
        hipError_t e;
        if (m - n0 > 32)
            e = launch_timed(head_gathered_kernel<2, WV>, dim3((unsigned)blocks), dim3(64 * WV), s, start,
                             stop, V, d, Wb, G, m, n0, hb, ldh_g, sl_off, sl_ids, ts, logits);
        else
            e = launch_timed(head_gathered_kernel<1, WV>, dim3((unsigned)blocks), dim3(64 * WV), s, start,
                             stop, V, d, Wb, G, m, n0, hb, ldh_g, sl_off, sl_ids, ts, logits);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t head_mfma_launch(hipStream_t s, int V, int d, const void *W, int G, int m,
                            const void *h, int64_t ldh_g, const int64_t *sl_off,
                            const int32_t *sl_ids, int64_t max_rows, float *logits, void *ws,
                            hipEvent_t t0, hipEvent_t t1)
{
    const uint16_t *Wb = reinterpret_cast<const uint16_t *>(W);
    const uint16_t *hb = reinterpret_cast<const uint16_t *>(h);
    if (m == 1) {
        const int nt = (V + 31) / 32;
        TileIx *tix = reinterpret_cast<TileIx *>(ws);
        // one entry per thread: each does a dependent search, so the
        // latency is hidden by having every entry in flight at once
        int64_t blocks = (max_rows + 255) / 256;
        if (blocks > 65535)
            blocks = 65535;
        if (blocks < 1)
            blocks = 1;
        hipError_t e = launch_timed(union_index_kernel, dim3((unsigned)blocks), dim3(256), s, t0,
                                    nullptr, G, nt, V, sl_off, sl_ids, tix, logits);
        if (e != hipSuccess)
            return e;
        return union_passes(s, V, d, Wb, G, hb, ldh_g, sl_off, tix, nt, logits, nullptr, t1);
    }
    return gathered_passes<8>(s, V, d, Wb, G, m, hb, ldh_g, sl_off, sl_ids, max_rows, logits, t0,
                              t1);
}

size_t router_l1_ws_bytes(int r)
{
    return (size_t)kRouterMaxWin * kRouterCols * (size_t)r * sizeof(float);
}

hipError_t router_l1_mfma_launch(hipStream_t s, int n, int d, int r, int act, const void *h,
                                 int64_t ldh, const void *W1, const void *b1, float *z, float *part)
{
    const int nwin = (d + kRouterWin - 1) / kRouterWin;
    const dim3 grid((unsigned)((r + 127) / 128), (unsigned)nwin);
    const uint16_t *Wb = reinterpret_cast<const uint16_t *>(W1);
    const uint16_t *hb = reinterpret_cast<const uint16_t *>(h);
    for (int c0 = 0; c0 < n; c0 += kRouterCols) {
        const int nc = n - c0 < kRouterCols ? n - c0 : kRouterCols;
        if (nc > 32)
            hipLaunchKernelGGL(router_l1_kernel<2>, grid, dim3(256), 0, s, n, d, r, Wb, hb, ldh, c0,
                               part);
        else
            hipLaunchKernelGGL(router_l1_kernel<1>, grid, dim3(256), 0, s, n, d, r, Wb, hb, ldh, c0,
                               part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        const int64_t cnt = (int64_t)nc * r;
        hipLaunchKernelGGL(router_l1_finish, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, s,
                           r, nwin, c0, nc, (const float *)part,
                           reinterpret_cast<const uint16_t *>(b1), act, z);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// layer 2 on the matrix cores: bf16 W2, r % 8 == 0, and the window
// partials of a column pass fit the first layer's partial buffer
static int router_l2_slices(int r, int M)
{
    if (r % 8)
        return 0;
    for (int nsw = 1; nsw <= 2; ++nsw) {
        const size_t need = (size_t)((r + nsw * kKs - 1) / (nsw * kKs)) * kRouterCols * M *
                            sizeof(float);
        if (need <= router_l1_ws_bytes(r))
            return nsw;
    }
    return 0;
}

bool router_l2_mfma_applies(int r, int M) { return router_l2_slices(r, M) > 0; }

int router_l2_windows(int r, int M)
{
    const int nsw = router_l2_slices(r, M);
    return nsw ? (r + nsw * kKs - 1) / (nsw * kKs) : 0;
}

// the second layer's window partials of column pass c0 into part
static hipError_t router_l2_pass(hipStream_t s, int n, int r, int M, int nsw, const float *z,
                                 const uint16_t *Wb, int c0, float *part)
{
    const dim3 grid((unsigned)((M + 127) / 128), (unsigned)router_l2_windows(r, M));
    const int nc = n - c0 < kRouterCols ? n - c0 : kRouterCols;
    if (nsw == 1) {
        if (nc > 32)
            hipLaunchKernelGGL((router_l2_kernel<2, 1>), grid, dim3(256), 0, s, n, r, M, Wb, z, c0,
                               part);
        else
            hipLaunchKernelGGL((router_l2_kernel<1, 1>), grid, dim3(256), 0, s, n, r, M, Wb, z, c0,
                               part);
    } else {
        if (nc > 32)
            hipLaunchKernelGGL((router_l2_kernel<2, 2>), grid, dim3(256), 0, s, n, r, M, Wb, z, c0,
                               part);
        else
            hipLaunchKernelGGL((router_l2_kernel<1, 2>), grid, dim3(256), 0, s, n, r, M, Wb, z, c0,
                               part);
    }
    return hipGetLastError();
}

hipError_t router_l2_mfma_partials(hipStream_t s, int n, int r, int M, const void *z,
                                   const void *W2, float *part)
{
    const int nsw = router_l2_slices(r, M);
    if (nsw == 0 || n > kRouterCols)
        return hipErrorInvalidValue;
    return router_l2_pass(s, n, r, M, nsw, reinterpret_cast<const float *>(z),
                          reinterpret_cast<const uint16_t *>(W2), 0, part);
}

hipError_t router_l2_mfma_launch(hipStream_t s, int n, int r, int M, const void *z_,
                                 const void *W2, const void *b2, float *scores, float *part)
{
    const int nsw = router_l2_slices(r, M);
    if (nsw == 0)
        return hipErrorInvalidValue;
    const int nwin = router_l2_windows(r, M);
    const uint16_t *Wb = reinterpret_cast<const uint16_t *>(W2);
    const float *z = reinterpret_cast<const float *>(z_);
    for (int c0 = 0; c0 < n; c0 += kRouterCols) {
        const int nc = n - c0 < kRouterCols ? n - c0 : kRouterCols;
        hipError_t e = router_l2_pass(s, n, r, M, nsw, z, Wb, c0, part);
        if (e != hipSuccess)
            return e;
        const int64_t cnt = (int64_t)nc * M;
        hipLaunchKernelGGL(router_l1_finish, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, s,
                           M, nwin, c0, nc, (const float *)part,
                           reinterpret_cast<const uint16_t *>(b2), -1, scores);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t head_union_prebuilt_launch(hipStream_t s, int V, int d, const void *W, int G,
                                      const void *h, int64_t ldh_g, const int64_t *sl_off,
                                      const TileIx *tix, float *logits, hipEvent_t t0,
                                      hipEvent_t t1)
{
    return union_passes(s, V, d, reinterpret_cast<const uint16_t *>(W), G,
                        reinterpret_cast<const uint16_t *>(h), ldh_g, sl_off, tix, (V + 31) / 32,
                        logits, t0, t1);
}

}  // namespace ds
