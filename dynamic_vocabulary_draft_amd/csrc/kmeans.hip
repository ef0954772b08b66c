// Spherical k-means over the rows of the LM head: the offline step that
// makes the vocabulary clusters the router selects from (DynaSpec summary
// page, "Key Novelty": clusters from the semantic similarity of LM-head
// weights; "Modeling / Key Hyperparameters": spherical k-means; "Key
// Terms": clusters by cosine similarity).  The algorithm is the published
// one (Dhillon and Modha, concept decompositions): unit rows x_y = w_y/|w_y|
// are assigned to the unit centroid of largest cosine, then every centroid
// becomes the normalised sum of its rows.  W is bf16.
//
// inverse norms: one wave per row, fp64 sums (once per W).
// assign:  the V x M x d contraction on v_mfma_f32_32x32x16_bf16 with the
//          argmax fused: a workgroup (8 waves, 4 high x 2 wide) owns 256
//          rows x 256 centroids, each wave a 64 x 128 block (2 x 4 MFMA
//          tiles: per slice, (256 + 256) rows pass through L2 for 256 x 256
//          outputs, a third fewer bytes per product than 256 x 128, and the
//          centroids, which do not fit one XCD's L2, are streamed V/256
//          times); per 64-wide slice of d both tiles arrive as whole
//          128-byte lines (8 rows per load) into a double-buffered,
//          XOR-swizzled LDS tile (128 KB, one barrier per slice; the
//          swizzle keeps the operand reads free of bank conflicts).  One slice
//          is in flight in registers while the previous one is multiplied
//          (a ring of two slices does not fit the 256 registers of a wave at
//          two waves per SIMD).
//          Workgroups that share a row tile are laid out on one XCD (blocks
//          are dealt round-robin over the 8 XCDs), so the tile is read from
//          HBM once and then from that XCD's L2.  The epilogue reduces each
//          row over its 128 columns (ties to the lower centroid) and keeps
//          the row's best with a 64-bit atomicMax of (order-preserving score
//          bits, ~centroid id): the maximum does not depend on the order the
//          workgroups finish in, so the result is deterministic.  The row
//          norm does not change the argmax, so the rows are not normalised.
// dense head: the same contraction with the hidden vectors of the full
//          drafter as the columns and a plain store epilogue (every logit,
//          [n][V]); used for the router's training labels.
// update:  members grouped by cluster in ascending row id without atomics
//          (per-chunk cluster counts, then a stable scatter: each 4096-row
//          chunk sorts its (cluster, row) keys in LDS); fp64 sums of
//          w_y * inv_norm[y] over member ranges of at most kUpdRange rows
//          (clusters are Zipf-sized, so ranges balance the work), then one
//          workgroup per cluster adds its ranges in order and normalises.
#include "common.h"
#include "kernels.h"

namespace ds {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer, CDNA encoding

constexpr int kTileR = 256;  // W rows per workgroup (4 waves high)
constexpr int kTileC = 256;  // centroids per workgroup (2 waves wide, 128 each)
constexpr int kAsgThreads = 512;
constexpr int kSlice = 64;   // hidden elements per LDS stage (128 B per row)
constexpr int kScatterChunk = 4096;
constexpr int kUpdRange = 128;   // member rows per partial sum
constexpr int kUpdBatch = 8;     // member rows in flight per workgroup
constexpr int kUpdGroup = 2048;  // hidden elements covered by one pass of 256 threads x 8

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

__device__ __forceinline__ f32x16 mfma(const u32x4 &a, const u32x4 &b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 -> order-preserving uint32 (larger float, larger integer; -0 and +0
// are one value, as in a floating-point comparison)
__device__ __forceinline__ uint32_t f32_key(float v)
{
    const uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_f32(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v)
{
    const uint32_t u = __float_as_uint(v);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return 0x7FC0;  // NaN
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// --------------------------------------------------------------- inverse norms
__global__ __launch_bounds__(256) void inv_norm_kernel(int V, int nch, const u32x4 *__restrict__ W,
                                                       float *__restrict__ inv_norm)
{
    const int lane = lane_id();
    const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t y = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); y < V; y += nw) {
        const u32x4 *row = W + y * nch;
        double ss = 0.0;
        for (int c = lane; c < nch; c += kWave) {
            const u32x4 v = __builtin_nontemporal_load(row + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double lo = bf16_lo(v[e]), hi = bf16_hi(v[e]);
                ss += lo * lo;
                ss += hi * hi;
            }
        }
        ss = wave_sum_f64(ss);
        if (lane == 0)
            inv_norm[y] = ss > 0.0 ? (float)(1.0 / sqrt(ss)) : 0.0f;
    }
}

// --------------------------------------------------------------------- assign
__global__ void fill_u64_kernel(uint64_t *p, int64_t n, uint64_t v)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// this thread's 16-byte pieces of an R-row tile's slice: piece q = tid +
// kAsgThreads i is row q/8, piece q%8 of the row's 128 bytes.  The per-lane
// part of the offset (row, piece) is fixed, vo[i]; the slice offset is
// wave-uniform and goes in the scalar offset (the range check uses vo[i]:
// rows past the tile read zero).
template <int R>
__device__ __forceinline__ void tile_offsets(int d, uint32_t vo[R * 8 / kAsgThreads])
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < R * 8 / kAsgThreads; ++i)
        vo[i] = (uint32_t)((tid >> 3) + (kAsgThreads / 8) * i) * (uint32_t)d * 2u +
                16u * (uint32_t)(tid & 7);
}
template <int R>
__device__ __forceinline__ void tile_load(rsrc_t r, const uint32_t vo[R * 8 / kAsgThreads], int k0,
                                          u32x4 v[R * 8 / kAsgThreads])
{
#pragma unroll
    for (int i = 0; i < R * 8 / kAsgThreads; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, vo[i], 2 * k0, 0);
}
// LDS tile: [row][64 bf16], piece p of row r in slot p ^ swz(r) with
// swz(r) = (r >> 1) & 7: rows 2k and 2k+1 (one 256-byte line of the banks)
// share a pattern, and the 8 pairs of 16 consecutive rows from a multiple
// of 16 take 8 different ones.  For the operand reads (lanes l and l + 32
// read pieces st and 4 + st of one row) this measured 185 bytes per cycle
// per CU against 114 for r & 7 and 138 for (r ^ (r >> 3)) & 7; the tile
// writes run at about 74 bytes per cycle with any of them.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
template <int R>
__device__ __forceinline__ void tile_store(uint16_t *t, const u32x4 v[R * 8 / kAsgThreads])
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < R * 8 / kAsgThreads; ++i) {
        const int row = (tid >> 3) + (kAsgThreads / 8) * i, p = tid & 7;
        *reinterpret_cast<u32x4 *>(t + row * kSlice + ((p ^ swz(row)) << 3)) = v[i];
    }
}
// MFMA operand: row `row` of a tile, pieces 4*(lane/32) + s (k permuted the
// same way for both operands, so the products pair up exactly)
__device__ __forceinline__ u32x4 frag(const uint16_t *t, int row, int s)
{
    const int p = 4 * (lane_id() >> 5) + s;
    return *reinterpret_cast<const u32x4 *>(t + row * kSlice + ((p ^ swz(row)) << 3));
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;
// 16 bytes per lane from the buffer (offset voff + soff) straight into LDS:
// the wave's 64 lanes fill 1 KB from lds on, in lane order
__device__ __forceinline__ void lds_load16(rsrc_t r, uint16_t *lds, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}
// wait until this wave's vector memory operations (LDS loads included) are done
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// STORE = false: the assignment (argmax epilogue into best); STORE = true:
// the plain product, out[c][y] = W[y] . C[c] (row stride ldo), which is the
// dense LM head when C holds hidden vectors.
// DMA (an even number of 64-wide slices): the slices go from L2 straight
// into LDS (buffer loads with the LDS destination), not through registers
// and LDS writes: two LDS stages, each wave's eight 1-KB loads of slice t+1
// issued before the products of slice t, one barrier per slice (which
// waits for them).  A load's 64 lanes fill 1 KB of LDS in lane order (8 rows
// of 128 bytes), so each lane fetches the global piece that the swizzle
// puts at its slot.  The stages are separate LDS arrays, so the compiler
// sees that the products' reads cannot alias the loads in flight.
template <bool STORE, int TC, bool DMA = false>
__global__ __launch_bounds__(kAsgThreads) void kmeans_assign_kernel(int V, int d, const uint16_t *__restrict__ W,
                                                            int M, const uint16_t *__restrict__ C,
                                                            int RT, int CT,
                                                            unsigned long long *__restrict__ best,
                                                            float *__restrict__ out, int64_t ldo)
{
    constexpr int WCOLS = TC / 2, JT = WCOLS / 32;  // columns per wave, its 32-wide tiles
    const int b = blockIdx.x;
    // a row tile stays on one XCD; the tile indices are read back as scalars
    // (the divisions go through vector registers; buffer descriptors built
    // from them must be scalar)
    const int rt = __builtin_amdgcn_readfirstlane((b / (8 * CT)) * 8 + (b % 8));
    const int ct = __builtin_amdgcn_readfirstlane((b / 8) % CT);
    if (rt >= RT)
        return;
    const int lane = lane_id(), wave = threadIdx.x >> 6, wr = wave >> 1, wc = wave & 1;  // 4 x 2 waves
    const int64_t y0 = (int64_t)rt * kTileR;
    const int c0 = ct * TC;
    const int rows = (int)min((int64_t)kTileR, (int64_t)V - y0), cols = min(TC, M - c0);
    const rsrc_t ra = make_rsrc(W + y0 * d, (uint32_t)rows * (uint32_t)d * 2u);
    const rsrc_t rb = make_rsrc(C + (int64_t)c0 * d, (uint32_t)cols * (uint32_t)d * 2u);
    f32x16 acc[2][JT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < JT; ++j)
            acc[i][j] = f32x16{};
    const int nsl = d / kSlice;
    if constexpr (DMA) {
        // two stages, each an A tile and a B tile, four separate arrays: the
        // compiler then tells every read from the loads in flight (an offset
        // folded into a constant loses that)
        __shared__ __attribute__((aligned(1024))) uint16_t sa0[kTileR * kSlice];
        __shared__ __attribute__((aligned(1024))) uint16_t sb0[TC * kSlice];
        __shared__ __attribute__((aligned(1024))) uint16_t sa1[kTileR * kSlice];
        __shared__ __attribute__((aligned(1024))) uint16_t sb1[TC * kSlice];
        const int wv = __builtin_amdgcn_readfirstlane(wave);  // LDS destinations are scalar
        // load q of this wave fills rows 8 * (8q + wave) .. +8 of a tile
        constexpr int QA = kTileR / 64, QB = TC / 64;
        uint32_t voa[QA], vob[QB];
#pragma unroll
        for (int q = 0; q < QA; ++q) {
            const int row = 8 * (8 * q + wv) + (lane >> 3);
            voa[q] = (uint32_t)row * (uint32_t)d * 2u + 16u * (uint32_t)((lane & 7) ^ swz(row));
        }
#pragma unroll
        for (int q = 0; q < QB; ++q) {
            const int row = 8 * (8 * q + wv) + (lane >> 3);
            vob[q] = (uint32_t)row * (uint32_t)d * 2u + 16u * (uint32_t)((lane & 7) ^ swz(row));
        }
#define KMD_LOAD(SA, SB, T)                                                                 \
    {                                                                                       \
        const int k0_ = min((T), nsl - 1) * kSlice;                                         \
        _Pragma("unroll") for (int q = 0; q < QA; ++q)                                      \
            lds_load16(ra, (SA) + (8 * q + wv) * 8 * kSlice, voa[q], 2 * k0_);              \
        _Pragma("unroll") for (int q = 0; q < QB; ++q)                                      \
            lds_load16(rb, (SB) + (8 * q + wv) * 8 * kSlice, vob[q], 2 * k0_);              \
    }
// the operands of piece st + 1 are read while piece st is multiplied (two
// register sets), one read between consecutive products
#define KMD_READ(SA, SB, ST, FA, FB)                                                        \
    {                                                                                       \
        _Pragma("unroll") for (int i = 0; i < 2; ++i)                                       \
            FA[i] = frag((SA), wr * 64 + i * 32 + (lane & 31), (ST));                       \
        _Pragma("unroll") for (int j = 0; j < JT; ++j)                                      \
            FB[j] = frag((SB), wc * WCOLS + j * 32 + (lane & 31), (ST));                    \
    }
#define KMD_MUL(FA, FB)                                                                     \
    {                                                                                       \
        _Pragma("unroll") for (int i = 0; i < 2; ++i)                                       \
            _Pragma("unroll") for (int j = 0; j < JT; ++j)                                  \
                acc[i][j] = mfma(FA[i], FB[j], acc[i][j]);                                  \
    }
#define KMD_PRODUCTS(SA, SB)                                                                \
    {                                                                                       \
        u32x4 fa0_[2], fb0_[JT], fa1_[2], fb1_[JT];                                         \
        KMD_READ(SA, SB, 0, fa0_, fb0_)                                                     \
        KMD_READ(SA, SB, 1, fa1_, fb1_)                                                     \
        KMD_MUL(fa0_, fb0_)                                                                 \
        KMD_READ(SA, SB, 2, fa0_, fb0_)                                                     \
        KMD_MUL(fa1_, fb1_)                                                                 \
        KMD_READ(SA, SB, 3, fa1_, fb1_)                                                     \
        KMD_MUL(fa0_, fb0_)                                                                 \
        KMD_MUL(fa1_, fb1_)                                                                 \
        /* order: piece 0's reads, then each of the first three pieces'   */                \
        /* products with the next piece's reads one by one between them   */                \
        __builtin_amdgcn_sched_group_barrier(0x100, 2 + JT, 0);                             \
        _Pragma("unroll") for (int g = 0; g < 3; ++g)                                       \
        {                                                                                   \
            _Pragma("unroll") for (int k = 0; k < 2 + JT; ++k)                              \
            {                                                                               \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          \
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                          \
            }                                                                               \
            __builtin_amdgcn_sched_group_barrier(0x008, JT - 2, 0);                         \
        }                                                                                   \
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * JT, 0);                             \
    }
        // a wave's LDS loads must have landed before the barrier that lets
        // the other waves read them (the barrier itself does not wait)
#define KMD_SYNC                                  \
    {                                             \
        wait_vmem();                              \
        __syncthreads();                          \
    }
        KMD_LOAD(sa0, sb0, 0)
        KMD_SYNC
        for (int t = 0; t < nsl; t += 2) {  // nsl is even (the launcher checks)
            // the scheduler would sink the loads below the products
            KMD_LOAD(sa1, sb1, t + 1)
            __builtin_amdgcn_sched_barrier(0);
            KMD_PRODUCTS(sa0, sb0)
            KMD_SYNC  // stage 1 loaded by every wave; stage 0 read by every wave
            KMD_LOAD(sa0, sb0, t + 2)
            __builtin_amdgcn_sched_barrier(0);
            KMD_PRODUCTS(sa1, sb1)
            KMD_SYNC
        }
#undef KMD_SYNC
#undef KMD_PRODUCTS
#undef KMD_MUL
#undef KMD_READ
#undef KMD_LOAD
    } else {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][(kTileR + TC) * kSlice];
    constexpr int NA = kTileR * 8 / kAsgThreads, NB = TC * 8 / kAsgThreads;
    // register ring of one slice (a 256-column slice holds enough MFMA work
    // to cover a memory round trip; 128-column tiles needed two slices in
    // flight): while slice t is multiplied, slice t+1 moves to LDS and slice
    // t+2 is requested.  Loads past the last slice re-read it (clamped), so
    // every load is unconditional and the compiler waits only for the slice
    // it stores.
    u32x4 a0[NA], b0[NB];
    uint32_t voa[NA], vob[NB];
    tile_offsets<kTileR>(d, voa);
    tile_offsets<TC>(d, vob);
#define KM_LOAD(T, VA, VB)                                      \
    {                                                           \
        const int k0_ = min((T), nsl - 1) * kSlice;             \
        tile_load<kTileR>(ra, voa, k0_, VA);                    \
        tile_load<TC>(rb, vob, k0_, VB);                        \
    }
    // one step: multiply slice T, move slice T+1 (held in VA/VB) to LDS,
    // request slice T+2 into VA/VB
#define KM_STEP(T, VA, VB)                                                          \
    {                                                                               \
        const uint16_t *ta_ = lds[(T) & 1], *tb_ = lds[(T) & 1] + kTileR * kSlice;  \
        _Pragma("unroll") for (int st = 0; st < 4; ++st)                            \
        {                                                                           \
            u32x4 fa_[2], fb_[JT];                                                  \
            _Pragma("unroll") for (int i = 0; i < 2; ++i)                           \
                fa_[i] = frag(ta_, wr * 64 + i * 32 + (lane & 31), st);             \
            _Pragma("unroll") for (int j = 0; j < JT; ++j)                          \
                fb_[j] = frag(tb_, wc * WCOLS + j * 32 + (lane & 31), st);          \
            _Pragma("unroll") for (int i = 0; i < 2; ++i)                           \
                _Pragma("unroll") for (int j = 0; j < JT; ++j)                      \
                    acc[i][j] = mfma(fa_[i], fb_[j], acc[i][j]);                    \
        }                                                                           \
        if ((T) + 1 < nsl) {                                                        \
            tile_store<kTileR>(lds[((T) + 1) & 1], VA);                             \
            tile_store<TC>(lds[((T) + 1) & 1] + kTileR * kSlice, VB);               \
        }                                                                           \
        KM_LOAD((T) + 2, VA, VB)                                                    \
        __syncthreads();                                                            \
    }
    KM_LOAD(0, a0, b0)
    tile_store<kTileR>(lds[0], a0);
    tile_store<TC>(lds[0] + kTileR * kSlice, b0);
    KM_LOAD(1, a0, b0)
    __syncthreads();
    for (int t = 0; t < nsl; ++t)
        KM_STEP(t, a0, b0)
#undef KM_STEP
#undef KM_LOAD
    }
    // epilogue: register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4 of
    // the 32 x 32 tile, column l%32
    if constexpr (STORE) {
        // lanes l and l + 32 cover 32 consecutive rows of one column over
        // their 16 registers, so each column's 128-byte run fills in L2
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < JT; ++j) {
                const int col = wc * WCOLS + j * 32 + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wr * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (col < cols && row < rows)
                        out[(int64_t)(c0 + col) * ldo + y0 + row] = acc[i][j][r];
                }
            }
        return;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // the lane's columns ascend with j: a strict > keeps the lower
            int c = wc * WCOLS + (lane & 31);
            float v = c < cols ? acc[i][0][r] : -INFINITY;
#pragma unroll
            for (int j = 1; j < JT; ++j) {
                const int cj = wc * WCOLS + j * 32 + (lane & 31);
                const float vj = cj < cols ? acc[i][j][r] : -INFINITY;
                if (vj > v) {
                    v = vj;
                    c = cj;
                }
            }
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) {  // within each 32-lane half
                const float ov = __shfl_xor(v, o);
                const int oc = __shfl_xor(c, o);
                if (ov > v || (ov == v && oc < c)) {
                    v = ov;
                    c = oc;
                }
            }
            const int row = wr * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if ((lane & 31) == 0 && row < rows && v > -INFINITY) {
                const uint64_t key = ((uint64_t)f32_key(v) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)(c0 + c));
                atomicMax(&best[y0 + row], (unsigned long long)key);
            }
        }
    }
}

__global__ void assign_finalize_kernel(int V, const unsigned long long *__restrict__ best,
                                       int32_t *__restrict__ assign, float *__restrict__ score)
{
    for (int64_t y = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; y < V;
         y += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t k = best[y];
        assign[y] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
        score[y] = key_f32((uint32_t)(k >> 32));
    }
}

// --------------------------------------------------------------------- update
// offsets: off[c] = first member slot of cluster c, item_off[c] = first
// partial-sum item of c (ceil(size/kUpdRange) items each); one workgroup
__global__ __launch_bounds__(1024) void update_offsets_kernel(int M, int nchunks,
                                                              const int32_t *__restrict__ index,
                                                              int32_t *__restrict__ off,
                                                              int32_t *__restrict__ item_off,
                                                              int32_t *__restrict__ size)
{
    __shared__ int64_t sh[kWave + 1];
    const int32_t *sizes = index + (int64_t)nchunks * M;
    int64_t carry_m = 0, carry_i = 0;
    for (int c0 = 0; c0 < M; c0 += 1024) {
        const int c = c0 + (int)threadIdx.x;
        const int64_t n = c < M ? sizes[c] : 0;
        const int64_t it = (n + kUpdRange - 1) / kUpdRange;
        int64_t tot_m, tot_i;
        const int64_t em = block_excl_scan_i64(n, sh, &tot_m);
        const int64_t ei = block_excl_scan_i64(it, sh, &tot_i);
        if (c < M) {
            off[c] = (int32_t)(carry_m + em);
            item_off[c] = (int32_t)(carry_i + ei);
            size[c] = (int32_t)n;
        }
        carry_m += tot_m;
        carry_i += tot_i;
    }
    if (threadIdx.x == 0) {
        off[M] = (int32_t)carry_m;
        item_off[M] = (int32_t)carry_i;
    }
}

// stable scatter of one 4096-row chunk: sort its (cluster, row) keys, then
// a row's slot is its cluster's start + the cluster's members in earlier
// chunks + its rank among the chunk's members of that cluster
__global__ __launch_bounds__(256) void update_scatter_kernel(int V, int M,
                                                             const int32_t *__restrict__ assign,
                                                             const int32_t *__restrict__ index,
                                                             const int32_t *__restrict__ off,
                                                             int32_t *__restrict__ members)
{
    __shared__ uint64_t key[kScatterChunk];
    __shared__ int s_wmax[4];
    const int chunk = blockIdx.x;
    const int64_t y0 = (int64_t)chunk * kScatterChunk;
    for (int i = threadIdx.x; i < kScatterChunk; i += blockDim.x) {
        const int64_t y = y0 + i;
        const int c = y < V ? assign[y] : -1;
        key[i] = (c >= 0 && c < M) ? (((uint64_t)(uint32_t)c << 32) | (uint32_t)y) : ~0ull;
    }
    __syncthreads();
    for (int k = 2; k <= kScatterChunk; k <<= 1) {  // bitonic sort, ascending
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int t = threadIdx.x; t < kScatterChunk / 2; t += blockDim.x) {
                const int i = 2 * t - (t & (j - 1));
                const bool up = (i & k) == 0;
                const uint64_t a = key[i], bk = key[i + j];
                if ((a > bk) == up) {
                    key[i] = bk;
                    key[i + j] = a;
                }
            }
            __syncthreads();
        }
    }
    // segment starts: thread t owns sorted slots 16t .. 16t+15
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int i0 = threadIdx.x * 16;
    int start[16];
    int run = -1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int i = i0 + e;
        const bool first = i == 0 || (key[i] >> 32) != (key[i - 1] >> 32);
        if (first)
            run = i;
        start[e] = run;
    }
    // carry the last start from earlier threads (inclusive max scan)
    int m = run;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_up(m, o);
        if (lane >= o)
            m = max(m, t);
    }
    if (lane == kWave - 1)
        s_wmax[wave] = m;
    __syncthreads();
    int carry = __shfl_up(m, 1);
    if (lane == 0)
        carry = -1;
    for (int w = 0; w < wave; ++w)
        carry = max(carry, s_wmax[w]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int i = i0 + e;
        const uint64_t kv = key[i];
        if (kv == ~0ull)
            continue;
        const int c = (int)(kv >> 32);
        const int st = start[e] >= 0 ? start[e] : carry;
        members[off[c] + index[(int64_t)chunk * M + c] + (i - st)] = (int32_t)(uint32_t)kv;
    }
}

// fp64 sum of w_y * inv_norm[y] over one member range (ascending y); thread
// t owns hidden elements 8t .. 8t+7 of every 2048-element group
template <int G>
__global__ __launch_bounds__(256) void update_partial_kernel(int d, const uint16_t *__restrict__ W,
                                                             const float *__restrict__ inv_norm,
                                                             int M, const int32_t *__restrict__ off,
                                                             const int32_t *__restrict__ item_off,
                                                             const int32_t *__restrict__ members,
                                                             double *__restrict__ partial)
{
    const int b = blockIdx.x;
    if (b >= item_off[M])
        return;
    int lo = 0, hi = M;  // cluster: last c with item_off[c] <= b
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (item_off[mid] <= b)
            lo = mid;
        else
            hi = mid;
    }
    const int c = lo;
    const int64_t j0 = (int64_t)off[c] + (int64_t)(b - item_off[c]) * kUpdRange;
    const int64_t j1 = min(j0 + kUpdRange, (int64_t)off[c + 1]);
    double acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[g][e] = 0.0;
    const int kt = threadIdx.x * 8;
    // ids and scales of the next batch are fetched while this batch's rows load
    int32_t yn[kUpdBatch];
#pragma unroll
    for (int q = 0; q < kUpdBatch; ++q)
        yn[q] = j0 + q < j1 ? members[j0 + q] : -1;
    for (int64_t j = j0; j < j1; j += kUpdBatch) {
        int32_t y[kUpdBatch];
#pragma unroll
        for (int q = 0; q < kUpdBatch; ++q)
            y[q] = yn[q];
        u32x4 v[kUpdBatch][G];
        double sc[kUpdBatch];
#pragma unroll
        for (int q = 0; q < kUpdBatch; ++q) {
            const bool in = y[q] >= 0;
            sc[q] = in ? (double)inv_norm[y[q]] : 0.0;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int k = g * kUpdGroup + kt;
                v[q][g] = (in && k < d)
                              ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(W + (int64_t)y[q] * d + k))
                              : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int q = 0; q < kUpdBatch; ++q)
            yn[q] = j + kUpdBatch + q < j1 ? members[j + kUpdBatch + q] : -1;
#pragma unroll
        for (int q = 0; q < kUpdBatch; ++q)  // members in ascending order
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[g][2 * e] += (double)bf16_lo(v[q][g][e]) * sc[q];
                    acc[g][2 * e + 1] += (double)bf16_hi(v[q][g][e]) * sc[q];
                }
    }
    double *out = partial + (int64_t)b * d;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int k = g * kUpdGroup + kt;
        if (k < d)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                out[k + e] = acc[g][e];
    }
}

// one workgroup per cluster: its ranges added in order, normalised
template <int G>
__global__ __launch_bounds__(256) void update_finalize_kernel(int d, int M,
                                                              const int32_t *__restrict__ item_off,
                                                              const int32_t *__restrict__ size,
                                                              const double *__restrict__ partial,
                                                              const float *__restrict__ C_prev,
                                                              float *__restrict__ C_out,
                                                              uint16_t *__restrict__ C_out_bf16,
                                                              double *__restrict__ norm)
{
    __shared__ double s_w[4];
    const int c = blockIdx.x;
    const int kt = threadIdx.x * 8;
    double sv[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            sv[g][e] = 0.0;
    for (int it = item_off[c]; it < item_off[c + 1]; ++it) {
        const double *p = partial + (int64_t)it * d;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int k = g * kUpdGroup + kt;
            if (k < d)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    sv[g][e] += p[k + e];
        }
    }
    double ss = 0.0;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            ss += sv[g][e] * sv[g][e];
    ss = wave_sum_f64(ss);
    if (lane_id() == 0)
        s_w[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = ((s_w[0] + s_w[1]) + s_w[2]) + s_w[3];
    const double nrm = sqrt(ss);
    const bool keep = size[c] <= 0 || !(nrm > 0.0);
    if (threadIdx.x == 0)
        norm[c] = size[c] > 0 ? nrm : 0.0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int k = g * kUpdGroup + kt;
        if (k < d)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t at = (int64_t)c * d + k + e;
                const float v = keep ? C_prev[at] : (float)(sv[g][e] / nrm);
                C_out[at] = v;
                C_out_bf16[at] = f32_to_bf16_rne(v);
            }
    }
}

struct UpdWs {
    int32_t *index, *off, *item_off, *members;
    double *partial;
};

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

UpdWs upd_ws(void *ws, int V, int d, int M)
{
    const int64_t nch = ((int64_t)V + kScatterChunk - 1) / kScatterChunk;
    char *p = reinterpret_cast<char *>(ws);
    UpdWs w;
    w.index = reinterpret_cast<int32_t *>(p);
    p += align256((size_t)(nch + 1) * M * 4);
    w.off = reinterpret_cast<int32_t *>(p);
    p += align256((size_t)(M + 1) * 4);
    w.item_off = reinterpret_cast<int32_t *>(p);
    p += align256((size_t)(M + 1) * 4);
    w.members = reinterpret_cast<int32_t *>(p);
    p += align256((size_t)V * 4);
    w.partial = reinterpret_cast<double *>(p);
    return w;
}

int64_t max_items(int V, int M) { return (int64_t)M + ((int64_t)V + kUpdRange - 1) / kUpdRange; }

template <int G>
hipError_t launch_update_g(hipStream_t s, int V, int d, const uint16_t *W, const float *inv_norm,
                           int M, const UpdWs &w, const float *C_prev, float *C_out,
                           uint16_t *C_out_bf16, int32_t *size, double *norm)
{
    hipLaunchKernelGGL((update_partial_kernel<G>), dim3((unsigned)max_items(V, M)), dim3(256), 0, s,
                       d, W, inv_norm, M, w.off, w.item_off, w.members, w.partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((update_finalize_kernel<G>), dim3((unsigned)M), dim3(256), 0, s, d, M,
                       w.item_off, size, w.partial, C_prev, C_out, C_out_bf16, norm);
    return hipGetLastError();
}

}  // namespace

hipError_t kmeans_inv_norm_launch(hipStream_t s, int V, int d, const void *W, float *inv_norm)
{
    int64_t blocks = ((int64_t)V + 3) / 4;
    const int64_t cap = 8LL * device_cu_count();
    if (blocks > cap)
        blocks = cap;
    hipLaunchKernelGGL(inv_norm_kernel, dim3((unsigned)blocks), dim3(256), 0, s, V, d / 8,
                       reinterpret_cast<const u32x4 *>(W), inv_norm);
    return hipGetLastError();
}

size_t kmeans_assign_ws_bytes(int V) { return (size_t)V * 8 + 256; }

hipError_t kmeans_assign_launch(hipStream_t s, int V, int d, const void *W, int M, const void *C,
                                int32_t *assign, float *score, void *ws, hipEvent_t t0,
                                hipEvent_t t1)
{
    unsigned long long *best = reinterpret_cast<unsigned long long *>(ws);
    const unsigned fb = (unsigned)min(((int64_t)V + 255) / 256, (int64_t)4096);
    hipLaunchKernelGGL(fill_u64_kernel, dim3(fb), dim3(256), 0, s, reinterpret_cast<uint64_t *>(best),
                       (int64_t)V, (uint64_t)0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int RT = (V + kTileR - 1) / kTileR, CT = (M + kTileC - 1) / kTileC;
    const int RTp = (RT + 7) / 8 * 8;  // row tiles padded to whole XCD rounds
    const dim3 grid((unsigned)((int64_t)RTp * CT));
    if ((d / kSlice) % 2 == 0)
        e = launch_timed(kmeans_assign_kernel<false, kTileC, true>, grid, dim3(kAsgThreads), s, t0,
                         t1, V, d, reinterpret_cast<const uint16_t *>(W), M,
                         reinterpret_cast<const uint16_t *>(C), RT, CT, best, (float *)nullptr,
                         (int64_t)0);
    else
        e = launch_timed(kmeans_assign_kernel<false, kTileC>, grid, dim3(kAsgThreads), s, t0, t1,
                         V, d, reinterpret_cast<const uint16_t *>(W), M,
                         reinterpret_cast<const uint16_t *>(C), RT, CT, best, (float *)nullptr,
                         (int64_t)0);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(assign_finalize_kernel, dim3(fb), dim3(256), 0, s, V,
                       (const unsigned long long *)best, assign, score);
    return hipGetLastError();
}

size_t kmeans_update_ws_bytes(int V, int d, int M)
{
    const int64_t nch = ((int64_t)V + kScatterChunk - 1) / kScatterChunk;
    return align256((size_t)(nch + 1) * M * 4) + 2 * align256((size_t)(M + 1) * 4) +
           align256((size_t)V * 4) + (size_t)max_items(V, M) * d * 8 + 256;
}

hipError_t kmeans_update_launch(hipStream_t s, int V, int d, const void *W, const float *inv_norm,
                                int M, const int32_t *assign, const float *C_prev, float *C_out,
                                void *C_out_bf16, int32_t *size, double *norm, int32_t *err_flag,
                                void *ws)
{
    UpdWs w = upd_ws(ws, V, d, M);
    const int nch = (V + kScatterChunk - 1) / kScatterChunk;
    hipError_t e = index_launch(s, M, V, assign, w.index, err_flag);  // per-chunk cluster counts
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(update_offsets_kernel, dim3(1), dim3(1024), 0, s, M, nch,
                       (const int32_t *)w.index, w.off, w.item_off, size);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(update_scatter_kernel, dim3((unsigned)nch), dim3(256), 0, s, V, M, assign,
                       (const int32_t *)w.index, (const int32_t *)w.off, w.members);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    const uint16_t *Wb = reinterpret_cast<const uint16_t *>(W);
    uint16_t *Cb = reinterpret_cast<uint16_t *>(C_out_bf16);
    const int G = (d + kUpdGroup - 1) / kUpdGroup;
    switch (G) {
    case 1:
        return launch_update_g<1>(s, V, d, Wb, inv_norm, M, w, C_prev, C_out, Cb, size, norm);
    case 2:
        return launch_update_g<2>(s, V, d, Wb, inv_norm, M, w, C_prev, C_out, Cb, size, norm);
    case 3:
        return launch_update_g<3>(s, V, d, Wb, inv_norm, M, w, C_prev, C_out, Cb, size, norm);
    default:
        return launch_update_g<4>(s, V, d, Wb, inv_norm, M, w, C_prev, C_out, Cb, size, norm);
    }
}

}  // namespace ds

namespace ds {

hipError_t dense_head_launch(hipStream_t s, int V, int d, const void *W, int n, const void *h,
                             float *logits, int64_t ldl, hipEvent_t t0, hipEvent_t t1)
{
    const int RT = (V + kTileR - 1) / kTileR, CT = (n + kTileC - 1) / kTileC;
    const int RTp = (RT + 7) / 8 * 8;
    // the register ring keeps two slices of W in flight against one for the
    // LDS-direct loads; W streams from HBM once here (one column tile), and
    // the ring measured as fast or faster
    return launch_timed(kmeans_assign_kernel<true, kTileC>, dim3((unsigned)((int64_t)RTp * CT)),
                        dim3(kAsgThreads), s, t0, t1, V, d, reinterpret_cast<const uint16_t *>(W),
                        n, reinterpret_cast<const uint16_t *>(h), RT, CT,
                        (unsigned long long *)nullptr, logits, ldl);
}

}  // namespace ds
