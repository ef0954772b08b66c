// Matrix-core building blocks shared by the gathered-head kernels (gfx950,
// v_mfma_f32_32x32x16_bf16): the buffer-load path that reads W rows as whole
// 128-byte lines, and the per-wave LDS slice that reorders a wave's 32 rows
// into MFMA operand order.  Loads and data movement only; no method
// arithmetic.
#pragma once

#include "common.h"

namespace ds {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kKs = 64;  // hidden-dimension slice per MFMA group
// W rows per workgroup: WV waves x 32.  The staged hidden vectors are shared
// by all of a workgroup's rows, so taller tiles move fewer hidden-vector
// bytes from L2 per W row.
template <int WV>
constexpr int tile_rows() { return 32 * WV; }

__device__ __forceinline__ f32x16 mfma(const u32x4 &a, const u32x4 &b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// W rows are read with raw buffer loads: one 32-bit byte offset per lane, the
// 16-byte piece offsets as instruction immediates, and the hardware range
// check (offset >= num_records reads zero) instead of clamping -- so every
// load is unconditional and the compiler waits only for the slice it uses.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer, CDNA encoding
// Cache policy of the W loads (the aux field of the buffer load).  The union
// kernel reads every row once: nontemporal (2) keeps W from displacing the
// hidden vectors.  The gathered kernel's trees share many rows, and groups
// with the same tile index run side by side, so its rows stay cacheable
// (0): measured 15% faster on the 8 x 64 tree than nontemporal, while the
// union kernel is 10% slower without the hint.
constexpr int kNonTemporal = 2;
constexpr int kCached = 0;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

// W is read in whole 128-byte lines: per 64-wide slice a wave's 32 rows are
// four loads of 8 rows x 128 B (lane l: row l/8 + 8i, bytes 16*(l%8) of the
// slice).  Loads that give each lane its own MFMA row instead (two lanes per
// row, 32 B of a line per load) stream at well under half the bandwidth.
// `voff[i]` = byte offset of this lane's row for load i plus 16*(l%8).
template <int AUX>
__device__ __forceinline__ void load_a(rsrc_t w, const uint32_t voff[4], int k0, u32x4 a[4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        a[i] = __builtin_amdgcn_raw_buffer_load_b128(w, voff[i] + 2u * (uint32_t)k0, 0,
                                                     AUX);
}

// Per-wave LDS slice of A: 32 rows x 64 bf16; the 16-byte piece p of row r
// sits in slot p ^ akey(r), so the row-wise writes and the MFMA-order reads
// (one piece of each of 8 consecutive rows per 128 bytes of banks, 16 rows
// per 256) both touch distinct banks: akey takes 8 distinct values on any 8
// aligned rows and on the even and the odd rows of any 16 aligned rows (with
// r & 7 alone, rows r and r + 8 share banks when 16 lanes are served at once).
constexpr int kASlice = 32 * kKs;  // bf16 elements per wave
__device__ __forceinline__ int akey(int r) { return (r & 7) ^ ((r >> 3) & 1); }

}  // namespace
}  // namespace ds
