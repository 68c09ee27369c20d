// Packed weight layout of the library (host and device side).
//
// Row tiles of 16 rows; slabs of KS weights along K (64 for Q8_0, 128 for the
// FP4 formats), 1024 bytes each, laid out so that 16-byte chunk L of a slab is
// exactly the operand that lane L of a wave feeds to a 16x16x32 bf16 MFMA for
// each 32-wide unit of the slab (row L % 16, k-group L / 16).  Scales follow,
// one contiguous record of the 16 rows per (row tile, slab) in the codes'
// order, so the scales of a slab are one 64-byte (128-byte for NVFP4) piece
// of a cache line; NVFP4 adds a 256-byte tensor-scale record.
#pragma once
#include <stdint.h>

#include "../../include/qgemm.h"

namespace qg {

enum { FMT_Q8 = 0, FMT_MX = 1, FMT_NV = 2, FMT_FP8 = 3 };

struct Layout {
    int64_t N, K;
    int64_t Np, Kp;      // padded rows (x16) and K (xKS)
    int64_t KS;          // weights per slab along K
    int64_t S;           // slabs per row tile
    int64_t RT;          // row tiles
    int64_t scale_off;   // byte offset of the scale region
    int64_t meta_off;    // byte offset of the NVFP4 tensor-scale record (or -1)
    int64_t total;       // total bytes
    int64_t blk;         // K granularity: weights per scale (FP8: per 32, its scales cover 128)
};

// Scale bytes of one row for one slab: Q8_0 two fp16, MXFP4 four E8M0,
// NVFP4 eight E4M3, FP8 the fp32 scale of the 128-wide block holding the slab.
__host__ __device__ constexpr int scale_bytes_per_slab(int fmt)
{
    return fmt == FMT_NV ? 8 : 4;
}

// Bytes of the scale record of one (row tile, slab): 16 rows.
__host__ __device__ constexpr int scale_record_bytes(int fmt)
{
    return 16 * scale_bytes_per_slab(fmt);
}

// Byte offset of the scales of row r (0..15) of row tile rt for slab s.
__host__ __device__ static inline int64_t scale_offset(int64_t scale_off, int64_t S, int fmt, int64_t rt, int r,
                                                       int64_t s)
{
    return scale_off + (rt * S + s) * scale_record_bytes(fmt) + r * scale_bytes_per_slab(fmt);
}

static inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

static inline int64_t block_of(int fmt) { return fmt == FMT_NV ? 16 : 32; }

// Weights per slab along K: 64 for the byte formats, 128 for the FP4 ones.
__host__ __device__ constexpr int slab_k(int fmt) { return fmt == FMT_Q8 || fmt == FMT_FP8 ? 64 : 128; }

constexpr int FP8_BLOCK = 128;  // weights per FP8 block scale along K

static inline bool make_layout(int fmt, int64_t N, int64_t K, Layout *L)
{
    if (fmt < FMT_Q8 || fmt > FMT_FP8 || N <= 0 || K <= 0)
        return false;
    if (K % block_of(fmt))
        return false;
    L->N = N;
    L->K = K;
    L->blk = block_of(fmt);
    L->KS = slab_k(fmt);
    L->Np = round_up(N, 16);
    L->Kp = round_up(K, L->KS);
    L->S = L->Kp / L->KS;
    L->RT = L->Np / 16;
    int64_t codes = L->RT * L->S * 1024;
    L->scale_off = round_up(codes, QGEMM_ALIGN);
    int64_t end = L->scale_off + L->RT * L->S * scale_record_bytes(fmt);
    if (fmt == FMT_NV) {
        L->meta_off = round_up(end, QGEMM_ALIGN);
        L->total = L->meta_off + 256;
    } else {
        L->meta_off = -1;
        L->total = round_up(end, QGEMM_ALIGN);
    }
    return true;
}

}  // namespace qg
