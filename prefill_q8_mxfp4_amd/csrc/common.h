// Shared device code of the block-quantized-weight batched GEMM on gfx950
// (CDNA4),
//
//   y[b][n] = sum_k x[b][k] * w[n][k],
//
// used by every tier: operand types, the per-format decoders, the split of
// fp32 activations into bf16 terms, the MFMA wrapper, epilogue helpers and the
// launch interface the host side (api.hip) calls.
//
// Block scales.  Where a tier keeps weights exact in its MFMA operand, int8 q
// and E2M1 codes are exact in bf16 and the fp32 block scale multiplies the
// fp32 partial of each 32-wide block.  NVFP4 (16-wide blocks) folds its E4M3
// scale into the operand (E2M1 x E4M3 is exact in bf16); the large-batch tier
// folds every format's scale into the bf16 operand (exact for the FP4
// formats; a Q8_0 weight d*q is rounded once to bf16 there).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace qg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { ACT_F32 = 0, ACT_BF16 = 1 };
enum { OUT_F32 = 0, OUT_BF16 = 1 };

struct KArgs {
    const uint8_t *w;
    const void *x;
    void *y;
    int B, N, K;
    int S;              // slabs per row tile
    int RT;             // row tiles
    int64_t scale_off;  // scale region offset
    int64_t meta_off;   // NVFP4 tensor-scale record offset (or -1)
};

// ------------------------------------------------------------ decoders

__device__ __forceinline__ float fp16_bits_to_f32(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// E8M0 byte -> fp32 2^(e-127); 0 -> 2^-127 (subnormal), 255 -> NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e)
{
    uint32_t bits = e == 0 ? 0x00400000u : (e == 255 ? 0x7FC00000u : (e << 23));
    return __uint_as_float(bits);
}

// FP8 E4M3 byte SEL of v -> fp32 (exact), one conversion: gfx950 decodes
// the OCP E4M3 format (subnormals 2^-9 * M, signed zero, 0x7F / 0xFF -> NaN);
// checked against a table of all 256 codes.
template <int SEL>
__device__ __forceinline__ float e4m3_byte_to_f32(uint32_t v)
{
    return __builtin_amdgcn_cvt_f32_fp8((int)v, SEL);
}

// FP8 E4M3 byte (the low byte of b) -> fp32 (exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b)
{
    return e4m3_byte_to_f32<0>(b);
}

// E2M1 code -> fp32 (exact).
__device__ __forceinline__ float e2m1_to_f32(uint32_t c)
{
    uint32_t m = c & 7u;
    // magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 as fp32 bit patterns
    uint32_t bits = m == 0 ? 0u
                  : m == 1 ? 0x3F000000u
                  : (((m >> 1) + 126u) << 23) | ((m & 1u) << 22);
    return __uint_as_float(bits | ((c & 8u) << 28));
}

// Signed byte BYTE of v -> fp32 (exact) in one SDWA conversion; written out
// because the compiler shifts bytes 1 and 3 down first.
template <int BYTE>
__device__ __forceinline__ float sbyte_to_f32(uint32_t v)
{
    float r;
    if constexpr (BYTE == 0)
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(v));
    else if constexpr (BYTE == 1)
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(v));
    else if constexpr (BYTE == 2)
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(v));
    else
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(v));
    return r;
}

// Eight int8 (two dwords) -> bf16x8, exact: 8 conversions and 4 packs.
__device__ __forceinline__ bf16x8 q8_to_bf16(uint32_t lo, uint32_t hi)
{
    bf16x8 r;
    r[0] = (__bf16)sbyte_to_f32<0>(lo); r[1] = (__bf16)sbyte_to_f32<1>(lo);
    r[2] = (__bf16)sbyte_to_f32<2>(lo); r[3] = (__bf16)sbyte_to_f32<3>(lo);
    r[4] = (__bf16)sbyte_to_f32<0>(hi); r[5] = (__bf16)sbyte_to_f32<1>(hi);
    r[6] = (__bf16)sbyte_to_f32<2>(hi); r[7] = (__bf16)sbyte_to_f32<3>(hi);
    return r;
}

// Eight FP8 E4M3 codes (two dwords, byte j = element j) -> bf16x8, exact
// (an E4M3 value has 4 significant bits): gfx950's packed FP8 conversion,
// unscaled; checked against all 256 codes.
__device__ __forceinline__ bf16x8 fp8_to_bf16(uint32_t lo, uint32_t hi)
{
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    bf16x8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// Eight FP8 E4M3 codes times an fp32 scale -> bf16x8 (codes to fp32 exactly,
// one fp32 multiply, one rounding to bf16).
__device__ __forceinline__ bf16x8 fp8_scaled_to_bf16(uint32_t lo, uint32_t hi, float d)
{
    const f32x2 f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
    const f32x2 f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
    const f32x2 f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
    const f32x2 f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
    bf16x8 r;
    r[0] = (__bf16)(f0[0] * d); r[1] = (__bf16)(f0[1] * d);
    r[2] = (__bf16)(f1[0] * d); r[3] = (__bf16)(f1[1] * d);
    r[4] = (__bf16)(f2[0] * d); r[5] = (__bf16)(f2[1] * d);
    r[6] = (__bf16)(f3[0] * d); r[7] = (__bf16)(f3[1] * d);
    return r;
}

// Eight int8 times an fp32 scale -> bf16x8 (one rounding each).
__device__ __forceinline__ bf16x8 q8_scaled_to_bf16(uint32_t lo, uint32_t hi, float d)
{
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        r[i] = (__bf16)((float)(int8_t)(lo >> (8 * i)) * d);
        r[4 + i] = (__bf16)((float)(int8_t)(hi >> (8 * i)) * d);
    }
    return r;
}

// Eight E2M1 codes (one dword, element 2j in the low nibble of byte j) times
// a power-of-two fp32 scale -> bf16x8, through the gfx950 scaled FP4
// conversion.  The conversion applies only the exponent of its scale operand
// (it is built for E8M0 scales), so it serves MXFP4 and unscaled E2M1 only.
__device__ __forceinline__ bf16x8 fp4_to_bf16(uint32_t v, float scale)
{
    bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0);
    bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1);
    bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2);
    bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3);
    bf16x8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// Eight E2M1 codes times an arbitrary fp32 scale (an E4M3 block scale) ->
// bf16x8: codes to fp32 exactly, one fp32 multiply (exact: at most 6
// significant bits), then a conversion that does not round.
__device__ __forceinline__ bf16x8 fp4_to_bf16_mul(uint32_t v, float scale)
{
    auto f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 0);
    auto f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 1);
    auto f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 2);
    auto f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 3);
    bf16x8 r;
    r[0] = (__bf16)(f0[0] * scale); r[1] = (__bf16)(f0[1] * scale);
    r[2] = (__bf16)(f1[0] * scale); r[3] = (__bf16)(f1[1] * scale);
    r[4] = (__bf16)(f2[0] * scale); r[5] = (__bf16)(f2[1] * scale);
    r[6] = (__bf16)(f3[0] * scale); r[7] = (__bf16)(f3[1] * scale);
    return r;
}

// ------------------------------------------------ activation operands

// CNT fp32 values -> NT bf16 terms each, whose sum is the fp32 value:
// NT = 1: nearest bf16; NT = 2: hi + lo, |residual| <= 2^-17 |x|;
// NT = 3: exact (truncated hi and mid carry 16 bits, the 8-bit rest is exact).
template <int NT>
struct Split {
    bf16x8 t[NT];
};

template <int NT, int CNT = 8>
__device__ __forceinline__ Split<NT> split_f32(const float *v)
{
    Split<NT> s;
#pragma unroll
    for (int i = 0; i < CNT; i++) {
        float f = v[i];
        if constexpr (NT == 1) {
            s.t[0][i] = (__bf16)f;
        } else if constexpr (NT == 2) {
            __bf16 h = (__bf16)f;
            float r = f - (float)h;
            s.t[0][i] = h;
            s.t[1][i] = (__bf16)r;
        } else {
            float h = __uint_as_float(__float_as_uint(f) & 0xFFFF0000u);
            float r1 = f - h;
            float m = __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);
            float r2 = r1 - m;
            s.t[0][i] = (__bf16)h;
            s.t[1][i] = (__bf16)m;
            s.t[2][i] = (__bf16)r2;
        }
    }
    return s;
}

// Raw buffer resource over [base, base + bytes) (clamped to 4 GiB); loads
// through it take a 32-bit per-lane offset plus a uniform (scalar) offset,
// and bytes past the end read as zero.  Descriptor word 3 is the gfx9-family
// raw-buffer setting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)(uint32_t)n, 0x00020000);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// The same loads with the nontemporal cache policy (gfx950 CPol NT = 2), for
// data a call reads exactly once (the small-batch weight stream): measured on
// MI355X, Q8_0 5120^2 weight loads alone at B = 16 run 0.5 us faster with it.
constexpr int CP_NT = 2;
// Scope bits of the same field for plain loads of data other workgroups
// stored with scoped stores: SC0 as the compiler sets for workgroup-scope
// atomics (served by the XCD's L2), SC1 for device scope.
constexpr int CP_SC0 = 1;
constexpr int CP_SC1 = 16;

__device__ __forceinline__ u32x4 bload16_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CP_NT));
}

__device__ __forceinline__ u32x2 bload8_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, CP_NT));
}

__device__ __forceinline__ uint32_t bload4_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, CP_NT));
}

// All-ones when `keep`, else zero, opaque to the optimiser.  Masking a loaded
// value with it (instead of `keep ? v : 0`) stops the compiler from turning the
// load into a conditional one issued late, which would make later waits drain
// every load in flight.
__device__ __forceinline__ uint32_t keep_mask(bool keep)
{
    uint32_t m = keep ? 0xFFFFFFFFu : 0u;
    asm volatile("" : "+v"(m));
    return m;
}

__device__ __forceinline__ u32x4 masked(u32x4 v, uint32_t m)
{
    return u32x4{v[0] & m, v[1] & m, v[2] & m, v[3] & m};
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float t)
{
    return t / (1.0f + __expf(-t));
}

// Scales of row r of row tile rt for slab s (see layout.h).
template <int FMT>
__device__ __forceinline__ const uint8_t *slab_scales(const KArgs &a, int64_t rt, int r, int s)
{
    return a.w + scale_offset(a.scale_off, a.S, FMT, rt, r, s);
}

__device__ __forceinline__ float tensor_scale(const KArgs &a, int n)
{
    const int *meta = (const int *)(a.w + a.meta_off);
    const float *g = (const float *)(a.w + a.meta_off + 16);
    int rpt = meta[1];
    return g[n / rpt];
}

template <int OUTT>
__device__ __forceinline__ void store_out(void *y, int64_t idx, float v)
{
    if constexpr (OUTT == OUT_F32)
        ((float *)y)[idx] = v;
    else
        ((__bf16 *)y)[idx] = (__bf16)v;
}

// Output stores that should not stay in L2 (written once, read by the next
// kernel): nontemporal.
template <int OUTT>
__device__ __forceinline__ void store_out_nt(void *y, int64_t idx, float v)
{
    if constexpr (OUTT == OUT_F32)
        __builtin_nontemporal_store(v, (float *)y + idx);
    else
        __builtin_nontemporal_store((__bf16)v, (__bf16 *)y + idx);
}

// ------------------------------------------------------------ launch API
// (host side; one translation unit per tier)

// Overrides of the tuned choices, read once from the environment when a plan
// is created (for measurements and tests; 0 or -1 keeps the tuned choice).
// Release builds honour only overrides that keep the documented results:
// the shape knobs (results stay within the same bounds) and QGEMM_ST_XLOCAL=0
// (the device-coherent exchange, bitwise the same result).  Builds with
// QGEMM_DEBUG_KNOBS also honour QGEMM_ST_XLOCAL=1, QGEMM_FP32_TERMS=1|2 (fewer
// activation terms: gives up the fp32-faithful bound) and QGEMM_XCC_FAKE=1
// (odd K splits report the next XCC, to exercise the per-launch check).
struct Knobs {
    int st_waves, st_nph;  // streaming-kernel shape (QGEMM_ST_WAVES, QGEMM_ST_NPH)
    int st_depth;          // streaming kernel's load depth in row tiles (QGEMM_ST_DEPTH)
    int gv_maxb;           // largest B sent to the GEMV kernel (QGEMM_GV_MAXB; 0 = none, -1 = the default rule)
    int sk_stream;         // 0: B <= 16 through the skinny kernel (QGEMM_SK_STREAM)
    int sk_nt;             // 1: one row tile per skinny wave (QGEMM_SK_NT)
    int vf;                // 0: no verify kernel for fp32-faithful 16 < B <= 80 (QGEMM_VF)
    int vf_bf16_maxb;      // largest B of bf16 math the verify kernel takes (QGEMM_VF_BF16_MAXB)
    int vf_swiglu_maxb;    // largest B the fused gate+up epilogue takes the verify kernel at (QGEMM_VF_SWIGLU_MAXB)
    int ti_bm, ti_split;   // large-batch row-tile height, K splits (QGEMM_TI_BM, QGEMM_TI_SPLIT)
    int ti_waves;          // large-batch waves per workgroup, 4 or 8 (QGEMM_TI_WAVES; 0 = default)
    int xlocal;            // -1 the probe decides, 0 device-coherent, 1 forced (debug)
    int fp32_terms;        // activation terms of fp32-faithful math (3; debug 1..3)
    int xcc_fake;          // debug: odd K splits report the next XCC to the placement check
};

struct Problem {
    int fmt, act, out, epi, math;
    int64_t N, K;
    Layout L;
    Knobs kn;
};

// Bits of the device status word (qgemm_device_status).
constexpr uint32_t DEV_XCD_MISMATCH = 1u;  // a workgroup ran off its probed XCD
constexpr uint32_t DEV_BAD_OFFSETS = 2u;   // routed-expert offsets broke their rules

// Small-batch tier shape: MB 16-row batch groups and 4*NT row tiles per
// workgroup, kc slabs of K per workgroup staged kch at a time, ksplit
// workgroups per output tile along K; grid ngroups x ksplit x nby.
constexpr int SK_RING = 8;  // weight slabs in flight per wave

struct SkCfg {
    int MB, NT;
    int ngroups, nby, ksplit, kc, kch;
    int lds;                        // dynamic LDS bytes (activation stage)
    int64_t cnt_bytes, part_bytes;  // workspace regions (0 without a K split)
};

// Workspace of the K split: tile counters, then partial tiles.
struct SkinnyWs {
    float *part;      // [ksplit][tiles][64 lanes][4]
    uint32_t *cnt;    // [nby][ngroups], zero between calls
    int ksplit;
    int kc;           // a multiple of kch
    int kch;          // a multiple of SK_RING
    // streaming kernel only: every K split of a row group runs on one XCD
    // (workgroup ids congruent mod 8; the dispatcher deals ids to the XCDs
    // round-robin), so partial tiles are exchanged through that XCD's L2
    // (workgroup-scope stores and loads) instead of device-coherent memory
    int xlocal;
    int xcc_fake;      // debug builds: odd splits report the next XCC (exercises the check)
    uint32_t *status;  // device status word (DEV_* bits), or null
};

// LDS bytes of one staged slab: NTA terms x MB x units x 64 lanes x 16 B.
__host__ __device__ constexpr int skinny_lds_per_slab(int fmt, int nta, int mb)
{
    return nta * mb * (slab_k(fmt) / 32) * 64 * 16;
}

// Small-batch streaming kernel for B <= 16: workgroups of W waves (8..16)
// over ST_RG row tiles, chunks of KC = W * NPH slabs with every load of a
// chunk issued at once; grid ngroups * ksplit.
constexpr int ST_RG = 8;
// wave limit per phase count: two phases hold twice the weight registers
__host__ __device__ constexpr int st_max_waves(int nph) { return nph == 2 ? 12 : 16; }

struct StCfg {
    int W, NPH, KC;
    int depth;  // weight items (phase, row tile) a wave keeps in flight (16: all of a chunk)
    int Nh;  // SwiGLU: gate rows (N / 2), else 0
    int ngroups, ksplit, kc;
    int xlocal, grid;  // XCD-local split exchange (SkinnyWs::xlocal); workgroups launched
    int64_t cnt_bytes, part_bytes;
};

// A K split's partial tile `tile` of split ks, a lane's 16 bytes in one
// store carrying the cache-scope bits of a scoped store at SCOPE (workgroup:
// kept in the XCD's L2; device: written through to the point of coherence).
template <int SCOPE>
__device__ __forceinline__ void publish_partial(uint64_t *part, int ks, int64_t tiles, int64_t tile, int lane,
                                                f32x4 v)
{
    constexpr int AUX = SCOPE == __HIP_MEMORY_SCOPE_WORKGROUP ? CP_SC0 : CP_SC1;
    const int64_t tbytes = tiles * 1024;
    const __amdgpu_buffer_rsrc_t r = make_rsrc((uint8_t *)part + ks * tbytes, tbytes);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)(tile * 1024) + lane * 16, 0, AUX);
}

// Last workgroup of a K split: sum the ksplit partial tiles of `tile` in
// split order (its own partial `own` in place ks).  A lane's 16 bytes of a
// partial are one load carrying the cache-scope bits of the stores (SCOPE:
// workgroup, served by the XCD's L2, or device), only the other splits are
// loaded, and the loads of up to 8 splits are issued before the first add.
template <int SCOPE>
__device__ __forceinline__ f32x4 reduce_partials_s(const uint64_t *part, int ksplit, int ks, int64_t tiles,
                                                   int64_t tile, int lane, f32x4 own)
{
    constexpr int AUX = SCOPE == __HIP_MEMORY_SCOPE_WORKGROUP ? CP_SC0 : CP_SC1;
    const int64_t tbytes = tiles * 1024;
    const int voff = (int)(tile * 1024) + lane * 16;
    f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < ksplit; k0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int kk = k0 + j;
            if (kk < ksplit && kk != ks) {  // uniform
                const __amdgpu_buffer_rsrc_t r = make_rsrc((const uint8_t *)part + kk * tbytes, tbytes);
                v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, AUX));
            } else {
                v[j] = own;
            }
        }
#pragma unroll
        for (int j = 0; j < 8; j++) {
            if (k0 + j >= ksplit)
                break;  // uniform
            sum[0] += v[j][0]; sum[1] += v[j][1]; sum[2] += v[j][2]; sum[3] += v[j][3];
        }
    }
    return sum;
}

__device__ __forceinline__ f32x4 reduce_partials(const uint64_t *part, int ksplit, int ks, int64_t tiles,
                                                 int64_t tile, int lane, f32x4 own)
{
    return reduce_partials_s<__HIP_MEMORY_SCOPE_AGENT>(part, ksplit, ks, tiles, tile, lane, own);
}

// Small-batch GEMV (B = 1, 2): one workgroup per row tile over all of K,
// fp32 FMA on the vector ALUs; no workspace.  gemv_lds_bytes: its dynamic
// LDS (the B activation rows as fp32).
hipError_t launch_gemv(const Problem &p, const KArgs &a, hipStream_t st);
int64_t gemv_lds_bytes(const Problem &p, int64_t B);
int gemv_waves(const Problem &p);

hipError_t launch_skinny(const Problem &p, const KArgs &a, const SkCfg &c, const SkinnyWs &ws,
                         int nterm, hipStream_t st);
hipError_t launch_stream(const Problem &p, const KArgs &a, const StCfg &c, const SkinnyWs &ws,
                         int nterm, hipStream_t st);
// 16 < B <= VF_MAX_B and K a whole number of slabs: the streaming kernel's
// row groups and K splits (StCfg) with all batch rows per workgroup (verify.h);
// partial tiles [ksplit][ngroups * 8][MB][64][4].  nterm: 3 (fp32-faithful,
// fp32 activations) or 1 (bf16 math).
constexpr int VF_MAX_B = 80;
constexpr int VF_BF16_MAXB = 80;  // bf16 math: the default of Knobs::vf_bf16_maxb
constexpr int VF_SWIGLU_MAXB = 48;  // fused gate+up: the default of Knobs::vf_swiglu_maxb
int verify_mb(int64_t B);
hipError_t launch_verify(const Problem &p, const KArgs &a, const StCfg &c, const SkinnyWs &ws, int nterm,
                         hipStream_t st);
hipError_t launch_verify_bf16(const Problem &p, const KArgs &a, const StCfg &c, const SkinnyWs &ws, hipStream_t st);
// Large-batch tier shape: BM x 256 tiles; the first `full` tiles run whole,
// the rest are split along K into S pieces each (one workgroup per piece),
// with partial tiles in `part` and one counter per split tile in `cnt`.
struct TiSplit {
    int full, S;
    uint32_t *cnt;
    float *part;
};

struct TiCfg {
    int BM, mtiles, ntiles, tiles, wgs;
    int NW;              // waves per workgroup: 8 (2 x 4), or 4 (2 x 2, bf16 math)
    TiSplit sp;
    int64_t part_bytes;  // workspace the split needs (0 without a split)
};

hipError_t launch_tiled(const Problem &p, const KArgs &a, const TiCfg &c, hipStream_t st);
hipError_t launch_tiled_w4(const Problem &p, const KArgs &a, const TiCfg &c, hipStream_t st);
hipError_t launch_tiled_fp32(const Problem &p, const KArgs &a, const TiCfg &c, hipStream_t st);
// x[n] fp32 -> xb[n] bf16, round to nearest even (n a multiple of 8, both
// 16-byte aligned).
hipError_t launch_x_to_bf16(const float *x, void *xb, int64_t n, hipStream_t st);

// Routed experts in the large-batch kernel: E packed weight buffers (device
// array of device pointers) and E + 1 row offsets (device int32, rows of
// expert e are off[e] .. off[e+1]-1); ntiles weight tiles per expert.
struct Groups {
    const uint8_t *const *wtab;
    const int *off;
    int E;
    int ntiles;
    int T;             // rows: off[0] = 0, off non-decreasing, off[E] = T
    uint32_t *status;  // device status word: DEV_BAD_OFFSETS when they are not
};
hipError_t launch_grouped(const Problem &p, const KArgs &a, const Groups &g, int BM, int64_t tiles,
                          hipStream_t st);
hipError_t launch_grouped_fp32(const Problem &p, const KArgs &a, const Groups &g, int BM, int64_t tiles,
                               hipStream_t st);
// Routed experts with few rows each, bf16 math: one workgroup per (expert,
// row-tile group), moe_groups(p) groups per expert (moe.hip).
hipError_t launch_moe(const Problem &p, const KArgs &a, const Groups &g, hipStream_t st);
int moe_groups(const Problem &p);
int moe_groups_per_wg(const Problem &p, int64_t E);
hipError_t launch_dequant(int fmt, const KArgs &a, float *out, hipStream_t st);
hipError_t launch_read_bytes(const void *buf, int64_t bytes, uint32_t *sink, int wgs, hipStream_t st);
hipError_t launch_mfma_rate(int mode, int iters, uint32_t *sink, hipStream_t st);

}  // namespace qg
