// HIP kernels for the block-quantized-weight batched GEMM on gfx950 (CDNA4).
//
//   y[b][n] = sum_k x[b][k] * w[n][k]
//
// Two tiers share the packed layout of layout.h:
//
//  * skinny: for small B.  Each wave streams packed weight slabs from HBM with
//    one 16-byte load per lane; the chunk a lane loads is already its operand
//    for v_mfma_f32_16x16x32_bf16 (row = lane % 16, k-group = lane / 16), so
//    weights go HBM -> VGPR -> decode -> MFMA with no LDS and no shuffles.
//    Batch rows are the MFMA's 16-row A operand (padded with zeros), loaded
//    straight from the activation matrix.  The waves of a workgroup split K and
//    their partial tiles are summed through LDS in a fixed order.
//  * tiled: for large B.  A workgroup owns a BM x BN output tile; activation
//    and decoded-weight tiles are staged through LDS as bf16 MFMA fragments,
//    with a register prefetch of the next K step.  Optional fused gate+up
//    epilogue: the tile holds gate rows j and up rows Nh + j so both
//    accumulators of an output sit in the same lane.
//
// Block scales.  Q8_0 and MXFP4 in the skinny tier keep the weight operand
// exact (int8 q and E2M1 are exact in bf16) and apply the fp32 block scale to
// the 16x16 partial of each 32-wide block (one 32-wide MFMA per block).  NVFP4
// (16-wide blocks) and every format in the tiled tier fold the scale into the
// bf16 operand: E2M1 x E4M3 and E2M1 x 2^e are exact in bf16; Q8_0 d*q is
// rounded once to bf16 (tiled tier only).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace qg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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
    int SP;             // scale pitch (bytes)
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

// FP8 E4M3 byte -> fp32 (exact).  Subnormals 2^-9 * M; 0x7F / 0xFF -> NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b)
{
    uint32_t s = (b & 0x80u) << 24;
    uint32_t em = b & 0x7Fu;
    float v;
    if ((em >> 3) == 0)
        v = (float)em * 0.001953125f;  // M * 2^-9, exact
    else
        v = __uint_as_float(((em >> 3) + 120u) << 23 | (em & 7u) << 20);
    v = __uint_as_float(__float_as_uint(v) | s);
    return em == 0x7Fu ? __uint_as_float(0x7FC00000u) : v;
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

// Eight int8 (two dwords) -> bf16x8, exact.
__device__ __forceinline__ bf16x8 q8_to_bf16(uint32_t lo, uint32_t hi)
{
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        r[i] = (__bf16)(float)(int8_t)(lo >> (8 * i));
        r[4 + i] = (__bf16)(float)(int8_t)(hi >> (8 * i));
    }
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

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float t)
{
    return t / (1.0f + __expf(-t));
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

// ================================================================ skinny
//
// A workgroup is 4 waves.  It owns RG = 4*NT row tiles (64*NT weight rows),
// one batch group of 16*MB rows and one range of K slabs; wave w computes
// row tiles w*NT .. w*NT+NT-1 over that range.  For every slab the workgroup
// stages the batch rows' activations in LDS once, already split into the
// bf16 terms the MFMAs take (exact for fp32 activations), double-buffered;
// all four waves read their A fragments from there.  Weight chunks stream
// HBM -> VGPR with a ring of D slabs in flight per wave.
//
// With a workspace, K is split over `ksplit` workgroups per output tile: each
// writes its partial tile, then bumps a device-scope counter; the last to
// arrive adds all partials in split order (so the result does not depend on
// arrival order), applies the epilogue and re-arms the counter to zero.

struct SkinnyWs {
    float *part;      // [ksplit][tiles][64 lanes][4]
    uint32_t *cnt;    // [nby][ngroups], zero between calls
    int ksplit;       // workgroups per output tile along K
    int kc;           // slabs per workgroup
};

template <int FMT, int ACT, int NTERM, int MB, int NT, int D, int OUTT>
__global__ __launch_bounds__(256) void skinny_kernel(KArgs a, SkinnyWs ws)
{
    constexpr int KS = FMT == FMT_Q8 ? 64 : 128;
    constexpr int U = KS / 32;                 // 32-wide units per slab
    constexpr bool POST = FMT != FMT_NV;       // block scale applied after the MFMA
    constexpr int NTA = ACT == ACT_F32 ? NTERM : 1;
    constexpr int BR = 16 * MB;                // batch rows per workgroup
    constexpr int CE = ACT == ACT_F32 ? 4 : 8; // activations per 16-byte chunk
    constexpr int NCH = BR * KS / CE;          // chunks per slab
    constexpr int XCH = (NCH + 255) / 256;     // chunks per thread

    __shared__ u32x4 xs[2][NTA][MB][U][64];
    __shared__ int s_is_last;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int r = lane & 15, gq = lane >> 4;
    const int grp = blockIdx.x, ks = blockIdx.y, by = blockIdx.z;
    const int ngroups = gridDim.x;
    const int rt0 = (grp * 4 + wid) * NT;
    const int b0 = by * BR;
    const int s_beg = ks * ws.kc;
    const int s_end = min(a.S, s_beg + ws.kc);
    const uint8_t *scl = a.w + a.scale_off;

    f32x4 acc[MB][NT];
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
            acc[mb][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- weight ring
    u32x4 wr[D][NT];
    uint32_t sr[D][NT][2];
    // Loads are unconditional (addresses clamped in bounds) so no register is
    // written on a side path while a load into it is in flight; tiles past the
    // last row tile compute on a copy of it and are never stored.
    auto wload = [&](int j, int s) {
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
            const int64_t rt = min(rt0 + nt, a.RT - 1);
            wr[j][nt] = *(const u32x4 *)(a.w + ((rt * a.S + s) << 10) + (lane << 4));
            const uint8_t *sp = scl + (rt * 16 + r) * (int64_t)a.SP;
            if constexpr (FMT == FMT_NV) {
                u32x2 v = *(const u32x2 *)(sp + s * 8);
                sr[j][nt][0] = v[0];
                sr[j][nt][1] = v[1];
            } else {
                sr[j][nt][0] = *(const uint32_t *)(sp + s * 4);
                sr[j][nt][1] = 0;
            }
        }
    };

    // ---- activation staging: global -> registers -> (split) -> LDS
    u32x4 xr[XCH];
    bool xin[XCH];
    auto xload = [&](int s) {
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            const int c = min(tid + i * 256, NCH - 1);
            const int row = c / (KS / CE), kk = (c % (KS / CE)) * CE;
            const int b = b0 + row, k = s * KS + kk;
            // K % 16 == 0: a chunk is all inside K or all past it
            xin[i] = b < a.B && k < a.K;
            const int bc = min(b, a.B - 1), kcl = min(k, a.K - CE);
            if constexpr (ACT == ACT_F32)
                xr[i] = *(const u32x4 *)((const float *)a.x + (int64_t)bc * a.K + kcl);
            else
                xr[i] = *(const u32x4 *)((const uint16_t *)a.x + (int64_t)bc * a.K + kcl);
        }
    };
    // Threads past the last chunk repeat it (same value to the same LDS
    // bytes) instead of branching around the store.
    auto xstore = [&](int p) {
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            const int c = min(tid + i * 256, NCH - 1);
            {
                const int row = c / (KS / CE), kk = (c % (KS / CE)) * CE;
                const int mb = row >> 4, b = row & 15;
                const int u = kk >> 5, g8 = (kk & 31) >> 3;
                const u32x4 xv = xin[i] ? xr[i] : u32x4{0u, 0u, 0u, 0u};
                if constexpr (ACT == ACT_F32) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        v[e] = __uint_as_float(xv[e]);
                    Split<NTA> sp = split_f32<NTA, 4>(v);
                    const int half = (kk & 7) >> 2;  // which 8 bytes of the entry
#pragma unroll
                    for (int t = 0; t < NTA; t++) {
                        u32x4 q = __builtin_bit_cast(u32x4, sp.t[t]);
                        u32x2 *dst = (u32x2 *)&xs[p][t][mb][u][g8 * 16 + b] + half;
                        *dst = u32x2{q[0], q[1]};
                    }
                } else {
                    xs[p][0][mb][u][g8 * 16 + b] = xv;
                }
            }
        }
    };

    // Every iteration issues the same loads (slab indices clamped to the last
    // real slab), so the compiler can count them statically and keep D weight
    // slabs in flight; only the arithmetic is skipped for padding slabs.
    // ws.kc is a multiple of D.
    const int s_last = s_end - 1;
    xload(s_beg);
    xstore(0);
    xload(min(s_beg + 1, s_last));
#pragma unroll
    for (int j = 0; j < D; j++)
        wload(j, min(s_beg + j, s_last));

    for (int s0 = s_beg; s0 < s_beg + ws.kc; s0 += D) {
#pragma unroll
        for (int j = 0; j < D; j++) {
            const int s = s0 + j;
            __syncthreads();  // slab s staged; the other buffer is free
            const int p = (s - s_beg) & 1;
            xstore(p ^ 1);
            xload(min(s + 2, s_last));
            u32x4 wc[NT];
            uint32_t sc[NT][2];
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                wc[nt] = wr[j][nt];
                sc[nt][0] = sr[j][nt][0];
                sc[nt][1] = sr[j][nt][1];
            }
            wload(j, min(s + D, s_last));
            if (s >= s_end)
                continue;  // padding slab (uniform)

#pragma unroll
            for (int u = 0; u < U; u++) {
                if (s * KS + 32 * u >= a.K)
                    break;  // padding units of the last slab (uniform)
                bf16x8 A[MB][NTA];
#pragma unroll
                for (int mb = 0; mb < MB; mb++)
#pragma unroll
                    for (int t = 0; t < NTA; t++)
                        A[mb][t] = __builtin_bit_cast(bf16x8, xs[p][t][mb][u][lane]);
#pragma unroll
                for (int nt = 0; nt < NT; nt++) {
                    bf16x8 Bw;
                    float ps = 1.f;
                    if constexpr (FMT == FMT_Q8) {
                        Bw = q8_to_bf16(wc[nt][2 * u], wc[nt][2 * u + 1]);
                        ps = fp16_bits_to_f32((sc[nt][0] >> (16 * u)) & 0xFFFFu);
                    } else if constexpr (FMT == FMT_MX) {
                        Bw = fp4_to_bf16(wc[nt][u], 1.0f);
                        ps = e8m0_to_f32((sc[nt][0] >> (8 * u)) & 0xFFu);
                    } else {
                        const int si = 2 * u + (gq >> 1);
                        const uint32_t sb = (si < 4 ? sc[nt][0] >> (8 * si) : sc[nt][1] >> (8 * (si - 4))) & 0xFFu;
                        Bw = fp4_to_bf16_mul(wc[nt][u], e4m3_to_f32(sb));
                    }
#pragma unroll
                    for (int mb = 0; mb < MB; mb++) {
                        if constexpr (POST) {
                            f32x4 t = mfma(A[mb][0], Bw, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                            for (int tt = 1; tt < NTA; tt++)
                                t = mfma(A[mb][tt], Bw, t);
#pragma unroll
                            for (int i = 0; i < 4; i++)
                                acc[mb][nt][i] = __builtin_fmaf(ps, t[i], acc[mb][nt][i]);
                        } else {
#pragma unroll
                            for (int tt = 0; tt < NTA; tt++)
                                acc[mb][nt] = mfma(A[mb][tt], Bw, acc[mb][nt]);
                        }
                    }
                }
            }
        }
    }

    // ---- split-K: publish the partial; the last workgroup of the tile reduces.
    // No device-wide fence (on gfx950 that writes back and invalidates the
    // whole L2 of the XCD): partials are written with device-scope stores that
    // go through to the point of coherence, each wave waits for its stores to
    // be acknowledged before the workgroup bumps the tile counter, and the
    // reducing workgroup reads partials with device-scope loads.
    if (ws.ksplit > 1) {
        const int64_t tiles = (int64_t)gridDim.z * ngroups * 4 * MB * NT;
        const int64_t tbase = (((int64_t)by * ngroups + grp) * 4 + wid) * (MB * NT);
        uint64_t *part = (uint64_t *)ws.part;
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                uint64_t *dst = part + (((int64_t)ks * tiles + tbase + mb * NT + nt) * 64 + lane) * 2;
                const u32x4 v = __builtin_bit_cast(u32x4, acc[mb][nt]);
                __hip_atomic_store(dst, (uint64_t)v[0] | ((uint64_t)v[1] << 32), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(dst + 1, (uint64_t)v[2] | ((uint64_t)v[3] << 32), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are acknowledged
        __syncthreads();
        if (tid == 0) {
            uint32_t old = __hip_atomic_fetch_add(&ws.cnt[by * ngroups + grp], 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
            s_is_last = old == (uint32_t)(ws.ksplit - 1);
        }
        __syncthreads();
        if (!s_is_last)
            return;
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
                for (int kk = 0; kk < ws.ksplit; kk++) {
                    f32x4 v;
                    if (kk == ks) {
                        v = acc[mb][nt];
                    } else {
                        const uint64_t *src =
                            part + (((int64_t)kk * tiles + tbase + mb * NT + nt) * 64 + lane) * 2;
                        const uint64_t lo = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        const uint64_t hi = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        v = __builtin_bit_cast(f32x4, u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi,
                                                            (uint32_t)(hi >> 32)});
                    }
                    sum[0] += v[0]; sum[1] += v[1]; sum[2] += v[2]; sum[3] += v[3];
                }
                acc[mb][nt] = sum;
            }
        if (tid == 0)
            __hip_atomic_store(&ws.cnt[by * ngroups + grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue: tensor scale, store (lane holds rows 4*gq..4*gq+3 of column r)
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        const int n = (rt0 + nt) * 16 + r;
        if (n >= a.N)
            continue;
        float g = 1.f;
        if constexpr (FMT == FMT_NV)
            g = tensor_scale(a, n);
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int b = b0 + 16 * mb + 4 * gq + i;
                if (b < a.B)
                    store_out<OUTT>(a.y, (int64_t)b * a.N + n, g * acc[mb][nt][i]);
            }
    }
}

// ================================================================= tiled
//
// Workgroup tile BM (batch) x BN (weight rows; for SwiGLU BN gate rows plus
// the matching BN up rows).  WM x WN waves, each owning (BM/WM) x (BN/WN).
// K advances one slab (KS) per step.  LDS holds fragments as 16-byte entries
// [k-group][row] with one spare row per k-group against bank conflicts.

template <int FMT, int ACT, int OUTT, bool DUAL, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void tiled_kernel(KArgs a, int Nh, int mtiles, int ntiles)
{
    constexpr int KS = FMT == FMT_Q8 ? 64 : 128;
    constexpr int U = KS / 32;
    constexpr int KG = KS / 8;                     // k-groups of 8 per step
    constexpr int NTHR = WM * WN * 64;
    constexpr int BNT = DUAL ? 2 * BN : BN;        // weight rows staged
    constexpr int XS = BM + 1;                     // LDS row pitch (entries)
    constexpr int WS = BNT + 1;
    constexpr int TM = BM / WM / 16;               // 16-row MFMA tiles per wave (batch)
    constexpr int TN = BN / WN / 16;               // 16-col MFMA tiles per wave (rows n)
    constexpr int XCH = BM * KG / NTHR;            // activation chunks per thread
    constexpr int WCH = (BNT / 16) * 64 / NTHR;    // weight chunks per thread
    static_assert(BM * KG % NTHR == 0, "x chunks");
    static_assert((BNT / 16) * 64 % NTHR == 0, "w chunks");

    __shared__ u32x4 xs[KG * XS];
    __shared__ u32x4 ws[KG * WS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wm = wid % WM;
    const int wn = wid / WM;

    // XCD-aware order: consecutive workgroup ids go to different XCDs, so
    // give each XCD a contiguous range of tiles; batch tiles vary fastest so
    // neighbours share a weight tile.
    const int nwg = gridDim.x;
    int t = blockIdx.x;
    {
        const int per = (nwg + 7) / 8;
        const int xcd = t % 8, loc = t / 8;
        const int full = nwg % 8 == 0 ? 8 : nwg % 8;  // XCDs that own 'per' tiles
        t = xcd < full ? xcd * per + loc : full * per + (xcd - full) * (per - 1) + loc;
    }
    const int mt = t % mtiles;
    const int ntl = t / mtiles;
    const int b0 = mt * BM;
    const int n0 = ntl * BN;                       // first row (gate row for DUAL)
    const int rt_base = n0 / 16;

    const uint8_t *scl = a.w + a.scale_off;

    // register stage for the next K step.  Loads are unconditional (addresses
    // clamped in bounds); out-of-range activations are zeroed when staged, and
    // weight tiles past the last row tile feed columns that are never stored.
    u32x4 xr[XCH][ACT == ACT_F32 ? 2 : 1];
    bool xin[XCH];
    u32x4 wr[WCH];
    uint32_t sr[WCH][2];

    auto load_stage = [&](int s) {
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            const int c = tid + i * NTHR;
            const int row = c / KG, kg = c % KG;
            const int b = b0 + row;
            const int k = s * KS + kg * 8;
            xin[i] = b < a.B && k < a.K;
            const int bc = min(b, a.B - 1), kc = min(k, a.K - 8);
            if constexpr (ACT == ACT_F32) {
                const float *xp = (const float *)a.x + (int64_t)bc * a.K + kc;
                xr[i][0] = *(const u32x4 *)xp;
                xr[i][1] = *(const u32x4 *)(xp + 4);
            } else {
                xr[i][0] = *(const u32x4 *)((const uint16_t *)a.x + (int64_t)bc * a.K + kc);
            }
        }
#pragma unroll
        for (int i = 0; i < WCH; i++) {
            const int c = tid + i * NTHR;
            const int tr = c >> 6, L = c & 63;     // staged row tile, lane chunk
            int rt;
            if constexpr (DUAL)
                rt = tr < BN / 16 ? rt_base + tr : (Nh / 16) + rt_base + (tr - BN / 16);
            else
                rt = rt_base + tr;
            rt = min(rt, a.RT - 1);
            wr[i] = *(const u32x4 *)(a.w + (((int64_t)rt * a.S + s) << 10) + (L << 4));
            const uint8_t *sp = scl + ((int64_t)rt * 16 + (L & 15)) * a.SP;
            if constexpr (FMT == FMT_NV) {
                u32x2 v = *(const u32x2 *)(sp + s * 8);
                sr[i][0] = v[0];
                sr[i][1] = v[1];
            } else {
                sr[i][0] = *(const uint32_t *)(sp + s * 4);
                sr[i][1] = 0;
            }
        }
    };

    auto store_stage = [&]() {
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            const int c = tid + i * NTHR;
            const int row = c / KG, kg = c % KG;
            u32x4 v;
            if constexpr (ACT == ACT_F32) {
                float f[8];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    f[j] = xin[i] ? __uint_as_float(xr[i][0][j]) : 0.f;
                    f[4 + j] = xin[i] ? __uint_as_float(xr[i][1][j]) : 0.f;
                }
                bf16x8 h;
#pragma unroll
                for (int j = 0; j < 8; j++)
                    h[j] = (__bf16)f[j];
                v = __builtin_bit_cast(u32x4, h);
            } else {
                v = xin[i] ? xr[i][0] : u32x4{0u, 0u, 0u, 0u};
            }
            xs[kg * XS + row] = v;
        }
#pragma unroll
        for (int i = 0; i < WCH; i++) {
            const int c = tid + i * NTHR;
            const int tr = c >> 6, L = c & 63;
            const int row = tr * 16 + (L & 15);
            const int g = L >> 4;
#pragma unroll
            for (int u = 0; u < U; u++) {
                bf16x8 h;
                if constexpr (FMT == FMT_Q8) {
                    const float d = fp16_bits_to_f32((sr[i][0] >> (16 * u)) & 0xFFFFu);
                    h = q8_scaled_to_bf16(wr[i][2 * u], wr[i][2 * u + 1], d);
                } else if constexpr (FMT == FMT_MX) {
                    h = fp4_to_bf16(wr[i][u], e8m0_to_f32((sr[i][0] >> (8 * u)) & 0xFFu));
                } else {
                    const int si = 2 * u + (g >> 1);
                    const uint32_t sb = (si < 4 ? sr[i][0] >> (8 * si) : sr[i][1] >> (8 * (si - 4))) & 0xFFu;
                    h = fp4_to_bf16_mul(wr[i][u], e4m3_to_f32(sb));
                }
                ws[(4 * u + g) * WS + row] = __builtin_bit_cast(u32x4, h);
            }
        }
    };

    f32x4 acc[TM][TN];
    f32x4 acc2[DUAL ? TM : 1][DUAL ? TN : 1];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) {
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (DUAL)
                acc2[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    const int nsteps = a.S;
    load_stage(0);
    for (int s = 0; s < nsteps; s++) {
        __syncthreads();  // previous step's fragment reads are done
        store_stage();
        __syncthreads();
        if (s + 1 < nsteps)
            load_stage(s + 1);
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (s * KS + 32 * u >= a.K)
                break;
            const int kg = 4 * u + (lane >> 4);
            bf16x8 af[TM];
#pragma unroll
            for (int i = 0; i < TM; i++)
                af[i] = __builtin_bit_cast(bf16x8, xs[kg * XS + wm * (BM / WM) + 16 * i + (lane & 15)]);
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const int col = wn * (BN / WN) + 16 * j + (lane & 15);
                bf16x8 bw = __builtin_bit_cast(bf16x8, ws[kg * WS + col]);
#pragma unroll
                for (int i = 0; i < TM; i++)
                    acc[i][j] = mfma(af[i], bw, acc[i][j]);
                if constexpr (DUAL) {
                    bf16x8 bu = __builtin_bit_cast(bf16x8, ws[kg * WS + BN + col]);
#pragma unroll
                    for (int i = 0; i < TM; i++)
                        acc2[i][j] = mfma(af[i], bu, acc2[i][j]);
                }
            }
        }
    }

    // ---- epilogue
#pragma unroll
    for (int j = 0; j < TN; j++) {
        const int col = n0 + wn * (BN / WN) + 16 * j + (lane & 15);
        if constexpr (DUAL) {
            if (col >= Nh)
                continue;
            float gg = 1.f, gu = 1.f;
            if constexpr (FMT == FMT_NV) {
                gg = tensor_scale(a, col);
                gu = tensor_scale(a, Nh + col);
            }
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int b = b0 + wm * (BM / WM) + 16 * i + 4 * (lane >> 4) + e;
                    if (b < a.B) {
                        const float G = gg * acc[i][j][e];
                        const float Uv = gu * acc2[i][j][e];
                        store_out<OUTT>(a.y, (int64_t)b * Nh + col, silu(G) * Uv);
                    }
                }
        } else {
            if (col >= a.N)
                continue;
            float g = 1.f;
            if constexpr (FMT == FMT_NV)
                g = tensor_scale(a, col);
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int b = b0 + wm * (BM / WM) + 16 * i + 4 * (lane >> 4) + e;
                    if (b < a.B)
                        store_out<OUTT>(a.y, (int64_t)b * a.N + col, g * acc[i][j][e]);
                }
        }
    }
}

// ============================================================ dequantize
// One thread per (row, 8 consecutive k): fp32 decode with the same decoders.
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(KArgs a, float *out)
{
    constexpr int KS = FMT == FMT_Q8 ? 64 : 128;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t groups = (int64_t)a.K / 8;
    if (idx >= (int64_t)a.N * groups)
        return;
    const int n = (int)(idx / groups);
    const int k0 = (int)(idx % groups) * 8;
    const int s = k0 / KS, u = (k0 % KS) / 32, g = (k0 % 32) / 8;
    const int rt = n / 16, r = n % 16;
    const int L = g * 16 + r;
    const uint8_t *chunk = a.w + (((int64_t)rt * a.S + s) << 10) + (L << 4);
    const uint8_t *sp = a.w + a.scale_off + (int64_t)n * a.SP;
    float v[8];
    if constexpr (FMT == FMT_Q8) {
        const float d = fp16_bits_to_f32(((const uint16_t *)sp)[k0 / 32]);
#pragma unroll
        for (int j = 0; j < 8; j++)
            v[j] = (float)(int8_t)chunk[8 * u + j] * d;
    } else {
        const uint32_t codes = *(const uint32_t *)(chunk + 4 * u);
        float sc;
        if constexpr (FMT == FMT_MX)
            sc = e8m0_to_f32(sp[k0 / 32]);
        else
            sc = e4m3_to_f32(sp[k0 / 16]);
        float gs = 1.f;
        if constexpr (FMT == FMT_NV)
            gs = tensor_scale(a, n);
#pragma unroll
        for (int j = 0; j < 8; j++) {
            float p = e2m1_to_f32((codes >> (4 * j)) & 0xFu) * sc;
            v[j] = FMT == FMT_NV ? gs * p : p;
        }
    }
    float *o = out + (int64_t)n * a.K + k0;
    *(f32x4 *)o = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4 *)(o + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

}  // namespace qg
