// Small-batch GEMV for the narrowest batches (B = 1, 2): fp32 FMA on the
// vector ALUs, one workgroup per 16-row output tile over the whole of K.
//
// The MFMA streaming kernel pads a batch of one or two rows to a 16-row
// matrix-core operand and needs several workgroups per row group along K,
// whose partial tiles then meet through memory at the end of the call (a
// store, a counter and the last workgroup's loads: about 2 us of a 10 us
// call at K = N = 5120).  Here a workgroup owns its rows for all of K, so
// nothing leaves the workgroup before the output store:
//
//  1. every wave issues the weight and scale loads of its first slabs
//     (slabs wid, wid + W, ... of the tile; 16-byte loads, nontemporal,
//     two ring stages of GV_D slabs in flight), then the workgroup stages
//     the B activation rows in LDS as fp32 (bf16 rows widened exactly);
//  2. lane L holds row L % 16 and k-group L / 16 of each 32-wide unit of a
//     slab (the packed layout's 16-byte chunk L); it decodes its 8 weights
//     of a unit to fp32 (int8 and E2M1 / E4M3 codes exactly), multiplies
//     them into the unit's partial with fp32 FMAs against the activations
//     read from LDS, and adds block scale x partial to its running sum;
//  3. the four k-groups of a row are added across lanes in a fixed order
//     (xor 16, then xor 32), the waves' sums in wave order through a small
//     LDS array, and the row sums stored (NVFP4 tensor scale applied; with
//     SwiGLU the workgroup owns a gate tile and the matching up tile and
//     stores SiLU(G) * U).
//
// Summation order is fixed by N and K: a row's result does not depend on B
// within this kernel, nor on the launch.  Products are rounded by fp32 FMA
// (no split of the activations is needed: x * w is formed exactly inside the
// FMA), so the error is that of an fp32 dot product.
#include "common.h"

namespace qg {

constexpr int GV_MAXW = 16;  // waves per workgroup

template <int FMT, int ACT, int NB, int OUTT, bool SWI>
__global__ __launch_bounds__(64 * GV_MAXW) void gemv_kernel(KArgs a, int Nh)
{
    constexpr int KS = slab_k(FMT);
    constexpr int U = KS / 32;                  // 32-wide units per slab
    constexpr int SB = scale_bytes_per_slab(FMT);
    constexpr int NTL = SWI ? 2 : 1;            // row tiles per workgroup
    constexpr int GV_D = SWI ? 2 : 4;           // slabs per ring stage (two stages in flight)
    extern __shared__ float xs[];               // [NB][Kp] fp32 activations, zero past K
    __shared__ float red[GV_MAXW][NTL][NB][16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int W = blockDim.x >> 6;
    const int r = lane & 15, gq = lane >> 4;
    const int Kp = a.S * KS;
    const int nsl = (a.S - wid + W - 1) / W;    // slabs of this wave: wid, wid + W, ...

    int64_t rt[NTL];
    rt[0] = blockIdx.x;
    if constexpr (SWI)
        rt[NTL - 1] = Nh / 16 + blockIdx.x;
    __amdgpu_buffer_rsrc_t wres[NTL], sres[NTL];
#pragma unroll
    for (int t = 0; t < NTL; t++) {
        wres[t] = make_rsrc(a.w + ((rt[t] * a.S) << 10), (int64_t)a.S << 10);
        sres[t] = make_rsrc(a.w + a.scale_off + rt[t] * a.S * (16 * SB), (int64_t)a.S * 16 * SB);
    }

    // ---- 1. ring of weight and scale registers: stage c holds the wave's
    // slabs c * GV_D .. c * GV_D + GV_D - 1 (past the last one: reads
    // through an empty resource, zeros, no memory traffic)
    const __amdgpu_buffer_rsrc_t none = make_rsrc(a.w, 0);
    u32x4 wb[2][GV_D][NTL];
    uint32_t sb[2][GV_D][NTL][2];
    auto load_stage = [&](int buf, int c) {
#pragma unroll
        for (int i = 0; i < GV_D; i++) {
            const int j = c * GV_D + i;
            const bool live = j < nsl;          // uniform
            const int s = live ? wid + W * j : 0;
#pragma unroll
            for (int t = 0; t < NTL; t++) {
                wb[buf][i][t] = bload16_nt(live ? wres[t] : none, lane << 4, s << 10);
                if constexpr (FMT == FMT_NV) {
                    const u32x2 v = bload8_nt(live ? sres[t] : none, r * SB, s * 16 * SB);
                    sb[buf][i][t][0] = v[0];
                    sb[buf][i][t][1] = v[1];
                } else {
                    sb[buf][i][t][0] = bload4_nt(live ? sres[t] : none, r * SB, s * 16 * SB);
                    sb[buf][i][t][1] = 0u;
                }
            }
        }
    };
    load_stage(0, 0);
    load_stage(1, 1);

    // ---- the activations, as fp32, in LDS (K is a multiple of 16, so a
    // 4-element piece is either all in or all out)
    for (int idx = tid * 4; idx < NB * Kp; idx += blockDim.x * 4) {
        const int b = idx / Kp, k = idx - b * Kp;
        f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
        if (k < a.K) {
            if constexpr (ACT == ACT_F32) {
                v = *(const f32x4 *)((const float *)a.x + (int64_t)b * a.K + k);
            } else {
                const u32x2 h = *(const u32x2 *)((const uint16_t *)a.x + (int64_t)b * a.K + k);
                v = f32x4{__uint_as_float(h[0] << 16), __uint_as_float(h[0] & 0xFFFF0000u),
                          __uint_as_float(h[1] << 16), __uint_as_float(h[1] & 0xFFFF0000u)};
            }
        }
        *(f32x4 *)(xs + idx) = v;
    }
    __syncthreads();

    float acc[NTL][NB];
#pragma unroll
    for (int t = 0; t < NTL; t++)
#pragma unroll
        for (int b = 0; b < NB; b++)
            acc[t][b] = 0.f;

    // ---- 2. one slab: per unit, the lane's 8 weights times the activations
    // into a partial, then block scale x partial into the running sum
    auto slab = [&](const u32x4 *w, const uint32_t (*sc)[2], int s) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            // the unit's 8 activations of each batch row (k-group gq)
            float xv[NB][8];
#pragma unroll
            for (int b = 0; b < NB; b++) {
                const float *p = xs + b * Kp + s * KS + 32 * u + 8 * gq;
                const f32x4 lo = *(const f32x4 *)p, hi = *(const f32x4 *)(p + 4);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    xv[b][e] = lo[e];
                    xv[b][4 + e] = hi[e];
                }
            }
#pragma unroll
            for (int t = 0; t < NTL; t++) {
                const u32x4 wc = w[t];
                const uint32_t s0 = sc[t][0], s1 = sc[t][1];
                float wv[8];
                float bs;
                if constexpr (FMT == FMT_Q8) {
                    const uint32_t lo = wc[2 * u], hi = wc[2 * u + 1];
                    wv[0] = sbyte_to_f32<0>(lo); wv[1] = sbyte_to_f32<1>(lo);
                    wv[2] = sbyte_to_f32<2>(lo); wv[3] = sbyte_to_f32<3>(lo);
                    wv[4] = sbyte_to_f32<0>(hi); wv[5] = sbyte_to_f32<1>(hi);
                    wv[6] = sbyte_to_f32<2>(hi); wv[7] = sbyte_to_f32<3>(hi);
                    bs = fp16_bits_to_f32((s0 >> (16 * u)) & 0xFFFFu);
                } else if constexpr (FMT == FMT_FP8) {
                    const uint32_t lo = wc[2 * u], hi = wc[2 * u + 1];
                    const f32x2 f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
                    const f32x2 f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
                    const f32x2 f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
                    const f32x2 f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
                    wv[0] = f0[0]; wv[1] = f0[1]; wv[2] = f1[0]; wv[3] = f1[1];
                    wv[4] = f2[0]; wv[5] = f2[1]; wv[6] = f3[0]; wv[7] = f3[1];
                    bs = __uint_as_float(s0);   // the slab's 128-wide block scale
                } else {
                    const uint32_t v = wc[u];
                    const f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 0);
                    const f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 1);
                    const f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 2);
                    const f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 3);
                    wv[0] = f0[0]; wv[1] = f0[1]; wv[2] = f1[0]; wv[3] = f1[1];
                    wv[4] = f2[0]; wv[5] = f2[1]; wv[6] = f3[0]; wv[7] = f3[1];
                    if constexpr (FMT == FMT_MX) {
                        bs = e8m0_to_f32((s0 >> (8 * u)) & 0xFFu);
                    } else {
                        // this lane's 16-wide block of unit u: scale byte 2u + gq/2
                        const uint32_t sv = (u < 2 ? s0 : s1) >> (16 * (u & 1) + 8 * (gq >> 1));
                        bs = e4m3_to_f32(sv & 0xFFu);
                    }
                }
#pragma unroll
                for (int b = 0; b < NB; b++) {
                    float p = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        p = __builtin_fmaf(xv[b][e], wv[e], p);
                    acc[t][b] = __builtin_fmaf(bs, p, acc[t][b]);
                }
            }
        }
    };

    // two stages per trip so every ring index is static
    for (int c = 0; c * GV_D < nsl; c += 2) {
#pragma unroll
        for (int i = 0; i < GV_D; i++)
            if (c * GV_D + i < nsl)  // uniform
                slab(wb[0][i], sb[0][i], wid + W * (c * GV_D + i));
        load_stage(0, c + 2);
        if ((c + 1) * GV_D >= nsl)
            break;
#pragma unroll
        for (int i = 0; i < GV_D; i++)
            if ((c + 1) * GV_D + i < nsl)
                slab(wb[1][i], sb[1][i], wid + W * ((c + 1) * GV_D + i));
        load_stage(1, c + 3);
    }

    // ---- 3. the row's four k-groups in a fixed order, then the waves
#pragma unroll
    for (int t = 0; t < NTL; t++)
#pragma unroll
        for (int b = 0; b < NB; b++) {
            float v = acc[t][b];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            if (lane < 16)
                red[wid][t][b][r] = v;
        }
    __syncthreads();
    if (tid >= NB * 16)
        return;
    const int b = tid / 16;
    float sum[NTL];
#pragma unroll
    for (int t = 0; t < NTL; t++) {
        sum[t] = 0.f;
        for (int w2 = 0; w2 < W; w2++)
            sum[t] += red[w2][t][b][r];
    }
    if constexpr (SWI) {
        const int col = (int)rt[0] * 16 + r;
        float g0 = 1.f, g1 = 1.f;
        if constexpr (FMT == FMT_NV) {
            g0 = tensor_scale(a, col);
            g1 = tensor_scale(a, Nh + col);
        }
        if (b < a.B && col < Nh)
            store_out_nt<OUTT>(a.y, (int64_t)b * Nh + col, silu(g0 * sum[0]) * (g1 * sum[1]));
    } else {
        const int n = (int)rt[0] * 16 + r;
        float gs = 1.f;
        if constexpr (FMT == FMT_NV)
            gs = tensor_scale(a, n);
        if (b < a.B && n < a.N)
            store_out_nt<OUTT>(a.y, (int64_t)b * a.N + n, gs * sum[0]);
    }
}

// ------------------------------------------------------------------ host

template <int FMT, int ACT, int NB, int OUTT>
static void launch_g(const KArgs &a, int W, int Nh, hipStream_t st)
{
    const size_t lds = (size_t)NB * a.S * slab_k(FMT) * sizeof(float);
    const unsigned grid = (unsigned)(Nh ? Nh / 16 : a.RT);
    if (Nh)
        hipLaunchKernelGGL((gemv_kernel<FMT, ACT, NB, OUTT, true>), dim3(grid), dim3(64 * W), lds, st, a, Nh);
    else
        hipLaunchKernelGGL((gemv_kernel<FMT, ACT, NB, OUTT, false>), dim3(grid), dim3(64 * W), lds, st, a, Nh);
}

template <int FMT>
static void launch_gf(const Problem &p, const KArgs &a, int W, int Nh, hipStream_t st)
{
    const bool f32 = p.act == QGEMM_F32, o32 = p.out == QGEMM_F32;
    if (a.B == 1) {
        if (f32) { if (o32) launch_g<FMT, ACT_F32, 1, OUT_F32>(a, W, Nh, st); else launch_g<FMT, ACT_F32, 1, OUT_BF16>(a, W, Nh, st); }
        else { if (o32) launch_g<FMT, ACT_BF16, 1, OUT_F32>(a, W, Nh, st); else launch_g<FMT, ACT_BF16, 1, OUT_BF16>(a, W, Nh, st); }
    } else {
        if (f32) { if (o32) launch_g<FMT, ACT_F32, 2, OUT_F32>(a, W, Nh, st); else launch_g<FMT, ACT_F32, 2, OUT_BF16>(a, W, Nh, st); }
        else { if (o32) launch_g<FMT, ACT_BF16, 2, OUT_F32>(a, W, Nh, st); else launch_g<FMT, ACT_BF16, 2, OUT_BF16>(a, W, Nh, st); }
    }
}

// 8 waves: a workgroup small enough that several are resident on a CU (16
// waves, one workgroup per CU, measured 10.8 against 9.4 us on Q8_0 5120^2
// at B = 1; 4 waves 9.1 there but 18.5 against 16.8 on MXFP4 5120x17408)
constexpr int GV_W = 8;
int gemv_waves(const Problem &p) { return (int)(p.L.S < GV_W ? p.L.S : GV_W); }

int64_t gemv_lds_bytes(const Problem &p, int64_t B) { return B * p.L.S * p.L.KS * 4; }

hipError_t launch_gemv(const Problem &p, const KArgs &a, hipStream_t st)
{
    const int W = gemv_waves(p);
    const int Nh = p.epi == QGEMM_EPI_SWIGLU ? (int)(p.N / 2) : 0;
    switch (p.fmt) {
    case FMT_Q8: launch_gf<FMT_Q8>(p, a, W, Nh, st); break;
    case FMT_MX: launch_gf<FMT_MX>(p, a, W, Nh, st); break;
    case FMT_FP8: launch_gf<FMT_FP8>(p, a, W, Nh, st); break;
    default: launch_gf<FMT_NV>(p, a, W, Nh, st); break;
    }
    return hipGetLastError();
}

}  // namespace qg
