// Small-batch tier: packed weights streamed once from HBM straight into MFMA
// operands.
//
// A workgroup is 4 waves.  It owns RG = 4*NT row tiles (64*NT weight rows),
// one batch group of 16*MB rows and a range of kc K-slabs; wave w computes
// row tiles w*NT .. w*NT+NT-1 over that range.
//
//  * Activations of the range are staged in LDS once per workgroup, already
//    split into the bf16 terms the MFMAs take (for fp32 input the terms add up
//    to the exact fp32 value), and shared by the four waves.
//  * Each lane's 16-byte chunk of a weight slab is already its B operand of
//    v_mfma_f32_16x16x32_bf16 (row lane % 16, k-group lane / 16); it is
//    decoded in registers (int8 and E2M1 exactly; NVFP4 times its E4M3 scale,
//    also exact).  Waves keep a ring of D slabs in flight with no barrier.
//  * Q8_0 and MXFP4 block scales multiply the fp32 partial of each 32-wide
//    block, so a block's sum is exact before it is scaled.
//  * Summation order, shared with the B <= 16 streaming kernel so a batch
//    row's result does not depend on B: per slab, its units in order into a
//    partial from zero, partials added to the running tile in slab order.
//
// Loads are unconditional (slab, row and column indices clamped in bounds;
// out-of-range activations zeroed when staged), so no register is written on
// a side path while a load into it is in flight, and the compiler can count
// loads across the ring.  Padding slabs skip only the arithmetic; tiles past
// the last row tile compute on a copy of it and are never stored.
//
// K split.  With a workspace, K is split over `ksplit` workgroups per output
// tile.  Each publishes its partial tile with device-scope stores (written
// through to the point of coherence), waits for them to be acknowledged and
// bumps a device-scope counter; the last to arrive reads the other partials
// with device-scope loads, adds all of them in split order (so the result
// does not depend on arrival order), applies the epilogue and re-arms the
// counter.  No device-wide fence is used: on gfx950 that would write back and
// invalidate the whole L2 of the XCD for every workgroup.
#include "common.h"

namespace qg {

template <int FMT, int ACT, int NTERM, int MB, int NT, int D, int OUTT>
__global__ __launch_bounds__(256) void skinny_kernel(KArgs a, SkinnyWs ws)
{
    constexpr int KS = slab_k(FMT);
    constexpr int U = KS / 32;                 // 32-wide units per slab
    constexpr bool POST = FMT != FMT_NV;       // block scale applied after the MFMA
    constexpr int NTA = ACT == ACT_F32 ? NTERM : 1;
    constexpr int BR = 16 * MB;                // batch rows per workgroup
    constexpr int CE = ACT == ACT_F32 ? 4 : 8; // activations per 16-byte chunk
    constexpr int NCH = BR * KS / CE;          // chunks per slab
    constexpr int XB = 8;                      // chunk loads in flight per thread
    constexpr int SLAB_E = NTA * MB * U * 64;  // 16-byte LDS entries per slab

    extern __shared__ u32x4 xs[];              // [kch][NTA][MB][U][64]
    __shared__ int s_is_last;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int r = lane & 15, gq = lane >> 4;
    const int grp = blockIdx.x, ks = blockIdx.y, by = blockIdx.z;
    const int ngroups = gridDim.x;
    const int rt0 = (grp * 4 + wid) * NT;
    const int b0 = by * BR;
    const int s_beg = ks * ws.kc;
    const int s_end = min(a.S, s_beg + ws.kc);
    const int s_last = s_end - 1;

    f32x4 acc[MB][NT];
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
            acc[mb][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- weight ring
    u32x4 wr[D][NT];
    uint32_t sr[D][NT][2];
    auto wload = [&](int j, int s) {
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
            const int64_t rt = min(rt0 + nt, a.RT - 1);
            wr[j][nt] = *(const u32x4 *)(a.w + ((rt * a.S + s) << 10) + (lane << 4));
            const uint8_t *sp = slab_scales<FMT>(a, rt, r, s);
            if constexpr (FMT == FMT_NV) {
                const u32x2 v = *(const u32x2 *)sp;
                sr[j][nt][0] = v[0];
                sr[j][nt][1] = v[1];
            } else {
                sr[j][nt][0] = *(const uint32_t *)sp;
                sr[j][nt][1] = 0;
            }
        }
    };

    // ---- activation staging: global -> registers -> (split) -> LDS, in
    // batches of XB chunks per thread.  Threads past the last chunk repeat it
    // (same bytes to the same place) instead of branching.
    auto xissue = [&](int c_beg, int total, int c0, u32x4 (&xr)[XB], bool (&xin)[XB]) {
#pragma unroll
        for (int i = 0; i < XB; i++) {
            const int c = min(c0 + tid + i * 256, total - 1);
            const int sl = c / NCH, cc = c % NCH;
            const int row = cc / (KS / CE), kk = (cc % (KS / CE)) * CE;
            const int b = b0 + row, k = (c_beg + sl) * KS + kk;
            xin[i] = b < a.B && k < a.K;  // K % 16 == 0: a chunk is all in or all out
            const int bc = min(b, a.B - 1), kcl = min(k, a.K - CE);
            if constexpr (ACT == ACT_F32)
                xr[i] = *(const u32x4 *)((const float *)a.x + (int64_t)bc * a.K + kcl);
            else
                xr[i] = *(const u32x4 *)((const uint16_t *)a.x + (int64_t)bc * a.K + kcl);
        }
    };
    auto xstore = [&](int total, int c0, const u32x4 (&xr)[XB], const bool (&xin)[XB]) {
#pragma unroll
        for (int i = 0; i < XB; i++) {
            const int c = min(c0 + tid + i * 256, total - 1);
            const int sl = c / NCH, cc = c % NCH;
            const int row = cc / (KS / CE), kk = (cc % (KS / CE)) * CE;
            const int mb = row >> 4, b = row & 15;
            const int u = kk >> 5, g8 = (kk & 31) >> 3;
            const u32x4 xv = masked(xr[i], keep_mask(xin[i]));
            u32x4 *slab = xs + sl * SLAB_E;
            if constexpr (ACT == ACT_F32) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; e++)
                    v[e] = __uint_as_float(xv[e]);
                const Split<NTA> sp = split_f32<NTA, 4>(v);
                const int half = (kk & 7) >> 2;  // which 8 bytes of the entry
#pragma unroll
                for (int t = 0; t < NTA; t++) {
                    const u32x4 q = __builtin_bit_cast(u32x4, sp.t[t]);
                    u32x2 *dst = (u32x2 *)&slab[((t * MB + mb) * U + u) * 64 + g8 * 16 + b] + half;
                    *dst = u32x2{q[0], q[1]};
                }
            } else {
                slab[(mb * U + u) * 64 + g8 * 16 + b] = xv;
            }
        }
    };
    auto stage = [&](int c_beg, int c0_from) {
        const int total = (min(s_end, c_beg + ws.kch) - c_beg) * NCH;
        for (int c0 = c0_from; c0 < total; c0 += 256 * XB) {
            u32x4 xr[XB];
            bool xin[XB];
            xissue(c_beg, total, c0, xr, xin);
            xstore(total, c0, xr, xin);
        }
    };

    // First chunk: its first activation batch is issued before the weight
    // ring, because a wave's loads return in issue order and the activations
    // (L2-resident) must not wait behind the HBM weight loads.
    {
        const int total = (min(s_end, s_beg + ws.kch) - s_beg) * NCH;
        u32x4 xr[XB];
        bool xin[XB];
        xissue(s_beg, total, 0, xr, xin);
#pragma unroll
        for (int j = 0; j < D; j++)
            wload(j, min(s_beg + j, s_last));
        xstore(total, 0, xr, xin);
        stage(s_beg, 256 * XB);
    }
    __syncthreads();

    for (int c_beg = s_beg;;) {
        // ---- stream the weights of slabs [c_beg, c_beg + kch)
        for (int s0 = c_beg; s0 < c_beg + ws.kch; s0 += D) {
#pragma unroll
            for (int j = 0; j < D; j++) {
                const int s = s0 + j;
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
                const u32x4 *slab = xs + (s - c_beg) * SLAB_E;
                f32x4 part[MB][NT];  // this slab's partial tiles, from zero
#pragma unroll
                for (int mb = 0; mb < MB; mb++)
#pragma unroll
                    for (int nt = 0; nt < NT; nt++)
                        part[mb][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
                for (int u = 0; u < U; u++) {
                    if (s * KS + 32 * u >= a.K)
                        break;  // padding units of the last slab (uniform)
                    bf16x8 A[MB][NTA];
#pragma unroll
                    for (int mb = 0; mb < MB; mb++)
#pragma unroll
                        for (int t = 0; t < NTA; t++)
                            A[mb][t] = __builtin_bit_cast(bf16x8, slab[((t * MB + mb) * U + u) * 64 + lane]);
#pragma unroll
                    for (int nt = 0; nt < NT; nt++) {
                        bf16x8 Bw;
                        float ps = 1.f;
                        if constexpr (FMT == FMT_Q8) {
                            Bw = q8_to_bf16(wc[nt][2 * u], wc[nt][2 * u + 1]);
                            ps = fp16_bits_to_f32((sc[nt][0] >> (16 * u)) & 0xFFFFu);
                        } else if constexpr (FMT == FMT_FP8) {
                            Bw = fp8_to_bf16(wc[nt][2 * u], wc[nt][2 * u + 1]);
                            ps = __uint_as_float(sc[nt][0]);  // the slab's block scale
                        } else if constexpr (FMT == FMT_MX) {
                            Bw = fp4_to_bf16(wc[nt][u], 1.0f);
                            ps = e8m0_to_f32((sc[nt][0] >> (8 * u)) & 0xFFu);
                        } else {
                            const int si = 2 * u + (gq >> 1);
                            const uint32_t sb =
                                (si < 4 ? sc[nt][0] >> (8 * si) : sc[nt][1] >> (8 * (si - 4))) & 0xFFu;
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
                                    part[mb][nt][i] = __builtin_fmaf(ps, t[i], part[mb][nt][i]);
                            } else {
#pragma unroll
                                for (int tt = 0; tt < NTA; tt++)
                                    part[mb][nt] = mfma(A[mb][tt], Bw, part[mb][nt]);
                            }
                        }
                    }
                }
#pragma unroll
                for (int mb = 0; mb < MB; mb++)
#pragma unroll
                    for (int nt = 0; nt < NT; nt++) {
                        acc[mb][nt][0] += part[mb][nt][0];
                        acc[mb][nt][1] += part[mb][nt][1];
                        acc[mb][nt][2] += part[mb][nt][2];
                        acc[mb][nt][3] += part[mb][nt][3];
                    }
            }
        }
        c_beg += ws.kch;
        if (c_beg >= s_beg + ws.kc)
            break;
        __syncthreads();  // every wave is done with the staged chunk
        stage(c_beg, 0);
        __syncthreads();
    }

    // ---- K split: publish the partial; the last workgroup of the tile reduces
    if (ws.ksplit > 1) {
        const int64_t tiles = (int64_t)gridDim.z * ngroups * 4 * MB * NT;
        const int64_t tbase = (((int64_t)by * ngroups + grp) * 4 + wid) * (MB * NT);
        uint64_t *part = (uint64_t *)ws.part;
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                publish_partial<__HIP_MEMORY_SCOPE_AGENT>(part, ks, tiles, tbase + mb * NT + nt, lane, acc[mb][nt]);
            }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are acknowledged
        __syncthreads();
        if (tid == 0) {
            const uint32_t old = __hip_atomic_fetch_add(&ws.cnt[by * ngroups + grp], 1u,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_is_last = old == (uint32_t)(ws.ksplit - 1);
        }
        __syncthreads();
        if (!s_is_last)
            return;
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
            for (int nt = 0; nt < NT; nt++)
                acc[mb][nt] = reduce_partials(part, ws.ksplit, ks, tiles, tbase + mb * NT + nt, lane, acc[mb][nt]);
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

// ------------------------------------------------------------------ host

template <int FMT, int ACT, int NTERM, int MB, int NT, int OUTT>
static void launch_k(const KArgs &a, const SkCfg &c, const SkinnyWs &ws, hipStream_t st)
{
    const dim3 grid((unsigned)c.ngroups, (unsigned)c.ksplit, (unsigned)c.nby);
    hipLaunchKernelGGL((skinny_kernel<FMT, ACT, NTERM, MB, NT, SK_RING, OUTT>), grid, dim3(256), c.lds, st,
                       a, ws);
}

template <int FMT, int ACT, int NTERM, int OUTT>
static void launch_t(const KArgs &a, const SkCfg &c, const SkinnyWs &ws, hipStream_t st)
{
#define QG_S(MB, NT) launch_k<FMT, ACT, NTERM, MB, NT, OUTT>(a, c, ws, st)
    if (c.NT == 1) {
        if (c.MB == 1) QG_S(1, 1); else if (c.MB == 2) QG_S(2, 1); else QG_S(4, 1);
    } else {
        if (c.MB == 1) QG_S(1, 2); else if (c.MB == 2) QG_S(2, 2); else QG_S(4, 2);
    }
#undef QG_S
}

template <int FMT>
static void launch_f(const Problem &p, const KArgs &a, const SkCfg &c, const SkinnyWs &ws, int nterm,
                     hipStream_t st)
{
    const bool o32 = p.out == QGEMM_F32;
    if (p.act != QGEMM_F32) {
        if (o32) launch_t<FMT, ACT_BF16, 1, OUT_F32>(a, c, ws, st);
        else launch_t<FMT, ACT_BF16, 1, OUT_BF16>(a, c, ws, st);
    } else if (nterm == 1) {
        if (o32) launch_t<FMT, ACT_F32, 1, OUT_F32>(a, c, ws, st);
        else launch_t<FMT, ACT_F32, 1, OUT_BF16>(a, c, ws, st);
    } else if (nterm == 2) {
        if (o32) launch_t<FMT, ACT_F32, 2, OUT_F32>(a, c, ws, st);
        else launch_t<FMT, ACT_F32, 2, OUT_BF16>(a, c, ws, st);
    } else {
        if (o32) launch_t<FMT, ACT_F32, 3, OUT_F32>(a, c, ws, st);
        else launch_t<FMT, ACT_F32, 3, OUT_BF16>(a, c, ws, st);
    }
}

hipError_t launch_skinny(const Problem &p, const KArgs &a, const SkCfg &c, const SkinnyWs &ws, int nterm,
                         hipStream_t st)
{
    switch (p.fmt) {
    case FMT_Q8: launch_f<FMT_Q8>(p, a, c, ws, nterm, st); break;
    case FMT_MX: launch_f<FMT_MX>(p, a, c, ws, nterm, st); break;
    case FMT_FP8: launch_f<FMT_FP8>(p, a, c, ws, nterm, st); break;
    default: launch_f<FMT_NV>(p, a, c, ws, nterm, st); break;
    }
    return hipGetLastError();
}

}  // namespace qg
