// Small-batch tier, B <= 16: weights streamed once from HBM straight into
// MFMA operands, every load of a workgroup issued at once.
//
// A workgroup is W waves (8..16) and owns 8 row tiles (128 weight rows) and a
// range of K slabs, walked in chunks of KC = W * NPH slabs (with a workspace
// the range is one chunk).  The host picks W and NPH so that the grid is at
// most one workgroup per CU with the least work on the busiest CU: a CU's
// memory requests drain at a bounded rate, so the busiest CU sets the time.
// Within a chunk, wave w owns the slabs w, w + W, ... (one per phase) across
// all 8 row tiles:
//
//  1. it loads the activations of its own slabs straight into registers (no
//     LDS, no barrier: each wave reads only the 16 batch rows x KS columns it
//     multiplies), then every weight and scale load of its slabs, each into
//     its own registers; nothing is loop-carried, so no wait ever drains the
//     loads still in flight;
//  2. it splits fp32 activations into bf16 terms that add up to the fp32
//     value (bf16 activations are used as they are), decodes each row tile's
//     slab in registers (int8 and E2M1 exact; NVFP4 times its E4M3 scale,
//     also exact) and runs v_mfma_f32_16x16x32_bf16 per 32-wide unit, Q8_0 /
//     MXFP4 block scales applied to the fp32 block partial, giving one
//     partial tile per (slab, row tile);
//  3. the waves exchange partial tiles through LDS and wave t < 8 adds the
//     partials of row tile t in slab order.
//
// Because each activation fragment is read by one wave only, LDS carries
// just the partial tiles, not eight copies of the activations.
//
// Fused gate+up (SwiGLU): a workgroup's 8 row tiles are 4 gate tiles and the
// 4 matching up tiles, so after the reduction G and U of an output column are
// exchanged through LDS and the workgroup stores SiLU(G) * U.
//
// Summation order (also used by the B > 16 kernel, so a batch row's result
// does not depend on B): per slab, its units in order into a partial from
// zero; partials added to the running tile in slab order; K splits added in
// split order by the last workgroup of a row group to arrive (partial-tile
// stores, a device-scope counter, no device-wide fence).  The partial tiles
// go through device-coherent memory, or, when the dispatcher is known to put
// workgroup ids congruent mod 8 on one XCD and all splits of a row group are
// given such ids, through that XCD's L2 (workgroup-scope stores, which that
// L2 acknowledges without writing them through to memory, and
// workgroup-scope loads).
#include "common.h"

namespace qg {

template <int FMT, int ACT, int NTERM, int NPH, int OUTT, bool FULLK, int PDEPTH>
__global__ __launch_bounds__(64 * st_max_waves(NPH)) void stream_kernel(KArgs a, SkinnyWs ws, int ngroups, int Nh)
{
    constexpr int KS = slab_k(FMT);
    constexpr int U = KS / 32;                 // 32-wide units per slab
    constexpr int NTA = ACT == ACT_F32 ? NTERM : 1;
    constexpr int XPU = ACT == ACT_F32 ? 2 : 1;  // 16-byte activation loads per unit
    constexpr int XB = ACT == ACT_F32 ? 4 : 2;   // bytes per activation
    constexpr int SBYTES = FMT == FMT_NV ? 8 : 4;    // scale bytes per row and slab

    extern __shared__ f32x4 red[];             // [W][ST_RG][64]: one phase's partial tiles
    __shared__ int s_is_last;

    const int tid = threadIdx.x, lane = tid & 63;
    // wave index as a scalar: everything derived from it (slab, offsets, the
    // idle-slab test) stays in scalar registers and branches
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int W = blockDim.x >> 6;             // waves = slabs per phase
    const int KC = W * NPH;                    // slabs per chunk
    const int r = lane & 15, gq = lane >> 4;

    // XCD-aware order: consecutive workgroup ids go to different XCDs (id mod
    // 8).  With the XCD-local exchange, XCD x runs the row groups x, x + 8,
    // ..., each with all its K splits in a row (workgroups past the last
    // group leave at once); otherwise each XCD gets a contiguous run of
    // (split, group) pairs, split major, so an XCD's workgroups share few
    // activation slices in its L2.
    int ks, grp;
    if (ws.xlocal) {
        const int xcd = blockIdx.x % 8, loc = blockIdx.x / 8;
        grp = (loc / ws.ksplit) * 8 + xcd;
        ks = loc % ws.ksplit;
        if (grp >= ngroups)
            return;  // uniform over the workgroup
    } else {
        const int nwg = gridDim.x;
        const int per = (nwg + 7) / 8;
        const int xcd = blockIdx.x % 8, loc = blockIdx.x / 8;
        const int full = nwg % 8 == 0 ? 8 : nwg % 8;
        const int t = xcd < full ? xcd * per + loc : full * per + (xcd - full) * (per - 1) + loc;
        ks = t / ngroups;
        grp = t % ngroups;
    }
    // the group's row tiles g = 0..7: 8 consecutive ones, or with SwiGLU
    // (Nh > 0) 4 gate tiles and the 4 matching up tiles Nh/16 further on
    const int rt0 = Nh ? grp * (ST_RG / 2) : grp * ST_RG;
    const int s_beg = ks * ws.kc;
    const int s_end = min(a.S, s_beg + ws.kc);
    // activation row of this lane: rows past B read row B-1 (they only feed
    // output rows that are never stored)
    const int xb = min(r, a.B - 1);

    // Per-lane byte offsets.  Every per-tile and per-slab part of an address
    // goes into a scalar buffer resource (or scalar offset), so no load needs
    // vector address arithmetic.
    const int xvoff = (xb * a.K + 8 * gq) * XB;
    const int wvoff = lane << 4, svoff = r * SBYTES;
    const uint32_t nvsh = 8 * (gq >> 1);  // NVFP4: this lane's scale byte within a unit's pair
    const __amdgpu_buffer_rsrc_t xres = make_rsrc(a.x, (int64_t)a.B * a.K * XB);
    // row tile of the group's tile g (tiles past the last read a copy of it;
    // their outputs are never stored)
    auto tile_of = [&](int g) -> int64_t {
        const int rt = Nh ? (g < ST_RG / 2 ? rt0 + g : Nh / 16 + rt0 + g - ST_RG / 2) : rt0 + g;
        return min(rt, a.RT - 1);
    };

    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};     // running sum of row tile `wid`

    for (int c_beg = s_beg; c_beg < s_end; c_beg += KC) {
        // ---- 1. activations of this wave's slabs, then their weights and
        // scales.  A wave with no slab in a phase (the end of the last split)
        // reads activations of a valid slab, and its weight and scale loads
        // go through empty resources: zeros, no memory traffic.  (Branching
        // around them instead costs registers the compiler then spills.)
        u32x4 xr[NPH][U][XPU];
        uint32_t xm[NPH][U];
#pragma unroll
        for (int ph = 0; ph < NPH; ph++) {
            const int sc = min(c_beg + ph * W + wid, a.S - 1);
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int k0 = sc * KS + 32 * u;  // first column of the unit
                int vo = xvoff, so = k0 * XB;
                if constexpr (FULLK) {
                    xm[ph][u] = 0xFFFFFFFFu;
                } else {
                    // K % 16 == 0: a lane's 8 columns are all in or all out
                    const int k = k0 + 8 * gq;
                    xm[ph][u] = keep_mask(k < a.K);
                    vo = (xb * a.K + min(k, a.K - 8)) * XB;
                    so = 0;
                }
                xr[ph][u][0] = bload16(xres, vo, so);
                if constexpr (XPU == 2)
                    xr[ph][u][1] = bload16(xres, vo, so + 16);
            }
        }
        // Keep the activation loads ahead of the weight loads: a wave's loads
        // return in issue order, and the compiler would otherwise sink some
        // of them below the weights, making the first MFMA wait for every
        // weight byte of the wave.
        __builtin_amdgcn_sched_barrier(0);
        // Weight and scale loads, one item per (phase, row tile): the first
        // PD items now, then item i + PD just before item i is computed, so a
        // wave's data arrive in the order it uses them and its decode and
        // MFMA work overlaps the rest of the stream (PD >= NI: all at once).
        constexpr int NI = NPH * ST_RG;
        constexpr int PD = PDEPTH < NI ? PDEPTH : NI;
        u32x4 wr[NPH][ST_RG];
        uint32_t sr[NPH][ST_RG][2];
        auto issue = [&](int i) {
            const int ph = i / ST_RG, g = i % ST_RG;
            const int s = c_beg + ph * W + wid;
            const int sc = min(s, a.S - 1);
            const bool live = s < s_end;
            const int64_t rt = tile_of(g);
            wr[ph][g] = bload16_nt(make_rsrc(a.w + ((rt * a.S + sc) << 10), live ? 1024 : 0), wvoff, 0);
            const __amdgpu_buffer_rsrc_t srs = make_rsrc(
                a.w + a.scale_off + (rt * a.S + sc) * (16 * SBYTES), live ? 16 * SBYTES : 0);
            if constexpr (FMT == FMT_NV) {
                const u32x2 v = bload8_nt(srs, svoff, 0);
                sr[ph][g][0] = v[0];
                sr[ph][g][1] = v[1];
            } else {
                sr[ph][g][0] = bload4_nt(srs, svoff, 0);
                sr[ph][g][1] = 0u;
            }
        };
#pragma unroll
        for (int i = 0; i < PD; i++)
            issue(i);
        __builtin_amdgcn_sched_barrier(0);

#pragma unroll
        for (int ph = 0; ph < NPH; ph++) {
            const int s = c_beg + ph * W + wid;  // this wave's slab
            const bool live = s < s_end;         // uniform
            // units past K (padding of the last slab) are left out
            const int nu = FULLK ? U : min(U, (a.K - s * KS + 31) / 32);

            // ---- 2. activation operands, then one partial tile per row tile
            bf16x8 A[U][NTA];
            if (live) {
#pragma unroll
                for (int u = 0; u < U; u++) {
                    if constexpr (ACT == ACT_F32) {
                        float v[8];
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            v[e] = __uint_as_float(xr[ph][u][0][e] & xm[ph][u]);
                            v[4 + e] = __uint_as_float(xr[ph][u][XPU - 1][e] & xm[ph][u]);
                        }
                        const Split<NTA> sp = split_f32<NTA, 8>(v);
#pragma unroll
                        for (int tt = 0; tt < NTA; tt++)
                            A[u][tt] = sp.t[tt];
                    } else {
                        A[u][0] = __builtin_bit_cast(bf16x8, masked(xr[ph][u][0], xm[ph][u]));
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < ST_RG; g++) {
                if (PD < NI && ph * ST_RG + g + PD < NI) {
                    issue(ph * ST_RG + g + PD);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (live) {
                    const u32x4 wc = wr[ph][g];
                    const uint32_t s0 = sr[ph][g][0], s1 = sr[ph][g][1];
                    f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int u = 0; u < U; u++) {
                        if (!FULLK && u >= nu)
                            continue;  // uniform
                        if constexpr (FMT == FMT_Q8) {
                            const bf16x8 Bw = q8_to_bf16(wc[2 * u], wc[2 * u + 1]);
                            f32x4 tacc = mfma(A[u][0], Bw, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                            for (int tt = 1; tt < NTA; tt++)
                                tacc = mfma(A[u][tt], Bw, tacc);
                            const float ps = fp16_bits_to_f32((s0 >> (16 * u)) & 0xFFFFu);
#pragma unroll
                            for (int i = 0; i < 4; i++)
                                part[i] = __builtin_fmaf(ps, tacc[i], part[i]);
                        } else if constexpr (FMT == FMT_FP8) {
                            const bf16x8 Bw = fp8_to_bf16(wc[2 * u], wc[2 * u + 1]);
                            f32x4 tacc = mfma(A[u][0], Bw, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                            for (int tt = 1; tt < NTA; tt++)
                                tacc = mfma(A[u][tt], Bw, tacc);
                            const float ps = __uint_as_float(s0);  // the slab's block scale
#pragma unroll
                            for (int i = 0; i < 4; i++)
                                part[i] = __builtin_fmaf(ps, tacc[i], part[i]);
                        } else if constexpr (FMT == FMT_MX) {
                            const bf16x8 Bw = fp4_to_bf16(wc[u], 1.0f);
                            f32x4 tacc = mfma(A[u][0], Bw, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                            for (int tt = 1; tt < NTA; tt++)
                                tacc = mfma(A[u][tt], Bw, tacc);
                            const float ps = e8m0_to_f32((s0 >> (8 * u)) & 0xFFu);
#pragma unroll
                            for (int i = 0; i < 4; i++)
                                part[i] = __builtin_fmaf(ps, tacc[i], part[i]);
                        } else {
                            // this lane's block of unit u: byte 2u + gq/2 of the row's
                            // 8 scale bytes (shifted to a fixed byte position first)
                            const uint32_t sv = (u < 2 ? s0 : s1) >> nvsh;
                            const float bs = (u & 1) ? e4m3_byte_to_f32<2>(sv) : e4m3_byte_to_f32<0>(sv);
                            const bf16x8 Bw = fp4_to_bf16_mul(wc[u], bs);
#pragma unroll
                            for (int tt = 0; tt < NTA; tt++)
                                part = mfma(A[u][tt], Bw, part);
                        }
                    }
                    red[(wid * ST_RG + g) * 64 + lane] = part;
                }
            }
            __syncthreads();

            // ---- 3. wave t < 8 adds row tile t's partials in slab order (all
            // read first, so the LDS latencies overlap)
            if (wid < ST_RG) {
                f32x4 v[st_max_waves(NPH)];
#pragma unroll
                for (int w2 = 0; w2 < st_max_waves(NPH); w2++)
                    v[w2] = red[(min(w2, W - 1) * ST_RG + wid) * 64 + lane];
                const int nv = min(W, s_end - (c_beg + ph * W));  // waves with a slab
#pragma unroll
                for (int w2 = 0; w2 < st_max_waves(NPH); w2++) {
                    if (w2 < nv) {  // uniform: a scalar branch, not a select per add
                        asm volatile("");
                        acc[0] += v[w2][0]; acc[1] += v[w2][1]; acc[2] += v[w2][2]; acc[3] += v[w2][3];
                    }
                }
            }
            __syncthreads();  // partials consumed before the next phase writes
        }
    }

    // ---- K split: publish the partial; the last workgroup of the group reduces
    if (ws.ksplit > 1) {
        const int64_t tiles = (int64_t)ngroups * ST_RG;
        const int64_t tile = (int64_t)grp * ST_RG + wid;
        uint64_t *part = (uint64_t *)ws.part;
        if (wid < ST_RG) {
            if (ws.xlocal)  // every reader of these lines runs on this XCD
                publish_partial<__HIP_MEMORY_SCOPE_WORKGROUP>(part, ks, tiles, tile, lane, acc);
            else
                publish_partial<__HIP_MEMORY_SCOPE_AGENT>(part, ks, tiles, tile, lane, acc);
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are acknowledged
        __syncthreads();
        if (tid == 0) {
            if (ws.xlocal) {
                // Per-launch check of the placement the exchange rests on:
                // each split adds one to the nibble of its XCC (at most 15
                // splits), so the last to arrive sees where all of them ran.
                // Splits spread over more than one XCD (a dispatcher that broke
                // the round-robin the probe saw) set DEV_XCD_MISMATCH: that
                // launch's result is not to be trusted.
                uint32_t xcc = __builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) & 7u;
                if (ws.xcc_fake && (ks & 1))
                    xcc = (xcc + 1) & 7u;  // debug builds: pretend odd splits ran next door
                const uint32_t mine = 1u << (4 * xcc);
                const uint32_t now = __hip_atomic_fetch_add(&ws.cnt[grp], mine, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT) + mine;
                uint32_t cnt = (now & 0x0F0F0F0Fu) + ((now >> 4) & 0x0F0F0F0Fu);
                cnt = (cnt + (cnt >> 8) + (cnt >> 16) + (cnt >> 24)) & 0xFFu;
                s_is_last = cnt == (uint32_t)ws.ksplit;
                if (s_is_last && now != (uint32_t)ws.ksplit << (4 * xcc) && ws.status)
                    __hip_atomic_fetch_or(ws.status, DEV_XCD_MISMATCH, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
            } else {
                const uint32_t old =
                    __hip_atomic_fetch_add(&ws.cnt[grp], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                s_is_last = old == (uint32_t)(ws.ksplit - 1);
            }
        }
        __syncthreads();
        if (!s_is_last)
            return;  // uniform over the workgroup
        if (wid < ST_RG) {
            if (ws.xlocal)
                acc = reduce_partials_s<__HIP_MEMORY_SCOPE_WORKGROUP>(part, ws.ksplit, ks, tiles, tile, lane, acc);
            else
                acc = reduce_partials(part, ws.ksplit, ks, tiles, tile, lane, acc);
        }
        if (tid == 0)
            __hip_atomic_store(&ws.cnt[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue (lane holds batch rows 4*(lane/16)+i of column r)
    if (Nh) {
        // SwiGLU: waves 4..7 hold the up tiles matching the gate tiles of
        // waves 0..3; out = SiLU(g_gate G) * (g_up U), stored [B][Nh]
        if (wid >= ST_RG / 2 && wid < ST_RG)
            red[(wid - ST_RG / 2) * 64 + lane] = acc;
        __syncthreads();
        const int col = (rt0 + wid) * 16 + r;
        if (wid >= ST_RG / 2 || col >= Nh)
            return;
        const f32x4 up = red[wid * 64 + lane];
        float g0 = 1.f, g1 = 1.f;
        if constexpr (FMT == FMT_NV) {
            g0 = tensor_scale(a, col);
            g1 = tensor_scale(a, Nh + col);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int b = 4 * gq + i;
            if (b < a.B)
                store_out_nt<OUTT>(a.y, (int64_t)b * Nh + col, silu(g0 * acc[i]) * (g1 * up[i]));
        }
        return;
    }
    const int n = (rt0 + wid) * 16 + r;
    if (wid >= ST_RG || n >= a.N)
        return;
    float gsc = 1.f;
    if constexpr (FMT == FMT_NV)
        gsc = tensor_scale(a, n);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int b = 4 * gq + i;
        if (b < a.B)
            store_out_nt<OUTT>(a.y, (int64_t)b * a.N + n, gsc * acc[i]);
    }
}

// ------------------------------------------------------------------ host

template <int FMT, int ACT, int NTERM, int OUTT, bool FULLK, int PD>
static void launch_kd(const KArgs &a, const StCfg &c, const SkinnyWs &ws, hipStream_t st)
{
    const dim3 grid((unsigned)c.grid);
    const dim3 block((unsigned)(64 * c.W));
    const size_t lds = (size_t)c.W * ST_RG * 1024;
    if (c.NPH == 2)
        hipLaunchKernelGGL((stream_kernel<FMT, ACT, NTERM, 2, OUTT, FULLK, PD>), grid, block, lds, st, a, ws,
                           c.ngroups, c.Nh);
    else
        hipLaunchKernelGGL((stream_kernel<FMT, ACT, NTERM, 1, OUTT, FULLK, PD>), grid, block, lds, st, a, ws,
                           c.ngroups, c.Nh);
}

// prefetch depth in (phase, row tile) items; 16 covers every item of a chunk
template <int FMT, int ACT, int NTERM, int OUTT, bool FULLK>
static void launch_kf(const KArgs &a, const StCfg &c, const SkinnyWs &ws, hipStream_t st)
{
    if constexpr (NTERM != 1 && NTERM != 2) {
        switch (c.depth) {
        case 2: launch_kd<FMT, ACT, NTERM, OUTT, FULLK, 2>(a, c, ws, st); return;
        case 3: launch_kd<FMT, ACT, NTERM, OUTT, FULLK, 3>(a, c, ws, st); return;
        case 4: launch_kd<FMT, ACT, NTERM, OUTT, FULLK, 4>(a, c, ws, st); return;
        default: break;
        }
    }
    launch_kd<FMT, ACT, NTERM, OUTT, FULLK, 16>(a, c, ws, st);
}

// K a whole number of slabs: no unit or activation masking at all
template <int FMT, int ACT, int NTERM, int OUTT>
static void launch_kc(const KArgs &a, const StCfg &c, const SkinnyWs &ws, hipStream_t st)
{
    constexpr int KS = slab_k(FMT);
    if (a.K % KS == 0)
        launch_kf<FMT, ACT, NTERM, OUTT, true>(a, c, ws, st);
    else
        launch_kf<FMT, ACT, NTERM, OUTT, false>(a, c, ws, st);
}

template <int FMT>
static void launch_sf(const Problem &p, const KArgs &a, const StCfg &c, const SkinnyWs &ws, int nterm,
                      hipStream_t st)
{
    const bool o32 = p.out == QGEMM_F32;
    if (p.act != QGEMM_F32) {
        if (o32) launch_kc<FMT, ACT_BF16, 0, OUT_F32>(a, c, ws, st);
        else launch_kc<FMT, ACT_BF16, 0, OUT_BF16>(a, c, ws, st);
    } else if (nterm == 1) {
        if (o32) launch_kc<FMT, ACT_F32, 1, OUT_F32>(a, c, ws, st);
        else launch_kc<FMT, ACT_F32, 1, OUT_BF16>(a, c, ws, st);
    } else if (nterm == 2) {
        if (o32) launch_kc<FMT, ACT_F32, 2, OUT_F32>(a, c, ws, st);
        else launch_kc<FMT, ACT_F32, 2, OUT_BF16>(a, c, ws, st);
    } else {
        if (o32) launch_kc<FMT, ACT_F32, 3, OUT_F32>(a, c, ws, st);
        else launch_kc<FMT, ACT_F32, 3, OUT_BF16>(a, c, ws, st);
    }
}

hipError_t launch_stream(const Problem &p, const KArgs &a, const StCfg &c, const SkinnyWs &ws, int nterm,
                         hipStream_t st)
{
    switch (p.fmt) {
    case FMT_Q8: launch_sf<FMT_Q8>(p, a, c, ws, nterm, st); break;
    case FMT_MX: launch_sf<FMT_MX>(p, a, c, ws, nterm, st); break;
    case FMT_FP8: launch_sf<FMT_FP8>(p, a, c, ws, nterm, st); break;
    default: launch_sf<FMT_NV>(p, a, c, ws, nterm, st); break;
    }
    return hipGetLastError();
}

}  // namespace qg
