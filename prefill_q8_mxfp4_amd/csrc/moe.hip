// Routed experts with few rows each (bf16 math): every expert's packed
// weights streamed once from HBM straight into MFMA operands, as in the
// small-batch tier, for all of that expert's rows at once.
//
// A workgroup is 4 waves and owns one expert and a run of its row-tile
// groups: a group is 4 * NTG output row tiles (with SwiGLU, NTG gate tiles
// per wave and the NTG matching up tiles, so SiLU(G) * U is formed in the
// lane that holds both).  An expert's groups are split over a few
// workgroups with consecutive ids on one XCD, so the expert's activation rows
// are read from that XCD's L2.  A workgroup walks the slabs of its (group,
// pass) items as one sequence, loading D slabs ahead across item boundaries.
//
//  * The expert's rows are taken 16 * MB at a time (one pass for up to 64
//    rows).  Each slab's activations are loaded into registers together with
//    its weights, written into an LDS stage one step before they are used,
//    in MFMA fragment order (16-byte entry [16-row group][unit]
//    [lane]), zero past the last row and past K, fp32 rounded to bf16; only
//    the 16-row groups that hold rows are loaded (all MB are multiplied:
//    fewer branches and registers than skipping the empty ones).  The
//    measured alternative, gfx950's direct loads into LDS, lets the compiler
//    order every fragment read after the newest such load, which serialises
//    the walk.
//  * Each lane's 16-byte chunk of a weight slab is its B operand, decoded in
//    registers (loads of dead slabs go through empty buffer resources).
//  * Summation order, the small-batch tier's: per (slab, row tile) its units
//    in order into a partial from zero (Q8_0 / MXFP4 / FP8 block scales
//    applied to the block's fp32 partial, NVFP4's E4M3 scale folded into the
//    operand), partials added to the running tile in slab order.  A row's
//    result therefore does not depend on the other rows, and each expert's
//    rows are bitwise those of an unsplit small-batch call of that expert.
//
// The offsets are checked by every workgroup before any load that uses them
// (offsets[0] = 0, non-decreasing, offsets[E] = T): when they break a rule no
// workgroup does any work and workgroup 0 sets DEV_BAD_OFFSETS.
#include "common.h"

namespace qg {

constexpr int MOE_MB = 4;        // 16-row groups per pass
constexpr int MOE_D = 2;         // weight slabs in flight per wave (a ring of D + 1 slots)
constexpr int MOE_NTG = 2;       // output row tiles per wave
constexpr int MOE_NTG_DUAL = 1;  // with SwiGLU: gate tiles per wave (and as many up tiles)
constexpr int MOE_W = 4;         // waves per workgroup (8, with half the activation staging, measured slower)

template <int FMT, int ACT, int OUTT, bool DUAL, int NTG, bool FULLK>
__global__ __launch_bounds__(64 * MOE_W, 8 / MOE_W) __attribute__((amdgpu_waves_per_eu(2, 2)))
void moe_kernel(KArgs a, Groups grp, int Nh, int ngroups, int gpw)
{
    constexpr int KS = slab_k(FMT);
    constexpr int U = KS / 32;                 // 32-wide units per slab
    constexpr int MB = MOE_MB, D = MOE_D;
    constexpr int WT = DUAL ? 2 * NTG : NTG;   // row tiles per wave
    constexpr int XSZ = ACT == ACT_F32 ? 4 : 2;
    constexpr int SBYTES = scale_bytes_per_slab(FMT);
    constexpr int SLAB_E = MB * U * 64;        // LDS entries per staged slab
    constexpr int NXF = (MB * U + MOE_W - 1) / MOE_W;  // activation fragments per wave and slab
    constexpr bool POST = FMT != FMT_NV;
    // Weight ring of R = D + 1 slots: the slot a step loads into held the
    // slab the previous step consumed, so no slot is copied and no register
    // of a load in flight is live elsewhere (a copy would make the compiler
    // wait for every load at the loop's back edge).  Activation stages in
    // LDS: NST, with R a multiple of NST, so the loop unrolled R times has
    // static slot and stage indices.
    constexpr int R = D + 1;
    constexpr int NST = R % 2 == 0 ? 2 : R;

    __shared__ u32x4 xs[NST * SLAB_E];  // activation stages, one slab each

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, gq = lane >> 4;

    // ---- this workgroup's expert and row-tile groups [g_beg, g_end):
    // consecutive ids (one expert's groups) on one XCD
    int t;
    {
        const int nwg = gridDim.x, per = (nwg + 7) / 8;
        const int xcd = blockIdx.x % 8, loc = blockIdx.x / 8;
        const int full = nwg % 8 == 0 ? 8 : nwg % 8;
        t = xcd < full ? xcd * per + loc : full * per + (xcd - full) * (per - 1) + loc;
    }
    const int nsplit = (ngroups + gpw - 1) / gpw;
    const int e = t / nsplit;
    const int g_beg = t % nsplit * gpw, g_end = min(ngroups, g_beg + gpw);

    // ---- offsets check (all of them, before any use; this expert's own
    // offsets and weights pointer are loaded in the same round)
    int bad = 0;
    for (int e2 = tid; e2 < grp.E; e2 += 64 * MOE_W) {
        const int lo2 = grp.off[e2], hi2 = grp.off[e2 + 1];
        bad |= (hi2 < lo2) | (e2 == 0 && lo2 != 0) | (e2 == grp.E - 1 && hi2 != grp.T);
    }
    // the expert's values are the same in every lane: kept in scalar registers
    const int lo = __builtin_amdgcn_readfirstlane(grp.off[e]);
    const int rows = __builtin_amdgcn_readfirstlane(grp.off[e + 1]) - lo;
    {
        // readfirstlane returns int: both words go through uint32_t, or a
        // low word with bit 31 set would sign-extend over the high one
        const uint64_t wp = (uint64_t)grp.wtab[e];
        const uint32_t whi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(wp >> 32));
        const uint32_t wlo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)wp);
        a.w = (const uint8_t *)(((uint64_t)whi << 32) | wlo);
    }
    if (__syncthreads_or(bad)) {
        if (blockIdx.x == 0 && tid == 0)
            __hip_atomic_fetch_or(grp.status, DEV_BAD_OFFSETS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;  // uniform
    }
    if (rows <= 0 || g_beg >= g_end)
        return;  // uniform
    const int ncols = DUAL ? Nh : a.N;
    const uint8_t *xe = (const uint8_t *)a.x + (int64_t)lo * a.K * XSZ;
    void *ye = (uint8_t *)a.y + (int64_t)lo * ncols * (OUTT == OUT_F32 ? 4 : 2);
    const __amdgpu_buffer_rsrc_t xres = make_rsrc(xe, (int64_t)rows * a.K * XSZ);
    const uint32_t nvsh = 8 * (gq >> 1);  // NVFP4: this lane's scale byte within a unit's pair

    // NVFP4 tensor scales: rows per tensor read once; a column's scale is a
    // buffer load (counted with the other vector loads, so waiting for it
    // never drains the weight stream)
    int rpt = 1;
    __amdgpu_buffer_rsrc_t gres = make_rsrc(a.w, 0);
    if constexpr (FMT == FMT_NV) {
        rpt = __builtin_amdgcn_readfirstlane(*(const int *)(a.w + a.meta_off + 4));
        gres = make_rsrc(a.w + a.meta_off + 16, (int64_t)((a.N + rpt - 1) / rpt) * 4);
    }
    auto gload = [&](int col) { return __uint_as_float(bload4(gres, col / rpt * 4, 0)); };

    // Work items: (row-tile group g, pass b0 over 16 * MB rows), g major.  The
    // walk over their slabs does not stop between items (position p is slab
    // p % S of item p / S), so a workgroup pays the load latency once.
    const int npass = (rows + 16 * MB - 1) / (16 * MB);
    const int nitems = (g_end - g_beg) * npass;
    const int S = a.S;
    const int P = nitems * S;

    // first output row tile of this wave in item it's group (with SwiGLU the
    // up tiles are Nh/16 further on); tiles past the last compute on a copy of
    // it and are never stored
    auto t0_of = [&](int it) { return ((g_beg + it / npass) * MOE_W + wid) * NTG; };
    auto b0_of = [&](int it) { return it % npass * 16 * MB; };
    auto tile_of = [&](int t0, int j) -> int64_t {
        const int rt = DUAL ? (j < NTG ? t0 + j : Nh / 16 + t0 + j - NTG) : t0 + j;
        return min(rt, a.RT - 1);
    };

    // ---- weight ring: position p's slab in slot p % R, loaded at step p - D
    u32x4 wr[R][WT];
    uint32_t sr[R][WT][2];
    auto wload = [&](int j, int t0, int s) {  // slot j <- slab s of the tiles from t0 (none past the last)
        const bool live = s < S;
        const int sc = min(s, S - 1);
#pragma unroll
        for (int q = 0; q < WT; q++) {
            const int64_t rt = tile_of(t0, q);
            wr[j][q] = bload16_nt(make_rsrc(a.w + ((rt * S + sc) << 10), live ? 1024 : 0), lane << 4, 0);
            const __amdgpu_buffer_rsrc_t srs =
                make_rsrc(a.w + a.scale_off + (rt * S + sc) * (16 * SBYTES), live ? 16 * SBYTES : 0);
            if constexpr (FMT == FMT_NV) {
                const u32x2 v = bload8_nt(srs, r * SBYTES, 0);
                sr[j][q][0] = v[0];
                sr[j][q][1] = v[1];
            } else {
                sr[j][q][0] = bload4_nt(srs, r * SBYTES, 0);
                sr[j][q][1] = 0u;
            }
        }
    };
    // weights of position p into ring slot j (tiles of p's item)
    auto wld = [&](int j, int p) {
        const int it2 = p / S, s2 = p - it2 * S;
        const bool live = it2 < nitems;
        wload(j, t0_of(live ? it2 : nitems - 1), live ? s2 : S);
    };

    // ---- activations.  Fragment (16-row group mb, unit u) of a slab is one
    // 1 KB block of LDS entries, lane l holding row 16 mb + l % 16, columns
    // 8 (l / 16) .. + 7 of the unit; wave w loads fragments w, w + 4, ...
    // (indices past the last repeat it: the same bytes to the same place, no
    // branch).  Position p's activations are loaded into registers at step
    // p - 2, before that step's weight loads (so waiting for them never waits
    // for a later weight load), and written at step p - 1 (masked past the
    // rows and past K, fp32 rounded to bf16) into LDS stage p % NST, which the
    // barrier opening step p makes visible; that barrier also ends every read
    // of the stage written next.  One register slot: a step writes it to LDS
    // before it loads the next position into it.  Positions past the last
    // item load zeros (offsets past the end).
    u32x4 xv0[NXF], xv1[NXF];
    auto xfrag = [&](int b0, int i, int s2, int &mb, int &u, int &row, int &k) {
        const int nfr = U * min(MB, (rows - b0 + 15) / 16);  // fragments of a slab
        const int f = min(wid + MOE_W * i, nfr - 1);
        mb = f / U;
        u = f % U;
        row = b0 + 16 * mb + r;
        k = s2 * KS + 32 * u + 8 * gq;
    };
    auto xld = [&](int p) {
        const int it2 = p / S, s2 = p - it2 * S;
        const bool live = it2 < nitems;
        const int b0 = b0_of(min(it2, nitems - 1));
#pragma unroll
        for (int i = 0; i < NXF; i++) {
            int mb, u, row, k;
            xfrag(b0, i, s2, mb, u, row, k);
            const int vo = live && row < rows && k < a.K ? (row * a.K + k) * XSZ : 0x7FFFFFE0;
            xv0[i] = bload16(xres, vo, 0);
            if constexpr (ACT == ACT_F32)
                xv1[i] = bload16(xres, vo + 16, 0);
        }
    };
    auto xst = [&](int stage, int p) {
        const int it2 = p / S, s2 = p - it2 * S;
        const int b0 = b0_of(min(it2, nitems - 1));
        u32x4 *st = xs + stage * SLAB_E;
#pragma unroll
        for (int i = 0; i < NXF; i++) {
            int mb, u, row, k;
            xfrag(b0, i, s2, mb, u, row, k);
            u32x4 v;
            if constexpr (ACT == ACT_F32) {
                float fv[8];
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++) {
                    fv[e2] = __uint_as_float(xv0[i][e2]);
                    fv[4 + e2] = __uint_as_float(xv1[i][e2]);
                }
                v = __builtin_bit_cast(u32x4, split_f32<1, 8>(fv).t[0]);
            } else {
                v = xv0[i];
            }
            st[(mb * U + u) * 64 + lane] = v;
        }
    };

    // ---- before step 0: weights of positions 0 .. D - 1, position 0's
    // activations in LDS stage 0, position 1's in the registers (loaded just
    // before the last weight slab, as in every step)
#pragma unroll
    for (int j = 0; j < D - 1; j++)
        wld(j, j);
    xld(0);
    xst(0, 0);
    xld(1);
    __builtin_amdgcn_sched_barrier(0);
    wld(D - 1, D - 1);
    // Nothing in flight when the walk starts: the loop's first step then
    // sees the same pending loads from the prologue as from its own back
    // edge (otherwise the compiler's wait counts, merged over both, demand
    // a near-drain at the top of every ring turn).  Costs one latency per
    // workgroup.
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)

    f32x4 acc[MB][WT];
    float g0 = 1.f, g1 = 1.f;
    for (int p0 = 0; p0 < P; p0 += R) {
#pragma unroll
        for (int j = 0; j < R; j++) {
            // Steps past the last position (the end of the last ring turn)
            // load nothing but zeros and compute nothing; they still run the
            // loads, so every path through a ring turn issues the same ones
            const int p = p0 + j;
            const bool on = p < P;  // uniform
            const int it = p / S, s = p - it * S;
            const int t0 = t0_of(it);
            __syncthreads();
            // Position p + 1's activations, into the next stage.  Only the
            // weight loads of position p + D - 1 (2 WT) were issued after
            // them; the explicit wait says so.
            __builtin_amdgcn_s_waitcnt(0xF70 | (2 * WT));  // vmcnt(2 WT), expcnt and lgkmcnt untouched
            xst((j + 1) % NST, p + 1);
            if (on && s == 0) {  // an item starts: accumulators, NVFP4 tensor scales
#pragma unroll
                for (int mb = 0; mb < MB; mb++)
#pragma unroll
                    for (int q = 0; q < WT; q++)
                        acc[mb][q] = f32x4{0.f, 0.f, 0.f, 0.f};
                if constexpr (FMT == FMT_NV) {
                    const int col = min(t0 * 16 + r, ncols - 1);  // clamped only for tiles never stored
                    g0 = gload(col);
                    if constexpr (DUAL)
                        g1 = gload(Nh + col);
                }
            }
            xld(p + 2);
            __builtin_amdgcn_sched_barrier(0);
            wld((j + D) % R, p + D);
            __builtin_amdgcn_sched_barrier(0);
            if (!on)
                continue;  // uniform
            const u32x4 *slab = xs + (j % NST) * SLAB_E;
            // units within K (FULLK: K is a whole number of slabs, so no unit
            // branch, and one step's loads, decode and MFMAs form one block)
            const int nu = FULLK ? U : min(U, (a.K - s * KS + 31) / 32);
            // per (row tile, group) a partial from zero over the units in
            // order; every group is multiplied (groups past the rows hold
            // stale entries; their outputs are never stored)
            f32x4 part[WT][MB];
#pragma unroll
            for (int q = 0; q < WT; q++)
#pragma unroll
                for (int mb = 0; mb < MB; mb++)
                    part[q][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
            // activation fragments one unit ahead of their MFMAs
            bf16x8 A2[2][MB];
#pragma unroll
            for (int mb = 0; mb < MB; mb++)
                A2[0][mb] = __builtin_bit_cast(bf16x8, slab[(mb * U) * 64 + lane]);
#pragma unroll
            for (int u = 0; u < U; u++) {
                if (u + 1 < U) {
#pragma unroll
                    for (int mb = 0; mb < MB; mb++)
                        A2[(u + 1) & 1][mb] = __builtin_bit_cast(bf16x8, slab[(mb * U + u + 1) * 64 + lane]);
                }
                if (!FULLK && u >= nu)
                    continue;  // uniform
                const bf16x8 *A = A2[u & 1];
#pragma unroll
                for (int q = 0; q < WT; q++) {
                    const u32x4 wc = wr[j][q];
                    const uint32_t sc0 = sr[j][q][0], sc1 = sr[j][q][1];
                    bf16x8 Bw;
                    float ps = 1.f;
                    if constexpr (FMT == FMT_Q8) {
                        Bw = q8_to_bf16(wc[2 * u], wc[2 * u + 1]);
                        ps = fp16_bits_to_f32((sc0 >> (16 * u)) & 0xFFFFu);
                    } else if constexpr (FMT == FMT_FP8) {
                        Bw = fp8_to_bf16(wc[2 * u], wc[2 * u + 1]);
                        ps = __uint_as_float(sc0);
                    } else if constexpr (FMT == FMT_MX) {
                        Bw = fp4_to_bf16(wc[u], 1.0f);
                        ps = e8m0_to_f32((sc0 >> (8 * u)) & 0xFFu);
                    } else {
                        const uint32_t sv = (u < 2 ? sc0 : sc1) >> nvsh;
                        const float bs = (u & 1) ? e4m3_byte_to_f32<2>(sv) : e4m3_byte_to_f32<0>(sv);
                        Bw = fp4_to_bf16_mul(wc[u], bs);
                    }
#pragma unroll
                    for (int mb = 0; mb < MB; mb++) {
                        if constexpr (POST) {
                            const f32x4 tq = mfma(A[mb], Bw, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                            for (int i = 0; i < 4; i++)
                                part[q][mb][i] = __builtin_fmaf(ps, tq[i], part[q][mb][i]);
                        } else {
                            part[q][mb] = mfma(A[mb], Bw, part[q][mb]);
                        }
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < WT; q++)
#pragma unroll
                for (int mb = 0; mb < MB; mb++) {
                    acc[mb][q][0] += part[q][mb][0];
                    acc[mb][q][1] += part[q][mb][1];
                    acc[mb][q][2] += part[q][mb][2];
                    acc[mb][q][3] += part[q][mb][3];
                }
            if (s != S - 1)
                continue;  // uniform

            // ---- the item's last slab: epilogue (lane holds rows 4 gq + i
            // of column r of each tile)
            const int b0 = b0_of(it);
            const int nmb = min(MB, (rows - b0 + 15) / 16);
#pragma unroll
            for (int q = 0; q < (DUAL ? NTG : WT); q++) {
                const int col = (t0 + q) * 16 + r;
                if (col >= ncols)
                    continue;
                float h0 = g0, h1 = g1;
                if constexpr (FMT == FMT_NV) {
                    if (q > 0) {  // tensor scales of the further tiles (NTG > 1)
                        h0 = gload(col);
                        if constexpr (DUAL)
                            h1 = gload(Nh + col);
                    }
                }
#pragma unroll
                for (int mb = 0; mb < MB; mb++)
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int b = b0 + 16 * mb + 4 * gq + i;
                        if (mb >= nmb || b >= rows)
                            continue;
                        if constexpr (DUAL)
                            store_out_nt<OUTT>(ye, (int64_t)b * Nh + col,
                                               silu(h0 * acc[mb][q][i]) * (h1 * acc[mb][q + NTG][i]));
                        else
                            store_out_nt<OUTT>(ye, (int64_t)b * a.N + col, h0 * acc[mb][q][i]);
                    }
            }
        }
    }
}

// ------------------------------------------------------------------ host

// Row-tile groups per expert (workgroups per expert).
int moe_groups(const Problem &p)
{
    const bool dual = p.epi == QGEMM_EPI_SWIGLU;
    const int64_t out_tiles = dual ? p.N / 2 / 16 : (p.N + 15) / 16;
    const int per = MOE_W * (dual ? MOE_NTG_DUAL : MOE_NTG);
    return (int)((out_tiles + per - 1) / per);
}

// Groups per workgroup: enough workgroups for about four rounds of two per
// CU (whole experts per workgroup would leave the kernel waiting for the
// experts with the most rows), each taking a run of one expert's groups.
int moe_groups_per_wg(const Problem &p, int64_t E)
{
    const int ng = moe_groups(p);
    const int64_t want = 2048;  // workgroups
    const int64_t split = E >= want ? 1 : (want + E - 1) / E;
    const int64_t gpw = (ng + (split < ng ? split : ng) - 1) / (split < ng ? split : ng);
    return (int)gpw;
}

template <int FMT, int ACT, int OUTT, bool DUAL>
static void launch_m(const KArgs &a, const Groups &g, int Nh, int ngroups, int gpw, hipStream_t st)
{
    constexpr int NTG = DUAL ? MOE_NTG_DUAL : MOE_NTG;
    const dim3 grid((unsigned)((int64_t)g.E * ((ngroups + gpw - 1) / gpw)));
    if (a.K % slab_k(FMT) == 0)  // no unit masking
        hipLaunchKernelGGL((moe_kernel<FMT, ACT, OUTT, DUAL, NTG, true>), grid, dim3(64 * MOE_W), 0, st, a, g, Nh, ngroups,
                           gpw);
    else
        hipLaunchKernelGGL((moe_kernel<FMT, ACT, OUTT, DUAL, NTG, false>), grid, dim3(64 * MOE_W), 0, st, a, g, Nh, ngroups,
                           gpw);
}

template <int FMT>
static void launch_mf(const Problem &p, const KArgs &a, const Groups &g, hipStream_t st)
{
    const bool f32 = p.act == QGEMM_F32, o32 = p.out == QGEMM_F32;
    const bool dual = p.epi == QGEMM_EPI_SWIGLU;
    const int Nh = (int)(p.N / 2);
    const int ng = moe_groups(p), gw = moe_groups_per_wg(p, g.E);
    if (f32) {
        if (o32) { if (dual) launch_m<FMT, ACT_F32, OUT_F32, true>(a, g, Nh, ng, gw, st); else launch_m<FMT, ACT_F32, OUT_F32, false>(a, g, Nh, ng, gw, st); }
        else { if (dual) launch_m<FMT, ACT_F32, OUT_BF16, true>(a, g, Nh, ng, gw, st); else launch_m<FMT, ACT_F32, OUT_BF16, false>(a, g, Nh, ng, gw, st); }
    } else {
        if (o32) { if (dual) launch_m<FMT, ACT_BF16, OUT_F32, true>(a, g, Nh, ng, gw, st); else launch_m<FMT, ACT_BF16, OUT_F32, false>(a, g, Nh, ng, gw, st); }
        else { if (dual) launch_m<FMT, ACT_BF16, OUT_BF16, true>(a, g, Nh, ng, gw, st); else launch_m<FMT, ACT_BF16, OUT_BF16, false>(a, g, Nh, ng, gw, st); }
    }
}

hipError_t launch_moe(const Problem &p, const KArgs &a, const Groups &g, hipStream_t st)
{
    switch (p.fmt) {
    case FMT_Q8: launch_mf<FMT_Q8>(p, a, g, st); break;
    case FMT_MX: launch_mf<FMT_MX>(p, a, g, st); break;
    case FMT_FP8: launch_mf<FMT_FP8>(p, a, g, st); break;
    default: launch_mf<FMT_NV>(p, a, g, st); break;
    }
    return hipGetLastError();
}

}  // namespace qg
