// Small-batch tier, B <= 16: every weight byte of a workgroup's K range is
// requested at once.
//
// A workgroup is R waves (8..16, chosen on the host from the problem shape);
// wave w owns one row tile (16 weight rows) and the workgroup a range of K
// slabs.
// Inside the range it works in chunks of KC slabs (with a workspace, the
// range is one chunk):
//
//  1. issue the activation loads of the chunk (16 batch rows; they are
//     L2-resident after the first workgroup of the XCD touched them), then
//     every weight and scale load of the wave's row tile for the chunk, each
//     into its own registers: nothing is loop-carried, so no wait ever drains
//     the loads still in flight;
//  2. split the activations into bf16 terms (fp32 input: the terms add up to
//     the fp32 value) and stage them in LDS in MFMA fragment order (waves
//     0..7 do this), shared by all the waves;
//  3. consume the slabs in order, each as soon as its load has returned:
//     decode in registers (int8 and E2M1 exact; NVFP4 times its E4M3 scale,
//     also exact), v_mfma_f32_16x16x32_bf16 with the weights as the A operand
//     of each 32-wide unit, Q8_0 / MXFP4 block scales applied to the fp32
//     block partial.
//
// Per 32-wide unit the accumulation is the one the B > 16 kernel uses (same
// MFMA chain, same scale step, slabs ascending, splits summed in split
// order), so a batch row's result does not depend on B.
//
// The K split and its fence-free reduction (device-scope stores, a counter,
// the last workgroup to arrive sums the partials in split order) follow the
// B > 16 kernel.
#include "common.h"

namespace qg {

constexpr int ST_STAGE_WAVES = 8;  // waves that stage the activations

template <int FMT, int ACT, int NTERM, int KC, int OUTT>
__global__ __launch_bounds__(64 * ST_MAX_WAVES(KC)) void stream_kernel(KArgs a, SkinnyWs ws, int ngroups)
{
    constexpr int KS = FMT == FMT_Q8 ? 64 : 128;
    constexpr int U = KS / 32;                 // 32-wide units per slab
    constexpr bool POST = FMT != FMT_NV;       // block scale applied after the MFMA
    constexpr int NTA = ACT == ACT_F32 ? NTERM : 1;
    constexpr int CE = ACT == ACT_F32 ? 4 : 8; // activations per 16-byte chunk
    constexpr int NCH = 16 * KS / CE;          // chunks per slab (16 batch rows)
    constexpr int NTHR = 64 * ST_STAGE_WAVES;  // staging threads
    constexpr int XL = KC * NCH / NTHR;        // activation loads per staging thread
    constexpr int SLAB_E = NTA * U * 64;       // 16-byte LDS entries per slab
    constexpr int G = FMT == FMT_NV ? 2 : 4;   // slabs per 256-byte scale record
    constexpr int NREC = KC / G;
    static_assert(XL * NTHR == KC * NCH, "activation chunks per thread");
    static_assert(KC % G == 0, "chunks start on a scale record");

    extern __shared__ u32x4 xs[];              // [KC][NTA][U][64]
    __shared__ int s_is_last;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int r = lane & 15;
    const int R = blockDim.x >> 6;             // waves = row tiles per workgroup
    const bool stager = wid < ST_STAGE_WAVES;

    // XCD-aware order: consecutive workgroup ids go to different XCDs (id mod
    // 8).  Give each XCD a contiguous run of (split, group) pairs, split
    // major, so an XCD's workgroups share few activation slices in its L2.
    int t = blockIdx.x;
    {
        const int nwg = gridDim.x;
        const int per = (nwg + 7) / 8;
        const int xcd = t % 8, loc = t / 8;
        const int full = nwg % 8 == 0 ? 8 : nwg % 8;
        t = xcd < full ? xcd * per + loc : full * per + (xcd - full) * (per - 1) + loc;
    }
    const int ks = t / ngroups, grp = t % ngroups;
    const int rtu = grp * R + wid;             // this wave's row tile
    const int64_t rt = min(rtu, a.RT - 1);     // clamped: a copy past the end, never stored
    const int s_beg = ks * ws.kc;
    const int s_end = min(a.S, s_beg + ws.kc);

    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c_beg = s_beg; c_beg < s_end; c_beg += KC) {
        // ---- 1. activation loads, then every weight and scale load of the chunk
        // Rows past B load a copy of row B-1: they only feed output rows that
        // are never stored.  Columns past K are zeroed when staged.
        u32x4 xr[XL];
        bool xin[XL];
        if (stager) {
#pragma unroll
        for (int i = 0; i < XL; i++) {
            const int c = tid + i * NTHR;
            const int sl = c / NCH, cc = c % NCH;
            const int b = cc / (KS / CE), kk = (cc % (KS / CE)) * CE;
            const int k = (c_beg + sl) * KS + kk;
            xin[i] = k < a.K;  // K % 16 == 0: a chunk is all in or all out
            const int bc = min(b, a.B - 1), kcl = min(k, a.K - CE);
            if constexpr (ACT == ACT_F32)
                xr[i] = *(const u32x4 *)((const float *)a.x + (int64_t)bc * a.K + kcl);
            else
                xr[i] = *(const u32x4 *)((const uint16_t *)a.x + (int64_t)bc * a.K + kcl);
        }
        }
        u32x4 wr[KC];
        u32x4 sr[NREC];
#pragma unroll
        for (int q = 0; q < NREC; q++) {
            // the record first, then its slabs: a slab's scales never wait
            // behind later slabs' weights
            const int sq = min(c_beg + q * G, a.S - 1);
            sr[q] = *(const u32x4 *)(a.w + a.scale_off + ((rt * a.SG + sq / G) << 8) + (r << 4));
#pragma unroll
            for (int j = q * G; j < q * G + G; j++) {
                const int s = min(c_beg + j, a.S - 1);
                wr[j] = *(const u32x4 *)(a.w + ((rt * a.S + s) << 10) + (lane << 4));
            }
        }

        // ---- 2. split and stage the activations
        if (stager) {
#pragma unroll
        for (int i = 0; i < XL; i++) {
            const int c = tid + i * NTHR;
            const int sl = c / NCH, cc = c % NCH;
            const int b = cc / (KS / CE), kk = (cc % (KS / CE)) * CE;
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
                for (int tt = 0; tt < NTA; tt++) {
                    const u32x4 qv = __builtin_bit_cast(u32x4, sp.t[tt]);
                    u32x2 *dst = (u32x2 *)&slab[(tt * U + u) * 64 + g8 * 16 + b] + half;
                    *dst = u32x2{qv[0], qv[1]};
                }
            } else {
                slab[u * 64 + g8 * 16 + b] = xv;
            }
        }
        }
        __syncthreads();

        // ---- 3. consume the slabs in order
#pragma unroll
        for (int j = 0; j < KC; j++) {
            const int s = c_beg + j;
            if (s >= s_end)
                continue;  // past the range (uniform)
            const u32x4 wc = wr[j];
            const uint32_t s0 = sr[j / G][FMT == FMT_NV ? 2 * (j % G) : j % G];
            const uint32_t s1 = FMT == FMT_NV ? sr[j / G][2 * (j % G) + 1] : 0u;
            const u32x4 *slab = xs + j * SLAB_E;
            // Units past K (padding of the last slab) are skipped.  Units are
            // taken two at a time: operands read and decoded up front so the
            // two MFMA chains interleave.
            const int nu = min(U, (a.K - s * KS + 31) / 32);
#pragma unroll
            for (int u0 = 0; u0 < U; u0 += 2) {
                bf16x8 A[2][NTA], Bw[2];
                float ps[2];
#pragma unroll
                for (int h = 0; h < 2; h++)
#pragma unroll
                    for (int tt = 0; tt < NTA; tt++)
                        A[h][tt] = __builtin_bit_cast(bf16x8, slab[(tt * U + u0 + h) * 64 + lane]);
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const int u = u0 + h;
                    ps[h] = 1.f;
                    if constexpr (FMT == FMT_Q8) {
                        Bw[h] = q8_to_bf16(wc[2 * u], wc[2 * u + 1]);
                        ps[h] = fp16_bits_to_f32((s0 >> (16 * u)) & 0xFFFFu);
                    } else if constexpr (FMT == FMT_MX) {
                        Bw[h] = fp4_to_bf16(wc[u], 1.0f);
                        ps[h] = e8m0_to_f32((s0 >> (8 * u)) & 0xFFu);
                    } else {
                        const int si = 2 * u + ((lane >> 4) >> 1);
                        const uint32_t sb = (si < 4 ? s0 >> (8 * si) : s1 >> (8 * (si - 4))) & 0xFFu;
                        Bw[h] = fp4_to_bf16_mul(wc[u], e4m3_to_f32(sb));
                    }
                }
                if constexpr (POST) {
                    f32x4 tacc[2];
#pragma unroll
                    for (int h = 0; h < 2; h++)
                        tacc[h] = mfma(A[h][0], Bw[h], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int tt = 1; tt < NTA; tt++)
#pragma unroll
                        for (int h = 0; h < 2; h++)
                            tacc[h] = mfma(A[h][tt], Bw[h], tacc[h]);
#pragma unroll
                    for (int h = 0; h < 2; h++) {
                        if (u0 + h >= nu)
                            continue;
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            acc[i] = __builtin_fmaf(ps[h], tacc[h][i], acc[i]);
                    }
                } else {
#pragma unroll
                    for (int h = 0; h < 2; h++) {
                        if (u0 + h >= nu)
                            continue;
#pragma unroll
                        for (int tt = 0; tt < NTA; tt++)
                            acc = mfma(A[h][tt], Bw[h], acc);
                    }
                }
            }
        }
        if (c_beg + KC < s_end)
            __syncthreads();  // every wave is done with the staged chunk
    }

    // ---- K split: publish the partial; the last workgroup of the group reduces
    if (ws.ksplit > 1) {
        const int64_t tiles = (int64_t)ngroups * R;
        const int64_t tile = (int64_t)grp * R + wid;
        uint64_t *part = (uint64_t *)ws.part;
        {
            uint64_t *dst = part + (((int64_t)ks * tiles + tile) * 64 + lane) * 2;
            const u32x4 v = __builtin_bit_cast(u32x4, acc);
            __hip_atomic_store(dst, (uint64_t)v[0] | ((uint64_t)v[1] << 32), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(dst + 1, (uint64_t)v[2] | ((uint64_t)v[3] << 32), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are acknowledged
        __syncthreads();
        if (tid == 0) {
            const uint32_t old =
                __hip_atomic_fetch_add(&ws.cnt[grp], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_is_last = old == (uint32_t)(ws.ksplit - 1);
        }
        __syncthreads();
        if (!s_is_last)
            return;
        acc = reduce_partials(part, ws.ksplit, ks, tiles, tile, lane, acc);
        if (tid == 0)
            __hip_atomic_store(&ws.cnt[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue: tensor scale, store (lane holds batch rows 4*(lane/16)+i of column r)
    const int n = rtu * 16 + r;
    if (n >= a.N)
        return;
    float g = 1.f;
    if constexpr (FMT == FMT_NV)
        g = tensor_scale(a, n);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int b = 4 * (lane >> 4) + i;
        if (b < a.B)
            store_out<OUTT>(a.y, (int64_t)b * a.N + n, g * acc[i]);
    }
}

// ------------------------------------------------------------------ host

template <int FMT, int ACT, int NTERM, int OUTT>
static void launch_kc(const KArgs &a, const StCfg &c, const SkinnyWs &ws, hipStream_t st)
{
    const dim3 grid((unsigned)(c.ngroups * c.ksplit));
    const dim3 block((unsigned)(64 * c.R));
    if (c.KC == 16)
        hipLaunchKernelGGL((stream_kernel<FMT, ACT, NTERM, 16, OUTT>), grid, block, c.lds, st, a, ws,
                           c.ngroups);
    else
        hipLaunchKernelGGL((stream_kernel<FMT, ACT, NTERM, 8, OUTT>), grid, block, c.lds, st, a, ws,
                           c.ngroups);
}

template <int FMT>
static void launch_sf(const Problem &p, const KArgs &a, const StCfg &c, const SkinnyWs &ws, int nterm,
                      hipStream_t st)
{
    const bool o32 = p.out == QGEMM_F32;
    if (p.act != QGEMM_F32) {
        if (o32) launch_kc<FMT, ACT_BF16, 1, OUT_F32>(a, c, ws, st);
        else launch_kc<FMT, ACT_BF16, 1, OUT_BF16>(a, c, ws, st);
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
    default: launch_sf<FMT_NV>(p, a, c, ws, nterm, st); break;
    }
    return hipGetLastError();
}

}  // namespace qg
