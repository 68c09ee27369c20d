// Small-batch tier, 16 < B <= 80: the MTP verify widths (64, 65, 70, 76 in
// the hipfire issue, Summary) in one pass over the weights.  fp32-faithful
// math (three exact bf16 terms per fp32 activation) is instantiated in
// verify.hip, bf16 math (bf16 activations as they are, fp32 ones rounded to
// bf16 once) in verify_bf16.hip.
//
// A workgroup owns the streaming kernel's row group (8 row tiles, 128 weight
// rows), all B batch rows as MB 16-row groups, and the streaming kernel's K
// split (the same slab ranges), so every output is summed in exactly the
// streaming kernel's order and a batch row's result does not depend on B
// across the small-batch tier.  It is 8 waves in two roles, one of each per
// SIMD, meeting at one barrier per step of one or two slabs:
//
//  * compute waves 0..3: wave w computes row tiles 2w and 2w + 1 (with the
//    fused gate+up epilogue, gate tile w and its up tile) over the whole slab
//    range.  Its weights arrive straight into registers as MFMA B
//    operands (a lane's 16-byte chunk of a slab is its operand; see
//    layout.h), D slabs ahead, through nontemporal buffer loads (past the
//    range through an empty resource: zeros, no traffic).  Only weight loads
//    are in its queue, so each step waits for the slab issued D steps before.
//  * staging waves 4..7: they load the activations of a slab (16*MB rows x 64
//    or 128 columns, L2-resident) VF_NSET steps ahead into registers, split
//    them into NTA bf16 terms (fp32 input) and store them into one of two LDS
//    buffers laid out as MFMA A fragments (a fragment read is 64 contiguous
//    16-byte entries), the step before they are used.  The split runs on the
//    vector ALUs while the compute wave of the same SIMD issues MFMAs.
//  * per 32-wide unit: both tiles' codes decoded once, then for each batch
//    group the NTA terms' MFMAs into a block partial from zero and the
//    Q8_0 / MXFP4 / FP8 block scale multiplied into the slab partial (NVFP4:
//    scale folded into the exact operand); slab partials added to the running
//    tile in slab order.
//
// With fp32-faithful math the products are exact (bf16 terms of fp32 x times
// exact codes), so only the fp32 accumulation rounds.  K splits meet as in
// the streaming kernel: partial tiles through the XCD's L2 when the
// dispatcher keeps a row group's splits on one XCD (checked every launch),
// else device-coherent, added in split order by the last workgroup of the
// group, all 8 of its waves sharing the adds.
#pragma once

#include "common.h"

namespace qg {

constexpr int VF_NT = 2;  // row tiles per compute wave
// Weight slabs in flight per compute wave (a multiple of VF_NSET): 8 of 64
// columns or 4 of 128 (the FP4 formats) while the accumulators leave room
// (MB <= 3), else half that.
__host__ __device__ constexpr int vf_depth(int fmt, int mb)
{
    return (slab_k(fmt) == 64 ? 8 : 4) / (mb <= 3 ? 1 : 2);
}
// Steps of activations in flight per staging wave: step t + VF_NSET is
// issued when step t + 1 is staged.
constexpr int VF_NSET = 2;
// Slabs per step (one barrier each): two of 64 columns up to 64 rows (half
// the barriers: Q8_0 5120^2 B = 64 24.1 -> 23.3 us on MI355X), else one (at 80 rows
// the ring would then hold only two steps: B = 65-80 ran 3-4 % slower).
__host__ __device__ constexpr int vf_sps(int fmt, int mb) { return slab_k(fmt) == 64 && mb <= 4 ? 2 : 1; }

// Splits of a chunk whose partial tiles the last workgroup loads together.
constexpr int VF_RCH = 8;

// The last workgroup's sum of one row tile's MB partial tiles over the
// ksplit splits, in split order: a lane's 16 bytes of a partial tile are one
// load with cache-scope bits AUX (those of the stores), and every load of a
// chunk of VF_RCH splits is issued before the first add.
template <int AUX, int MB>
__device__ __forceinline__ void vf_sum_splits(const uint8_t *part, int ksplit, int64_t tbytes, int tvo,
                                              f32x4 (&sum)[MB])
{
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
        sum[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < ksplit; k0 += VF_RCH) {
        u32x4 v[VF_RCH][MB];
#pragma unroll
        for (int j = 0; j < VF_RCH; j++) {
            if (k0 + j < ksplit) {  // uniform
                const __amdgpu_buffer_rsrc_t pr = make_rsrc(part + (int64_t)(k0 + j) * tbytes, tbytes);
#pragma unroll
                for (int mb = 0; mb < MB; mb++)
                    v[j][mb] = __builtin_bit_cast(u32x4,
                                                  __builtin_amdgcn_raw_buffer_load_b128(pr, tvo + mb * 1024, 0, AUX));
            }
        }
#pragma unroll
        for (int j = 0; j < VF_RCH; j++) {
            if (k0 + j < ksplit) {  // uniform
#pragma unroll
                for (int mb = 0; mb < MB; mb++) {
                    const f32x4 f = __builtin_bit_cast(f32x4, v[j][mb]);
                    sum[mb][0] += f[0]; sum[mb][1] += f[1]; sum[mb][2] += f[2]; sum[mb][3] += f[3];
                }
            }
        }
    }
}

template <int FMT, int MB, int OUTT, int NTA, int ACT>
__global__ __launch_bounds__(512) void verify_kernel(KArgs a, SkinnyWs ws, int ngroups, int Nh)
{
    static_assert(NTA == 1 || (NTA == 3 && ACT == ACT_F32), "three terms of fp32 input, or one");
    constexpr int KS = slab_k(FMT);
    constexpr int U = KS / 32;                   // 32-wide units per slab
    constexpr int NT = VF_NT, D = vf_depth(FMT, MB), NSET = VF_NSET;
    constexpr int SPS = vf_sps(FMT, MB), DS = D / SPS;  // slabs per step, steps of weights in flight
    static_assert(D % SPS == 0 && DS % NSET == 0 && DS % 2 == 0, "sets and buffers known at compile time");
    constexpr bool POST = FMT != FMT_NV;         // block scale after the MFMA
    constexpr int SBYTES = FMT == FMT_NV ? 8 : 4;  // scale bytes per row and slab
    constexpr int XB = ACT == ACT_F32 ? 4 : 2;   // bytes per activation
    constexpr int CPR = KS * XB / 16;            // 16-byte chunks per row and slab
    constexpr int NCH = 16 * MB * CPR;           // chunks per slab
    constexpr int XPT = (NCH + 255) / 256;       // chunk loads per thread per slab
    constexpr bool XWHOLE = NCH % 256 == 0;      // every thread's chunks all in the slab
    constexpr int TSTR = MB * U * 64;            // entries per term
    constexpr int SLAB_E = NTA * TSTR;           // 16-byte entries per staged slab

    __shared__ u32x4 xs[2][SPS * SLAB_E];        // [buffer][slab of the step][term][mb][unit][64]
    __shared__ int s_is_last;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool stager = wid >= 4;  // uniform per wave
    const int r = lane & 15, gq = lane >> 4;

    // the streaming kernel's (split, group) order, so the same exchange and
    // the same per-launch placement check apply
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
    // The group's 8 tile slots: 8 consecutive row tiles, or with SwiGLU
    // (Nh > 0) 4 gate tiles and the 4 matching up tiles Nh/16 further on.
    // A compute wave holds slots 2w, 2w + 1, or with SwiGLU gate slot w and
    // its up slot 4 + w, so G and U of an output column meet in one lane.
    static_assert(NT == 2, "two tile slots per compute wave");
    auto slot_of = [&](int t) { return Nh ? (wid & 3) + 4 * t : (wid & 3) * NT + t; };
    auto row_of = [&](int g) { return Nh ? (g < 4 ? grp * 4 + g : Nh / 16 + grp * 4 + g - 4) : grp * ST_RG + g; };
    const int s_beg = ks * ws.kc;
    const int s_end = min(a.S, s_beg + ws.kc);
    const int s_last = s_end - 1;

    // ---- activation staging.  Chunk c of a slab (c = stid + 256 i, stid the
    // thread's index among the staging waves) is, for fp32 input, 4 values of
    // batch row 16*mb + b at columns 32*u + 8*g8 + 4*h (a wave's 64 chunks
    // cover 16 rows x both halves of two k-groups, so its 8-byte LDS writes of
    // one term fall on distinct bank pairs), for bf16 input the 8 values of
    // one whole fragment entry (row 16*mb + b, columns 32*u + 8*g8; a wave
    // writes 64 consecutive entries).  Rows past B, and chunks past the slab
    // (bf16, odd MB), read as zero (the resource ends at row B); the latter
    // are not stored.
    const __amdgpu_buffer_rsrc_t xres = make_rsrc(a.x, (int64_t)a.B * a.K * XB);
    int xvo[XPT], xeo[XPT];
    const int stid = tid & 255;
#pragma unroll
    for (int i = 0; i < XPT; i++) {
        const int c = stid + 256 * i;
        if constexpr (ACT == ACT_F32) {
            const int b = c & 15, h = (c >> 4) & 1, q = c >> 5;
            const int g8 = q & 3, u = (q >> 2) % U, mb = (q >> 2) / U;
            xvo[i] = ((16 * mb + b) * a.K + 32 * u + 8 * g8 + 4 * h) * 4;
            xeo[i] = 2 * ((mb * U + u) * 64 + g8 * 16 + b) + h;  // 8-byte slot of term 0
        } else {
            const int b = c & 15, q = c >> 4;
            const int g8 = q & 3, u = (q >> 2) % U, mb = (q >> 2) / U;
            xvo[i] = ((16 * mb + b) * a.K + 32 * u + 8 * g8) * 2;
            xeo[i] = (mb * U + u) * 64 + g8 * 16 + b;  // 16-byte entry
        }
    }
    u32x4 xr[NSET][SPS][XPT];  // step t (its first slab s_beg + t * SPS) in set t % NSET
    auto xload = [&](int set, int s) {
#pragma unroll
        for (int sl = 0; sl < SPS; sl++)
#pragma unroll
            for (int i = 0; i < XPT; i++)
                xr[set][sl][i] = bload16(xres, xvo[i], min(s + sl, s_last) * KS * XB);
    };
    auto xstore = [&](int set, u32x4 *buf) {
#pragma unroll
        for (int sl = 0; sl < SPS; sl++) {
            if constexpr (ACT == ACT_BF16) {
#pragma unroll
                for (int i = 0; i < XPT; i++)
                    if (XWHOLE || stid + 256 * i < NCH)
                        buf[sl * SLAB_E + xeo[i]] = xr[set][sl][i];
                continue;
            }
            u32x2 *b2 = (u32x2 *)(buf + sl * SLAB_E);
#pragma unroll
            for (int i = 0; i < XPT; i++) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; e++)
                    v[e] = __uint_as_float(xr[set][sl][i][e]);
                const Split<NTA> sp = split_f32<NTA, 4>(v);
#pragma unroll
                for (int t = 0; t < NTA; t++) {
                    const u32x4 q = __builtin_bit_cast(u32x4, sp.t[t]);  // elements 0..3 hold the values
                    b2[xeo[i] + 2 * t * TSTR] = u32x2{q[0], q[1]};
                }
            }
        }
    };

    // ---- weight ring: slot j holds one slab of both row tiles
    const int wvoff = lane << 4, svoff = r * SBYTES;
    u32x4 wr[D][NT];
    uint32_t sr[D][NT][2];
    auto wload = [&](int j, int s) {
        const bool live = s < s_end;  // uniform
        const int sc = min(s, s_last);
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const int64_t rt = min(row_of(slot_of(t)), a.RT - 1);
            wr[j][t] = bload16_nt(make_rsrc(a.w + ((rt * a.S + sc) << 10), live ? 1024 : 0), wvoff, 0);
            const __amdgpu_buffer_rsrc_t srs = make_rsrc(
                a.w + a.scale_off + (rt * a.S + sc) * (16 * SBYTES), live ? 16 * SBYTES : 0);
            if constexpr (FMT == FMT_NV) {
                const u32x2 v = bload8_nt(srs, svoff, 0);
                sr[j][t][0] = v[0];
                sr[j][t][1] = v[1];
            } else {
                sr[j][t][0] = bload4_nt(srs, svoff, 0);
                sr[j][t][1] = 0u;
            }
        }
    };

    f32x4 acc[NT][MB];
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
            acc[t][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One slab: per unit both tiles decoded, then every batch group's three
    // MFMAs per tile (the streaming kernel's order, see the file comment).
    const uint32_t nvsh = 8 * (gq >> 1);  // NVFP4: this lane's scale byte within a unit's pair
    auto compute = [&](const u32x4 *slab, const u32x4 (&wc)[NT], const uint32_t (&sc)[NT][2]) {
        f32x4 part[NT][MB];
#pragma unroll
        for (int t = 0; t < NT; t++)
#pragma unroll
            for (int mb = 0; mb < MB; mb++)
                part[t][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < U; u++) {
            bf16x8 Bw[NT];
            float ps[NT];
#pragma unroll
            for (int t = 0; t < NT; t++) {
                if constexpr (FMT == FMT_Q8) {
                    Bw[t] = q8_to_bf16(wc[t][2 * u], wc[t][2 * u + 1]);
                    ps[t] = fp16_bits_to_f32((sc[t][0] >> (16 * u)) & 0xFFFFu);
                } else if constexpr (FMT == FMT_FP8) {
                    Bw[t] = fp8_to_bf16(wc[t][2 * u], wc[t][2 * u + 1]);
                    ps[t] = __uint_as_float(sc[t][0]);  // the slab's block scale
                } else if constexpr (FMT == FMT_MX) {
                    Bw[t] = fp4_to_bf16(wc[t][u], 1.0f);
                    ps[t] = e8m0_to_f32((sc[t][0] >> (8 * u)) & 0xFFu);
                } else {
                    const uint32_t sv = (u < 2 ? sc[t][0] : sc[t][1]) >> nvsh;
                    const float bs = (u & 1) ? e4m3_byte_to_f32<2>(sv) : e4m3_byte_to_f32<0>(sv);
                    Bw[t] = fp4_to_bf16_mul(wc[t][u], bs);
                    ps[t] = 1.f;
                }
            }
            // term-major: the NT x MB chains of the unit advance together,
            // so no MFMA waits for the one just issued (the same per-output
            // order as one chain at a time)
            f32x4 tacc[NT][MB];
#pragma unroll
            for (int tt = 0; tt < NTA; tt++) {
#pragma unroll
                for (int mb = 0; mb < MB; mb++) {
                    const bf16x8 A = __builtin_bit_cast(bf16x8, slab[tt * TSTR + (mb * U + u) * 64 + lane]);
#pragma unroll
                    for (int t = 0; t < NT; t++) {
                        if constexpr (POST)
                            tacc[t][mb] = mfma(A, Bw[t], tt == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : tacc[t][mb]);
                        else
                            part[t][mb] = mfma(A, Bw[t], part[t][mb]);
                    }
                }
            }
            if constexpr (POST) {
#pragma unroll
                for (int t = 0; t < NT; t++)
#pragma unroll
                    for (int mb = 0; mb < MB; mb++)
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            part[t][mb][i] = __builtin_fmaf(ps[t], tacc[t][mb][i], part[t][mb][i]);
            }
        }
#pragma unroll
        for (int t = 0; t < NT; t++)
#pragma unroll
            for (int mb = 0; mb < MB; mb++) {
                acc[t][mb][0] += part[t][mb][0];
                acc[t][mb][1] += part[t][mb][1];
                acc[t][mb][2] += part[t][mb][2];
                acc[t][mb][3] += part[t][mb][3];
            }
    };

    // ---- the two roles, each in a loop of its own with one barrier per step
    // of SPS slabs (the same count in both).  Step t: compute waves compute
    // its slabs (in slab order) from its LDS buffer and the ring slots
    // holding their weights, then refill those slots with the slabs D
    // further on; staging waves split step t + 1 into the other buffer and
    // issue the loads of step t + 1 + NSET into the register set that freed.
    // The steps of a ring turn are unrolled and DS is a multiple of NSET and
    // of 2, so slots, sets and buffers are known at compile time.  Each
    // prologue leaves the same loads in flight as a step does, so the
    // compiler's waits need no drain on entry.  Both loops run whole ring
    // turns; past the range the staging repeats the last slab into a buffer
    // nobody reads and the compute waves only keep the barrier count.  (One
    // loop with a branch per role, or early exits from the unrolled steps,
    // made the compiler merge or copy load results, draining every load at
    // every step.)
    const int nsteps = (s_end - s_beg + SPS - 1) / SPS;
    if (stager) {
#pragma unroll
        for (int k = 0; k < NSET; k++)
            xload(k, s_beg + k * SPS);
        xstore(0, xs[0]);
        xload(0, s_beg + NSET * SPS);
        __syncthreads();
        for (int t0 = 0; t0 < nsteps; t0 += DS) {
#pragma unroll
            for (int j = 0; j < DS; j++) {
                xstore((j + 1) % NSET, xs[(j + 1) & 1]);
                xload((j + 1) % NSET, s_beg + (t0 + j + 1 + NSET) * SPS);
                __syncthreads();
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < D; j++)
            wload(j, s_beg + j);
        __syncthreads();
        for (int t0 = 0; t0 < nsteps; t0 += DS) {
#pragma unroll
            for (int j = 0; j < DS; j++) {
#pragma unroll
                for (int sl = 0; sl < SPS; sl++) {
                    const int s = s_beg + (t0 + j) * SPS + sl;
                    if (s < s_end)  // uniform; padding only keeps the barrier count
                        compute(xs[j & 1] + sl * SLAB_E, wr[j * SPS + sl], sr[j * SPS + sl]);
                }
                // refill the slots after their last use, so the new slabs
                // load into the same registers and nothing is copied at the
                // back edge (a copy would wait for every load in flight)
#pragma unroll
                for (int sl = 0; sl < SPS; sl++)
                    wload(j * SPS + sl, s_beg + (t0 + j) * SPS + sl + D);
                __syncthreads();
            }
        }
    }
    // The staging waves stay to the end: they take part in every barrier
    // below and skip the work.

    // Store row tile rt (lane: batch rows 16*mb + 4*gq + i of column r).
    auto store_tile = [&](int rt, const f32x4 (&v)[MB]) {
        const int n = rt * 16 + r;
        if (n >= a.N)
            return;
        float gsc = 1.f;
        if constexpr (FMT == FMT_NV)
            gsc = tensor_scale(a, n);
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int b = 16 * mb + 4 * gq + i;
                if (b < a.B)
                    store_out_nt<OUTT>(a.y, (int64_t)b * a.N + n, gsc * v[mb][i]);
            }
    };

    // SwiGLU: store SiLU(G) * U of gate tile gt (lane: batch rows
    // 16*mb + 4*gq + i of column r), y being [B][Nh].
    auto store_swiglu = [&](int gt, const f32x4 (&G)[MB], const f32x4 (&Up)[MB]) {
        const int col = gt * 16 + r;
        if (col >= Nh)
            return;
        float g0 = 1.f, g1 = 1.f;
        if constexpr (FMT == FMT_NV) {
            g0 = tensor_scale(a, col);
            g1 = tensor_scale(a, Nh + col);
        }
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int b = 16 * mb + 4 * gq + i;
                if (b < a.B)
                    store_out_nt<OUTT>(a.y, (int64_t)b * Nh + col, silu(g0 * G[mb][i]) * (g1 * Up[mb][i]));
            }
    };

    // ---- K split: publish the partial tiles; the last workgroup of the
    // group adds them in split order
    if (ws.ksplit > 1) {
        const int64_t tiles = (int64_t)ngroups * ST_RG * MB;  // 16x16 partial tiles per split
        uint64_t *part = (uint64_t *)ws.part;
#pragma unroll
        for (int t = 0; t < NT; t++)
#pragma unroll
            for (int mb = 0; mb < MB; mb++) {
                if (stager)
                    break;  // uniform
                const int64_t tile = ((int64_t)grp * ST_RG + slot_of(t)) * MB + mb;
                if (ws.xlocal)  // every reader of these lines runs on this XCD
                    publish_partial<__HIP_MEMORY_SCOPE_WORKGROUP>(part, ks, tiles, tile, lane, acc[t][mb]);
                else
                    publish_partial<__HIP_MEMORY_SCOPE_AGENT>(part, ks, tiles, tile, lane, acc[t][mb]);
            }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are acknowledged
        __syncthreads();
        if (tid == 0) {
            if (ws.xlocal) {
                // the streaming kernel's per-launch placement check: one per
                // split in the nibble of its XCC; splits on more than one XCD
                // set DEV_XCD_MISMATCH
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
        // The last workgroup of the group: all 8 waves, wave w adding row
        // tile w of the group for every batch group, its ksplit partials
        // (this workgroup's own included, read back) in split order.  A
        // lane's 16 bytes of a partial tile are one load, with the cache
        // scope of the stores (workgroup: this XCD's L2; else device), and
        // every load of a chunk of splits is issued before the first add.
        // With SwiGLU, waves 0..3 each add gate slot w and up slot 4 + w.
        const int64_t tbytes = tiles * 1024;
        if (tid == 0)
            __hip_atomic_store(&ws.cnt[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        auto sum_slot = [&](int g, f32x4 (&sum)[MB]) {
            const int tvo = (int)((((int64_t)grp * ST_RG + g) * MB) * 1024) + lane * 16;
            if (ws.xlocal)
                vf_sum_splits<CP_SC0, MB>((const uint8_t *)ws.part, ws.ksplit, tbytes, tvo, sum);
            else
                vf_sum_splits<CP_SC1, MB>((const uint8_t *)ws.part, ws.ksplit, tbytes, tvo, sum);
        };
        f32x4 sum[MB];
        if (Nh) {
            if (wid >= 4)
                return;  // uniform per wave; no barrier follows
            f32x4 up[MB];
            sum_slot(wid, sum);
            sum_slot(4 + wid, up);
            store_swiglu(grp * 4 + wid, sum, up);
            return;
        }
        sum_slot(wid, sum);
        store_tile(row_of(wid), sum);
        return;
    }

    // ---- unsplit: each compute wave stores its two tile slots
    if (stager)
        return;  // uniform
    if (Nh) {
        store_swiglu(grp * 4 + (wid & 3), acc[0], acc[1]);
        return;
    }
#pragma unroll
    for (int t = 0; t < NT; t++)
        store_tile(row_of(slot_of(t)), acc[t]);
}

}  // namespace qg
