// Large-batch tier: one BM x BN output tile per workgroup, bf16 MFMA from
// LDS-staged fragments.
//
// 8 waves (two per SIMD) arranged 2 (batch) x 4 (weight rows); each wave owns
// BM/2 x 64 outputs as (BM/32) x 4 tiles of v_mfma_f32_16x16x32_bf16.  A
// 4-wave form (NW = 4: one wave per SIMD, 2 x 2, each wave BM/2 x 128
// outputs, its 256 accumulator registers in AGPRs) reads a third fewer LDS
// fragment bytes per MFMA but hides less latency; it measured 4-15 % slower
// at B = 2048 and is selected only by QGEMM_TI_WAVES=4.  K advances 64 per
// step:
//
//  * activations: BM x 64 (fp32 input rounded to bf16 on the way);
//  * weights: BN rows x 64, i.e. one Q8_0 slab or half an FP4 slab of each of
//    the BN/16 row tiles; a thread's 16-byte (Q8_0) or 8-byte (FP4) piece of a
//    slab chunk is decoded with its block scale folded in (exact for the FP4
//    formats, one rounding for Q8_0) into the two bf16 fragments it feeds;
//    MXFP4 instead stages the codes with their scale and decodes each
//    fragment as it is read (half the LDS bytes, the same values).
//
// LDS holds both operands as 16-byte fragment entries [k-group][row ^
// k-group], a swizzle under which neither the stage writes nor the fragment
// reads collide in banks; it is double-buffered.  Global loads go through buffer
// resources (fixed per-lane offsets, the step in the scalar offset, zero
// past the data) into register stages two steps ahead of their use (three or
// four for routed experts), and the conversion and LDS stores of the next
// step are interleaved by hand with the MFMA groups of the current one, so
// each step ends in one barrier.
//
// Tile counts: whole rounds of 256 tiles (one per CU) run unsplit; the tiles
// of a last, partial round may be split along K into pieces, one workgroup
// each, whose partial tiles tiled_reduce adds in piece order.
//
// SwiGLU: the staged rows are BN/2 gate rows j and the BN/2 up rows Nh + j,
// and every wave owns matching gate and up columns, so G and U of an output
// sit in the same lane for the epilogue.
//
// fp32-faithful variant (FAITH): fp32 activations are staged as three bf16
// terms that add up to the exact value, weights as their exact unscaled
// codes (NVFP4: times its E4M3 scale, also exact), so every MFMA product is
// exact; the three terms' MFMAs of a 32-wide block run into a block partial
// from zero, and the Q8_0 / MXFP4 / FP8 block scale (staged in LDS beside the
// weights, one fp32 per staged row and block) multiplies that partial into
// the accumulator.  Tiles are BM = 64 or 96 rows so the three activation
// planes fit in LDS.
#include <type_traits>

#include "common.h"

namespace qg {

// Output column (in the staged BN rows) of n-tile j of wave column wn, for
// NW waves in 2 x NW/2 (SwiGLU: the first half of a wave's tiles are gate
// columns, the second half the matching up columns BN/2 further on).
template <bool DUAL, int NW>
__device__ __forceinline__ int tiled_wcol(int wn, int j)
{
    constexpr int BN = 256, WCOLS = BN / (NW / 2), TN = WCOLS / 16;
    if constexpr (DUAL)
        return j < TN / 2 ? wn * (WCOLS / 2) + 16 * j : BN / 2 + wn * (WCOLS / 2) + 16 * (j - TN / 2);
    else
        return wn * WCOLS + 16 * j;
}

template <int FMT, int ACT, int OUTT, bool DUAL, int BM, bool GROUPED, bool FAITH, int NW = 8>
__global__ __launch_bounds__(NW * 64) void tiled_kernel(KArgs a, int Nh, int mtiles, TiSplit sp, Groups grp)
{
    constexpr int BN = 256;                    // staged weight rows
    constexpr int KT = 64;                     // K per step
    constexpr int KG = KT / 8;                 // 16-byte k-groups per step
    constexpr int NTHR = NW * 64;
    constexpr int XP = BM, WP = BN;            // LDS entries per k-group
    constexpr int TM = BM / 2 / 16;            // 16-row MFMA tiles per wave (batch)
    constexpr int TN = BN / (NW / 2) / 16;     // 16-col MFMA tiles per wave (weights)
    static_assert(NW == 8 || (NW == 4 && !FAITH), "8 waves, or 4 for bf16 math");
    constexpr int CE = ACT == ACT_F32 ? 4 : 8; // activations per 16-byte load
    constexpr int XCH = BM * KT / CE / NTHR;   // activation loads per thread per step
    constexpr int WCH = (BN / 16) * 64 / NTHR; // weight chunks per thread per step (2 or 4)
    constexpr int WCH2 = WCH / 2;              // chunks per half (gate / up) of the staged rows
    constexpr bool FP4 = FMT == FMT_MX || FMT == FMT_NV;  // 128-wide slabs, two steps each
    constexpr int NTA = FAITH && ACT == ACT_F32 ? 3 : 1;  // activation terms
    constexpr bool POST = FAITH && FMT != FMT_NV;         // block scale after the MFMA
    static_assert(XCH * NTHR * CE == BM * KT, "activation staging");
    static_assert(!FAITH || BM == 64 || BM == 96, "the faithful variant runs 64- or 96-row tiles");

    // LDS entry of (k-group kg, row): rows XOR kg.  Fragment reads (16 rows of
    // one k-group per 16 lanes) then cover all 64 banks without conflict, and
    // so do the activation stage writes (8 k-groups of one row per 8 lanes),
    // which a plain [kg][row] layout would put in one bank group (measured on
    // gfx950: 4 and 13 cycles per wave-wide 16-byte read and write, against 8
    // for the reads of a layout padded by one entry per k-group).
    auto lx = [](int kg, int row) { return kg * XP + (row ^ kg); };
    auto lw = [](int kg, int col) { return kg * WP + (col ^ kg); };
    __shared__ u32x4 xs[2][NTA][KG * XP];
    // MXFP4 (bf16 math) stages the packed codes instead of decoded bf16: each
    // entry is one lane's 8 codes of a fragment and its E8M0 scale as fp32
    // (8 bytes, not 16), decoded when the fragment is read
    constexpr bool CMX = FMT == FMT_MX && !FAITH;
    __shared__ u32x4 ws[2][CMX ? 1 : KG * WP];
    __shared__ u32x2 wsc[2][CMX ? KG * WP : 1];
    __shared__ float ss[POST ? 2 * 2 * BN : 1];  // [buf][32-wide block of the step][staged row]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int wm = wid & 1, wn = wid >> 1;

    int tile = 0, ks = 0, mt = 0, ntl = 0;
    bool split = false;
    if constexpr (GROUPED) {
        // Routed experts: workgroup ids run over the experts' row tiles in
        // expert order (weight tiles fastest).  A block scan of the per-expert
        // row-tile counts finds this workgroup's expert and row tile; the rest
        // of the kernel then runs on that expert's weights and rows, unsplit.
        __shared__ int s_wsum[NTHR / 64];
        __shared__ int s_e, s_mt;
        const int j = (int)blockIdx.x / grp.ntiles;
        ntl = (int)blockIdx.x % grp.ntiles;
        if (tid == 0)
            s_e = -1;
        // Every workgroup also checks the offsets it scans (all of them):
        // off[0] = 0, non-decreasing, off[E] = T.  If they break a rule no
        // workgroup does any work, and workgroup 0 sets DEV_BAD_OFFSETS in the
        // device status word, so bad offsets never move a load or a store
        // outside x and y.
        int base = 0;  // row tiles of the experts before this chunk
        int bad = 0;
        for (int e0 = 0; e0 < grp.E; e0 += NTHR) {
            const int e = e0 + tid;
            int c = 0;
            if (e < grp.E) {
                const int lo = grp.off[e], hi = grp.off[e + 1];
                bad |= (hi < lo) | (e == 0 && lo != 0) | (e == grp.E - 1 && hi != grp.T);
                c = hi > lo ? (int)(((int64_t)hi - lo + BM - 1) / BM) : 0;
            }
            int v = c;  // inclusive scan within the wave
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int up = __shfl_up(v, d, 64);
                if (lane >= d)
                    v += up;
            }
            if (lane == 63)
                s_wsum[wid] = v;
            __syncthreads();
            int pre = 0, tot = 0;
#pragma unroll
            for (int w2 = 0; w2 < NTHR / 64; w2++) {
                const int ws2 = s_wsum[w2];
                pre += w2 < wid ? ws2 : 0;
                tot += ws2;
            }
            const int inc = base + pre + v;  // row tiles of experts <= e
            if (c > 0 && j >= inc - c && j < inc) {
                s_e = e;
                s_mt = j - (inc - c);
            }
            base += tot;
            __syncthreads();  // s_wsum is rewritten by the next chunk
        }
        if (__syncthreads_or(bad)) {
            if (blockIdx.x == 0 && tid == 0)
                __hip_atomic_fetch_or(grp.status, DEV_BAD_OFFSETS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;  // uniform over the workgroup
        }
        if (s_e < 0)
            return;  // past the experts' last row tile (uniform)
        const int e = s_e;
        mt = s_mt;
        const int r0 = grp.off[e];
        constexpr int XSZ = ACT == ACT_F32 ? 4 : 2, YSZ = OUTT == OUT_F32 ? 4 : 2;
        a.B = grp.off[e + 1] - r0;
        a.w = grp.wtab[e];
        a.x = (const uint8_t *)a.x + (int64_t)r0 * a.K * XSZ;
        a.y = (uint8_t *)a.y + (int64_t)r0 * (DUAL ? Nh : a.N) * YSZ;
    } else {
        // XCD-aware order: hardware hands consecutive workgroup ids to different
        // XCDs (id mod 8); give each XCD a contiguous range of tiles, batch tiles
        // fastest, so the workgroups sharing an XCD's L2 share weight tiles and
        // the same activation rows.  Whole tiles and split pieces are remapped as
        // two separate groups (ids below and from sp.full), so both spread evenly
        // over the XCDs.
        const bool piece = (int)blockIdx.x >= sp.full;
        const int g0 = piece ? sp.full : 0;
        const int ng = piece ? (int)gridDim.x - sp.full : sp.full;
        int t = (int)blockIdx.x - g0;
        {
            const int per = (ng + 7) / 8;
            const int xcd = t % 8, loc = t / 8;
            const int full = ng % 8 == 0 ? 8 : ng % 8;  // XCDs that own 'per' tiles
            t = xcd < full ? xcd * per + loc : full * per + (xcd - full) * (per - 1) + loc;
        }
        t += g0;
        // Tiles below sp.full run whole; each later tile is split along K into
        // sp.S pieces (workgroups).
        tile = t;
        if (piece) {
            tile = sp.full + (t - sp.full) / sp.S;
            ks = (t - sp.full) % sp.S;
        }
        split = piece && sp.S > 1;
        mt = tile % mtiles;
        ntl = tile / mtiles;
    }
    const int b0 = mt * BM;
    const int n0 = ntl * (DUAL ? BN / 2 : BN);  // first output column
    const int nsteps = (a.K + KT - 1) / KT;
    // this workgroup's K steps [sb, se)
    const int spp = split ? (nsteps + sp.S - 1) / sp.S : nsteps;
    const int sb = split ? min(nsteps, ks * spp) : 0;
    const int se = split ? min(nsteps, sb + spp) : nsteps;

    // ---- register stage of one K step.  Loads go through buffer resources:
    // per-lane offsets are fixed, the step only moves the scalar offset, and
    // rows or tiles past the end of the data read as zero.
    constexpr int ESZ = ACT == ACT_F32 ? 4 : 2;
    const int gate_rt0 = n0 / 16;                          // first (gate) row tile
    const int up_rt0 = DUAL ? (Nh + n0) / 16 : gate_rt0 + BN / 32;
    const int64_t code_bytes = (int64_t)a.RT * a.S * 1024;
    constexpr int SREC = 16 * scale_bytes_per_slab(FMT);  // scale record of a (row tile, slab)
    const int64_t sc_bytes = (int64_t)a.RT * a.S * SREC;
    const __amdgpu_buffer_rsrc_t xres =
        make_rsrc((const uint8_t *)a.x + (int64_t)b0 * a.K * ESZ, (int64_t)(a.B - b0) * a.K * ESZ);
    // weight chunk i of a thread covers staged row tile c >> 6 with c = tid +
    // NTHR i: chunks i < WCH2 the first BN/32 tiles, the rest the second
    // (SwiGLU: gate, then up); within a half, chunk i starts (i % WCH2) *
    // NTHR/64 tiles on (in the scalar offset)
    const int64_t wb0 = (int64_t)gate_rt0 * a.S * 1024, wb1 = (int64_t)up_rt0 * a.S * 1024;
    const int64_t sb0 = (int64_t)gate_rt0 * a.S * SREC, sb1 = (int64_t)up_rt0 * a.S * SREC;
    const __amdgpu_buffer_rsrc_t wres[2] = {make_rsrc(a.w + wb0, code_bytes - wb0),
                                            make_rsrc(a.w + wb1, code_bytes - wb1)};
    const __amdgpu_buffer_rsrc_t sres[2] = {make_rsrc(a.w + a.scale_off + sb0, sc_bytes - sb0),
                                            make_rsrc(a.w + a.scale_off + sb1, sc_bytes - sb1)};
    // activation chunk i of a thread is row tid / (KT / CE) + i * XRI of the
    // tile: one per-lane offset, the chunk's rows in the scalar offset
    constexpr int XRI = NTHR / (KT / CE);
    const int xoff = ((tid / (KT / CE)) * a.K + (tid % (KT / CE)) * CE) * ESZ;
    const int xrow_bytes = XRI * a.K * ESZ;
    const int woff = (((tid >> 6) * a.S) << 10) + (lane << 4);
    const int soff = (tid >> 6) * a.S * SREC + (lane & 15) * scale_bytes_per_slab(FMT);
    const int wtile_step = (NTHR / 64) * a.S;  // slabs between chunk i and i + 1 of a half
    const bool ktail = a.K % KT != 0;  // the last step has columns past K

    // Register stages: PF slots, each one step's global loads; slot r is
    // refilled PF steps after it was loaded.  Routed experts in 64- and
    // 128-row tiles, whose workgroups have little MFMA work per step, keep
    // two or three steps in flight (as many as the registers hold; deeper
    // stages measured no faster for the dense GEMM).
    constexpr int PF = GROUPED && BM <= 128 ? (ACT == ACT_BF16 ? 3 : 2) : 1;
    u32x4 xr[PF][XCH];
    uint32_t wr[PF][WCH][FP4 ? 2 : 4];
    uint32_t sr[PF][WCH][2];

    auto load_wstage = [&](int r, int step) {
        const int s = FP4 ? step >> 1 : step;   // slab
        const int half = FP4 ? step & 1 : 0;    // which 64 k of an FP4 slab
        const int ssc = s * SREC;
#pragma unroll
        for (int i = 0; i < WCH; i++) {
            const int h = i / WCH2, t = (i % WCH2) * wtile_step;  // half, slabs from its first tile
            if constexpr (FP4) {
                const u32x2 v = bload8(wres[h], woff, ((s + t) << 10) + 8 * half);
                wr[r][i][0] = v[0];
                wr[r][i][1] = v[1];
            } else {
                const u32x4 v = bload16(wres[h], woff, (s + t) << 10);
                wr[r][i][0] = v[0]; wr[r][i][1] = v[1]; wr[r][i][2] = v[2]; wr[r][i][3] = v[3];
            }
            if constexpr (FMT == FMT_NV) {
                const u32x2 v = bload8(sres[h], soff, ssc + t * SREC);
                sr[r][i][0] = v[0];
                sr[r][i][1] = v[1];
            } else {
                sr[r][i][0] = bload4(sres[h], soff, ssc + t * SREC);
                sr[r][i][1] = 0;
            }
        }
    };

    // The last step of a K that is not a multiple of the step reads the next
    // row's first columns: zero them (rare; a branch of its own so the common
    // steps carry no masking work).
    auto tail_mask = [&](int r, int step) {
        if (ktail && step == nsteps - 1) {
#pragma unroll
            for (int i = 0; i < XCH; i++) {
                const int c = tid + i * NTHR;
                if (step * KT + (c % (KT / CE)) * CE >= a.K)
                    xr[r][i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    // One activation chunk (i < XCH) of the next stage into LDS buffer buf.
    // The swizzle permutes only the low three bits of a row (or column), so
    // every LDS access below is a per-lane base plus a compile-time offset.
    // Activation chunk i of this thread: row tid / (KT/CE) + i * XRI, columns
    // xkk .. xkk + CE - 1 of the step.
    const int xkk = (tid % (KT / CE)) * CE;
    const int xw0 = lx(xkk >> 3, tid / (KT / CE));
    auto xpiece = [&](int r, int buf, int i) {
        const int e = xw0 + i * XRI;
        const int kk = xkk;
        const u32x4 v = xr[r][i];
        if constexpr (NTA > 1) {
            float f[4];
#pragma unroll
            for (int e = 0; e < 4; e++)
                f[e] = __uint_as_float(v[e]);
            const Split<NTA> s = split_f32<NTA, 4>(f);
#pragma unroll
            for (int t = 0; t < NTA; t++) {
                const u32x4 q = __builtin_bit_cast(u32x4, s.t[t]);
                u32x2 *dst = (u32x2 *)&xs[buf][t][e] + ((kk & 7) >> 2);
                *dst = u32x2{q[0], q[1]};
            }
        } else if constexpr (ACT == ACT_F32) {
            bf16x2 p0, p1;
            p0[0] = (__bf16)__uint_as_float(v[0]);
            p0[1] = (__bf16)__uint_as_float(v[1]);
            p1[0] = (__bf16)__uint_as_float(v[2]);
            p1[1] = (__bf16)__uint_as_float(v[3]);
            u32x2 *dst = (u32x2 *)&xs[buf][0][e] + ((kk & 7) >> 2);
            *dst = u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
        } else {
            xs[buf][0][e] = v;
        }
    };
    // One decoded weight unit (p < 2 * WCH: chunk p / 2, unit p % 2) of the
    // next stage (step `step`) into LDS buffer buf, block scale folded in.
    // Weight unit ul of chunk i: k-group 4 ul + lane / 16 of staged column
    // (tid / 64 + i NTHR / 64) * 16 + lane % 16.
    const int ww0[2] = {lw(lane >> 4, (tid >> 6) * 16 + (lane & 15)), lw(4 + (lane >> 4), (tid >> 6) * 16 + (lane & 15))};
    auto wpiece = [&](int r, int buf, int step, int p) {
        const int i = p >> 1, ul = p & 1;
        const int half = FP4 ? step & 1 : 0;
        const int col = ((tid >> 6) + i * (NTHR / 64)) * 16 + (lane & 15);
        const int g = lane >> 4;
        const int e = ww0[ul] + i * (NTHR / 64) * 16;
        bf16x8 h;
        if constexpr (POST) {
            // exact codes; the block scale goes to LDS once per staged row
            float d;
            if constexpr (FMT == FMT_Q8) {
                h = q8_to_bf16(wr[r][i][2 * ul], wr[r][i][2 * ul + 1]);
                d = fp16_bits_to_f32((sr[r][i][0] >> (16 * ul)) & 0xFFFFu);
            } else if constexpr (FMT == FMT_FP8) {
                h = fp8_to_bf16(wr[r][i][2 * ul], wr[r][i][2 * ul + 1]);
                d = __uint_as_float(sr[r][i][0]);
            } else {
                h = fp4_to_bf16(wr[r][i][ul], 1.0f);
                d = e8m0_to_f32((sr[r][i][0] >> (8 * (2 * half + ul))) & 0xFFu);
            }
            if (g == 0)
                ss[(buf * 2 + ul) * BN + col] = d;
        } else if constexpr (FMT == FMT_Q8) {
            const float d = fp16_bits_to_f32((sr[r][i][0] >> (16 * ul)) & 0xFFFFu);
            h = q8_scaled_to_bf16(wr[r][i][2 * ul], wr[r][i][2 * ul + 1], d);
        } else if constexpr (FMT == FMT_FP8) {
            h = fp8_scaled_to_bf16(wr[r][i][2 * ul], wr[r][i][2 * ul + 1], __uint_as_float(sr[r][i][0]));
        } else if constexpr (FMT == FMT_MX) {
            const int u = 2 * half + ul;
            const float d = e8m0_to_f32((sr[r][i][0] >> (8 * u)) & 0xFFu);
            wsc[buf][e] = u32x2{wr[r][i][ul], __float_as_uint(d)};
            return;
        } else {
            const int u = 2 * half + ul;
            const int si = 2 * u + (g >> 1);
            // byte si of the 8 scale bytes, by one 64-bit shift (a select of
            // the dword turned into an indexed private array, i.e. scratch)
            const uint64_t sc8 = ((uint64_t)sr[r][i][1] << 32) | sr[r][i][0];
            const uint32_t sb = (uint32_t)(sc8 >> (8 * si)) & 0xFFu;
            h = fp4_to_bf16_mul(wr[r][i][ul], e4m3_to_f32(sb));
        }
        ws[buf][e] = __builtin_bit_cast(u32x4, h);
    };
    auto store_stage = [&](int r, int buf, int step) {
#pragma unroll
        for (int i = 0; i < XCH; i++)
            xpiece(r, buf, i);
#pragma unroll
        for (int p = 0; p < 2 * WCH; p++)
            wpiece(r, buf, step, p);
    };

    // staged column of the wave's n-tile j
    auto wcol = [&](int j) { return tiled_wcol<DUAL, NW>(wn, j); };
    // fragment reads of MFMA k-step kk: k-group 4 kk + lane / 16, row (or
    // column) base + lane % 16 for a base that is a multiple of 16
    const int xa[2] = {lx(lane >> 4, wm * (BM / 2) + (lane & 15)), lx(4 + (lane >> 4), wm * (BM / 2) + (lane & 15))};
    const int wb[2] = {lw(lane >> 4, lane & 15), lw(4 + (lane >> 4), lane & 15)};

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (NW == 4) {
        // 4 waves: the 256 (BM = 256) accumulator registers live in AGPRs for
        // the whole kernel.  Binding them there once (an empty asm, no
        // instruction) keeps the register allocator from splitting them
        // between the two register files and copying them every step.
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++)
                asm volatile("" : "+a"(acc[i][j]));
    }

    auto load_xstage = [&](int r, int step) {
#pragma unroll
        for (int i = 0; i < XCH; i++)
            xr[r][i] = bload16(xres, xoff, i * xrow_bytes + step * KT * ESZ);
    };

    load_xstage(0, sb);
    load_wstage(0, sb);
    tail_mask(0, sb);
    store_stage(0, sb & 1, sb);
#pragma unroll
    for (int r = 0; r < PF; r++) {
        load_xstage(r, min(sb + 1 + r, se - 1));
        load_wstage(r, min(sb + 1 + r, se - 1));
    }
    __syncthreads();

    // One step: the MFMAs of step s from LDS buffer s & 1, interleaved by
    // hand (fences keep the order) with the next stage: after each group of
    // TN MFMAs (one A fragment: a batch tile, or one term of it) pieces of
    // work on step s + 1 (weight units during the first k-step, activation
    // chunks during the second, dealt round-robin over the groups), whose
    // register slot is then refilled by the global loads of step s + 1 + PF.
    // Past the last step the pieces repeat the last step's data into a
    // buffer no one reads.
    constexpr int NG = TM * NTA;  // MFMA groups per k-step
    // With 8 waves the loop exists twice: with the K-tail masking (K not a
    // multiple of the step) and without it, so the common case carries no
    // masking work; with 4 waves once, masking behind a uniform branch (two
    // copies of a loop carrying 256 accumulators defeat the allocator).
    auto main_loop = [&](auto masking) {
    for (int step0 = sb; step0 < se; step0 += PF) {
#pragma unroll
    for (int r = 0; r < PF; r++) {  // slot r holds step + 1
        const int step = step0 + r;
        if (step >= se)
            break;  // uniform
        const int buf = step & 1;
        const int nst = min(step + 1, se - 1);
        if constexpr (decltype(masking)::value)
            tail_mask(r, nst);
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {        // two 32-wide MFMA k-steps
            // A fragment q: batch tile q / NTA, term q % NTA
            auto afrag = [&](int q) {
                return __builtin_bit_cast(
                    bf16x8, xs[buf][q % NTA][xa[kk] + 16 * (q / NTA)]);
            };
            bf16x8 bw[TN];
            float bsc[TN];  // block scale of each n-tile's column (POST)
#pragma unroll
            for (int j = 0; j < TN; j++) {
                if constexpr (CMX) {
                    const u32x2 e = wsc[buf][wb[kk] + wcol(j)];
                    bw[j] = fp4_to_bf16(e[0], __uint_as_float(e[1]));
                } else {
                    bw[j] = __builtin_bit_cast(bf16x8, ws[buf][wb[kk] + wcol(j)]);
                }
                if constexpr (POST)
                    bsc[j] = ss[(buf * 2 + kk) * BN + wcol(j) + (lane & 15)];
            }
            f32x4 part[POST ? TM : 1][TN];  // block partials (POST)
            bf16x8 af = afrag(0);
#pragma unroll
            for (int q = 0; q < NG; q++) {
                const int i = q / NTA, t = q % NTA;
                bf16x8 afn = af;
                if (q + 1 < NG)
                    afn = afrag(q + 1);
#pragma unroll
                for (int j = 0; j < TN; j++) {
                    if constexpr (POST)
                        part[i][j] = mfma(af, bw[j], t == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : part[i][j]);
                    else
                        acc[i][j] = mfma(af, bw[j], acc[i][j]);
                }
#pragma unroll
                for (int p = q; p < 2 * WCH; p += NG)
                    if (kk == 0)
                        wpiece(r, buf ^ 1, nst, p);
#pragma unroll
                for (int p = q; p < XCH; p += NG)
                    if (kk == 1)
                        xpiece(r, buf ^ 1, p);
                __builtin_amdgcn_sched_barrier(0);
                af = afn;
            }
            if constexpr (POST) {
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN; j++)
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            acc[i][j][e] = __builtin_fmaf(bsc[j], part[i][j][e], acc[i][j][e]);
            }
            // refill the slot this half consumed, PF steps ahead of its use
            if (kk == 0)
                load_wstage(r, min(step + 1 + PF, se - 1));
            else
                load_xstage(r, min(step + 1 + PF, se - 1));
        }
        __syncthreads();
    }
    }
    };
    if (NW == 4 || ktail)
        main_loop(std::true_type{});
    else
        main_loop(std::false_type{});

    // ---- K split: this piece's tile goes to the workspace; tiled_reduce (the
    // next kernel on the stream) adds the pieces in order and stores y
    if (split) {
        const int r = tile - sp.full;               // split tile index
        f32x4 *dst = (f32x4 *)sp.part + ((int64_t)r * sp.S + ks) * (NTHR * TM * TN) + tid;
#pragma unroll
        for (int i = 0; i < TM; i++) {
            if (b0 + wm * (BM / 2) + 16 * i >= a.B)
                continue;  // a 16-row block wholly past B: tiled_reduce skips it too
#pragma unroll
            for (int j = 0; j < TN; j++)
                dst[(i * TN + j) * NTHR] = acc[i][j];
        }
        return;
    }

    // ---- epilogue (lane holds rows 4*(lane/16)+e of each 16x16 tile, column lane%16)
#pragma unroll
    for (int j = 0; j < (DUAL ? TN / 2 : TN); j++) {
        const int col = n0 + wcol(j) + (lane & 15);
        if (col >= (DUAL ? Nh : a.N))
            continue;
        float g0 = 1.f, g1 = 1.f;
        if constexpr (FMT == FMT_NV) {
            g0 = tensor_scale(a, col);
            if constexpr (DUAL)
                g1 = tensor_scale(a, Nh + col);
        }
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int b = b0 + wm * (BM / 2) + 16 * i + 4 * (lane >> 4) + e;
                if (b >= a.B)
                    continue;
                if constexpr (DUAL) {
                    const float G = g0 * acc[i][j][e];
                    const float U = g1 * acc[i][j + TN / 2][e];
                    store_out<OUTT>(a.y, (int64_t)b * Nh + col, silu(G) * U);
                } else {
                    store_out<OUTT>(a.y, (int64_t)b * a.N + col, g0 * acc[i][j][e]);
                }
            }
    }
}

// Sum of the K-split pieces of the split tiles, in piece order, then the
// tiled_kernel epilogue.  The partial layout is the one tiled_kernel writes:
// [split tile][piece][MFMA tile i * TN + j][thread][4], one thread of this
// kernel per (split tile, i, j-pair, thread of the tiled workgroup).
template <int FMT, int OUTT, bool DUAL, int BM, int NW>
__global__ __launch_bounds__(256) void tiled_reduce(KArgs a, int Nh, int mtiles, TiSplit sp, int nsplit)
{
    constexpr int NTHR = NW * 64, TM = BM / 2 / 16, TN = 256 / (NW / 2) / 16;
    constexpr int JN = DUAL ? TN / 2 : TN;      // output column tiles per wave
    const int64_t per_piece = (int64_t)NTHR * TM * TN;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)nsplit * TM * JN * NTHR)
        return;
    const int th = (int)(idx % NTHR);
    const int64_t q = idx / NTHR;
    const int jj = (int)(q % JN);
    const int i = (int)(q / JN % TM);
    const int r = (int)(q / JN / TM);
    const int tile = sp.full + r;
    const int mt = tile % mtiles, ntl = tile / mtiles;
    const int lane = th & 63, wid = th >> 6, wm = wid & 1, wn = wid >> 1;
    const int b0 = mt * BM, n0 = ntl * (DUAL ? 128 : 256);
    if (b0 + wm * (BM / 2) + 16 * i >= a.B)
        return;  // a 16-row block wholly past B: its partials were never stored
    const f32x4 *src = (const f32x4 *)sp.part + (int64_t)r * sp.S * per_piece + th;
    // pieces in order; up to 8 loads in flight before the first add (a piece
    // index past S re-reads the last piece and is not added)
    f32x4 v0 = f32x4{0.f, 0.f, 0.f, 0.f}, v1 = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < sp.S; k0 += 8) {
        f32x4 t0[8], t1[8];
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int k = min(k0 + u, sp.S - 1);
            t0[u] = src[k * per_piece + (i * TN + jj) * NTHR];
            if constexpr (DUAL)
                t1[u] = src[k * per_piece + (i * TN + jj + TN / 2) * NTHR];
        }
#pragma unroll
        for (int u = 0; u < 8; u++) {
            if (k0 + u >= sp.S)
                break;
            v0[0] += t0[u][0]; v0[1] += t0[u][1]; v0[2] += t0[u][2]; v0[3] += t0[u][3];
            if constexpr (DUAL) {
                v1[0] += t1[u][0]; v1[1] += t1[u][1]; v1[2] += t1[u][2]; v1[3] += t1[u][3];
            }
        }
    }
    const int col = n0 + tiled_wcol<DUAL, NW>(wn, jj) + (lane & 15);
    if (col >= (DUAL ? Nh : a.N))
        return;
    float g0 = 1.f, g1 = 1.f;
    if constexpr (FMT == FMT_NV) {
        g0 = tensor_scale(a, col);
        if constexpr (DUAL)
            g1 = tensor_scale(a, Nh + col);
    }
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const int b = b0 + wm * (BM / 2) + 16 * i + 4 * (lane >> 4) + e;
        if (b >= a.B)
            continue;
        if constexpr (DUAL)
            store_out<OUTT>(a.y, (int64_t)b * Nh + col, silu(g0 * v0[e]) * (g1 * v1[e]));
        else
            store_out<OUTT>(a.y, (int64_t)b * a.N + col, g0 * v0[e]);
    }
}

// ------------------------------------------------------------------ host

template <int FMT, int ACT, int OUTT, bool DUAL, int BM, bool FAITH, int NW = 8>
static void launch_tiled_bm(const KArgs &a, const TiCfg &c, hipStream_t st, int Nh)
{
    constexpr int TN = 256 / (NW / 2) / 16;
    const int nsplit = c.tiles - c.sp.full;
    const Groups none = {nullptr, nullptr, 0, 0};
    hipLaunchKernelGGL((tiled_kernel<FMT, ACT, OUTT, DUAL, BM, false, FAITH, NW>), dim3((unsigned)c.wgs),
                       dim3(NW * 64), 0, st, a, Nh, c.mtiles, c.sp, none);
    if (c.sp.S > 1) {
        const int64_t n = (int64_t)nsplit * (BM / 32) * (DUAL ? TN / 2 : TN) * NW * 64;
        hipLaunchKernelGGL((tiled_reduce<FMT, OUTT, DUAL, BM, NW>), dim3((unsigned)((n + 255) / 256)), dim3(256),
                           0, st, a, Nh, c.mtiles, c.sp, nsplit);
    }
}

// Routed experts: one launch over every expert's row tiles (grid: an upper
// bound, extra workgroups leave after the scan), BM rows per tile.
template <int FMT, int ACT, int OUTT, bool DUAL, int BM, bool FAITH>
static void launch_grouped_bm(const KArgs &a, const Groups &g, int64_t tiles, hipStream_t st, int Nh)
{
    const TiSplit none = {0, 1, nullptr, nullptr};
    const dim3 grid((unsigned)(tiles * g.ntiles));
    hipLaunchKernelGGL((tiled_kernel<FMT, ACT, OUTT, DUAL, BM, true, FAITH>), grid, dim3(512), 0, st, a, Nh, 1,
                       none, g);
}

// One (format, math) pair: the activation, output and epilogue variants.
// bf16 math runs 128- or 256-row tiles, fp32-faithful math 64-row tiles.
// NW: waves per workgroup of the plain GEMM (routed experts and the
// fp32-faithful variant always run 8; they are instantiated with NW = 8 only).
template <int FMT, bool FAITH, int NW>
static void launch_tiled_f(const Problem &p, const KArgs &a, const TiCfg *c, hipStream_t st, const Groups *g,
                           int BM, int64_t gtiles)
{
    const bool f32 = p.act == QGEMM_F32, o32 = p.out == QGEMM_F32;
    const bool dual = p.epi == QGEMM_EPI_SWIGLU;
    const int Nh = (int)(p.N / 2);
    auto go = [&](auto act, auto out, auto du) {
        constexpr int A = decltype(act)::value, O = decltype(out)::value;
        constexpr bool D = decltype(du)::value;
        auto bm = [&](auto bmv) {
            constexpr int M = decltype(bmv)::value;
            if constexpr (NW == 8) {
                if (g)
                    launch_grouped_bm<FMT, A, O, D, M, FAITH>(a, *g, gtiles, st, Nh);
                else
                    launch_tiled_bm<FMT, A, O, D, M, FAITH>(a, *c, st, Nh);
            } else {
                launch_tiled_bm<FMT, A, O, D, M, FAITH, NW>(a, *c, st, Nh);
            }
        };
        if constexpr (FAITH) {
            // 64-row tiles, or 96 for B in (64, 96] (plain GEMM only)
            if (!g && BM == 96)
                launch_tiled_bm<FMT, A, O, D, 96, FAITH>(a, *c, st, Nh);
            else
                bm(std::integral_constant<int, 64>{});
        } else if (NW == 8 && g && BM == 64) {
            // routed experts with few rows each
            if constexpr (NW == 8)
                launch_grouped_bm<FMT, A, O, D, 64, FAITH>(a, *g, gtiles, st, Nh);
        } else if (BM == 128) {
            bm(std::integral_constant<int, 128>{});
        } else {
            bm(std::integral_constant<int, 256>{});
        }
    };
    using F32 = std::integral_constant<int, ACT_F32>;
    using B16 = std::integral_constant<int, ACT_BF16>;
    using OF = std::integral_constant<int, OUT_F32>;
    using OB = std::integral_constant<int, OUT_BF16>;
    if constexpr (FAITH) {
        // fp32 math takes fp32 activations and no fused epilogue (checked at
        // plan creation)
        if (o32) go(F32{}, OF{}, std::false_type{}); else go(F32{}, OB{}, std::false_type{});
    } else if (f32) {
        if (o32) { if (dual) go(F32{}, OF{}, std::true_type{}); else go(F32{}, OF{}, std::false_type{}); }
        else { if (dual) go(F32{}, OB{}, std::true_type{}); else go(F32{}, OB{}, std::false_type{}); }
    } else {
        if (o32) { if (dual) go(B16{}, OF{}, std::true_type{}); else go(B16{}, OF{}, std::false_type{}); }
        else { if (dual) go(B16{}, OB{}, std::true_type{}); else go(B16{}, OB{}, std::false_type{}); }
    }
}

// Every format of one math mode (c: the plain GEMM's shape; g: routed
// experts instead, BM-row tiles, gtiles row tiles).
template <bool FAITH, int NW = 8>
static hipError_t launch_tiled_math(const Problem &p, const KArgs &a, const TiCfg *c, const Groups *g, int BM,
                                    int64_t gtiles, hipStream_t st)
{
    switch (p.fmt) {
    case FMT_Q8: launch_tiled_f<FMT_Q8, FAITH, NW>(p, a, c, st, g, BM, gtiles); break;
    case FMT_MX: launch_tiled_f<FMT_MX, FAITH, NW>(p, a, c, st, g, BM, gtiles); break;
    case FMT_FP8: launch_tiled_f<FMT_FP8, FAITH, NW>(p, a, c, st, g, BM, gtiles); break;
    default: launch_tiled_f<FMT_NV, FAITH, NW>(p, a, c, st, g, BM, gtiles); break;
    }
    return hipGetLastError();
}

}  // namespace qg
