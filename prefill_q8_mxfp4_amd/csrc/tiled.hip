// Large-batch tier: a BM x BN output tile per workgroup, activation and
// decoded-weight tiles staged through LDS as bf16 MFMA fragments.
#include "common.h"

namespace qg {

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
            const uint8_t *sp = slab_scales<FMT>(a, rt, L & 15, s);
            if constexpr (FMT == FMT_NV) {
                const u32x2 v = *(const u32x2 *)sp;
                sr[i][0] = v[0];
                sr[i][1] = v[1];
            } else {
                sr[i][0] = *(const uint32_t *)sp;
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

constexpr int TBM = 128, TBN = 128, TWM = 2, TWN = 2;

template <int FMT, int ACT, int OUTT, bool DUAL>
static void launch_tiled_t(const KArgs &a, hipStream_t st, int Nh)
{
    const int mtiles = (a.B + TBM - 1) / TBM;
    const int nrows = DUAL ? Nh : a.N;
    const int ntiles = (nrows + TBN - 1) / TBN;
    dim3 grid(mtiles * ntiles);
    hipLaunchKernelGGL((tiled_kernel<FMT, ACT, OUTT, DUAL, TBM, TBN, TWM, TWN>), grid,
                       dim3(TWM * TWN * 64), 0, st, a, Nh, mtiles, ntiles);
}

template <int FMT>
static void launch_tiled_f(const Problem *p, const KArgs &a, hipStream_t st)
{
    const bool f32 = p->act == QGEMM_F32, o32 = p->out == QGEMM_F32;
    const bool dual = p->epi == QGEMM_EPI_SWIGLU;
    const int Nh = (int)(p->N / 2);
#define QG_T(A, O, D) launch_tiled_t<FMT, A, O, D>(a, st, Nh)
    if (f32) {
        if (o32) { if (dual) QG_T(ACT_F32, OUT_F32, true); else QG_T(ACT_F32, OUT_F32, false); }
        else { if (dual) QG_T(ACT_F32, OUT_BF16, true); else QG_T(ACT_F32, OUT_BF16, false); }
    } else {
        if (o32) { if (dual) QG_T(ACT_BF16, OUT_F32, true); else QG_T(ACT_BF16, OUT_F32, false); }
        else { if (dual) QG_T(ACT_BF16, OUT_BF16, true); else QG_T(ACT_BF16, OUT_BF16, false); }
    }
#undef QG_T
}

hipError_t launch_tiled(const Problem &p, const KArgs &a, hipStream_t st)
{
    switch (p.fmt) {
    case FMT_Q8: launch_tiled_f<FMT_Q8>(&p, a, st); break;
    case FMT_MX: launch_tiled_f<FMT_MX>(&p, a, st); break;
    default: launch_tiled_f<FMT_NV>(&p, a, st); break;
    }
    return hipGetLastError();
}

}  // namespace qg
