// C ABI of the library: plans, argument validation, the host packer, tier
// dispatch and kernel launch on the caller's stream.  See include/qgemm.h.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "kernels.hip"

namespace qg {

static thread_local char g_err[512];

static int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

static int hip_fail(hipError_t e, const char *what)
{
    return fail(QGEMM_EHIP, "%s: %s", what, hipGetErrorString(e));
}

static const uint32_t PLAN_MAGIC = 0x51474D31u;  // "QGM1"

}  // namespace qg

struct qgemm_plan {
    uint32_t magic;
    int fmt, act, out, epi, math;
    int64_t N, K;
    int forced_tier;  // 0 = automatic
    qg::Layout L;
};

namespace qg {

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// ------------------------------------------------------------ dispatch

// ---- skinny tier configuration
//
// MB: 16-row batch groups per workgroup; NT: row tiles per wave (a workgroup
// covers 4*NT); D: weight slabs in flight per wave; ksplit / kc: workgroups
// per output tile along K and slabs per workgroup.

struct SkCfg {
    int MB, NT, D;
    int ngroups, nby, ksplit, kc;
    int64_t cnt_bytes, part_bytes;
};

static int env_int(const char *name, int dflt)
{
    const char *v = getenv(name);
    return (v && *v) ? atoi(v) : dflt;
}

static SkCfg skinny_cfg(const qgemm_plan *p, int64_t B, bool split)
{
    SkCfg c;
    c.MB = B <= 16 ? 1 : (B <= 32 ? 2 : 4);
    const int U = p->fmt == FMT_Q8 ? 2 : 4;
    const int nta = p->act == QGEMM_F32 && p->math == QGEMM_MATH_FP32 ? 3 : 1;
    while (c.MB > 1 && 2 * nta * c.MB * U > 96)  // activation LDS (KB) per workgroup
        c.MB /= 2;
    c.NT = env_int("QGEMM_SK_NT", 2) == 1 ? 1 : 2;
    c.D = 4;
    c.ngroups = (int)((p->L.RT + 4 * c.NT - 1) / (4 * c.NT));
    c.nby = (int)((B + 16 * c.MB - 1) / (16 * c.MB));
    const int S = (int)p->L.S;
    c.ksplit = 1;
    if (split) {
        const int64_t target = env_int("QGEMM_SK_WGS", 512);
        const int64_t cols = (int64_t)c.ngroups * c.nby;
        int64_t ks = (target + cols - 1) / cols;
        ks = ks < 1 ? 1 : (ks > S ? S : ks);
        c.ksplit = (int)ks;
    }
    c.kc = (S + c.ksplit - 1) / c.ksplit;
    c.kc = (c.kc + c.D - 1) / c.D * c.D;  // the kernel walks whole rings of D slabs
    c.ksplit = (S + c.kc - 1) / c.kc;
    if (c.ksplit > 1) {
        const int64_t tiles = (int64_t)c.nby * c.ngroups * 4 * c.MB * c.NT;
        c.cnt_bytes = round_up((int64_t)c.nby * c.ngroups * 4, 256);
        c.part_bytes = (int64_t)c.ksplit * tiles * 1024;
    } else {
        c.cnt_bytes = c.part_bytes = 0;
    }
    return c;
}

template <int FMT, int ACT, int NTERM, int MB, int NT, int OUTT>
static void launch_skinny_k(const KArgs &a, const SkCfg &c, const SkinnyWs &ws, hipStream_t st)
{
    dim3 grid(c.ngroups, c.ksplit, c.nby);
    hipLaunchKernelGGL((skinny_kernel<FMT, ACT, NTERM, MB, NT, 4, OUTT>), grid, dim3(256), 0, st, a, ws);
}

template <int FMT, int ACT, int NTERM, int OUTT>
static void launch_skinny_t(const KArgs &a, const SkCfg &c, const SkinnyWs &ws, hipStream_t st)
{
#define QG_S(MB, NT) launch_skinny_k<FMT, ACT, NTERM, MB, NT, OUTT>(a, c, ws, st)
    if (c.NT == 1) {
        if (c.MB == 1) QG_S(1, 1); else if (c.MB == 2) QG_S(2, 1); else QG_S(4, 1);
    } else {
        if (c.MB == 1) QG_S(1, 2); else if (c.MB == 2) QG_S(2, 2); else QG_S(4, 2);
    }
#undef QG_S
}

template <int FMT>
static void launch_skinny_f(const qgemm_plan *p, const KArgs &a, const SkCfg &c, const SkinnyWs &ws,
                            hipStream_t st, int nterm)
{
    const bool f32 = p->act == QGEMM_F32, o32 = p->out == QGEMM_F32;
    if (!f32) {
        if (o32) launch_skinny_t<FMT, ACT_BF16, 1, OUT_F32>(a, c, ws, st);
        else launch_skinny_t<FMT, ACT_BF16, 1, OUT_BF16>(a, c, ws, st);
    } else if (nterm == 1) {
        if (o32) launch_skinny_t<FMT, ACT_F32, 1, OUT_F32>(a, c, ws, st);
        else launch_skinny_t<FMT, ACT_F32, 1, OUT_BF16>(a, c, ws, st);
    } else if (nterm == 2) {
        if (o32) launch_skinny_t<FMT, ACT_F32, 2, OUT_F32>(a, c, ws, st);
        else launch_skinny_t<FMT, ACT_F32, 2, OUT_BF16>(a, c, ws, st);
    } else {
        if (o32) launch_skinny_t<FMT, ACT_F32, 3, OUT_F32>(a, c, ws, st);
        else launch_skinny_t<FMT, ACT_F32, 3, OUT_BF16>(a, c, ws, st);
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
static void launch_tiled_f(const qgemm_plan *p, const KArgs &a, hipStream_t st)
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

static int choose_tier(const qgemm_plan *p, int64_t B)
{
    if (p->forced_tier)
        return p->forced_tier;
    if (p->math == QGEMM_MATH_FP32 || p->epi == QGEMM_EPI_NONE) {
        if (p->math == QGEMM_MATH_FP32)
            return QGEMM_TIER_SKINNY;
        return B <= 64 ? QGEMM_TIER_SKINNY : QGEMM_TIER_TILED;
    }
    return QGEMM_TIER_TILED;  // fused gate+up
}

static KArgs make_args(const qgemm_plan *p, int64_t B, const void *w, const void *x, void *y)
{
    KArgs a;
    a.w = (const uint8_t *)w;
    a.x = x;
    a.y = y;
    a.B = (int)B;
    a.N = (int)p->N;
    a.K = (int)p->K;
    a.S = (int)p->L.S;
    a.RT = (int)p->L.RT;
    a.SP = (int)p->L.SP;
    a.scale_off = p->L.scale_off;
    a.meta_off = p->L.meta_off;
    return a;
}

}  // namespace qg

using namespace qg;

extern "C" {

int qgemm_version(void) { return (1 << 16) | 0; }

const char *qgemm_strerror(int status)
{
    switch (status) {
    case QGEMM_OK: return "ok";
    case QGEMM_EINVAL: return "invalid argument";
    case QGEMM_ENOTSUP: return "not supported";
    case QGEMM_EHIP: return "HIP error";
    case QGEMM_ENOMEM: return "out of memory";
    }
    return "unknown status";
}

const char *qgemm_last_error(void) { return g_err; }

size_t qgemm_weight_bytes(qgemm_format fmt, int64_t N, int64_t K)
{
    Layout L;
    if (!make_layout((int)fmt, N, K, &L))
        return 0;
    return (size_t)L.total;
}

int qgemm_pack(qgemm_format fmt, int64_t N, int64_t K, const void *codes, const void *scales,
               const float *tensor_scales, int64_t ntensors, void *out, size_t out_bytes)
{
    Layout L;
    if (!make_layout((int)fmt, N, K, &L))
        return fail(QGEMM_EINVAL, "qgemm_pack: bad format/shape (fmt=%d N=%lld K=%lld)", (int)fmt,
                    (long long)N, (long long)K);
    if (!codes || !scales || !out)
        return fail(QGEMM_EINVAL, "qgemm_pack: null pointer");
    if (out_bytes < (size_t)L.total)
        return fail(QGEMM_EINVAL, "qgemm_pack: output buffer %zu bytes < %lld needed", out_bytes,
                    (long long)L.total);
    if (fmt == QGEMM_NVFP4) {
        if (!tensor_scales || ntensors < 1 || ntensors > QGEMM_MAX_TENSORS || N % ntensors)
            return fail(QGEMM_EINVAL, "qgemm_pack: NVFP4 needs 1..%d tensor scales dividing N",
                        QGEMM_MAX_TENSORS);
    } else if (tensor_scales || ntensors) {
        return fail(QGEMM_EINVAL, "qgemm_pack: tensor scales are for NVFP4 only");
    }
    if (fmt != QGEMM_Q8_0) {
        const uint8_t *c = (const uint8_t *)codes;
        for (int64_t i = 0; i < N * K; i++)
            if (c[i] > 15)
                return fail(QGEMM_EINVAL, "qgemm_pack: FP4 code %u > 15 at %lld", c[i], (long long)i);
    }
    uint8_t *o = (uint8_t *)out;
    memset(o, 0, (size_t)L.total);
    // codes
    for (int64_t n = 0; n < N; n++) {
        const int64_t rt = n / 16, r = n % 16;
        for (int64_t k = 0; k < K; k++) {
            const int64_t s = k / L.KS, kk = k % L.KS;
            const int64_t u = kk / 32, g = (kk % 32) / 8, j = kk % 8;
            uint8_t *chunk = o + ((rt * L.S + s) << 10) + ((g * 16 + r) << 4);
            if (fmt == QGEMM_Q8_0) {
                chunk[8 * u + j] = ((const uint8_t *)codes)[n * K + k];
            } else {
                const uint8_t c = ((const uint8_t *)codes)[n * K + k];
                chunk[4 * u + j / 2] |= (uint8_t)(c << (4 * (j & 1)));
            }
        }
    }
    // scales
    const int64_t nsc = K / L.blk;
    const int64_t esz = fmt == QGEMM_Q8_0 ? 2 : 1;
    for (int64_t n = 0; n < N; n++)
        memcpy(o + L.scale_off + n * L.SP, (const uint8_t *)scales + n * nsc * esz, (size_t)(nsc * esz));
    // tensor scales
    if (fmt == QGEMM_NVFP4) {
        int32_t hdr[4] = {(int32_t)ntensors, (int32_t)(N / ntensors), 0, 0};
        memcpy(o + L.meta_off, hdr, sizeof hdr);
        memcpy(o + L.meta_off + 16, tensor_scales, (size_t)ntensors * sizeof(float));
    }
    return QGEMM_OK;
}

int qgemm_create(qgemm_plan **plan, qgemm_format fmt, qgemm_dtype act, qgemm_dtype out,
                 qgemm_epilogue epi, qgemm_math math, int64_t N, int64_t K, uint32_t flags)
{
    if (!plan)
        return fail(QGEMM_EINVAL, "qgemm_create: null plan pointer");
    *plan = nullptr;
    if ((int)fmt < 0 || (int)fmt > 2)
        return fail(QGEMM_EINVAL, "qgemm_create: unknown format %d", (int)fmt);
    if ((act != QGEMM_F32 && act != QGEMM_BF16) || (out != QGEMM_F32 && out != QGEMM_BF16))
        return fail(QGEMM_EINVAL, "qgemm_create: unknown dtype");
    if (epi != QGEMM_EPI_NONE && epi != QGEMM_EPI_SWIGLU)
        return fail(QGEMM_EINVAL, "qgemm_create: unknown epilogue %d", (int)epi);
    if (math != QGEMM_MATH_FP32 && math != QGEMM_MATH_BF16)
        return fail(QGEMM_EINVAL, "qgemm_create: unknown math mode %d", (int)math);
    if (N <= 0 || K <= 0)
        return fail(QGEMM_EINVAL, "qgemm_create: N and K must be positive (N=%lld K=%lld)",
                    (long long)N, (long long)K);
    if (N > (1ll << 30) || K > (1ll << 30))
        return fail(QGEMM_EINVAL, "qgemm_create: N or K above 2^30");
    const int64_t blk = fmt == QGEMM_NVFP4 ? 16 : 32;
    if (K % blk)
        return fail(QGEMM_EINVAL, "qgemm_create: K=%lld is not a multiple of the %lld-wide block",
                    (long long)K, (long long)blk);
    if (epi == QGEMM_EPI_SWIGLU && (N % 2))
        return fail(QGEMM_EINVAL, "qgemm_create: SwiGLU needs an even N (gate and up halves)");
    if (epi == QGEMM_EPI_SWIGLU && (N / 2) % 16)
        return fail(QGEMM_ENOTSUP, "qgemm_create: SwiGLU needs N/2 to be a multiple of 16");
    if (math == QGEMM_MATH_FP32 && act != QGEMM_F32)
        return fail(QGEMM_EINVAL, "qgemm_create: fp32 math needs fp32 activations");
    if ((flags & ~(QGEMM_FLAG_FORCE_SKINNY | QGEMM_FLAG_FORCE_TILED)) ||
        ((flags & QGEMM_FLAG_FORCE_SKINNY) && (flags & QGEMM_FLAG_FORCE_TILED)))
        return fail(QGEMM_EINVAL, "qgemm_create: bad flags 0x%x", flags);
    int forced = (flags & QGEMM_FLAG_FORCE_SKINNY) ? QGEMM_TIER_SKINNY
               : (flags & QGEMM_FLAG_FORCE_TILED) ? QGEMM_TIER_TILED : 0;
    if (!forced) {
        const char *e = getenv("QGEMM_FORCE_TIER");
        if (e && !strcmp(e, "skinny"))
            forced = QGEMM_TIER_SKINNY;
        else if (e && !strcmp(e, "tiled"))
            forced = QGEMM_TIER_TILED;
    }
    if (forced == QGEMM_TIER_TILED && math == QGEMM_MATH_FP32)
        return fail(QGEMM_ENOTSUP, "qgemm_create: the tiled tier computes in bf16; fp32 math runs "
                                   "in the skinny tier");
    if (forced == QGEMM_TIER_SKINNY && epi == QGEMM_EPI_SWIGLU)
        return fail(QGEMM_ENOTSUP, "qgemm_create: the fused gate+up epilogue runs in the tiled tier");
    qgemm_plan *p = new (std::nothrow) qgemm_plan;
    if (!p)
        return fail(QGEMM_ENOMEM, "qgemm_create: out of host memory");
    p->magic = PLAN_MAGIC;
    p->fmt = (int)fmt;
    p->act = (int)act;
    p->out = (int)out;
    p->epi = (int)epi;
    p->math = (int)math;
    p->N = N;
    p->K = K;
    p->forced_tier = forced;
    make_layout((int)fmt, N, K, &p->L);
    *plan = p;
    return QGEMM_OK;
}

int qgemm_destroy(qgemm_plan *plan)
{
    if (!plan)
        return QGEMM_OK;
    if (plan->magic != PLAN_MAGIC)
        return fail(QGEMM_EINVAL, "qgemm_destroy: not a live plan");
    plan->magic = 0;
    delete plan;
    return QGEMM_OK;
}

int qgemm_plan_tier(const qgemm_plan *plan, int64_t B)
{
    if (!plan || plan->magic != PLAN_MAGIC || B < 0)
        return 0;
    return choose_tier(plan, B);
}

size_t qgemm_workspace_bytes(const qgemm_plan *plan, int64_t B)
{
    if (!plan || plan->magic != PLAN_MAGIC || B <= 0 || B > (1ll << 30))
        return 0;
    if (choose_tier(plan, B) != QGEMM_TIER_SKINNY)
        return 0;
    const SkCfg c = skinny_cfg(plan, B, true);
    return (size_t)(c.cnt_bytes + c.part_bytes);
}

int qgemm_run_ws(const qgemm_plan *plan, int64_t B, const void *w, const void *x, void *y,
                 void *workspace, size_t ws_bytes, void *stream)
{
    if (!plan || plan->magic != PLAN_MAGIC)
        return fail(QGEMM_EINVAL, "qgemm_run: not a live plan");
    if (B < 0)
        return fail(QGEMM_EINVAL, "qgemm_run: B=%lld < 0", (long long)B);
    if (B > (1ll << 30))
        return fail(QGEMM_EINVAL, "qgemm_run: B=%lld above 2^30", (long long)B);
    if (B == 0)
        return QGEMM_OK;
    if (!w || !x || !y)
        return fail(QGEMM_EINVAL, "qgemm_run: null pointer");
    if (!aligned16(w) || !aligned16(x) || !aligned16(y))
        return fail(QGEMM_EINVAL, "qgemm_run: w, x and y must be 16-byte aligned");
    if (workspace && ((uintptr_t)workspace & 255u))
        return fail(QGEMM_EINVAL, "qgemm_run: workspace must be 256-byte aligned");
    const int64_t ncols = plan->epi == QGEMM_EPI_SWIGLU ? plan->N / 2 : plan->N;
    if (B * plan->K > (1ll << 31) - 1 || B * ncols > (1ll << 31) - 1)
        return fail(QGEMM_EINVAL, "qgemm_run: B*K or B*N above 2^31 elements");
    const KArgs a = make_args(plan, B, w, x, y);
    hipStream_t st = (hipStream_t)stream;
    const int tier = choose_tier(plan, B);
    if (tier == QGEMM_TIER_SKINNY) {
        SkCfg c = skinny_cfg(plan, B, workspace != nullptr);
        if (c.ksplit > 1 && (size_t)(c.cnt_bytes + c.part_bytes) > ws_bytes)
            c = skinny_cfg(plan, B, false);  // workspace too small: no K split
        if (c.nby > 65535)
            return fail(QGEMM_EINVAL, "qgemm_run: B=%lld exceeds the skinny tier's grid",
                        (long long)B);
        SkinnyWs ws;
        ws.cnt = c.ksplit > 1 ? (uint32_t *)workspace : nullptr;
        ws.part = c.ksplit > 1 ? (float *)((uint8_t *)workspace + c.cnt_bytes) : nullptr;
        ws.ksplit = c.ksplit;
        ws.kc = c.kc;
        const int nterm = plan->math == QGEMM_MATH_BF16 ? 1 : env_int("QGEMM_FP32_TERMS", 3);
        if (nterm < 1 || nterm > 3)
            return fail(QGEMM_EINVAL, "qgemm_run: QGEMM_FP32_TERMS must be 1..3");
        switch (plan->fmt) {
        case FMT_Q8: launch_skinny_f<FMT_Q8>(plan, a, c, ws, st, nterm); break;
        case FMT_MX: launch_skinny_f<FMT_MX>(plan, a, c, ws, st, nterm); break;
        default: launch_skinny_f<FMT_NV>(plan, a, c, ws, st, nterm); break;
        }
    } else {
        switch (plan->fmt) {
        case FMT_Q8: launch_tiled_f<FMT_Q8>(plan, a, st); break;
        case FMT_MX: launch_tiled_f<FMT_MX>(plan, a, st); break;
        default: launch_tiled_f<FMT_NV>(plan, a, st); break;
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e, "qgemm_run: kernel launch");
    return QGEMM_OK;
}

int qgemm_run(const qgemm_plan *plan, int64_t B, const void *w, const void *x, void *y, void *stream)
{
    return qgemm_run_ws(plan, B, w, x, y, nullptr, 0, stream);
}

int qgemm_dequantize(qgemm_format fmt, const void *w, float *w_out, int64_t N, int64_t K, void *stream)
{
    Layout L;
    if (!make_layout((int)fmt, N, K, &L))
        return fail(QGEMM_EINVAL, "qgemm_dequantize: bad format/shape");
    if (!w || !w_out)
        return fail(QGEMM_EINVAL, "qgemm_dequantize: null pointer");
    if (!aligned16(w) || !aligned16(w_out))
        return fail(QGEMM_EINVAL, "qgemm_dequantize: pointers must be 16-byte aligned");
    if (N * K > (1ll << 40))
        return fail(QGEMM_EINVAL, "qgemm_dequantize: too large");
    KArgs a;
    a.w = (const uint8_t *)w;
    a.x = nullptr;
    a.y = w_out;
    a.B = 0;
    a.N = (int)N;
    a.K = (int)K;
    a.S = (int)L.S;
    a.RT = (int)L.RT;
    a.SP = (int)L.SP;
    a.scale_off = L.scale_off;
    a.meta_off = L.meta_off;
    const int64_t threads = N * (K / 8);
    dim3 grid((unsigned)((threads + 255) / 256));
    hipStream_t st = (hipStream_t)stream;
    switch ((int)fmt) {
    case FMT_Q8: hipLaunchKernelGGL(dequant_kernel<FMT_Q8>, grid, dim3(256), 0, st, a, w_out); break;
    case FMT_MX: hipLaunchKernelGGL(dequant_kernel<FMT_MX>, grid, dim3(256), 0, st, a, w_out); break;
    default: hipLaunchKernelGGL(dequant_kernel<FMT_NV>, grid, dim3(256), 0, st, a, w_out); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e, "qgemm_dequantize: kernel launch");
    return QGEMM_OK;
}

}  // extern "C"
