// C ABI of the library: plans, argument validation, the host packer, tier
// dispatch and kernel launch on the caller's stream.  See include/qgemm.h.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>

#include "common.h"

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

static int env_int(const char *name, int dflt)
{
    const char *v = getenv(name);
    return (v && *v) ? atoi(v) : dflt;
}

// The environment overrides of a plan, read once at creation (see Knobs).
static void read_knobs(Knobs *k)
{
    k->st_waves = env_int("QGEMM_ST_WAVES", 0);
    k->st_nph = env_int("QGEMM_ST_NPH", 0);
    k->st_depth = env_int("QGEMM_ST_DEPTH", 0);
    k->gv_maxb = env_int("QGEMM_GV_MAXB", -1);
    k->sk_stream = env_int("QGEMM_SK_STREAM", 1);
    k->sk_nt = env_int("QGEMM_SK_NT", 2);
    k->vf = env_int("QGEMM_VF", 1);
    k->vf_bf16_maxb = env_int("QGEMM_VF_BF16_MAXB", VF_BF16_MAXB);
    k->vf_swiglu_maxb = env_int("QGEMM_VF_SWIGLU_MAXB", VF_SWIGLU_MAXB);
    k->ti_bm = env_int("QGEMM_TI_BM", 0);
    k->ti_split = env_int("QGEMM_TI_SPLIT", 0);
    k->ti_waves = env_int("QGEMM_TI_WAVES", 0);
    k->xlocal = env_int("QGEMM_ST_XLOCAL", -1) == 0 ? 0 : -1;
    k->fp32_terms = 3;
    k->xcc_fake = 0;
#ifdef QGEMM_DEBUG_KNOBS
    if (env_int("QGEMM_ST_XLOCAL", -1) == 1)
        k->xlocal = 1;
    const int t = env_int("QGEMM_FP32_TERMS", 3);
    k->fp32_terms = t >= 1 && t <= 3 ? t : 3;
    k->xcc_fake = env_int("QGEMM_XCC_FAKE", 0) != 0;
#endif
}

}  // namespace qg

struct qgemm_plan {
    uint32_t magic;
    int forced_tier;  // 0 = automatic
    qg::Problem p;
};

namespace qg {

static bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// ---- small-batch tier shape
//
// With a workspace, K is split into ranges of split_kc() slabs, a choice that
// depends on the problem (format, activation terms, N, K) and not on B: every
// batch row is then summed in the same order by both small-batch kernels, up
// to SK_SPLIT_NBY batch groups (larger batches have enough tiles unsplit).
// The counter region has one size for every B, so no call's partial tiles
// land on another call's counters.
static const int SK_LDS_MAX = 96 * 1024;
static const int SK_SPLIT_NBY = 8;  // batch groups up to which K is split
static const int ST_MAX_B = 16;     // the streaming kernel's batch limit

static int act_terms(const Problem &p)
{
    return p.act == QGEMM_F32 && p.math == QGEMM_MATH_FP32 ? 3 : 1;
}

// Shape of the streaming kernel (B <= 16): W waves per workgroup, NPH slabs
// per wave, so KC = W * NPH slabs per K split.  The search minimises the
// slabs of the busiest SIMD (a CU's four SIMDs share its W waves, and a
// wave's decode and MFMA work is per slab), assuming one workgroup per CU and
// rounds of 256; ties go to fewer rounds, then to fewer splits (fewer
// partial tiles to publish and add), then to fewer waves.  It depends on N
// and K only.
struct StShape {
    int W, NPH;
};

static StShape stream_shape(const Problem &p)
{
    const int64_t groups = (p.L.RT + ST_RG - 1) / ST_RG;
    const int64_t S = p.L.S;
    const int fw = p.kn.st_waves, fp = p.kn.st_nph;
    StShape best = {8, 1};
    int64_t best_cost = -1, best_rounds = 0, best_splits = 0;
    for (int nph = 1; nph <= 2; nph++) {
        if (fp && nph != fp)
            continue;
        for (int w = 8; w <= st_max_waves(nph); w++) {
            if (fw && w != fw)
                continue;
            const int64_t kc = (int64_t)w * nph;
            const int64_t splits = (S + kc - 1) / kc;
            const int64_t rounds = (groups * splits + 255) / 256;
            const int64_t per_wave = (kc < S ? kc : S) < w ? 1 : nph;  // slabs a wave walks
            const int64_t cost = rounds * ((w + 3) / 4) * per_wave;
            if (best_cost < 0 || cost < best_cost ||
                (cost == best_cost &&
                 (rounds < best_rounds || (rounds == best_rounds && splits < best_splits)))) {
                best = {w, nph};
                best_cost = cost;
                best_rounds = rounds;
                best_splits = splits;
            }
        }
    }
    return best;
}

// Slabs per K split (with a workspace), shared by both small-batch kernels.
static int split_kc(const Problem &p)
{
    const StShape sh = stream_shape(p);
    return sh.W * sh.NPH;
}

static int64_t split_cnt_bytes(const Problem &p)
{
    return round_up((int64_t)SK_SPLIT_NBY * ((p.L.RT + 3) / 4) * 4, 256);
}

// Workspace layout of a plan: the small-batch tiers' counters, then the
// large-batch tier's counters (at most 255 split tiles), then partial tiles
// (whichever tier the call used).  Counters are zero between calls.
static const int64_t TI_CNT_BYTES = 1024;

static int64_t ws_data_off(const Problem &p)
{
    return split_cnt_bytes(p) + TI_CNT_BYTES;
}

static bool use_stream(const Problem &p, int64_t B)
{
    return B <= ST_MAX_B && p.kn.sk_stream != 0;
}

// 16 < B <= 80 (the MTP verify widths), K a whole number of slabs: the
// verify kernel, one pass over the weights for all batch rows in the
// streaming kernel's summation order; fp32-faithful math (three terms) up to
// 80 rows, bf16 math up to QGEMM_VF_BF16_MAXB rows (80), the fused gate+up
// epilogue up to QGEMM_VF_SWIGLU_MAXB (48: NVFP4 gate+up 2x17408x5120 ran
// 39.8 / 55.3 us at B = 17 / 48 against the tiled tier's 64.2 / 66.3, but
// 69.9 / 86.9 at 64 / 80 against 68.4 / 72.0).  QGEMM_VF=0 turns it off (the
// skinny kernel, or the tiled tier by default).
static int plan_nterm(const Problem &p) { return p.math == QGEMM_MATH_BF16 ? 1 : p.kn.fp32_terms; }

static bool use_verify(const Problem &p, int64_t B, int nterm)
{
    if (p.kn.vf == 0 || (p.epi == QGEMM_EPI_SWIGLU && B > p.kn.vf_swiglu_maxb) || B <= ST_MAX_B || B > VF_MAX_B ||
        p.K % slab_k(p.fmt) != 0 ||
        (p.L.RT + 7) / 8 * 8 * (VF_MAX_B / 16) * 1024 >= (1ll << 31))  // a split's partials: 32-bit offsets
        return false;
    if (p.math == QGEMM_MATH_FP32)
        return p.act == QGEMM_F32 && nterm == 3;
    return nterm == 1 && B <= p.kn.vf_bf16_maxb;
}

// The GEMV kernel takes B = 1 and 2 when its activation rows fit in LDS
// with room for two workgroups per CU (one workgroup per row tile, so a grid
// above 256 tiles needs them resident two at a time).
static const int GV_MAX_B = 2;
static const int64_t GV_LDS_MAX = 72 * 1024;

static bool gemv_fits(const Problem &p, int64_t B)
{
    return B <= GV_MAX_B && gemv_lds_bytes(p, B) <= GV_LDS_MAX;
}

// Automatic choice: B = 1 when the activation row takes at most 32 KB of
// LDS (K <= 8192), so that four or more GEMV workgroups of 8 waves fit on a
// CU and the CUs that hold a tile more than others keep HBM busy.  Measured
// on MI355X against the MFMA streaming kernel: Q8_0 5120^2 B = 1 9.37 vs
// 10.19 us, FP8 5120^2 8.95 vs 9.85, NVFP4 gate+up 2x17408x5120 23.7 vs
// 29.0; MXFP4 5120x17408 (K = 17408, 70 KB of LDS) 16.8 vs 14.0; at B = 2
// the streaming kernel wins everywhere (Q8_0 11.2 vs 10.2, FP8 10.6 vs 9.9,
// NVFP4 gate+up 32.5 vs 29.3).  QGEMM_GV_MAXB=0|1|2 overrides the rule
// (0: never).
static const int64_t GV_AUTO_LDS = 32 * 1024;

static bool use_gemv(const Problem &p, int64_t B)
{
    if (p.kn.gv_maxb >= 0) {
        const int maxb = p.kn.gv_maxb < GV_MAX_B ? p.kn.gv_maxb : GV_MAX_B;
        return B <= maxb && gemv_fits(p, B);
    }
    return B == 1 && gemv_lds_bytes(p, 1) <= GV_AUTO_LDS;
}

// XCD dispatch probe.  The streaming kernel's XCD-local split exchange
// needs every workgroup id congruent mod 8 to run on one XCD, so that one L2
// holds all partial tiles of a row group (the hardware dispatcher deals
// consecutive workgroup ids to the XCDs round-robin).  qgemm_init_device
// checks this once per device: a probe kernel records the XCC id (hardware
// register XCC_ID) of 2048 workgroups, three times, and the exchange is
// enabled on a device only if ids b and b mod 8 always ran on the same XCC.
// Devices never probed, or that fail, use the device-coherent exchange; both
// give bitwise the same result (same partials, same split order).  Every
// launch with the exchange still checks that the K splits of each row group
// ran on one XCD (the kernel's own check, see the streaming kernel).
static const int XCC_PROBE_WGS = 2048;
static const int MAX_DEVICES = 64;
static std::atomic<int> g_xlocal[MAX_DEVICES];  // 0 not probed, 1 round-robin, 2 not
static std::atomic<uint32_t *> g_status_ptr[MAX_DEVICES];  // device address of g_status there
static std::mutex g_probe_mu;
static __device__ uint32_t g_xcc_probe[XCC_PROBE_WGS];  // the probe's output, one word per workgroup
// Device status word, one per device (DEV_* bits): kernels that detect a
// broken assumption at run time set a bit here; qgemm_device_status reads it.
static __device__ uint32_t g_status;

// Scratch of the allocation-free entry point (qgemm_run_noalloc), one array
// per device for the life of the process: QGEMM_SCRATCH_COUNTER_BYTES of
// counter words (zero between calls: each call re-arms those it used), then
// the partial tiles and the rounded copy of x.  Counters of every plan sit in
// the first region and data only in the second, so a call of one plan never
// finds another plan's partial tiles in its counter words.  In host code
// `scratch` is a stand-in, not a device address: kernels get the address
// hipGetSymbolAddress returned for the current device (g_scratch_ptr).
static __device__ __align__(256) uint8_t scratch[QGEMM_SCRATCH_BYTES];
static std::atomic<uint8_t *> g_scratch_ptr[MAX_DEVICES];
static std::mutex g_scratch_mu;

__global__ void zero_words_kernel(uint32_t *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

__global__ void xcc_probe_kernel(uint32_t *o)
{
    // s_getreg of HW_REG_XCC_ID (id 20), bits [3:0]
    if (threadIdx.x == 0)
        o[blockIdx.x] = __builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) & 15u;
}

static int current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
        (void)hipGetLastError();
        return -1;
    }
    return dev;
}

// Address of this device's status word (null when it cannot be had).  The
// lookup runs once per device, with the calling thread in relaxed capture
// mode so that a graph being captured stays valid.
static uint32_t *status_word(int dev)
{
    if (dev < 0)
        return nullptr;
    uint32_t *p = g_status_ptr[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
    (void)hipThreadExchangeStreamCaptureMode(&mode);
    if (hipGetSymbolAddress((void **)&p, HIP_SYMBOL(g_status)) != hipSuccess)
        p = nullptr;
    (void)hipGetLastError();
    (void)hipThreadExchangeStreamCaptureMode(&mode);
    if (p)
        g_status_ptr[dev].store(p, std::memory_order_release);
    return p;
}

// Device address of `scratch` on device dev, set up once: the address from
// hipGetSymbolAddress (checked), and the counter region zeroed by a kernel
// on `st` (stream-ordered before any use on st; graph-capturable, no memset).
// sync: wait for the zeroing (the init call), else leave it queued.
static uint8_t *scratch_setup(int dev, hipStream_t st, bool sync)
{
    if (dev < 0)
        return nullptr;
    uint8_t *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
    (void)hipThreadExchangeStreamCaptureMode(&mode);
    hipError_t e = hipGetSymbolAddress((void **)&p, HIP_SYMBOL(scratch));
    (void)hipThreadExchangeStreamCaptureMode(&mode);
    if (e != hipSuccess || !p) {
        (void)hipGetLastError();
        return nullptr;
    }
    hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, st, (uint32_t *)p,
                       (int64_t)(QGEMM_SCRATCH_COUNTER_BYTES / 4));
    e = hipGetLastError();
    if (e == hipSuccess && sync)
        e = hipStreamSynchronize(st);
    if (e != hipSuccess)
        return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

static int probe_xcd_dispatch(int dev)
{
    if (g_xlocal[dev].load() != 0)
        return QGEMM_OK;
    std::lock_guard<std::mutex> lock(g_probe_mu);
    if (g_xlocal[dev].load() != 0)
        return QGEMM_OK;
    // relaxed capture mode for this thread and a stream of its own, so a
    // graph being captured on another stream is not disturbed
    hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
    (void)hipThreadExchangeStreamCaptureMode(&mode);
    bool good = false, ran = false;
    uint32_t *d = nullptr;  // device address of g_xcc_probe on this device
    hipStream_t st = nullptr;
    static uint32_t h[XCC_PROBE_WGS];
    if (hipGetSymbolAddress((void **)&d, HIP_SYMBOL(g_xcc_probe)) == hipSuccess && d &&
        hipStreamCreateWithFlags(&st, hipStreamNonBlocking) == hipSuccess) {
        good = true;
        for (int rep = 0; rep < 3 && good; rep++) {
            hipLaunchKernelGGL(xcc_probe_kernel, dim3(XCC_PROBE_WGS), dim3(64), 0, st, d);
            good = hipMemcpyAsync(h, d, sizeof h, hipMemcpyDeviceToHost, st) == hipSuccess &&
                   hipStreamSynchronize(st) == hipSuccess;
            ran = ran || good;
            for (int b = 8; good && b < XCC_PROBE_WGS; b++)
                good = h[b] == h[b % 8];
        }
    }
    if (st)
        (void)hipStreamDestroy(st);
    const hipError_t e = hipGetLastError();
    (void)hipThreadExchangeStreamCaptureMode(&mode);
    if (!ran)
        return hip_fail(e != hipSuccess ? e : hipErrorUnknown, "qgemm_init_device: dispatch probe");
    g_xlocal[dev].store(good ? 1 : 2);
    return QGEMM_OK;
}

// Whether the current device passed the probe.  QGEMM_ST_XLOCAL=0 turns the
// exchange off; forcing it on is for debug builds only.
static bool xcd_local_exchange(const Problem &p)
{
    if (p.kn.xlocal == 0)
        return false;
#ifdef QGEMM_DEBUG_KNOBS
    if (p.kn.xlocal == 1)
        return true;
#endif
    const int dev = current_device();
    return dev >= 0 && g_xlocal[dev].load(std::memory_order_relaxed) == 1;
}

// The streaming kernel's shape: 8 row tiles per workgroup and KC-slab splits
// (split_kc).  Depends on the problem only, not on B.
static StCfg stream_cfg(const Problem &p, bool split)
{
    StCfg c;
    const int S = (int)p.L.S;
    const StShape sh = stream_shape(p);
    c.W = sh.W;
    c.NPH = sh.NPH;
    c.Nh = p.epi == QGEMM_EPI_SWIGLU ? (int)(p.N / 2) : 0;
    c.KC = sh.W * sh.NPH;
    // weight items a wave keeps in flight, fastest on MI355X per format:
    // Q8_0 4, MXFP4 and FP8 3 (MXFP4 down projection B = 1: 16.6 -> 13.9 us
    // against all at once), NVFP4 all at once (16)
    c.depth = p.kn.st_depth ? p.kn.st_depth
            : p.fmt == FMT_Q8 ? 4 : (p.fmt == FMT_MX || p.fmt == FMT_FP8) ? 3 : 16;
    c.kc = split ? c.KC : (S + c.KC - 1) / c.KC * c.KC;
    c.ksplit = (S + c.kc - 1) / c.kc;
    c.ngroups = (int)((p.L.RT + 7) / 8);
    // the per-launch placement check counts splits in 4-bit fields
    c.xlocal = c.ksplit > 1 && c.ksplit <= 15 && xcd_local_exchange(p);
    // XCD-local exchange: 8 XCDs x ceil(groups / 8) groups x ksplit
    c.grid = c.xlocal ? (c.ngroups + 7) / 8 * 8 * c.ksplit : c.ngroups * c.ksplit;
    if (c.ksplit > 1) {
        c.cnt_bytes = ws_data_off(p);
        c.part_bytes = (int64_t)c.ksplit * c.ngroups * 8 * 1024;
    } else {
        c.cnt_bytes = c.part_bytes = 0;
    }
    return c;
}

static SkCfg skinny_cfg(const Problem &p, int64_t B, bool split)
{
    SkCfg c;
    const int nta = act_terms(p);
    c.MB = B <= 16 ? 1 : (B <= 32 ? 2 : 4);
    while (c.MB > 1 && skinny_lds_per_slab(p.fmt, nta, c.MB) * SK_RING > SK_LDS_MAX)
        c.MB /= 2;
    const int per_slab = skinny_lds_per_slab(p.fmt, nta, c.MB);
    const int kch_max = SK_LDS_MAX / per_slab / SK_RING * SK_RING;  // >= SK_RING by the MB choice
    c.NT = p.kn.sk_nt == 1 ? 1 : 2;
    c.ngroups = (int)((p.L.RT + 4 * c.NT - 1) / (4 * c.NT));
    c.nby = (int)((B + 16 * c.MB - 1) / (16 * c.MB));
    const int S = (int)p.L.S;
    c.kc = split && c.nby <= SK_SPLIT_NBY ? split_kc(p) : S;
    c.kch = c.kc <= kch_max ? c.kc : kch_max;  // the last chunk of a range may be shorter
    c.ksplit = (S + c.kc - 1) / c.kc;
    c.lds = c.kch * per_slab;
    if (c.ksplit > 1) {
        const int64_t tiles = (int64_t)c.nby * c.ngroups * 4 * c.MB * c.NT;
        c.cnt_bytes = ws_data_off(p);
        c.part_bytes = (int64_t)c.ksplit * tiles * 1024;
    } else {
        c.cnt_bytes = c.part_bytes = 0;
    }
    return c;
}

// Large-batch tier shape.  Whole rounds of 256 tiles (one per CU) run
// unsplit; the tiles of a last, partial round may be split along K into S
// pieces whose partial tiles a reduce kernel adds.  A cost model in
// microseconds picks the row-tile height (bf16 math: 128 or 256 rows; the
// fp32-faithful variant: 64, or 96 for 64 < B <= 96) and S: rounds of tile
// work plus the partial tiles' traffic.  Its constants are fits to times
// measured on MI355X: a 256 x 256 tile takes about 0.03 us per K column on
// one CU (MXFP4, which stages packed codes, 0.026), a 128-row tile 0.6 of
// that (its weight decode is shared by half the rows), the fp32-faithful
// variant three times the MFMA work, and partial tiles cost about 0.25 us
// per MB (written, then read by the reduce kernel).  On the measured shapes it picks the fastest of the
// forced choices: e.g. FP8 5120^2 at B = 2048 takes 128-row tiles (320
// tiles, 123 us, against 137 us for 160 256-row tiles split in three), the
// other formats keep 256 rows at B = 1024 and 2048, and 128-row tiles win
// at B = 384.  Without a large enough workspace nothing is split.
struct TiPick {
    int S;
    double us;
};

static TiPick pick_split(int tiles, int nsteps, int BM, double tile_us, bool split, int forced)
{
    const int full = tiles / 256 * 256, rem = tiles - full;
    TiPick best = {1, (double)(full / 256 + (rem ? 1 : 0)) * tile_us};
    if (!split || rem == 0)
        return best;
    if (forced)
        best.us = 1e30;  // a valid forced S replaces the unsplit choice
    for (int s = 1; s <= 16; s++) {
        const int spp = (nsteps + s - 1) / s;
        if (s > 1 && (s - 1) * spp >= nsteps)
            continue;  // a piece would be empty
        if (forced && s != forced)
            continue;
        const int64_t rounds = ((int64_t)rem * s + 255) / 256;
        const double part_mb = s > 1 ? (double)rem * s * BM * 256 * 4 / 1e6 : 0.0;
        const double t = (double)(full / 256) * tile_us + (double)rounds * tile_us / s + 0.25 * part_mb;
        if (t < best.us - 1e-9)
            best = {s, t};
    }
    return best;
}

static TiCfg tiled_cfg(const Problem &p, int64_t B, bool split)
{
    TiCfg c;
    const bool faith = p.math == QGEMM_MATH_FP32;
    const bool dual = p.epi == QGEMM_EPI_SWIGLU;
    const int64_t cols = dual ? p.N / 2 : p.N;
    const int ntiles = (int)((cols + (dual ? 127 : 255)) / (dual ? 128 : 256));
    const int nsteps = (int)((p.K + 63) / 64);
    const int fbm = p.kn.ti_bm;
    int cand[2], nc = 1;
    if (faith) {
        cand[0] = (fbm == 64 || fbm == 96) ? fbm : (B > 64 && B <= 96 ? 96 : 64);
    } else if (fbm == 128 || fbm == 256) {
        cand[0] = fbm;
    } else {
        cand[0] = 128;
        if (B > 128)
            cand[nc++] = 256;
    }
    TiPick best = {1, 1e300};
    c.BM = cand[0];
    for (int i = 0; i < nc; i++) {
        const int bm = cand[i];
        const int tiles = (int)((B + bm - 1) / bm) * ntiles;
        const double per_k = p.fmt == FMT_MX ? 0.026 : 0.03;  // MXFP4 stages packed codes
        const double tile_us = per_k * (double)p.K * (bm / 256.0) * (faith ? 3.0 : 1.0) * (bm == 128 ? 1.2 : 1.0);
        const TiPick t = pick_split(tiles, nsteps, bm, tile_us, split, p.kn.ti_split);
        if (t.us < best.us) {
            best = t;
            c.BM = bm;
        }
    }
    c.NW = faith ? 8 : (p.kn.ti_waves == 4 ? 4 : 8);
    c.mtiles = (int)((B + c.BM - 1) / c.BM);
    c.ntiles = ntiles;
    c.tiles = c.mtiles * c.ntiles;
    const int full = c.tiles / 256 * 256, rem = c.tiles - full;
    const int S = best.S;
    c.sp.S = S;
    c.sp.full = S > 1 ? full : c.tiles;
    c.wgs = S > 1 ? full + rem * S : c.tiles;
    c.sp.cnt = nullptr;
    c.sp.part = nullptr;
    c.part_bytes = S > 1 ? (int64_t)rem * S * c.BM * 256 * 4 : 0;
    return c;
}

// Workspace bytes the small-batch tier uses for B (0: no K split).
static int64_t skinny_ws_bytes(const Problem &p, int64_t B)
{
    if (use_stream(p, B)) {
        const StCfg c = stream_cfg(p, true);
        return c.cnt_bytes + c.part_bytes;
    }
    if (use_verify(p, B, plan_nterm(p))) {
        const StCfg c = stream_cfg(p, true);
        return c.ksplit > 1 ? c.cnt_bytes + c.part_bytes * verify_mb(B) : 0;
    }
    const SkCfg c = skinny_cfg(p, B, true);
    return c.cnt_bytes + c.part_bytes;
}

static int choose_tier(const qgemm_plan *plan, int64_t B)
{
    const Problem &p = plan->p;
    if (plan->forced_tier)
        return plan->forced_tier;
    if (use_gemv(p, B))  // B = 1, 2: the GEMV kernel (no K split, no workspace)
        return QGEMM_TIER_GEMV;
    if (p.math == QGEMM_MATH_FP32)  // the streaming and verify kernels, else the faithful tiled variant
        return B <= ST_MAX_B || use_verify(p, B, plan_nterm(p)) ? QGEMM_TIER_SKINNY : QGEMM_TIER_TILED;
    if (p.epi == QGEMM_EPI_SWIGLU)  // fused gate+up: the streaming or verify kernel, or the tiled tier
        return B <= ST_MAX_B || use_verify(p, B, 1) ? QGEMM_TIER_SKINNY : QGEMM_TIER_TILED;
    if (use_verify(p, B, 1))
        return QGEMM_TIER_SKINNY;
    // bf16 math: the skinny kernel's cost grows per 16-row group, the tiled
    // kernel's 128-row tile costs about the same from B = 17 to 128; measured
    // on MI355X the tiled tier wins from B = 48 in every format (and at 32 for
    // MXFP4 and Q8_0).  Both give way to the verify kernel where it applies.
    return B <= 32 ? QGEMM_TIER_SKINNY : QGEMM_TIER_TILED;
}

static KArgs make_args(const Problem &p, int64_t B, const void *w, const void *x, void *y)
{
    KArgs a;
    a.w = (const uint8_t *)w;
    a.x = x;
    a.y = y;
    a.B = (int)B;
    a.N = (int)p.N;
    a.K = (int)p.K;
    a.S = (int)p.L.S;
    a.RT = (int)p.L.RT;
    a.scale_off = p.L.scale_off;
    a.meta_off = p.L.meta_off;
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
    if (fmt == QGEMM_MXFP4 || fmt == QGEMM_NVFP4) {
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
            if (fmt == QGEMM_Q8_0 || fmt == QGEMM_FP8) {
                chunk[8 * u + j] = ((const uint8_t *)codes)[n * K + k];
            } else {
                const uint8_t c = ((const uint8_t *)codes)[n * K + k];
                chunk[4 * u + j / 2] |= (uint8_t)(c << (4 * (j & 1)));
            }
        }
    }
    // scales: per row and slab, the slab's blocks in k order (blocks past K stay 0)
    if (fmt == QGEMM_FP8) {
        // one fp32 scale per 128-wide block: each slab's record holds its block's
        const int64_t nb = (K + FP8_BLOCK - 1) / FP8_BLOCK;
        for (int64_t n = 0; n < N; n++)
            for (int64_t s = 0; s * L.KS < K; s++)
                memcpy(o + scale_offset(L.scale_off, L.S, (int)fmt, n / 16, (int)(n % 16), s),
                       (const float *)scales + n * nb + s * L.KS / FP8_BLOCK, sizeof(float));
        return QGEMM_OK;
    }
    const int64_t nsc = K / L.blk;                       // scales per row
    const int64_t esz = fmt == QGEMM_Q8_0 ? 2 : 1;        // bytes per scale
    const int64_t per_slab = L.KS / L.blk;               // scales per row per slab
    for (int64_t n = 0; n < N; n++) {
        const uint8_t *src = (const uint8_t *)scales + n * nsc * esz;
        for (int64_t s = 0; s < L.S; s++) {
            const int64_t first = s * per_slab;
            const int64_t cnt = first >= nsc ? 0 : (nsc - first < per_slab ? nsc - first : per_slab);
            if (cnt > 0)
                memcpy(o + scale_offset(L.scale_off, L.S, (int)fmt, n / 16, (int)(n % 16), (int)s),
                       src + first * esz, (size_t)(cnt * esz));
        }
    }
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
    if ((int)fmt < 0 || (int)fmt > 3)
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
    // K: a workgroup's activation rows (up to 256 of K fp32 values) and
    // weight rows stay below 2^31 bytes, so the kernels' 32-bit offsets hold
    if (N > (1ll << 30) || K > (1ll << 20))
        return fail(QGEMM_EINVAL, "qgemm_create: N above 2^30 or K above 2^20");
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
    if (math == QGEMM_MATH_FP32 && epi == QGEMM_EPI_SWIGLU)
        return fail(QGEMM_ENOTSUP, "qgemm_create: the fused gate+up epilogue computes in bf16 "
                                   "(QGEMM_MATH_BF16)");
    const uint32_t force = flags & (QGEMM_FLAG_FORCE_SKINNY | QGEMM_FLAG_FORCE_TILED | QGEMM_FLAG_FORCE_GEMV);
    if ((flags & ~(QGEMM_FLAG_FORCE_SKINNY | QGEMM_FLAG_FORCE_TILED | QGEMM_FLAG_FORCE_GEMV)) ||
        (force & (force - 1)))
        return fail(QGEMM_EINVAL, "qgemm_create: bad flags 0x%x", flags);
    int forced = (flags & QGEMM_FLAG_FORCE_SKINNY) ? QGEMM_TIER_SKINNY
               : (flags & QGEMM_FLAG_FORCE_TILED) ? QGEMM_TIER_TILED
               : (flags & QGEMM_FLAG_FORCE_GEMV) ? QGEMM_TIER_GEMV : 0;
    if (!forced) {
        const char *e = getenv("QGEMM_FORCE_TIER");
        if (e && !strcmp(e, "skinny"))
            forced = QGEMM_TIER_SKINNY;
        else if (e && !strcmp(e, "tiled"))
            forced = QGEMM_TIER_TILED;
        else if (e && !strcmp(e, "gemv"))
            forced = QGEMM_TIER_GEMV;
    }
    qgemm_plan *p = new (std::nothrow) qgemm_plan;
    if (!p)
        return fail(QGEMM_ENOMEM, "qgemm_create: out of host memory");
    p->magic = PLAN_MAGIC;
    p->forced_tier = forced;
    p->p.fmt = (int)fmt;
    p->p.act = (int)act;
    p->p.out = (int)out;
    p->p.epi = (int)epi;
    p->p.math = (int)math;
    p->p.N = N;
    p->p.K = K;
    make_layout((int)fmt, N, K, &p->p.L);
    read_knobs(&p->p.kn);
    *plan = p;
    return QGEMM_OK;
}

int qgemm_init_device(void)
{
    const int dev = current_device();
    if (dev < 0)
        return fail(QGEMM_EHIP, "qgemm_init_device: no current HIP device");
    if (!status_word(dev))
        return fail(QGEMM_EHIP, "qgemm_init_device: device status word unavailable");
    if (!g_scratch_ptr[dev].load()) {
        hipStream_t st = nullptr;
        hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
        (void)hipThreadExchangeStreamCaptureMode(&mode);
        hipError_t e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
        uint8_t *sp = e == hipSuccess ? scratch_setup(dev, st, true) : nullptr;
        if (st)
            (void)hipStreamDestroy(st);
        (void)hipThreadExchangeStreamCaptureMode(&mode);
        if (!sp)
            return fail(QGEMM_EHIP, "qgemm_init_device: static scratch unavailable");
    }
    return probe_xcd_dispatch(dev);
}

int qgemm_device_status(uint32_t *bits, int clear, void *stream)
{
    if (!bits)
        return fail(QGEMM_EINVAL, "qgemm_device_status: null pointer");
    *bits = 0;
    uint32_t *d = status_word(current_device());
    if (!d)
        return fail(QGEMM_EHIP, "qgemm_device_status: no device status word");
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e == hipSuccess)
        e = hipMemcpy(bits, d, sizeof *bits, hipMemcpyDeviceToHost);
    if (e == hipSuccess && clear) {
        const uint32_t zero = 0;
        e = hipMemcpy(d, &zero, sizeof zero, hipMemcpyHostToDevice);
    }
    if (e != hipSuccess)
        return hip_fail(e, "qgemm_device_status");
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

int qgemm_xcd_local(void)
{
    const int dev = current_device();
    if (dev < 0)
        return -1;
    const int v = g_xlocal[dev].load();
    return v == 0 ? -1 : v == 1 ? 1 : 0;
}

int qgemm_plan_tier(const qgemm_plan *plan, int64_t B)
{
    if (!plan || plan->magic != PLAN_MAGIC || B < 0)
        return 0;
    return choose_tier(plan, B);
}

// Large-batch tier, fp32 activations with bf16 math: bytes of the bf16 copy
// of x that a workspace can hold (converted once per call instead of once
// per weight tile by every workgroup that stages it).
static int64_t xconv_bytes(const Problem &p, int64_t B)
{
    return p.act == QGEMM_F32 && p.math == QGEMM_MATH_BF16 ? round_up(B * p.K * 2, 256) : 0;
}

size_t qgemm_workspace_bytes(const qgemm_plan *plan, int64_t B)
{
    if (!plan || plan->magic != PLAN_MAGIC || B <= 0 || B > (1ll << 30))
        return 0;
    const int tier = choose_tier(plan, B);
    if (tier == QGEMM_TIER_GEMV)
        return 0;
    if (tier != QGEMM_TIER_SKINNY) {
        const TiCfg c = tiled_cfg(plan->p, B, true);
        const int64_t extra = round_up(c.part_bytes, 256) + xconv_bytes(plan->p, B);
        return extra ? (size_t)(ws_data_off(plan->p) + extra) : 0;
    }
    return (size_t)skinny_ws_bytes(plan->p, B);
}

}  // extern "C"

namespace qg {

// Checks shared by the run entry points.
static int check_run(const qgemm_plan *plan, int64_t B, const void *w, const void *x, const void *y)
{
    if (!plan || plan->magic != PLAN_MAGIC)
        return fail(QGEMM_EINVAL, "qgemm_run: not a live plan");
    const Problem &p = plan->p;
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
    const int64_t ncols = p.epi == QGEMM_EPI_SWIGLU ? p.N / 2 : p.N;
    if (B * p.K > (1ll << 31) - 1 || B * ncols > (1ll << 31) - 1)
        return fail(QGEMM_EINVAL, "qgemm_run: B*K or B*N above 2^31 elements");
    return QGEMM_OK;
}

// One call on arguments check_run accepted, with B > 0.  Scratch is two
// regions: counter words at `cnt` (ws_data_off(p) bytes, zero between calls:
// every call re-arms the ones it used) and partial tiles and the rounded
// copy of x at `data` (data_bytes).  cnt == nullptr: no scratch at all, the
// unsplit route.
static int run_with(const qgemm_plan *plan, int64_t B, const void *w, const void *x, void *y,
                    uint8_t *cnt, uint8_t *data, int64_t data_bytes, hipStream_t st)
{
    const Problem &p = plan->p;
    if (!cnt)
        data_bytes = -1;
    const KArgs a = make_args(p, B, w, x, y);
    hipError_t e;
    const int tier = choose_tier(plan, B);
    if (tier == QGEMM_TIER_GEMV) {
        if (!gemv_fits(p, B))
            return fail(QGEMM_ENOTSUP, "qgemm_run: the GEMV tier takes B <= %d with B*K*4 <= %lld bytes "
                                       "of activations (B=%lld, K=%lld)", GV_MAX_B, (long long)GV_LDS_MAX,
                        (long long)B, (long long)p.K);
        e = launch_gemv(p, a, st);
        if (e != hipSuccess)
            return hip_fail(e, "qgemm_run: kernel launch");
        return QGEMM_OK;
    }
    if (tier == QGEMM_TIER_SKINNY) {
        if (p.epi == QGEMM_EPI_SWIGLU && !use_stream(p, B) && !use_verify(p, B, plan_nterm(p)))
            return fail(QGEMM_ENOTSUP, "qgemm_run: the small-batch tier runs the fused gate+up epilogue "
                                       "for B <= %d, or B <= %d with K a whole number of slabs (B=%lld)",
                        ST_MAX_B, p.kn.vf_swiglu_maxb < VF_MAX_B ? p.kn.vf_swiglu_maxb : VF_MAX_B,
                        (long long)B);
        const int nterm = plan_nterm(p);
        const int64_t need = skinny_ws_bytes(p, B);
        const bool split = cnt != nullptr && (need == 0 || need - ws_data_off(p) <= data_bytes);
        const bool vf = use_verify(p, B, nterm);
        if (use_stream(p, B) || vf) {
            const StCfg c = stream_cfg(p, split);
            SkinnyWs ws;
            ws.cnt = c.ksplit > 1 ? (uint32_t *)cnt : nullptr;
            ws.part = c.ksplit > 1 ? (float *)data : nullptr;
            ws.ksplit = c.ksplit;
            ws.kc = c.kc;
            ws.kch = c.KC;
            ws.xlocal = c.xlocal;
            ws.xcc_fake = p.kn.xcc_fake;
            ws.status = c.xlocal ? status_word(current_device()) : nullptr;
            e = vf ? launch_verify(p, a, c, ws, nterm, st) : launch_stream(p, a, c, ws, nterm, st);
            if (e != hipSuccess)
                return hip_fail(e, "qgemm_run: kernel launch");
            return QGEMM_OK;
        }
        SkCfg c = skinny_cfg(p, B, split);
        if (c.ksplit > 1 && c.part_bytes > data_bytes)
            c = skinny_cfg(p, B, false);  // workspace too small: no K split
        if (c.nby > 65535)
            return fail(QGEMM_EINVAL, "qgemm_run: B=%lld exceeds the small-batch tier's grid",
                        (long long)B);
        SkinnyWs ws;
        ws.cnt = c.ksplit > 1 ? (uint32_t *)cnt : nullptr;
        ws.part = c.ksplit > 1 ? (float *)data : nullptr;
        ws.ksplit = c.ksplit;
        ws.kc = c.kc;
        ws.kch = c.kch;
        ws.xlocal = 0;
        ws.xcc_fake = 0;
        ws.status = nullptr;
        e = launch_skinny(p, a, c, ws, nterm, st);
    } else {
        TiCfg c = tiled_cfg(p, B, cnt != nullptr);
        if (c.part_bytes && c.part_bytes > data_bytes)
            c = tiled_cfg(p, B, false);  // workspace too small: no K split
        if (c.part_bytes) {
            c.sp.cnt = (uint32_t *)(cnt + split_cnt_bytes(p));
            c.sp.part = (float *)data;
        }
        // fp32 activations, bf16 math: with room after the partial tiles, x is
        // rounded to bf16 once into the workspace (the same rounding the
        // kernel applies when it stages fp32 rows) and the bf16 kernel runs
        const int64_t xoff = round_up(c.part_bytes, 256), xcb = xconv_bytes(p, B);
        if (cnt && xcb && xoff + xcb <= data_bytes) {
            void *xb = data + xoff;
            e = launch_x_to_bf16((const float *)x, xb, B * p.K, st);
            if (e != hipSuccess)
                return hip_fail(e, "qgemm_run: kernel launch");
            Problem pb = p;
            pb.act = QGEMM_BF16;
            KArgs ab = a;
            ab.x = xb;
            e = launch_tiled(pb, ab, c, st);
        } else {
            e = launch_tiled(p, a, c, st);
        }
    }
    if (e != hipSuccess)
        return hip_fail(e, "qgemm_run: kernel launch");
    return QGEMM_OK;
}

}  // namespace qg

extern "C" {

int qgemm_run_ws(const qgemm_plan *plan, int64_t B, const void *w, const void *x, void *y,
                 void *workspace, size_t ws_bytes, void *stream)
{
    const int r = check_run(plan, B, w, x, y);
    if (r != QGEMM_OK || B == 0)
        return r;
    if (workspace && ((uintptr_t)workspace & 255u))
        return fail(QGEMM_EINVAL, "qgemm_run: workspace must be 256-byte aligned");
    const int64_t off = ws_data_off(plan->p);
    uint8_t *ws = (uint8_t *)workspace;
    if (!ws || (int64_t)ws_bytes < off)
        return run_with(plan, B, w, x, y, nullptr, nullptr, 0, (hipStream_t)stream);
    return run_with(plan, B, w, x, y, ws, ws + off, (int64_t)ws_bytes - off, (hipStream_t)stream);
}

int qgemm_run_noalloc(const qgemm_plan *plan, int64_t B, const void *w, const void *x, void *y,
                      void *stream)
{
    const int r = check_run(plan, B, w, x, y);
    if (r != QGEMM_OK || B == 0)
        return r;
    const int64_t need = (int64_t)qgemm_workspace_bytes(plan, B);
    const int64_t off = ws_data_off(plan->p);
    if (need > 0 && (off > (int64_t)QGEMM_SCRATCH_COUNTER_BYTES ||
                     need - off > (int64_t)(QGEMM_SCRATCH_BYTES - QGEMM_SCRATCH_COUNTER_BYTES)))
        return fail(QGEMM_EINVAL,
                    "qgemm_run_noalloc: this call needs %lld bytes of scratch (%lld of counters), above "
                    "the static %lld (%lld); use qgemm_run_ws with a workspace or qgemm_run",
                    (long long)need, (long long)off, (long long)QGEMM_SCRATCH_BYTES,
                    (long long)QGEMM_SCRATCH_COUNTER_BYTES);
    if (need == 0)
        return run_with(plan, B, w, x, y, nullptr, nullptr, 0, (hipStream_t)stream);
    uint8_t *sp = scratch_setup(current_device(), (hipStream_t)stream, false);
    if (!sp)
        return fail(QGEMM_EHIP, "qgemm_run_noalloc: static scratch unavailable on this device");
    return run_with(plan, B, w, x, y, sp, sp + QGEMM_SCRATCH_COUNTER_BYTES,
                    (int64_t)(QGEMM_SCRATCH_BYTES - QGEMM_SCRATCH_COUNTER_BYTES), (hipStream_t)stream);
}

// Route of a routed-expert call: bf16 math with fewer than 64 rows per
// expert on average takes the streaming kernel over (expert, row-tile group)
// work items (the small-batch tier's order); otherwise, or for a plan forced
// to the large-batch tier, the large-batch kernel.  0: not runnable.
static int grouped_tier(const qgemm_plan *plan, int64_t E, int64_t T)
{
    const Problem &p = plan->p;
    if (plan->forced_tier == QGEMM_TIER_GEMV)
        return 0;
    const int64_t xsz = p.act == QGEMM_F32 ? 4 : 2;
    const bool small_ok = p.math == QGEMM_MATH_BF16 && T * p.K * xsz < (1ll << 31) &&
                          E * moe_groups(p) <= 0x7FFFFFFFll && moe_groups_per_wg(p, E) >= 1;
    if (plan->forced_tier == QGEMM_TIER_SKINNY)
        return small_ok ? QGEMM_TIER_SKINNY : 0;
    if (plan->forced_tier == QGEMM_TIER_TILED)
        return QGEMM_TIER_TILED;
    return small_ok && T < 64 * E ? QGEMM_TIER_SKINNY : QGEMM_TIER_TILED;
}

int qgemm_grouped_tier(const qgemm_plan *plan, int64_t E, int64_t T)
{
    if (!plan || plan->magic != PLAN_MAGIC || E < 1 || E > (1 << 16) || T < 0 || T > (1ll << 30))
        return 0;
    return grouped_tier(plan, E, T);
}

int qgemm_run_grouped(const qgemm_plan *plan, int64_t E, int64_t T, const void *const *w_table,
                      const int32_t *offsets, const void *x, void *y, void *stream)
{
    if (!plan || plan->magic != PLAN_MAGIC)
        return fail(QGEMM_EINVAL, "qgemm_run_grouped: not a live plan");
    const Problem &p = plan->p;
    if (E < 1 || E > (1 << 16))
        return fail(QGEMM_EINVAL, "qgemm_run_grouped: E=%lld outside 1..2^16", (long long)E);
    if (T < 0 || T > (1ll << 30))
        return fail(QGEMM_EINVAL, "qgemm_run_grouped: T=%lld outside 0..2^30", (long long)T);
    const int tier = grouped_tier(plan, E, T);
    if (!tier)
        return fail(QGEMM_ENOTSUP, "qgemm_run_grouped: a plan forced to the GEMV tier, or to the small-batch "
                                   "tier with fp32 math or T*K beyond 2^31 bytes, has no routed-expert route");
    if (T == 0)
        return QGEMM_OK;
    if (!w_table || !offsets || !x || !y)
        return fail(QGEMM_EINVAL, "qgemm_run_grouped: null pointer");
    if (!aligned16(x) || !aligned16(y) || ((uintptr_t)w_table & 7u) || ((uintptr_t)offsets & 3u))
        return fail(QGEMM_EINVAL, "qgemm_run_grouped: misaligned pointer");
    const int64_t ncols = p.epi == QGEMM_EPI_SWIGLU ? p.N / 2 : p.N;
    if (T * p.K > (1ll << 31) - 1 || T * ncols > (1ll << 31) - 1)
        return fail(QGEMM_EINVAL, "qgemm_run_grouped: T*K or T*N above 2^31 elements");
    KArgs a = make_args(p, T, nullptr, x, y);
    if (tier == QGEMM_TIER_SKINNY) {
        Groups g;
        g.wtab = (const uint8_t *const *)w_table;
        g.off = offsets;
        g.E = (int)E;
        g.T = (int)T;
        g.ntiles = moe_groups(p);
        g.status = status_word(current_device());
        if (!g.status)
            return fail(QGEMM_EHIP, "qgemm_run_grouped: no device status word");
        const hipError_t e = launch_moe(p, a, g, (hipStream_t)stream);
        if (e != hipSuccess)
            return hip_fail(e, "qgemm_run_grouped: kernel launch");
        return QGEMM_OK;
    }
    // BM by the mean rows per expert; an upper bound on the experts' row tiles
    // (each expert adds at most one partial tile, and at most T experts have rows)
    const int BM = p.math == QGEMM_MATH_FP32 ? 64 : T / E >= 192 ? 256 : T / E >= 64 ? 128 : 64;
    const int64_t tiles = T / BM + (E < T ? E : T);
    Groups g;
    g.wtab = (const uint8_t *const *)w_table;
    g.off = offsets;
    g.E = (int)E;
    g.T = (int)T;
    g.status = status_word(current_device());
    if (!g.status)
        return fail(QGEMM_EHIP, "qgemm_run_grouped: no device status word");
    g.ntiles = (int)((ncols + (p.epi == QGEMM_EPI_SWIGLU ? 127 : 255)) / (p.epi == QGEMM_EPI_SWIGLU ? 128 : 256));
    if (tiles * g.ntiles > 0x7FFFFFFFll)
        return fail(QGEMM_EINVAL, "qgemm_run_grouped: grid too large");
    const hipError_t e = launch_grouped(p, a, g, BM, tiles, (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "qgemm_run_grouped: kernel launch");
    return QGEMM_OK;
}

int qgemm_run(const qgemm_plan *plan, int64_t B, const void *w, const void *x, void *y, void *stream)
{
    return qgemm_run_ws(plan, B, w, x, y, nullptr, 0, stream);
}

int qgemm_read_bytes(const void *buf, size_t bytes, uint32_t *sink, int wgs, void *stream)
{
    if (!buf || !sink || !aligned16(buf) || (bytes & 15u) || bytes == 0)
        return fail(QGEMM_EINVAL, "qgemm_read_bytes: null, misaligned or empty buffer, or bytes %% 16");
    if (wgs < 0 || wgs > (1 << 20))
        return fail(QGEMM_EINVAL, "qgemm_read_bytes: wgs outside 0..2^20");
    const hipError_t e = launch_read_bytes(buf, (int64_t)bytes, sink, wgs ? wgs : 2048, (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "qgemm_read_bytes: kernel launch");
    return QGEMM_OK;
}

int qgemm_mfma_rate(int mode, int iters, uint32_t *sink, void *stream)
{
    if (mode < 0 || mode > 7 || iters < 1 || iters > (1 << 24) || !sink)
        return fail(QGEMM_EINVAL, "qgemm_mfma_rate: mode 0..7, iters 1..2^24, sink not null");
    const hipError_t e = launch_mfma_rate(mode, iters, sink, (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "qgemm_mfma_rate: kernel launch");
    return QGEMM_OK;
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
    a.scale_off = L.scale_off;
    a.meta_off = L.meta_off;
    hipError_t e0 = launch_dequant((int)fmt, a, w_out, (hipStream_t)stream);
    if (e0 != hipSuccess)
        return hip_fail(e0, "qgemm_dequantize: kernel launch");
    return QGEMM_OK;
}

}  // extern "C"
