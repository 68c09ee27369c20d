/*
 * qgemm.h - block-quantized-weight batched GEMM for AMD Instinct MI355X (gfx950)
 *
 *     y[b][n] = sum_k x[b][k] * dequant(W)[n][k],   0 <= b < B, 0 <= n < N
 *
 * The operation is the Q8_0 batched GEMM that speculative-decoding verify and
 * prefill call with any batch width (hipfire issue "Qwen3.8-27B native MTP
 * crashes when Q8 batched GEMM exceeds MAX_BATCH=64", Summary and Expected
 * behavior: widths 70, 76, 256 must run, not abort), and its 4-bit siblings
 * MXFP4 (HF model card "Qwen3.8-27B - MXFP4 (AMD Quark) for RDNA4", "What's
 * 4-bit") and NVFP4 (Atlas issue "[job] Qwen3.8-27B on Strix Halo: prefill
 * 2.4x gap + DP4A verify tiers for K=5..9", section "Kernel-level root cause
 * of the gfx1151 NVFP4 prefill gap", Fix), plus the fused gate+up
 * dual-accumulator GEMM with a SiLU*mul epilogue that the same Atlas issue
 * asks for in "What's the job?", and the FP8-weight (W8A16) GEMM of the
 * attention and GDN projections in the same issue's "Kernel ranking".
 *
 * There is no batch limit: every B >= 0 runs in one call, with no host loop
 * over batch chunks (B = 0 is a no-op).
 *
 * Conventions for every entry point
 *  - Return value: QGEMM_OK (0) or a positive qgemm_status.  On failure,
 *    qgemm_last_error() returns a message for the calling thread.  The library
 *    never aborts, asserts, prints or exits.
 *  - "device pointer": memory the caller allocated on the current HIP device
 *    (hipMalloc or a framework allocator).  The caller owns every buffer.
 *  - stream: a hipStream_t passed as void* (NULL = the default stream).  GPU
 *    work is enqueued asynchronously on it; errors raised while a kernel runs
 *    surface at the caller's next synchronisation, as in HIP.
 *
 * Weight formats (the logical arrays; N rows of K weights, blocks along K)
 *  - QGEMM_Q8_0:  int8 q[N][K] and fp16 d[N][K/32];   w = d * q.
 *  - QGEMM_MXFP4: E2M1 codes c[N][K] (4 bits) and E8M0 e[N][K/32];
 *                 w = E2M1(c) * 2^(e-127)  (e = 255 is NaN).
 *  - QGEMM_NVFP4: E2M1 codes c[N][K] and FP8-E4M3 s[N][K/16], plus an fp32
 *                 tensor scale g per tensor;  w = g * E2M1(c) * E4M3(s), with
 *                 g applied to the finished sum.
 *  - QGEMM_FP8:   FP8-E4M3 codes c[N][K] (OCP E4M3: bias 7, no infinities,
 *                 0x7F/0xFF NaN) and one fp32 scale s[N][ceil(K/128)] per
 *                 128-wide block along K (the last block may be shorter);
 *                 w = s * E4M3(c).  (The pages fix no block rule for their
 *                 FP8 weights; per-row 128-blocks also carry per-channel and
 *                 128x128-block scales.)
 *  E2M1 code bits: sign (bit 3), exponent (bits 2-1, bias 1), mantissa (bit 0):
 *  magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qgemm_status {
    QGEMM_OK = 0,
    QGEMM_EINVAL = 1,  /* bad argument: null/misaligned pointer, B < 0, N or K <= 0,
                          K not a multiple of the block, odd N with SwiGLU, ... */
    QGEMM_ENOTSUP = 2, /* combination of format / dtypes / epilogue / tier not built */
    QGEMM_EHIP = 3,    /* a HIP call failed; qgemm_last_error() holds its message */
    QGEMM_ENOMEM = 4   /* host allocation failed */
} qgemm_status;

typedef enum qgemm_format {
    QGEMM_Q8_0 = 0,
    QGEMM_MXFP4 = 1,
    QGEMM_NVFP4 = 2,
    QGEMM_FP8 = 3
} qgemm_format;

typedef enum qgemm_dtype {
    QGEMM_F32 = 0,  /* IEEE binary32 */
    QGEMM_BF16 = 1  /* bfloat16, passed as its 16-bit pattern */
} qgemm_dtype;

typedef enum qgemm_epilogue {
    QGEMM_EPI_NONE = 0,
    /* Fused gate+up: W has N = 2*Nh rows, rows [0, Nh) the gate projection and
     * rows [Nh, 2Nh) the up projection.  y is [B][Nh]:
     *     y[b][j] = SiLU(G) * U,  G = sum_k x w[j],  U = sum_k x w[Nh + j],
     * SiLU(t) = t / (1 + exp(-t)).  G and U never reach memory. */
    QGEMM_EPI_SWIGLU = 1
} qgemm_epilogue;

typedef enum qgemm_math {
    /* fp32-faithful: used with fp32 activations, in both tiers.  Weights enter
     * exactly and activations are split into bf16 terms that together hold
     * their full fp32 value; relative Frobenius error against an exact
     * product <= 1e-5. */
    QGEMM_MATH_FP32 = 0,
    /* bf16 operands: fp32 activations are rounded to bf16 (nearest even) in the
     * kernel; bf16 activations enter as they are.  Decoded MXFP4 and NVFP4
     * weights are exact in bf16; a Q8_0 weight d*q or an FP8 weight s*E4M3(c)
     * is rounded once to bf16 in the large-batch tier.  Relative Frobenius
     * error <= 1e-2. */
    QGEMM_MATH_BF16 = 1
} qgemm_math;

/* Tiers (how a call maps onto kernels); qgemm_create flags may force one. */
typedef enum qgemm_tier {
    QGEMM_TIER_SKINNY = 1, /* weights streamed once per 16..80 batch rows straight
                              into matrix-core operands; for small B (B <= 80
                              when K is a whole number of slabs, B <= 48 with
                              the fused epilogue; else B <= 16, or B <= 32 with
                              bf16 math).  Each math mode keeps one summation
                              order per output across the tier, so a batch
                              row's result does not depend on B there */
    QGEMM_TIER_TILED = 2,  /* batch x weight tiles staged through LDS; for large B
                              (above the small-batch limits) */
    QGEMM_TIER_GEMV = 3    /* B = 1, 2: one workgroup per 16-row tile over all of
                              K, fp32 FMA on the vector ALUs, a fixed-order
                              cross-lane sum; no K split and no workspace.
                              Chosen automatically for B = 1 when the row, as
                              fp32, takes at most 32 KB (K <= 8192; measured
                              faster than the streaming kernel there on
                              MI355X), else only when forced; a forced call
                              needs the B rows, as fp32, to fit in 72 KB of
                              LDS, and returns QGEMM_ENOTSUP otherwise */
} qgemm_tier;

#define QGEMM_FLAG_FORCE_SKINNY 0x1u
#define QGEMM_FLAG_FORCE_TILED 0x2u
#define QGEMM_FLAG_FORCE_GEMV 0x4u

/* ---------------------------------------------------------------- layout
 * The packed device buffer that qgemm_pack writes and every kernel reads.
 *
 * Rows are grouped in row tiles of 16 (Np = N rounded up to 16) and K is cut
 * into slabs of KS = 64 (Q8_0, FP8) or 128 (MXFP4, NVFP4) weights (Kp = K rounded
 * up to KS; S = Kp / KS).  Padding rows and columns hold zero codes and zero
 * scale bytes.
 *
 * 1. Codes: slab (rt, s) is 1024 bytes at ((rt * S) + s) * 1024.  Its 16-byte
 *    chunk L (0..63) belongs to row r = L % 16 of the tile and k-group
 *    g = L / 16, and holds, for each 32-wide unit u of the slab, the eight
 *    weights k = s*KS + 32u + 8g + 0..7 of that row:
 *      Q8_0 : byte 8u + j is q (int8) for j = 0..7, u = 0..1;
 *      FP8  : byte 8u + j is the E4M3 code, as for Q8_0;
 *      FP4  : byte 4u + j holds the codes of k = ... + 2j (low nibble) and
 *             ... + 2j + 1 (high nibble), u = 0..3.
 * 2. Scales: at a QGEMM_ALIGN-rounded offset, one record per slab, in the
 *    codes' order: record (rt, s) is at ((rt * S) + s) * 16 * E and its bytes
 *    E*r .. E*r+E-1 hold row r's scales of the slab, blocks in k order:
 *      Q8_0 : E = 4, 2 fp16 d;
 *      MXFP4: E = 4, 4 E8M0 bytes;
 *      NVFP4: E = 8, 8 E4M3 bytes (one per 16 weights);
 *      FP8  : E = 4, the fp32 scale of the 128-wide block holding the slab
 *             (each block's scale appears in both of its slabs' records).
 * 3. NVFP4 only, at the next QGEMM_ALIGN offset, 256 bytes:
 *      int32 ntensors, int32 rows_per_tensor, int32 0, int32 0,
 *      float g[QGEMM_MAX_TENSORS];  row n uses g[n / rows_per_tensor].
 */
#define QGEMM_ALIGN 256
#define QGEMM_MAX_TENSORS 60

/* Size in bytes of the packed buffer for an N x K weight.  0 on bad input. */
size_t qgemm_weight_bytes(qgemm_format fmt, int64_t N, int64_t K);

/* Host-side packer: logical arrays (host pointers) -> packed buffer (host
 * pointer, out_bytes >= qgemm_weight_bytes).  codes: Q8_0 int8 [N][K]; FP4
 * uint8 [N][K], one code (0..15) per byte; FP8 uint8 [N][K] E4M3 codes.
 * scales: Q8_0 uint16 fp16 bits [N][K/32]; MXFP4 uint8 [N][K/32]; NVFP4
 * uint8 [N][K/16]; FP8 float [N][ceil(K/128)].  tensor_scales:
 * NVFP4 only, ntensors (1..QGEMM_MAX_TENSORS, dividing N) fp32 values; NULL
 * and 0 for the other formats.  Pure host code, callable without a GPU. */
int qgemm_pack(qgemm_format fmt, int64_t N, int64_t K, const void *codes, const void *scales,
               const float *tensor_scales, int64_t ntensors, void *out, size_t out_bytes);

/* ------------------------------------------------------------------ plan */
typedef struct qgemm_plan qgemm_plan;

/* Validate and record a problem shape: 1 <= N <= 2^30, 1 <= K <= 2^20, K a
 * multiple of the format's block.  act: activation dtype; out: output
 * dtype; math: see qgemm_math (QGEMM_MATH_FP32 needs act = QGEMM_F32; the
 * SwiGLU epilogue needs QGEMM_MATH_BF16, else QGEMM_ENOTSUP); flags:
 * 0 or one QGEMM_FLAG_FORCE_* bit (also settable with the environment
 * variable QGEMM_FORCE_TIER=skinny|tiled|gemv).  Host-only: allocates the small
 * plan object, makes no HIP call and works without a device.  Tuning
 * overrides in the environment (QGEMM_ST_*, QGEMM_SK_*, QGEMM_TI_*) are read
 * here, once.  *plan receives the handle. */
int qgemm_create(qgemm_plan **plan, qgemm_format fmt, qgemm_dtype act, qgemm_dtype out,
                 qgemm_epilogue epi, qgemm_math math, int64_t N, int64_t K, uint32_t flags);

/* y = x * W^T (or the SwiGLU of the two halves) for B rows.  SwiGLU runs in
 * the small-batch tier for B <= 16 and in the large-batch tier otherwise (a
 * plan forced to the small-batch tier returns QGEMM_ENOTSUP for B > 16).
 *   w: packed weights (device, 16-byte aligned), laid out as above for the
 *      plan's N and K;
 *   x: activations [B][K] row-major (device, 16-byte aligned, act dtype);
 *   y: output [B][N] (or [B][N/2] for SwiGLU) row-major (device, out dtype);
 *      must not overlap x or w.
 * Any B >= 0; B = 0 returns QGEMM_OK and enqueues nothing.  No allocation,
 * no synchronisation.  Plans are immutable, so several threads may run one
 * plan at once.  Results are deterministic: no atomics, fixed summation order
 * for a given plan, tier and B. */
int qgemm_run(const qgemm_plan *plan, int64_t B, const void *w, const void *x, void *y,
              void *stream);

/* Routed experts (the Atlas issue's routed-expert GEMMs reached through an
 * expert pointer table, "Per-32-K-step hot loop" and the 512-expert, top-10
 * routed MoE of its validation plan): E experts share the plan's format,
 * shape, dtypes and epilogue; rows offsets[e] .. offsets[e+1]-1 of x and y
 * use expert e's packed weights w_table[e].
 *   w_table: device array of E device pointers (each 16-byte aligned, laid out
 *            as above for the plan's N and K; NVFP4 tensor scales per expert);
 *   offsets: device int32 [E + 1], offsets[0] = 0, non-decreasing,
 *            offsets[E] = T (the caller sorts the routed rows by expert);
 *            1 <= E <= 2^16;
 *   x: [T][K] routed activation rows; y: [T][N] (or [T][N/2] with SwiGLU).
 * Experts with no rows cost only a scan.  One launch, on one of two routes
 * (qgemm_grouped_tier tells which):
 *   QGEMM_TIER_SKINNY: bf16 math with fewer than 64 rows per expert on
 *     average (T < 64 E) and under 2^31 bytes of activations, or a plan
 *     forced to the small-batch tier (bf16 math): each expert's weights are streamed once for all of its rows, in
 *     the small-batch tier's summation order, so each expert's rows are
 *     bitwise those of qgemm_run of that expert in the small-batch tier
 *     without a workspace (a row's result does not depend on the other rows;
 *     with SwiGLU, calls of at most 16 rows);
 *   QGEMM_TIER_TILED: otherwise (fp32-faithful math, more rows per expert,
 *     or a plan forced to the large-batch tier): the large-batch kernel,
 *     unsplit, so each expert's rows are bitwise those of qgemm_run of that
 *     expert in the large-batch tier without a workspace.
 * A plan forced to the GEMV tier, or to the small-batch tier with fp32 math,
 * returns QGEMM_ENOTSUP.  T = 0 returns QGEMM_OK and enqueues nothing.
 * The offsets are read and checked on the device: when they break a rule
 * above, the kernel reads and writes nothing outside the offsets array and
 * the table and sets QGEMM_DEV_BAD_OFFSETS in the device status word (y is
 * left unwritten; qgemm_device_status reports it). */
int qgemm_run_grouped(const qgemm_plan *plan, int64_t E, int64_t T, const void *const *w_table,
                      const int32_t *offsets, const void *x, void *y, void *stream);

/* The route qgemm_run_grouped takes for E experts and T rows
 * (QGEMM_TIER_SKINNY or QGEMM_TIER_TILED, as described there), or 0 for a bad
 * plan or sizes, or a plan with no routed-expert route.  Host only. */
int qgemm_grouped_tier(const qgemm_plan *plan, int64_t E, int64_t T);

/* Bytes of device workspace with which qgemm_run_ws may split K across
 * workgroups for this plan and B (0 when the chosen tier does not use one). */
size_t qgemm_workspace_bytes(const qgemm_plan *plan, int64_t B);

/* qgemm_run with a caller-owned workspace (device memory, 256-byte aligned).
 * With at least qgemm_workspace_bytes(plan, B) bytes, the small-batch tier
 * splits K over several workgroups per output tile (the last workgroup of a
 * tile to finish adds the partial tiles in a fixed order), and the
 * large-batch tier splits the tiles of a last, partial round of tiles along K
 * (a second kernel on the stream adds the pieces in order) and, for fp32
 * activations with bf16 math, first rounds x to bf16 once into the workspace
 * (the rounding its kernel applies anyway: results are unchanged by it).
 * Results stay
 * deterministic; they can differ in rounding from the unsplit route, and in
 * the large-batch tier from one B to another.
 * Contract: the workspace must be all zero before its first use with a plan;
 * every call returns its counter words to zero, so it can be reused by later
 * calls of that plan on the same stream, at any B.  A workspace moved to
 * another plan must be zeroed again.  Calls that may overlap in time need
 * distinct workspaces.  A NULL or smaller workspace selects the unsplit
 * route. */
int qgemm_run_ws(const qgemm_plan *plan, int64_t B, const void *w, const void *x, void *y,
                 void *workspace, size_t workspace_bytes, void *stream);

/* qgemm_run_ws with the library's own scratch instead of a workspace, for
 * callers that cannot allocate (code under graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): it calls no hipMalloc, hipFree or
 * other allocating routine.  The scratch is one static device array of
 * QGEMM_SCRATCH_BYTES per device (the first QGEMM_SCRATCH_COUNTER_BYTES hold
 * counter words), held from the library's load until the process ends; it
 * is set up by qgemm_init_device or by the first call on a device (which
 * then also enqueues a small zeroing kernel on `stream` before its work).
 * The call takes the same route, and gives bitwise the same result, as
 * qgemm_run_ws with a workspace of qgemm_workspace_bytes(plan, B) bytes.  A
 * call that needs more scratch than the array holds returns QGEMM_EINVAL
 * (with the sizes in qgemm_last_error) and enqueues nothing.  Every call on
 * a device shares that device's array and leaves its counters at zero:
 * calls that may overlap in time on one device race (use one stream, or
 * qgemm_run_ws with distinct workspaces). */
#define QGEMM_SCRATCH_BYTES (64u << 20)
#define QGEMM_SCRATCH_COUNTER_BYTES (1u << 20)
int qgemm_run_noalloc(const qgemm_plan *plan, int64_t B, const void *w, const void *x, void *y,
                      void *stream);

/* The tier qgemm_run would use for B (QGEMM_TIER_*), or 0 for a bad plan. */
int qgemm_plan_tier(const qgemm_plan *plan, int64_t B);

/* Optional one-time set-up of the current device; calling it again is cheap.
 * It runs a dispatch probe there (a small kernel on a stream of its own, in
 * relaxed capture mode so a graph being captured elsewhere stays valid, and
 * a synchronous 8 KB copy) that decides whether the small-batch kernel's K
 * splits may meet in one XCD's L2: the hardware deals workgroup ids to the
 * XCDs round-robin, and the probe checks that ids congruent mod 8 share an
 * XCC.  Until it has run on a device, or where the probe fails, the K splits
 * meet in device-coherent memory; results are bitwise the same either way.
 * (The XCD that id 0 lands on can change from launch to launch; only the
 * congruence matters.)  Every launch that uses the XCD-local exchange checks
 * it again: the K splits of each row group count themselves per XCC, and
 * when the last one finds them spread over more than one XCD it sets
 * QGEMM_DEV_XCD_MISMATCH in the device status word; that launch's output is
 * then not to be trusted (rerun with the exchange off).  QGEMM_ST_XLOCAL=0
 * in the environment (read at plan creation) turns the exchange off.
 * Returns QGEMM_EHIP when there is no device or the probe cannot run. */
int qgemm_init_device(void);

/* Outcome of qgemm_init_device's dispatch probe on the current device: 1 when
 * workgroup ids congruent mod 8 ran on one XCD, 0 when they did not, -1 when
 * the device was not initialised or there is no device. */
int qgemm_xcd_local(void);

/* Device status word bits: conditions a kernel detected while it ran. */
#define QGEMM_DEV_XCD_MISMATCH 0x1u /* the K splits of a row group ran on different XCDs */
#define QGEMM_DEV_BAD_OFFSETS 0x2u  /* qgemm_run_grouped offsets broke their rules; no work done */

/* Read the current device's status word into *bits (the OR of every bit set
 * since it was last cleared), after synchronising `stream` (the word is set
 * by kernels, so the caller names the stream whose work it asks about);
 * clear != 0 then zeroes it.  Synchronous; not for use during graph
 * capture. */
int qgemm_device_status(uint32_t *bits, int clear, void *stream);

/* Release a plan (NULL is accepted). */
int qgemm_destroy(qgemm_plan *plan);

/* Device decode of a packed buffer to fp32 w_out[N][K] (device pointer),
 * using the kernels' own decoders: Q8_0 d*q; MXFP4 E2M1 * 2^(e-127); NVFP4
 * g * (E2M1 * E4M3) rounded once to fp32; FP8 s * E4M3(c) rounded once to
 * fp32.  Every other value is exact. */
int qgemm_dequantize(qgemm_format fmt, const void *w, float *w_out, int64_t N, int64_t K,
                     void *stream);

/* Measurement aid, not part of the GEMM: read `bytes` (a positive multiple
 * of 16) of device memory at buf (16-byte aligned) once, with the 16-byte
 * loads the streaming kernel uses, over `wgs` workgroups of 256 threads
 * (0 = 2048), and write one XOR-folded word per workgroup to sink (device,
 * wgs words) so the loads are kept.  The plain read rate of the same bytes
 * is the achieved-bandwidth ceiling the weight stream is compared with. */
int qgemm_read_bytes(const void *buf, size_t bytes, uint32_t *sink, int wgs, void *stream);

/* Measurement aid, not part of the GEMM: one launch of a matrix-core loop
 * (512 workgroups of 8 waves, each wave `iters` trips of eight independent
 * accumulator chains) that shows whether an int8-activation tier could beat
 * the bf16 tier for Q8_0 weights, whose scales change every 32 weights, and
 * what the hardware block-scaled route would give the MX formats:
 *   0 v_mfma_f32_16x16x32_bf16; 1 v_mfma_i32_16x16x32_i8 (one 32-wide block
 *   per MFMA); 2 v_mfma_i32_16x16x64_i8 (two blocks, no per-block scale);
 *   3 mode 1 plus each block's int32 -> fp32 conversion and scale product
 *   d_w * d_x into an fp32 accumulator; 4 mode 0 plus a per-block fp32 scale
 *   FMA; 5 v_mfma_scale_f32_16x16x128_f8f6f4 with E4M3 A and E2M1 B (E8M0
 *   scale per row and 32-wide block on each side); 6 the same with E2M1 on
 *   both sides; 7 the same with E4M3 on both sides.  mode outside 0..7 ->
 *   QGEMM_EINVAL.  sink: device, 4096 words.  The caller times the launch. */
int qgemm_mfma_rate(int mode, int iters, uint32_t *sink, void *stream);

/* Text for a status code (static storage). */
const char *qgemm_strerror(int status);

/* Message of the last failure on the calling thread ("" if none). */
const char *qgemm_last_error(void);

/* Library version, (major << 16) | minor. */
int qgemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
