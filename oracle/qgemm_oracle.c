/*
 * CPU oracle for the block-quantized-weight batched GEMM
 *
 *     y[b][n] = sum_k x[b][k] * w[n][k]
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant with the HIP library; it reads the *logical*
 * arrays (one code per byte, scales in their own arrays), never the packed
 * device layout.
 *
 * Sources (the pages; see the oracle/__init__.py docstring for page titles):
 *  - hipfire issue "Qwen3.8-27B native MTP crashes when Q8 batched GEMM
 *    exceeds MAX_BATCH=64", Summary and Expected behavior: the Q8 batched GEMM
 *    must accept batch widths such as 65, 70, 76, 256 (no fixed maximum).
 *  - hipfire PR "fix(mtp): chunk scalar Q8 batched GEMM above 64 rows", Root
 *    cause and fix + Scalar-Q8 boundary matrix: an f32 reduction contract, and
 *    a batch split into contiguous chunks (70 = 64 + 6) gives the same rows.
 *  - Atlas issue "[job] Qwen3.8-27B on Strix Halo ...", section "Kernel-level
 *    root cause of the gfx1151 NVFP4 prefill gap", Fix paragraph: NVFP4 is
 *    E2M1 codes times an E4M3 block scale (exact), with the fp32 tensor scale
 *    applied in the epilogue; validation against an FP64 host reference with
 *    exact weights.
 *  - HF model card "Qwen3.8-27B — MXFP4 (AMD Quark) for RDNA4", Model
 *    details: MXFP4 = E2M1 codes with a shared power-of-two (E8M0) scale.
 *  - The workload definitions (Q8_0: 32 int8 + fp16 scale, w = d*q; MXFP4:
 *    32 E2M1 + E8M0; NVFP4: 16 E2M1 + E4M3 + fp32 tensor scale; fused
 *    gate+up output SiLU(gate)*up).
 *  - Atlas issue, "Kernel ranking" and "Next lever" sections: the FP8-weight
 *    GEMM (FP8 weights times 16-bit activations) of the GDN and attention
 *    projections.  The pages give no block rule for it; this oracle reads it
 *    as E4M3 codes times one fp32 scale per row and 128-wide K block (the
 *    last block may be shorter): w = s * E4M3(c).
 *
 * Arithmetic: every decoded weight is exact in double (Q8_0 d*q has at most
 * 19 significant bits, FP4 values times their scales at most 6, an fp32
 * scale times an E4M3 value at most 28), and every
 * product x*w is exact in double (fp32 x has 24 bits).  Sums run in fp64 in
 * increasing k.  Compile with -ffp-contract=off.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

#define OR_Q8_0 0
#define OR_MXFP4 1
#define OR_NVFP4 2
#define OR_FP8 3

#define OR_ACT_F32 0
#define OR_ACT_BF16 1

/* ---- element and scale decoders, written from the format definitions ---- */

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_fp16(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + m, e - 25);          /* (1 + m/1024) * 2^(e-15) */
    return s ? -v : v;
}

/* bfloat16: the upper half of an IEEE binary32. */
double oracle_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* E2M1 (FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit; no inf/NaN. */
double oracle_e2m1(uint8_t c)
{
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* E8M0: unsigned power-of-two exponent, bias 127; 0xFF is NaN. */
double oracle_e8m0(uint8_t b)
{
    return (b == 0xFF) ? NAN : ldexp(1.0, (int)b - 127);
}

/* FP8 E4M3 (the "fn" variant): 1 sign, 4 exponent (bias 7), 3 mantissa; no
 * infinities; S.1111.111 is NaN; largest finite value 448. */
double oracle_e4m3(uint8_t b)
{
    int s = (b >> 7) & 1, E = (b >> 3) & 15, M = b & 7;
    double v;
    if (E == 15 && M == 7)
        return NAN;
    if (E == 0)
        v = ldexp((double)M, -9);               /* 2^-6 * M/8 */
    else
        v = ldexp(8.0 + M, E - 10);             /* 2^(E-7) * (1 + M/8) */
    return s ? -v : v;
}

/* Decoded weight w[n][k] without the NVFP4 tensor scale. */
static double weight(int fmt, const void *codes, const void *scales,
                     int64_t K, int64_t n, int64_t k)
{
    switch (fmt) {
    case OR_Q8_0: {
        const int8_t *q = (const int8_t *)codes;
        const uint16_t *d = (const uint16_t *)scales;
        return oracle_fp16(d[n * (K / 32) + k / 32]) * (double)q[n * K + k];
    }
    case OR_MXFP4: {
        const uint8_t *c = (const uint8_t *)codes;
        const uint8_t *e = (const uint8_t *)scales;
        return oracle_e2m1(c[n * K + k]) * oracle_e8m0(e[n * (K / 32) + k / 32]);
    }
    case OR_NVFP4: {
        const uint8_t *c = (const uint8_t *)codes;
        const uint8_t *s = (const uint8_t *)scales;
        return oracle_e2m1(c[n * K + k]) * oracle_e4m3(s[n * (K / 16) + k / 16]);
    }
    case OR_FP8: {
        const uint8_t *c = (const uint8_t *)codes;
        const float *s = (const float *)scales;
        const int64_t nb = (K + 127) / 128;  /* blocks per row */
        return (double)s[n * nb + k / 128] * oracle_e4m3(c[n * K + k]);
    }
    }
    return NAN;
}

/* Tensor scale of row n: rows are split into `ntensors` equal groups, each
 * with its own fp32 scale (NVFP4 only; 1 elsewhere). */
static double tensor_scale(int fmt, const float *g, int64_t ntensors, int64_t N, int64_t n)
{
    if (fmt != OR_NVFP4 || g == 0 || ntensors <= 0)
        return 1.0;
    return (double)g[n / (N / ntensors)];
}

static double act(int act_dtype, const void *x, int64_t K, int64_t b, int64_t k)
{
    if (act_dtype == OR_ACT_F32)
        return (double)((const float *)x)[b * K + k];
    return oracle_bf16(((const uint16_t *)x)[b * K + k]);
}

/* Dense decode: w_out[n][k] = weight (times the tensor scale when apply_g). */
void oracle_dequant(int fmt, const void *codes, const void *scales, const float *g,
                    int64_t ntensors, int apply_g, int64_t N, int64_t K, double *w_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        double gs = apply_g ? tensor_scale(fmt, g, ntensors, N, n) : 1.0;
        for (int64_t k = 0; k < K; k++) {
            double w = weight(fmt, codes, scales, K, n, k);
            w_out[n * K + k] = apply_g ? gs * w : w;
        }
    }
}

/* One output: y[b][n] = g(n) * sum_k x[b][k] * w[n][k], k increasing. */
static double dot_row(int fmt, const void *codes, const void *scales, const float *g,
                      int64_t ntensors, int act_dtype, const void *x, int64_t N, int64_t K,
                      int64_t b, int64_t n)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; k++)
        acc += act(act_dtype, x, K, b, k) * weight(fmt, codes, scales, K, n, k);
    return tensor_scale(fmt, g, ntensors, N, n) * acc;
}

/* Full product y[B][N] (fp64). */
void oracle_gemm(int fmt, const void *codes, const void *scales, const float *g,
                 int64_t ntensors, int act_dtype, const void *x, int64_t B, int64_t N,
                 int64_t K, double *y)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t b = 0; b < B; b++)
            y[b * N + n] = dot_row(fmt, codes, scales, g, ntensors, act_dtype, x, N, K, b, n);
    }
}

/* Selected outputs y[bidx[i]][nidx[i]] (fp64), for full-size workloads. */
void oracle_gemm_at(int fmt, const void *codes, const void *scales, const float *g,
                    int64_t ntensors, int act_dtype, const void *x, int64_t N, int64_t K,
                    const int64_t *bidx, const int64_t *nidx, int64_t count, double *y)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; i++)
        y[i] = dot_row(fmt, codes, scales, g, ntensors, act_dtype, x, N, K, bidx[i], nidx[i]);
}

/* Magnitude sum behind the floating-point error bound of a dot product,
 * M[b][n] = |g(n)| * sum_k |x[b][k]| * |w[n][k]|: a summation of the K
 * products in any order, rounding each addition to precision u, lies within
 * gamma_n * M of the exact sum, gamma_n = n u / (1 - n u) (the standard
 * recursive-summation bound).  Selected outputs, as oracle_gemm_at. */
void oracle_gemm_abs_at(int fmt, const void *codes, const void *scales, const float *g,
                        int64_t ntensors, int act_dtype, const void *x, int64_t N, int64_t K,
                        const int64_t *bidx, const int64_t *nidx, int64_t count, double *m)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; i++) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; k++)
            acc += fabs(act(act_dtype, x, K, bidx[i], k)) *
                   fabs(weight(fmt, codes, scales, K, nidx[i], k));
        m[i] = fabs(tensor_scale(fmt, g, ntensors, N, nidx[i])) * acc;
    }
}

/* SiLU(t) = t * sigmoid(t) = t / (1 + e^-t). */
/* Threads an OpenMP region of this library runs on (for reporting only). */
int oracle_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}

/* Threads the parallel loops use from now on (n >= 1); for the timing of
 * the benchmark's one-thread baseline.  Results do not depend on it: every
 * output is one sequential sum. */
void oracle_set_threads(int n)
{
    omp_set_num_threads(n > 0 ? n : 1);
}

double oracle_silu(double t)
{
    return t / (1.0 + exp(-t));
}

/* Fused gate+up: rows [0, Nh) of w are the gate, rows [Nh, 2Nh) the up
 * projection (each its own tensor scale); out[b][j] = SiLU(G) * U with
 * G = y[b][j], U = y[b][Nh + j].  N = 2 Nh. */
void oracle_swiglu_at(int fmt, const void *codes, const void *scales, const float *g,
                      int64_t ntensors, int act_dtype, const void *x, int64_t N, int64_t K,
                      const int64_t *bidx, const int64_t *jidx, int64_t count, double *out)
{
    int64_t Nh = N / 2;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; i++) {
        double G = dot_row(fmt, codes, scales, g, ntensors, act_dtype, x, N, K, bidx[i], jidx[i]);
        double U = dot_row(fmt, codes, scales, g, ntensors, act_dtype, x, N, K, bidx[i],
                           Nh + jidx[i]);
        out[i] = oracle_silu(G) * U;
    }
}

void oracle_swiglu(int fmt, const void *codes, const void *scales, const float *g,
                   int64_t ntensors, int act_dtype, const void *x, int64_t B, int64_t N,
                   int64_t K, double *out)
{
    int64_t Nh = N / 2;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t j = 0; j < Nh; j++) {
        for (int64_t b = 0; b < B; b++) {
            double G = dot_row(fmt, codes, scales, g, ntensors, act_dtype, x, N, K, b, j);
            double U = dot_row(fmt, codes, scales, g, ntensors, act_dtype, x, N, K, b, Nh + j);
            out[b * Nh + j] = oracle_silu(G) * U;
        }
    }
}
