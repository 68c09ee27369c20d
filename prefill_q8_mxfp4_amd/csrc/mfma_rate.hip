// Measurement aid, not part of the GEMM: matrix-core throughput of the inner
// loops an int8-activation tier for Q8_0 weights would run, next to the bf16
// loop the library runs.  Q8_0 scales change every 32 weights along K, so an
// int8 product needs one 32-deep integer sum per block before its two scales
// (weight row x activation row) can be applied; gfx950's double-rate int8
// MFMA sums 64 products, i.e. two blocks, at once.
//
// Every wave runs `iters` trips of eight independent accumulator chains
// (8 waves per workgroup, two workgroups per CU on a 512-workgroup grid):
//
//   mode 0  v_mfma_f32_16x16x32_bf16                 (bf16 math: scales folded
//                                                     into the bf16 weights)
//   mode 1  v_mfma_i32_16x16x32_i8                   (one Q8_0 block per MFMA)
//   mode 2  v_mfma_i32_16x16x64_i8                   (two blocks: no per-block scale)
//   mode 3  mode 1 from a zero accumulator, then per block the int32 -> fp32
//           conversion and the scale product d_w * d_x[row] into an fp32
//           accumulator (4 cvt, 4 mul, 4 fma per lane): the int8 tier's loop
//   mode 4  mode 0 from a zero accumulator plus a per-block fp32 scale FMA
//           (4 fma per lane): the block-scale pattern of the fp32-faithful path
//
// and the block-scaled matrix-core route for the MX formats (one E8M0 scale
// per operand row and 32-wide block, applied by the hardware), K = 128 per
// instruction:
//
//   mode 5  v_mfma_scale_f32_16x16x128_f8f6f4, A E4M3, B E2M1 (MXFP4 weights
//           against fp8 activations)
//   mode 6  the same, A and B E2M1 (fp4 activations)
//   mode 7  the same, A and B E4M3 (FP8 weights against fp8 activations)
//
// Operands are derived from the thread id and a seed so nothing folds; each
// wave writes one word to sink.  Throughput = MFMAs x 2 x 16 x 16 x K / time.
#include "common.h"

namespace qg {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int MODE>
__global__ __launch_bounds__(512) void mfma_rate_kernel(int iters, uint32_t seed, uint32_t *sink)
{
    const uint32_t v = seed ^ (threadIdx.x * 2654435761u) ^ (blockIdx.x * 40503u);
    const u32x4 bits = u32x4{v & 0x3F7F3F7Fu, (v * 3u) & 0x3F7F3F7Fu, (v * 5u) & 0x3F7F3F7Fu, (v * 7u) & 0x3F7F3F7Fu};
    const bf16x8 ab = __builtin_bit_cast(bf16x8, bits);
    const i32x4 a8 = __builtin_bit_cast(i32x4, bits);
    const long a4 = (long)bits[0] | ((long)bits[1] << 32);
    constexpr int NC = 8;  // independent chains: enough to cover the MFMA latency
    f32x4 acc[NC];
    i32x4 iacc[NC];
#pragma unroll
    for (int j = 0; j < NC; j++) {
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        iacc[j] = i32x4{0, 0, 0, 0};
    }
    float dw = __uint_as_float(0x3F800000u | (v & 0xFFFu));
    f32x4 dx = f32x4{1.f, 1.5f, 2.f, 2.5f};
    // modes 3 and 4: each chain its own B operand, and an A operand that
    // changes every trip (one XOR a trip for all chains), so the products
    // from a zero accumulator are neither hoisted out of the loop nor merged
    bf16x8 bb[NC];
    long b8[NC];
#pragma unroll
    for (int j = 0; j < NC; j++) {
        bb[j] = __builtin_bit_cast(bf16x8, bits ^ (uint32_t)(0x00010001u * (j + 1)));
        b8[j] = a4 ^ (long)(0x0101010101010101ll * (j + 1));
    }
    // modes 5-7: 32 fp8 codes (or 32 fp4 codes in the low four words) per
    // lane, without the E4M3 NaN pattern; E8M0 scales near 1
    const uint32_t m8 = 0x3B3B3B3Bu;
    const i32x8 q8 = i32x8{(int)(v & m8), (int)((v * 3u) & m8), (int)((v * 5u) & m8), (int)((v * 7u) & m8),
                           (int)((v * 9u) & m8), (int)((v * 11u) & m8), (int)((v * 13u) & m8), (int)((v * 15u) & m8)};
    const int sa = 125 + (int)(v & 3u), sb = 126 + (int)((v >> 2) & 1u);
    for (int it = 0; it < iters; it++) {
        const long a4t = a4 ^ (long)it;
        const bf16x8 abt = __builtin_bit_cast(bf16x8, bits ^ (uint32_t)(it & 0x003F003F));
#pragma unroll
        for (int j = 0; j < NC; j++) {
            if constexpr (MODE == 0) {
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, ab, acc[j], 0, 0, 0);
            } else if constexpr (MODE == 1) {
                iacc[j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a4, a4, iacc[j], 0, 0, 0);
            } else if constexpr (MODE == 2) {
                iacc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a8, a8, iacc[j], 0, 0, 0);
            } else if constexpr (MODE == 3) {
                // operands differ per trip (one XOR a trip), so the product
                // from a zero accumulator cannot be hoisted out of the loop
                const i32x4 t = __builtin_amdgcn_mfma_i32_16x16x32_i8(a4t, b8[j], i32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; e++)
                    acc[j][e] = __builtin_fmaf(dw * dx[e], (float)t[e], acc[j][e]);
            } else if constexpr (MODE == 5) {
                acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q8, q8, acc[j], 0, 4, 0, sa, 0, sb);
            } else if constexpr (MODE == 6) {
                acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q8, q8, acc[j], 4, 4, 0, sa, 0, sb);
            } else if constexpr (MODE == 7) {
                acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q8, q8, acc[j], 0, 0, 0, sa, 0, sb);
            } else {
                const f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abt, bb[j], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; e++)
                    acc[j][e] = __builtin_fmaf(dw, t[e], acc[j][e]);
            }
        }
        dw += 0.5f;  // the next block's scale
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NC; j++)
#pragma unroll
        for (int e = 0; e < 4; e++)
            s += acc[j][e] + (float)iacc[j][e];
    if ((threadIdx.x & 63) == 0)
        sink[blockIdx.x * 8 + (threadIdx.x >> 6)] = __float_as_uint(s);
}

hipError_t launch_mfma_rate(int mode, int iters, uint32_t *sink, hipStream_t st)
{
    const dim3 grid(512), block(512);
    switch (mode) {
    case 0: hipLaunchKernelGGL(mfma_rate_kernel<0>, grid, block, 0, st, iters, 12345u, sink); break;
    case 1: hipLaunchKernelGGL(mfma_rate_kernel<1>, grid, block, 0, st, iters, 12345u, sink); break;
    case 2: hipLaunchKernelGGL(mfma_rate_kernel<2>, grid, block, 0, st, iters, 12345u, sink); break;
    case 3: hipLaunchKernelGGL(mfma_rate_kernel<3>, grid, block, 0, st, iters, 12345u, sink); break;
    case 4: hipLaunchKernelGGL(mfma_rate_kernel<4>, grid, block, 0, st, iters, 12345u, sink); break;
    case 5: hipLaunchKernelGGL(mfma_rate_kernel<5>, grid, block, 0, st, iters, 12345u, sink); break;
    case 6: hipLaunchKernelGGL(mfma_rate_kernel<6>, grid, block, 0, st, iters, 12345u, sink); break;
    default: hipLaunchKernelGGL(mfma_rate_kernel<7>, grid, block, 0, st, iters, 12345u, sink); break;
    }
    return hipGetLastError();
}

}  // namespace qg
