// Device decode of a packed weight buffer to fp32, with the same decoders
// the GEMM kernels use.
#include "common.h"

namespace qg {

// ============================================================ dequantize
// One thread per (row, 8 consecutive k): fp32 decode with the same decoders.
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(KArgs a, float *out)
{
    constexpr int KS = slab_k(FMT);
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t groups = (int64_t)a.K / 8;
    if (idx >= (int64_t)a.N * groups)
        return;
    const int n = (int)(idx / groups);
    const int k0 = (int)(idx % groups) * 8;
    const int s = k0 / KS, u = (k0 % KS) / 32, g = (k0 % 32) / 8;
    const int rt = n / 16, r = n % 16;
    const int L = g * 16 + r;
    const uint8_t *chunk = a.w + (((int64_t)rt * a.S + s) << 10) + (L << 4);
    const uint8_t *sp = slab_scales<FMT>(a, rt, r, s);  // this row's scales of slab s
    float v[8];
    if constexpr (FMT == FMT_Q8) {
        const float d = fp16_bits_to_f32(((const uint16_t *)sp)[u]);
#pragma unroll
        for (int j = 0; j < 8; j++)
            v[j] = (float)(int8_t)chunk[8 * u + j] * d;
    } else if constexpr (FMT == FMT_FP8) {
        const float d = *(const float *)sp;  // the slab's block scale
#pragma unroll
        for (int j = 0; j < 8; j++)
            v[j] = e4m3_to_f32(chunk[8 * u + j]) * d;
    } else {
        const uint32_t codes = *(const uint32_t *)(chunk + 4 * u);
        float sc;
        if constexpr (FMT == FMT_MX)
            sc = e8m0_to_f32(sp[u]);
        else
            sc = e4m3_to_f32(sp[(k0 % KS) / 16]);
        float gs = 1.f;
        if constexpr (FMT == FMT_NV)
            gs = tensor_scale(a, n);
#pragma unroll
        for (int j = 0; j < 8; j++) {
            float p = e2m1_to_f32((codes >> (4 * j)) & 0xFu) * sc;
            v[j] = FMT == FMT_NV ? gs * p : p;
        }
    }
    float *o = out + (int64_t)n * a.K + k0;
    *(f32x4 *)o = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4 *)(o + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

hipError_t launch_dequant(int fmt, const KArgs &a, float *out, hipStream_t st)
{
    const int64_t threads = (int64_t)a.N * (a.K / 8);
    const dim3 grid((unsigned)((threads + 255) / 256));
    switch (fmt) {
    case FMT_Q8: hipLaunchKernelGGL(dequant_kernel<FMT_Q8>, grid, dim3(256), 0, st, a, out); break;
    case FMT_MX: hipLaunchKernelGGL(dequant_kernel<FMT_MX>, grid, dim3(256), 0, st, a, out); break;
    case FMT_FP8: hipLaunchKernelGGL(dequant_kernel<FMT_FP8>, grid, dim3(256), 0, st, a, out); break;
    default: hipLaunchKernelGGL(dequant_kernel<FMT_NV>, grid, dim3(256), 0, st, a, out); break;
    }
    return hipGetLastError();
}

}  // namespace qg
