// Large-batch tier, bf16 math: the kernel instantiations for 128- and
// 256-row tiles.  fp32-faithful math has its own translation unit
// (tiled_fp32.hip) so the two compile in parallel.
#include "tiled.h"

namespace qg {

// fp32 activations rounded to bf16 once per call, 8 per thread.
__global__ __launch_bounds__(256) void x_to_bf16_kernel(const f32x4 *x, u32x4 *xb, int64_t n8)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8)
        return;
    const f32x4 v0 = x[2 * i], v1 = x[2 * i + 1];
    bf16x8 h;
#pragma unroll
    for (int e = 0; e < 4; e++) {
        h[e] = (__bf16)v0[e];
        h[4 + e] = (__bf16)v1[e];
    }
    xb[i] = __builtin_bit_cast(u32x4, h);
}

hipError_t launch_x_to_bf16(const float *x, void *xb, int64_t n, hipStream_t st)
{
    const int64_t n8 = n / 8;
    if (n8 > 0)
        hipLaunchKernelGGL(x_to_bf16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                           (const f32x4 *)x, (u32x4 *)xb, n8);
    return hipGetLastError();
}

hipError_t launch_tiled(const Problem &p, const KArgs &a, const TiCfg &c, hipStream_t st)
{
    if (p.math == QGEMM_MATH_FP32)
        return launch_tiled_fp32(p, a, c, st);
    if (c.NW == 4)
        return launch_tiled_w4(p, a, c, st);
    return launch_tiled_math<false>(p, a, &c, nullptr, c.BM, 0, st);
}

hipError_t launch_grouped(const Problem &p, const KArgs &a, const Groups &g, int BM, int64_t tiles,
                          hipStream_t st)
{
    if (p.math == QGEMM_MATH_FP32)
        return launch_grouped_fp32(p, a, g, BM, tiles, st);
    return launch_tiled_math<false>(p, a, nullptr, &g, BM, tiles, st);
}

}  // namespace qg
