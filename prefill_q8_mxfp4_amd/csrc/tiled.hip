// Large-batch tier, bf16 math: the kernel instantiations for 128- and
// 256-row tiles.  fp32-faithful math has its own translation unit
// (tiled_fp32.hip) so the two compile in parallel.
#include "tiled.h"

namespace qg {

hipError_t launch_tiled(const Problem &p, const KArgs &a, const TiCfg &c, hipStream_t st)
{
    if (p.math == QGEMM_MATH_FP32)
        return launch_tiled_fp32(p, a, c, st);
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
