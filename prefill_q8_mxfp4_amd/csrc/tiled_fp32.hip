// Large-batch tier, fp32-faithful math: the kernel instantiations for 64-
// and 96-row tiles (three exact bf16 activation terms, exact weight codes,
// block scales applied to each block's fp32 partial).
#include "tiled.h"

namespace qg {

hipError_t launch_tiled_fp32(const Problem &p, const KArgs &a, const TiCfg &c, hipStream_t st)
{
    return launch_tiled_math<true>(p, a, &c, nullptr, c.BM, 0, st);
}

hipError_t launch_grouped_fp32(const Problem &p, const KArgs &a, const Groups &g, int BM, int64_t tiles,
                               hipStream_t st)
{
    (void)BM;  // always 64 rows
    return launch_tiled_math<true>(p, a, nullptr, &g, 64, tiles, st);
}

}  // namespace qg
