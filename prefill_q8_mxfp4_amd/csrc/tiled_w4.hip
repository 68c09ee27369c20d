// Large-batch tier, bf16 math, plain GEMM: the 4-wave instantiations (one
// wave per SIMD, each owning 128 x 128 outputs of a 256 x 256 tile, or
// 64 x 128 of a 128 x 256 tile), in a translation unit of their own so they
// compile beside the 8-wave ones.
#include "tiled.h"

namespace qg {

hipError_t launch_tiled_w4(const Problem &p, const KArgs &a, const TiCfg &c, hipStream_t st)
{
    return launch_tiled_math<false, 4>(p, a, &c, nullptr, c.BM, 0, st);
}

}  // namespace qg
