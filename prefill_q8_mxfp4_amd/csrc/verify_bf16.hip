// Verify kernel, bf16 math (bf16 activations as they are, fp32 ones rounded
// to bf16 once, nearest even, as every bf16-math kernel does): the
// instantiations (the kernel is in verify.h).
#include "verify_launch.h"

namespace qg {

template <int ACT>
static void launch_vb(const Problem &p, const KArgs &a, const StCfg &c, const SkinnyWs &ws, hipStream_t st)
{
    switch (p.fmt) {
    case FMT_Q8: launch_vf<FMT_Q8, 1, ACT>(p, a, c, ws, st); break;
    case FMT_MX: launch_vf<FMT_MX, 1, ACT>(p, a, c, ws, st); break;
    case FMT_FP8: launch_vf<FMT_FP8, 1, ACT>(p, a, c, ws, st); break;
    default: launch_vf<FMT_NV, 1, ACT>(p, a, c, ws, st); break;
    }
}

hipError_t launch_verify_bf16(const Problem &p, const KArgs &a, const StCfg &c, const SkinnyWs &ws, hipStream_t st)
{
    if (p.act == QGEMM_F32)
        launch_vb<ACT_F32>(p, a, c, ws, st);
    else
        launch_vb<ACT_BF16>(p, a, c, ws, st);
    return hipGetLastError();
}

}  // namespace qg
