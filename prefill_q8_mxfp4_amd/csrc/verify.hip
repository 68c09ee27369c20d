// Verify kernel, fp32-faithful math (three exact bf16 terms per fp32
// activation): host-side dispatch and instantiations (the kernel is in
// verify.h; the bf16-math instantiations are in verify_bf16.hip, compiled
// in parallel).
#include "verify.h"
#include "verify_launch.h"

namespace qg {

int verify_mb(int64_t B) { return (int)((B + 15) / 16); }

hipError_t launch_verify(const Problem &p, const KArgs &a, const StCfg &c, const SkinnyWs &ws, int nterm,
                         hipStream_t st)
{
    if (a.B <= 16 || a.B > VF_MAX_B || a.K % slab_k(p.fmt) != 0 || (nterm != 1 && nterm != 3) ||
        (nterm == 3 && p.act != QGEMM_F32))
        return hipErrorInvalidValue;
    if (nterm == 1)
        return launch_verify_bf16(p, a, c, ws, st);
    switch (p.fmt) {
    case FMT_Q8: launch_vf<FMT_Q8, 3, ACT_F32>(p, a, c, ws, st); break;
    case FMT_MX: launch_vf<FMT_MX, 3, ACT_F32>(p, a, c, ws, st); break;
    case FMT_FP8: launch_vf<FMT_FP8, 3, ACT_F32>(p, a, c, ws, st); break;
    default: launch_vf<FMT_NV, 3, ACT_F32>(p, a, c, ws, st); break;
    }
    return hipGetLastError();
}

}  // namespace qg
