// Launchers of the verify kernel's instantiations, shared by the
// translation units that instantiate it (verify.hip, verify_bf16.hip).
#pragma once

#include "verify.h"

namespace qg {

template <int FMT, int MB, int NTA, int ACT>
static void launch_vm(const Problem &p, const KArgs &a, const StCfg &c, const SkinnyWs &ws, hipStream_t st)
{
    if (p.out == QGEMM_F32)
        hipLaunchKernelGGL((verify_kernel<FMT, MB, OUT_F32, NTA, ACT>), dim3((unsigned)c.grid), dim3(512), 0, st,
                           a, ws, c.ngroups, c.Nh);
    else
        hipLaunchKernelGGL((verify_kernel<FMT, MB, OUT_BF16, NTA, ACT>), dim3((unsigned)c.grid), dim3(512), 0, st,
                           a, ws, c.ngroups, c.Nh);
}

template <int FMT, int NTA, int ACT>
static void launch_vf(const Problem &p, const KArgs &a, const StCfg &c, const SkinnyWs &ws, hipStream_t st)
{
    switch (verify_mb(a.B)) {
    case 2: launch_vm<FMT, 2, NTA, ACT>(p, a, c, ws, st); break;
    case 3: launch_vm<FMT, 3, NTA, ACT>(p, a, c, ws, st); break;
    case 4: launch_vm<FMT, 4, NTA, ACT>(p, a, c, ws, st); break;
    default: launch_vm<FMT, 5, NTA, ACT>(p, a, c, ws, st); break;
    }
}

}  // namespace qg
