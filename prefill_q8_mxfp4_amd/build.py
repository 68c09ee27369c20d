"""Build libqgemm.so (HIP, gfx950) in-tree with hipcc.

Each tier is its own translation unit, compiled in parallel, then linked:

    python -m prefill_q8_mxfp4_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqgemm.so")
# the same kernels with the host side built to honour the debug-only
# environment overrides (QGEMM_DEBUG_KNOBS in api.hip); for tests
LIB_DEBUG = os.path.join(HERE, "libqgemm_debug.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
UNITS = ("api.hip", "skinny.hip", "stream.hip", "tiled.hip", "tiled_w4.hip", "tiled_fp32.hip", "dequant.hip",
         "readbw.hip", "gemv.hip", "mfma_rate.hip", "moe.hip", "verify.hip",
         "verify_bf16.hip")
HEADERS = ("common.h", "layout.h", "tiled.h", "verify.h", "verify_launch.h")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
    # packed fp32 VALU ops stay off: scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return ([os.path.join(CSRC, f) for f in UNITS + HEADERS]
            + [os.path.join(ROOT, "include", "qgemm.h")])


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = [ln for ln in (res.stdout + res.stderr).splitlines()
             if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        sys.stderr.write("\n".join(noise) + "\n")
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))
    if verbose and noise:
        print("\n".join(noise))


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(OBJ, exist_ok=True)
    objs = [os.path.join(OBJ, u.replace(".hip", ".o")) for u in UNITS]
    cmds = [[HIPCC] + FLAGS + list(extra) + ["-c", os.path.join(CSRC, u), "-o", o]
            for u, o in zip(UNITS, objs)]
    dbg_obj = os.path.join(OBJ, "api_debug.o")
    cmds.append([HIPCC] + FLAGS + list(extra) + ["-DQGEMM_DEBUG_KNOBS", "-c",
                                                 os.path.join(CSRC, "api.hip"), "-o", dbg_obj])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    for lib, parts in ((LIB, objs), (LIB_DEBUG, [dbg_obj] + objs[1:])):
        tmp = lib + ".tmp%d" % os.getpid()
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + parts + ["-o", tmp], verbose)
        os.replace(tmp, lib)
    return LIB


def is_stale() -> bool:
    if not (os.path.exists(LIB) and os.path.exists(LIB_DEBUG)):
        return True
    t = min(os.path.getmtime(LIB), os.path.getmtime(LIB_DEBUG))
    return any(os.path.getmtime(s) > t for s in sources())


if __name__ == "__main__":
    print(build(verbose=True))
