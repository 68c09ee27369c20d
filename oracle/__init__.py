"""CPU oracle (fp64) for the block-quantized-weight batched GEMM.

TEST INFRASTRUCTURE ONLY: it is loaded by ``tests/``, by the smoke check and
by the benchmark's CPU-baseline leg, never by the library.  It reads the
logical arrays produced by ``synth`` (one code per byte, scales in their own
arrays) and shares no code with the HIP library.

What it computes (plain definitions, see qgemm_oracle.c for the decoders):

* ``y[b][n] = g(n) * sum_k x[b][k] * w[n][k]`` in fp64, k increasing, with
  ``w`` decoded per format: Q8_0 ``d*q``; MXFP4 ``E2M1(c) * 2**(e-127)``;
  NVFP4 ``E2M1(c) * E4M3(s)`` and ``g(n)`` the fp32 tensor scale of row n's
  tensor, applied after the sum (Atlas issue "[job] Qwen3.8-27B on Strix
  Halo: prefill 2.4x gap + DP4A verify tiers for K=5..9", section
  "Kernel-level root cause of the gfx1151 NVFP4 prefill gap", Fix); FP8
  ``s * E4M3(c)`` with one fp32 scale per row and 128-wide K block (the same
  issue's FP8-weight projection GEMM; the pages do not fix the block width, 128 is a reading).
* fused gate+up: ``out[b][j] = SiLU(G) * U`` with G from row j and U from row
  Nh + j (Atlas issue, "What's the job?" asks for the fused gate+up
  dual-accumulator GEMM; the workload names SiLU(gate)*up).

Every function here is pinned by ``tests/test_oracle_pins.py`` against
library decoders (numpy float16, torch float8, transformers' FP4 table),
closed forms, exact rational brute force and invariants.
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qgemm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FMT = {"q8_0": 0, "mxfp4": 1, "nvfp4": 2, "fp8": 3}
ACT = {"f32": 0, "bf16": 1}

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, OpenMP, no fp contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        d, i64, vp, u8, u16, i32 = (ctypes.c_double, ctypes.c_int64, ctypes.c_void_p,
                                    ctypes.c_uint8, ctypes.c_uint16, ctypes.c_int)
        for name, arg in (("oracle_fp16", u16), ("oracle_bf16", u16), ("oracle_e2m1", u8),
                          ("oracle_e8m0", u8), ("oracle_e4m3", u8), ("oracle_silu", d)):
            f = getattr(lib, name)
            f.restype = d
            f.argtypes = [arg]
        lib.oracle_threads.restype = i32
        lib.oracle_threads.argtypes = []
        lib.oracle_set_threads.restype = None
        lib.oracle_set_threads.argtypes = [i32]
        lib.oracle_dequant.restype = None
        lib.oracle_dequant.argtypes = [i32, vp, vp, vp, i64, i32, i64, i64, vp]
        lib.oracle_gemm.restype = None
        lib.oracle_gemm.argtypes = [i32, vp, vp, vp, i64, i32, vp, i64, i64, i64, vp]
        lib.oracle_swiglu.restype = None
        lib.oracle_swiglu.argtypes = [i32, vp, vp, vp, i64, i32, vp, i64, i64, i64, vp]
        for name in ("oracle_gemm_at", "oracle_swiglu_at", "oracle_gemm_abs_at"):
            f = getattr(lib, name)
            f.restype = None
            f.argtypes = [i32, vp, vp, vp, i64, i32, vp, i64, i64, vp, vp, i64, vp]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _prep(w: dict):
    codes = np.ascontiguousarray(w["codes"])
    scales = np.ascontiguousarray(w["scales"])
    g = w.get("g")
    g = None if g is None else np.ascontiguousarray(g, dtype=np.float32)
    nt = 0 if g is None else len(g)
    return FMT[w["fmt"]], codes, scales, g, nt


def _act(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return ACT["f32"], x
    if x.dtype == np.uint16:
        return ACT["bf16"], x
    raise TypeError("activations must be float32 or bf16 bits (uint16)")


# ---- scalar decoders (exposed for the pins) ----

def fp16(h):
    return _load().oracle_fp16(int(h))


def bf16(h):
    return _load().oracle_bf16(int(h))


def e2m1(c):
    return _load().oracle_e2m1(int(c))


def e8m0(b):
    return _load().oracle_e8m0(int(b))


def e4m3(b):
    return _load().oracle_e4m3(int(b))


def threads() -> int:
    """Threads the oracle's parallel loops use."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Threads the oracle's parallel loops use from now on (timing only:
    every output is one sequential sum, whatever the thread count)."""
    _load().oracle_set_threads(int(n))


def silu(t):
    return _load().oracle_silu(float(t))


# ---- array entry points ----

def dequant(w: dict, apply_g: bool = False) -> np.ndarray:
    """Dense fp64 [N][K] decoded weights (times the tensor scale if apply_g)."""
    fmt, codes, scales, g, nt = _prep(w)
    n, k = codes.shape
    out = np.empty((n, k), dtype=np.float64)
    _load().oracle_dequant(fmt, _ptr(codes), _ptr(scales), _ptr(g), nt, int(apply_g), n, k,
                           _ptr(out))
    return out


def gemm(w: dict, x: np.ndarray) -> np.ndarray:
    """y[B][N] in fp64."""
    fmt, codes, scales, g, nt = _prep(w)
    a, x = _act(x)
    n, k = codes.shape
    b = x.shape[0]
    assert x.shape[1] == k
    y = np.empty((b, n), dtype=np.float64)
    _load().oracle_gemm(fmt, _ptr(codes), _ptr(scales), _ptr(g), nt, a, _ptr(x), b, n, k, _ptr(y))
    return y


def gemm_at(w: dict, x: np.ndarray, bidx, nidx) -> np.ndarray:
    """y[bidx[i]][nidx[i]] in fp64."""
    fmt, codes, scales, g, nt = _prep(w)
    a, x = _act(x)
    n, k = codes.shape
    bi = np.ascontiguousarray(bidx, dtype=np.int64)
    ni = np.ascontiguousarray(nidx, dtype=np.int64)
    assert bi.shape == ni.shape
    assert bi.size == 0 or (bi.max() < x.shape[0] and ni.max() < n and bi.min() >= 0
                            and ni.min() >= 0)
    y = np.empty(bi.size, dtype=np.float64)
    _load().oracle_gemm_at(fmt, _ptr(codes), _ptr(scales), _ptr(g), nt, a, _ptr(x), n, k,
                           _ptr(bi), _ptr(ni), bi.size, _ptr(y))
    return y


def gemm_abs_at(w: dict, x: np.ndarray, bidx, nidx) -> np.ndarray:
    """M[bidx[i]][nidx[i]] = |g(n)| * sum_k |x[b][k]| * |w[n][k]| in fp64: the
    magnitude sum that bounds the rounding error of any fp summation order of
    y[b][n] (|computed - exact| <= gamma(n_adds, u) * M, see :func:`gamma`)."""
    fmt, codes, scales, g, nt = _prep(w)
    a, x = _act(x)
    n, k = codes.shape
    bi = np.ascontiguousarray(bidx, dtype=np.int64)
    ni = np.ascontiguousarray(nidx, dtype=np.int64)
    assert bi.shape == ni.shape
    assert bi.size == 0 or (bi.max() < x.shape[0] and ni.max() < n and bi.min() >= 0
                            and ni.min() >= 0)
    m = np.empty(bi.size, dtype=np.float64)
    _load().oracle_gemm_abs_at(fmt, _ptr(codes), _ptr(scales), _ptr(g), nt, a, _ptr(x), n, k,
                               _ptr(bi), _ptr(ni), bi.size, _ptr(m))
    return m


def gamma(n: int, u: float) -> float:
    """gamma_n = n u / (1 - n u): a sum of n + 1 terms computed with n
    roundings of relative size at most u, in any order, differs from the
    exact sum by at most gamma_n times the sum of the terms' magnitudes
    (the standard forward error bound of recursive summation)."""
    nu = n * u
    if nu >= 1.0:
        return math.inf
    return nu / (1.0 - nu)


def swiglu(w: dict, x: np.ndarray) -> np.ndarray:
    """out[B][N/2] = SiLU(gate) * up, fp64."""
    fmt, codes, scales, g, nt = _prep(w)
    a, x = _act(x)
    n, k = codes.shape
    assert n % 2 == 0
    b = x.shape[0]
    out = np.empty((b, n // 2), dtype=np.float64)
    _load().oracle_swiglu(fmt, _ptr(codes), _ptr(scales), _ptr(g), nt, a, _ptr(x), b, n, k,
                          _ptr(out))
    return out


def swiglu_at(w: dict, x: np.ndarray, bidx, jidx) -> np.ndarray:
    fmt, codes, scales, g, nt = _prep(w)
    a, x = _act(x)
    n, k = codes.shape
    bi = np.ascontiguousarray(bidx, dtype=np.int64)
    ji = np.ascontiguousarray(jidx, dtype=np.int64)
    assert bi.size == 0 or (bi.max() < x.shape[0] and ji.max() < n // 2)
    out = np.empty(bi.size, dtype=np.float64)
    _load().oracle_swiglu_at(fmt, _ptr(codes), _ptr(scales), _ptr(g), nt, a, _ptr(x), n, k,
                             _ptr(bi), _ptr(ji), bi.size, _ptr(out))
    return out


def gemm_grouped(ws: list, offsets, x: np.ndarray, swiglu_epi: bool = False) -> np.ndarray:
    """Routed experts (Atlas issue, "Per-32-K-step hot loop" table: the routed
    expert GEMMs reached through an expert pointer table): rows
    offsets[e] .. offsets[e+1]-1 of x use expert e's weights ws[e].  Each
    expert's rows are the plain GEMM (or fused gate+up) of that expert."""
    off = np.asarray(offsets, dtype=np.int64)
    n = ws[0]["codes"].shape[0]
    out = np.zeros((x.shape[0], n // 2 if swiglu_epi else n), dtype=np.float64)
    for e, w in enumerate(ws):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 > r0:
            out[r0:r1] = swiglu(w, x[r0:r1]) if swiglu_epi else gemm(w, x[r0:r1])
    return out


def rel_fro(y, ref) -> float:
    """||y - ref||_F / ||ref||_F in fp64.  A zero reference gives 0 when y is
    zero too and inf otherwise (a relative error is undefined there, so it
    must not pass any bound); NaN anywhere gives NaN (which fails every
    ``err <= tol``)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if y.shape != ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {ref.shape}")
    d = (y - ref).ravel()
    r = ref.ravel()
    if np.isnan(d).any() or np.isnan(r).any():
        return math.nan
    # both norms in units of the largest magnitude, so that squares of very
    # small or very large outputs neither underflow nor overflow
    s = max(float(np.max(np.abs(d), initial=0.0)), float(np.max(np.abs(r), initial=0.0)))
    if s == 0.0:
        return 0.0
    if math.isinf(s):
        return math.nan if np.isinf(r).any() else math.inf
    num = np.linalg.norm(d / s)
    den = np.linalg.norm(r / s)
    if den > 0:
        return float(num / den)
    return 0.0 if num == 0 else math.inf


def rel_fro_groups(y, ref, groups, ngroups: int) -> np.ndarray:
    """Per-group relative Frobenius error: element i belongs to group
    groups[i] (0 <= groups[i] < ngroups); result[g] is rel_fro over the
    elements of group g (an output tile, say), with rel_fro's conventions,
    and NaN for a group with no element."""
    y = np.asarray(y, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    gi = np.asarray(groups, dtype=np.int64).ravel()
    if not (y.shape == ref.shape == gi.shape):
        raise ValueError("y, ref and groups must have the same size")
    if gi.size and (gi.min() < 0 or gi.max() >= ngroups):
        raise ValueError("group index out of range")
    d = y - ref
    cnt = np.bincount(gi, minlength=ngroups)
    bad = np.bincount(gi, weights=(np.isnan(d) | np.isnan(ref)).astype(np.float64),
                      minlength=ngroups) > 0
    # per-group scale: the largest |d| or |ref| of the group (no under/overflow)
    s = np.zeros(ngroups)
    np.maximum.at(s, gi, np.where(np.isnan(d), 0.0, np.maximum(np.abs(d), np.abs(ref))))
    si = s[gi]
    safe = np.where((si > 0) & np.isfinite(si), si, 1.0)
    num = np.sqrt(np.bincount(gi, weights=np.where(np.isnan(d), 0.0, d / safe) ** 2,
                              minlength=ngroups))
    den = np.sqrt(np.bincount(gi, weights=np.where(np.isnan(ref), 0.0, ref / safe) ** 2,
                              minlength=ngroups))
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, math.inf, 0.0))
    out[np.isinf(s) & ~bad] = math.inf
    out[bad] = math.nan
    out[cnt == 0] = math.nan
    return out
