"""Seeded synthetic inputs for the block-quantized batched GEMM.

This module is the only code shared by the CPU oracle side and the HIP side.
It produces *inputs*: random weights and activations, and the quantized
logical arrays (integer codes plus block scales) that the three weight
formats store.  It contains no decoder and no GEMM arithmetic: turning codes
back into values and contracting them is done independently by ``oracle/``
and by the HIP library.

Random numbers
--------------
SplitMix64, used in counter form: element ``i`` of stream ``(seed, sid)`` is
``mix64(base + (i + 1) * GOLDEN)`` with ``base = mix64(mix64(seed) + sid)``
and ``mix64`` the SplitMix64 output finaliser (Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014).  Because
every element is a pure function of its index, tensors are generated in row
chunks and any sub-block can be regenerated on its own.

Uniforms are ``((v >> 11) + 1) * 2**-53`` in (0, 1].  Normals use the
Box-Muller transform on consecutive pairs ``(u1, u2)``:
``r = sqrt(-2 ln u1)``, ``z0 = r cos(2 pi u2)``, ``z1 = r sin(2 pi u2)``.

Quantizers (input recipes)
--------------------------
The pages name the three block formats but give no quantizer, so these follow
the plainest reading of the workloads:

* Q8_0 (32-wide blocks): ``d32 = amax / 127`` in fp32, ``q = clamp(round
  half away from zero (w / d32), -127, 127)``, stored scale ``d = fp16(d32)``
  (round to nearest even).  An all-zero block stores d = 0, q = 0.
* MXFP4 (32-wide blocks, OCP MX rule): ``e = clamp(floor(log2 amax) - 2,
  -127, 127)`` stored as the E8M0 byte ``e + 127``; elements are
  ``E2M1_rne_sat(w / 2**e)``.  An all-zero block stores byte 0 and codes 0.
* NVFP4 (16-wide blocks): per-tensor fp32 ``g = amax_tensor / (448 * 6)``;
  block scale ``s = E4M3_rne(amax_block / (6 g))``; elements
  ``E2M1_rne_sat(w / (g s))``; a zero scale stores zero codes.
* FP8 (E4M3 weights, 128-wide blocks along K, the last one possibly
  shorter): block scale ``s = amax_block / 448`` in fp32; elements
  ``E4M3_rne(clamp(w / s, -448, 448))``; an all-zero block stores s = 0 and
  zero codes.

E2M1 codes are 4-bit sign-magnitude: bit 3 is the sign, bits 0-2 index the
magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Rounding to nearest with ties to the
even (mantissa-0) neighbour is done by comparing against the midpoints.
"""

from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# stream ids: one per tensor role, so every tensor has its own sequence
SID_W = 1
SID_X = 2
SID_OUTLIER = 3
SID_W_UP = 4
SID_ROUTE = 5
SID_EXPERT0 = 1000  # expert e's weights use stream SID_EXPERT0 + 2e (gate) and + 2e + 1 (up)

QK8_0 = 32
QK_MX = 32
QK_NV = 16
QK_FP8 = 128  # weights per FP8 block scale along K

FORMATS = ("q8_0", "mxfp4", "nvfp4", "fp8")


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def _scalar_mix64(v: int) -> int:
    return int(_mix64(np.array([v & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))[0])


def stream_base(seed: int, sid: int) -> np.uint64:
    return np.uint64((_scalar_mix64(seed) + sid) & 0xFFFFFFFFFFFFFFFF)


def raw_u64(seed: int, sid: int, start: int, count: int) -> np.ndarray:
    """Elements ``start .. start+count-1`` of stream (seed, sid) as uint64."""
    base = stream_base(seed, sid)
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(base + idx * GOLDEN)


def uniform(seed: int, sid: int, start: int, count: int) -> np.ndarray:
    v = raw_u64(seed, sid, start, count)
    return ((v >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * (2.0 ** -53)


def normal(seed: int, sid: int, start: int, count: int) -> np.ndarray:
    """Standard normals ``start .. start+count-1`` (float64)."""
    p0 = start // 2
    p1 = (start + count + 1) // 2
    u = uniform(seed, sid, 2 * p0, 2 * (p1 - p0))
    u1 = u[0::2]
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    t = 2.0 * np.pi * u2
    z = np.empty(2 * (p1 - p0), dtype=np.float64)
    z[0::2] = r * np.cos(t)
    z[1::2] = r * np.sin(t)
    off = start - 2 * p0
    return z[off:off + count]


def normal_f32(seed, sid, rows, cols, std=1.0, row0=0):
    """fp32 matrix ``rows x cols`` of N(0, std^2), element (r, c) at index (row0+r)*cols+c."""
    z = normal(seed, sid, row0 * cols, rows * cols)
    return (z * std).astype(np.float32).reshape(rows, cols)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- quantizers

def _round_half_away(v: np.ndarray) -> np.ndarray:
    v64 = v.astype(np.float64)
    return np.sign(v64) * np.floor(np.abs(v64) + 0.5)


def quantize_q8_0(w: np.ndarray):
    """w fp32 [N][K] -> (qs int8 [N][K], d fp16 bits uint16 [N][K/32])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    if k % QK8_0:
        raise ValueError("K must be a multiple of 32")
    blk = w.reshape(n, k // QK8_0, QK8_0)
    amax = np.max(np.abs(blk), axis=2)
    d32 = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(d32 > 0, d32, np.float32(1.0)).astype(np.float32)
    r = (blk / safe[:, :, None]).astype(np.float32)
    q = np.clip(_round_half_away(r), -127, 127)
    q = np.where(d32[:, :, None] > 0, q, 0).astype(np.int8)
    d = d32.astype(np.float16).view(np.uint16)
    return q.reshape(n, k), d


def _e2m1_encode(r: np.ndarray) -> np.ndarray:
    """Round real values (already divided by the block scale) to E2M1 codes,
    nearest with ties to even mantissa, saturating at +-6."""
    a = np.abs(r)
    mag = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
           + (a > 2.5) + (a >= 3.5) + (a > 5.0))
    sign = np.signbit(r).astype(np.uint8) << 3
    return (sign | mag.astype(np.uint8)).astype(np.uint8)


def quantize_mxfp4(w: np.ndarray):
    """w fp32 [N][K] -> (codes uint8 [N][K] in 0..15, e8m0 uint8 [N][K/32])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    if k % QK_MX:
        raise ValueError("K must be a multiple of 32")
    blk = w.reshape(n, k // QK_MX, QK_MX).astype(np.float64)
    amax = np.max(np.abs(blk), axis=2)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.clip(ex.astype(np.int64) - 1 - 2, -127, 127)
    r = np.ldexp(blk, (-e)[:, :, None])
    codes = _e2m1_encode(r)
    zero = amax == 0
    codes[zero] = 0
    ebyte = (e + 127).astype(np.uint8)
    ebyte[zero] = 0
    return codes.reshape(n, k), ebyte


def _e4m3_rne(v: np.ndarray):
    """fp32 -> (E4M3 bytes, their fp32 values), via torch's float8_e4m3fn cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    f8 = t.to(torch.float8_e4m3fn)
    return f8.view(torch.uint8).numpy().copy(), f8.to(torch.float32).numpy()


def quantize_nvfp4(w: np.ndarray):
    """w fp32 [N][K] -> (codes uint8 [N][K], e4m3 uint8 [N][K/16], g float32)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    if k % QK_NV:
        raise ValueError("K must be a multiple of 16")
    amax_t = np.float32(np.max(np.abs(w))) if w.size else np.float32(0)
    g = np.float32(amax_t / np.float32(448.0 * 6.0))
    blk = w.reshape(n, k // QK_NV, QK_NV)
    amax_b = np.max(np.abs(blk), axis=2)
    if g > 0:
        sb = (amax_b / (np.float32(6.0) * g)).astype(np.float32)
    else:
        sb = np.zeros_like(amax_b)
    sbyte, sval = _e4m3_rne(sb)
    denom = (g * sval).astype(np.float32)
    safe = np.where(denom > 0, denom, np.float32(1.0)).astype(np.float32)
    r = (blk / safe[:, :, None]).astype(np.float32)
    codes = _e2m1_encode(r)
    codes[denom == 0] = 0
    return codes.reshape(n, k), sbyte, np.float32(g)


def quantize_fp8(w: np.ndarray):
    """w fp32 [N][K] -> (e4m3 uint8 [N][K], s float32 [N][ceil(K/128)])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    nb = -(-k // QK_FP8)
    wp = np.zeros((n, nb * QK_FP8), dtype=np.float32)
    wp[:, :k] = w
    blk = wp.reshape(n, nb, QK_FP8)
    amax = np.max(np.abs(blk), axis=2)
    s = (amax / np.float32(448.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    r = np.clip((blk / safe[:, :, None]).astype(np.float32), -448.0, 448.0).astype(np.float32)
    codes, _ = _e4m3_rne(r)
    codes = codes.reshape(n, nb, QK_FP8)
    codes[s == 0] = 0
    return np.ascontiguousarray(codes.reshape(n, nb * QK_FP8)[:, :k]), s


def quantize(fmt: str, w: np.ndarray) -> dict:
    """Quantize fp32 weights into the logical arrays of ``fmt``."""
    if fmt == "q8_0":
        q, d = quantize_q8_0(w)
        return {"fmt": fmt, "codes": q, "scales": d, "g": None}
    if fmt == "mxfp4":
        c, e = quantize_mxfp4(w)
        return {"fmt": fmt, "codes": c, "scales": e, "g": None}
    if fmt == "nvfp4":
        c, s, g = quantize_nvfp4(w)
        return {"fmt": fmt, "codes": c, "scales": s, "g": np.array([g], dtype=np.float32)}
    if fmt == "fp8":
        c, s = quantize_fp8(w)
        return {"fmt": fmt, "codes": c, "scales": s, "g": None}
    raise ValueError(fmt)


def concat_rows(parts: list) -> dict:
    """Stack quantized tensors along N (e.g. gate on top of up); NVFP4 tensor
    scales are kept one per part."""
    fmt = parts[0]["fmt"]
    out = {
        "fmt": fmt,
        "codes": np.concatenate([p["codes"] for p in parts], axis=0),
        "scales": np.concatenate([p["scales"] for p in parts], axis=0),
        "g": None,
    }
    if fmt == "nvfp4":
        out["g"] = np.concatenate([p["g"] for p in parts]).astype(np.float32)
    return out


# ------------------------------------------------------------------ workloads

def gen_weights(fmt, n, k, seed=0, sid=SID_W, std=0.02, outlier_p=0.0,
                outlier_mult=20.0, chunk_rows=2048):
    """fp32 N(0, std^2) weights (optionally with a Bernoulli(outlier_p) mask of
    weights multiplied by outlier_mult) quantized to ``fmt``, built in row
    chunks to bound memory."""
    codes_parts, scale_parts = [], []
    amax_t = np.float32(0)
    w_chunks = []
    for r0 in range(0, n, chunk_rows):
        rows = min(chunk_rows, n - r0)
        w = normal_f32(seed, sid, rows, k, std, row0=r0)
        if outlier_p > 0:
            u = uniform(seed, sid + 100, r0 * k, rows * k).reshape(rows, k)
            w = np.where(u < outlier_p, w * np.float32(outlier_mult), w).astype(np.float32)
        if fmt == "nvfp4":
            # the tensor scale needs the global amax before any block is coded
            amax_t = max(amax_t, np.float32(np.max(np.abs(w))))
            w_chunks.append(w)
            continue
        qd = quantize(fmt, w)
        codes_parts.append(qd["codes"])
        scale_parts.append(qd["scales"])
    if fmt == "nvfp4":
        w = np.concatenate(w_chunks, axis=0)
        del w_chunks
        c, s, g = quantize_nvfp4(w)
        return {"fmt": fmt, "codes": c, "scales": s, "g": np.array([g], dtype=np.float32)}
    return {"fmt": fmt, "codes": np.concatenate(codes_parts, axis=0),
            "scales": np.concatenate(scale_parts, axis=0), "g": None}


def gen_x_f32(b, k, seed=0, sid=SID_X):
    return normal_f32(seed, sid, b, k, 1.0)


def gen_x_bf16(b, k, seed=0, sid=SID_X):
    """bf16 activations ~N(0,1): fp32 normals rounded to nearest-even bf16 (bits)."""
    return f32_to_bf16_bits(normal_f32(seed, sid, b, k, 1.0))


# The workloads (all seed 0), named by format, role and N x K; Bs are the
# batch widths each is checked and measured at.
CONFIGS = {
    # the small Q8_0 parity case (crosses the old 64-row limit)
    "q8_0_256x512": dict(fmt="q8_0", act="f32", N=256, K=512, Bs=(70,), out="f32", epi="none",
                         math="fp32"),
    # Q8_0 attention projection over the verify widths
    "q8_0_5120x5120": dict(fmt="q8_0", act="f32", N=5120, K=5120,
                           Bs=(1, 4, 8, 16, 64, 65, 70, 76, 256), out="f32", epi="none", math="fp32"),
    # Q8_0 FFN gate/up prefill chunk, weights with 0.1 % outliers x20
    "q8_0_ffn_17408x5120": dict(fmt="q8_0", act="f32", N=17408, K=5120, Bs=(2048,), out="f32",
                                epi="none", math="bf16", outlier_p=0.001),
    # MXFP4 FFN down projection
    "mxfp4_down_5120x17408": dict(fmt="mxfp4", act="bf16", N=5120, K=17408, Bs=(1, 16, 256, 2048),
                                  out="f32", epi="none", math="bf16"),
    # NVFP4 fused gate+up (SwiGLU), two 17408 x 5120 halves
    "nvfp4_gate_up_34816x5120": dict(fmt="nvfp4", act="bf16", N=2 * 17408, K=5120, Bs=(2048,),
                                     out="bf16", epi="swiglu", math="bf16"),
    # the FP8-weight (W8A16) attention-projection shape of the follow-on format
    "fp8_5120x5120": dict(fmt="fp8", act="bf16", N=5120, K=5120, Bs=(1, 16, 256, 2048), out="f32",
                          epi="none", math="bf16"),
}


def gen_config_weights(name: str, seed: int = 0) -> dict:
    c = CONFIGS[name]
    if c["epi"] == "swiglu":
        nh = c["N"] // 2
        gate = gen_weights(c["fmt"], nh, c["K"], seed=seed, sid=SID_W)
        up = gen_weights(c["fmt"], nh, c["K"], seed=seed, sid=SID_W_UP)
        return concat_rows([gate, up])
    return gen_weights(c["fmt"], c["N"], c["K"], seed=seed, sid=SID_W,
                       outlier_p=c.get("outlier_p", 0.0))


def gen_config_x(name: str, b: int, seed: int = 0) -> np.ndarray:
    c = CONFIGS[name]
    return gen_x_f32(b, c["K"], seed) if c["act"] == "f32" else gen_x_bf16(b, c["K"], seed)


# ------------------------------------------------------------ routed experts

def gen_routing(tokens: int, topk: int, experts: int, seed: int = 0):
    """Top-k routing of `tokens` tokens over `experts` experts, each token to
    `topk` distinct experts drawn uniformly (the experts with the k smallest
    of its per-expert uniform keys).  Returns (token index of each routed
    row, rows sorted by expert, stable in token order) and the expert offsets
    [E + 1] (rows of expert e are offsets[e] .. offsets[e+1]-1)."""
    keys = uniform(seed, SID_ROUTE, 0, tokens * experts).reshape(tokens, experts)
    choice = np.argsort(keys, axis=1, kind="stable")[:, :topk]          # [T][topk]
    tok = np.repeat(np.arange(tokens, dtype=np.int64), topk)
    exp = choice.reshape(-1)
    order = np.lexsort((tok, exp))                                       # by expert, then token
    counts = np.bincount(exp, minlength=experts)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return tok[order], offsets


def gen_expert_weights(fmt: str, n: int, k: int, e: int, seed: int = 0, swiglu: bool = False) -> dict:
    """Weights of expert e: N(0, 0.02) from the expert's own streams; with
    swiglu, n = 2*nh rows (gate on top of up), each half its own tensor."""
    if swiglu:
        nh = n // 2
        gate = gen_weights(fmt, nh, k, seed=seed, sid=SID_EXPERT0 + 2 * e)
        up = gen_weights(fmt, nh, k, seed=seed, sid=SID_EXPERT0 + 2 * e + 1)
        return concat_rows([gate, up])
    return gen_weights(fmt, n, k, seed=seed, sid=SID_EXPERT0 + 2 * e)
