"""Pins for the CPU oracle: every part of it is checked against something
other than itself (library decoders, facts the pages state, closed forms,
exact rational brute force, a library matmul, invariants).

CPU only.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")
FACTS = json.load(open(GOLDEN))


def _same(a: float, b: float) -> bool:
    """Bitwise-equal doubles (NaN == NaN, -0 != +0)."""
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return np.float64(a).view(np.uint64) == np.float64(b).view(np.uint64)


# ------------------------------------------------------------- decoders

def test_fp16_exhaustive_vs_numpy():
    ref = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    for h in range(65536):
        assert _same(oracle.fp16(h), ref[h]), hex(h)


def test_bf16_exhaustive_vs_torch():
    ref = (torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
           .to(torch.float64).numpy())
    for h in range(65536):
        assert _same(oracle.bf16(h), ref[h]), hex(h)


def test_e4m3_exhaustive_vs_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        assert _same(oracle.e4m3(b), ref[b]), hex(b)


def test_e4m3_page_f16_rule_and_nan_count():
    """Atlas issue, 'Kernel-level root cause ...', Fix: E4M3 -> f16 by a left
    shift of 7 then x256, exact for all non-NaN bytes; there are 254 of them."""
    f = FACTS["e4m3_to_f16_rule"]
    nan_free = [b for b in range(256) if not math.isnan(oracle.e4m3(b))]
    assert len(nan_free) == FACTS["e4m3_non_nan_bytes"]["value"]
    for b in nan_free:
        bits = ((b & 0x7F) << f["shift"]) | ((b & 0x80) << 8)
        h = np.array([bits], dtype=np.uint16).view(np.float16)[0]
        assert _same(float(h) * f["multiplier"], oracle.e4m3(b)), hex(b)


def test_e8m0_exhaustive_vs_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for b in range(256):
        assert _same(oracle.e8m0(b), ref[b]), hex(b)


def test_e2m1_vs_transformers_table_and_page_invariant():
    from transformers.integrations.mxfp4 import FP4_VALUES

    assert len(FP4_VALUES) == FACTS["e2m1_codes"]["value"]
    for c in range(16):
        assert _same(oracle.e2m1(c), float(FP4_VALUES[c])), c
        # the page: every E2M1 value has a zero low byte in f16
        h = np.array([oracle.e2m1(c)], dtype=np.float16).view(np.uint16)[0]
        assert h & 0xFF == 0, c


def test_nvfp4_element_products_exact_in_f16_and_bf16():
    """All 254 x 16 products E2M1(c) * E4M3(s) are exact in f16 and bf16
    (Atlas issue, Fix paragraph; the HIP path relies on the bf16 half)."""
    for s in range(256):
        sv = oracle.e4m3(s)
        if math.isnan(sv):
            continue
        for c in range(16):
            p = oracle.e2m1(c) * sv
            assert float(np.float16(p)) == p
            assert float(torch.tensor(p, dtype=torch.float64).to(torch.bfloat16).double()) == p


def test_q8_0_decode_exhaustive():
    """Every finite fp16 scale times every int8 code (the decoded value must
    equal the exact product of numpy's fp16 value and q)."""
    pats = np.concatenate([np.arange(0x0000, 0x7C00), np.arange(0x8000, 0xFC00)]).astype(np.uint16)
    n = pats.size
    k = 256
    q = np.tile(np.arange(-128, 128, dtype=np.int16).astype(np.int8), (n, 1))
    d = np.repeat(pats[:, None], k // 32, axis=1)
    w = {"fmt": "q8_0", "codes": q, "scales": d, "g": None}
    got = oracle.dequant(w)
    ref = pats.view(np.float16).astype(np.float64)[:, None] * q.astype(np.float64)
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))


def test_mxfp4_dequant_vs_transformers():
    """MXFP4 decode against transformers' packed-block dequantizer (library),
    packing the logical codes two per byte, even element in the low nibble."""
    from transformers.integrations.mxfp4 import convert_moe_packed_tensors

    rng = np.random.default_rng(7)
    n, k = 24, 128
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    e = rng.integers(2, 251, size=(n, k // 32), dtype=np.uint8)
    e[0, 0] = 127
    e[1, 1] = 2
    e[2, 2] = 250
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    blocks = torch.from_numpy(packed.reshape(1, n, k // 32, 16).copy())
    scales = torch.from_numpy(e.reshape(1, n, k // 32).copy())
    ref = convert_moe_packed_tensors(blocks, scales, dtype=torch.float32)
    assert tuple(ref.shape) == (1, k, n)
    ref = ref[0].transpose(0, 1).double().numpy()
    got = oracle.dequant({"fmt": "mxfp4", "codes": codes, "scales": e, "g": None})
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- GEMM

def _lib_decode(w):
    """Decoded weights from library routines only (numpy fp16, torch fp8,
    transformers FP4 table), times the tensor scale."""
    from transformers.integrations.mxfp4 import FP4_VALUES

    fp4 = np.array(FP4_VALUES, dtype=np.float64)
    c, s = w["codes"], w["scales"]
    n, k = c.shape
    if w["fmt"] == "q8_0":
        d = s.view(np.float16).astype(np.float64)
        return np.repeat(d, 32, axis=1) * c.astype(np.float64)
    if w["fmt"] == "mxfp4":
        sc = torch.from_numpy(s.copy()).view(torch.float8_e8m0fnu).double().numpy()
        return fp4[c] * np.repeat(sc, 32, axis=1)
    if w["fmt"] == "fp8":
        v = torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).double().numpy()
        return v * np.repeat(s.astype(np.float64), 128, axis=1)[:, :k]
    sc = torch.from_numpy(s.copy()).view(torch.float8_e4m3fn).double().numpy()
    v = fp4[c] * np.repeat(sc, 16, axis=1)
    g = w["g"].astype(np.float64)
    return v * np.repeat(g, n // len(g))[:, None]


def _lib_x(x):
    if x.dtype == np.float32:
        return x.astype(np.float64)
    return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).double().numpy()


def _rand_weights(fmt, n, k, rng, ntensors=1):
    if fmt == "fp8":
        c = rng.integers(0, 0x7F, size=(n, k), dtype=np.uint8)   # no NaN codes
        c |= (rng.integers(0, 2, size=c.shape, dtype=np.uint8) << 7)
        s = (rng.random((n, -(-k // 128))) * 0.01 + 1e-4).astype(np.float32)
        return {"fmt": fmt, "codes": c, "scales": s, "g": None}
    if fmt == "q8_0":
        q = rng.integers(-128, 128, size=(n, k), dtype=np.int16).astype(np.int8)
        d = np.float16(rng.standard_normal((n, k // 32)) * 0.01).view(np.uint16)
        return {"fmt": fmt, "codes": q, "scales": d, "g": None}
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    if fmt == "mxfp4":
        e = rng.integers(110, 140, size=(n, k // 32), dtype=np.uint8)
        return {"fmt": fmt, "codes": codes, "scales": e, "g": None}
    s = rng.integers(0, 0x7F, size=(n, k // 16), dtype=np.uint8)
    s |= (rng.integers(0, 2, size=s.shape, dtype=np.uint8) << 7)
    g = (rng.random(ntensors) * 0.01 + 1e-4).astype(np.float32)
    return {"fmt": fmt, "codes": codes, "scales": s, "g": g}


def _rand_x(act, b, k, rng):
    x = rng.standard_normal((b, k)).astype(np.float32)
    return x if act == "f32" else synth.f32_to_bf16_bits(x)


CASES = [(f, a) for f in ("q8_0", "mxfp4", "nvfp4", "fp8") for a in ("f32", "bf16")]


@pytest.mark.parametrize("fmt,act", CASES)
def test_gemm_bruteforce_exact_rational(fmt, act):
    """Tiny shapes against the exact rational sum (library-decoded operands):
    the fp64 oracle must lie within the recursive-summation error bound
    |err| <= gamma_K * sum |x w|, gamma_K = K u / (1 - K u), u = 2^-53."""
    rng = np.random.default_rng(11)
    for k in (32, 64) if fmt != "nvfp4" else (16, 48, 64):
        for b, n in ((1, 1), (3, 4), (2, 3)):
            w = _rand_weights(fmt, n, k, rng, ntensors=1)
            x = _rand_x(act, b, k, rng)
            W = _lib_decode(w)
            X = _lib_x(x)
            got = oracle.gemm(w, x)
            u = 2.0 ** -53
            gam = k * u / (1 - k * u)
            for bi in range(b):
                for ni in range(n):
                    exact = sum(Fraction(X[bi, kk]) * Fraction(W[ni, kk]) for kk in range(k))
                    mag = sum(abs(X[bi, kk] * W[ni, kk]) for kk in range(k))
                    assert abs(Fraction(got[bi, ni]) - exact) <= Fraction(gam * mag * 1.0001)


@pytest.mark.parametrize("fmt", ["q8_0", "mxfp4", "nvfp4", "fp8"])
def test_gemm_bruteforce_dyadic_equal(fmt):
    """Operands whose every partial sum is exact: the oracle must equal the
    exact rational result exactly."""
    rng = np.random.default_rng(5)
    n, k, b = 3, 64, 2
    w = _rand_weights(fmt, n, k, rng)
    if fmt == "q8_0":
        w["scales"][:] = np.float16(0.25).view(np.uint16)
    elif fmt == "mxfp4":
        w["scales"][:] = 125
    elif fmt == "fp8":
        w["scales"][:] = 0.125
    else:
        w["scales"][:] = 0x38  # 1.0
        w["g"] = np.array([0.5], dtype=np.float32)
    x = synth.f32_to_bf16_bits(rng.integers(-4, 5, size=(b, k)).astype(np.float32) * 0.5)
    W = _lib_decode(w)
    X = _lib_x(x)
    got = oracle.gemm(w, x)
    for bi in range(b):
        for ni in range(n):
            exact = sum(Fraction(X[bi, kk]) * Fraction(W[ni, kk]) for kk in range(k))
            assert Fraction(got[bi, ni]) == exact


@pytest.mark.parametrize("fmt,act", CASES)
def test_gemm_vs_numpy_matmul(fmt, act):
    """Medium shape (the 256x512, B=70 workload) against numpy's float64
    matmul on library-decoded operands."""
    rng = np.random.default_rng(3)
    n, k, b = 256, 512, 70
    w = _rand_weights(fmt, n, k, rng, ntensors=2 if fmt == "nvfp4" else 1)
    x = _rand_x(act, b, k, rng)
    ref = _lib_x(x) @ _lib_decode(w).T
    got = oracle.gemm(w, x)
    assert oracle.rel_fro(got, ref) < 1e-14
    bound = 2 * k * 2.0 ** -53 * (np.abs(_lib_x(x)) @ np.abs(_lib_decode(w)).T)
    assert np.all(np.abs(got - ref) <= bound + 1e-300)


def test_closed_form_constant_q8_0():
    """Constant q, d and x: every output is K*d*q*x and each output row sums
    to N*K*d*q*x (the workload's closed form)."""
    n, k, b = 48, 5120, 3
    d = np.float16(2.0 ** -7)
    q8, xv = 3, 0.5
    w = {"fmt": "q8_0", "codes": np.full((n, k), q8, dtype=np.int8),
         "scales": np.full((n, k // 32), d.view(np.uint16), dtype=np.uint16), "g": None}
    x = np.full((b, k), xv, dtype=np.float32)
    y = oracle.gemm(w, x)
    assert np.all(y == k * float(d) * q8 * xv)
    assert np.all(y == 60.0)
    assert np.all(y.sum(axis=1) == n * k * float(d) * q8 * xv)


def test_closed_form_constant_fp4():
    n, k, b = 8, 1024, 2
    x = synth.f32_to_bf16_bits(np.full((b, k), 2.0, dtype=np.float32))
    w = {"fmt": "mxfp4", "codes": np.full((n, k), 0x3, dtype=np.uint8),      # 1.5
         "scales": np.full((n, k // 32), 126, dtype=np.uint8), "g": None}      # 0.5
    assert np.all(oracle.gemm(w, x) == k * 1.5 * 0.5 * 2.0)
    w = {"fmt": "nvfp4", "codes": np.full((n, k), 0xB, dtype=np.uint8),      # -1.5
         "scales": np.full((n, k // 16), 0x40, dtype=np.uint8),                # 2.0
         "g": np.array([0.25, 4.0], dtype=np.float32)}
    y = oracle.gemm(w, x)
    assert np.all(y[:, : n // 2] == 0.25 * k * -1.5 * 2.0 * 2.0)
    assert np.all(y[:, n // 2:] == 4.0 * k * -1.5 * 2.0 * 2.0)


def test_closed_form_constant_fp8():
    """Constant E4M3 code and block scale: y = K * s * E4M3(c) * x exactly."""
    n, k, b = 8, 1024, 2
    x = synth.f32_to_bf16_bits(np.full((b, k), 0.5, dtype=np.float32))
    w = {"fmt": "fp8", "codes": np.full((n, k), 0x40, dtype=np.uint8),      # 2.0
         "scales": np.full((n, k // 128), 0.25, dtype=np.float32), "g": None}
    assert np.all(oracle.gemm(w, x) == k * 0.25 * 2.0 * 0.5)


def test_fp8_block_boundaries():
    """One fp32 scale per 128 columns, the last block shorter: a code of 1.0
    decodes to the scale of its own block (an off-by-one block index or a
    32-wide block would show here)."""
    n, k = 3, 320
    s = np.array([[1.0, 2.0, 4.0], [8.0, 16.0, 32.0], [0.5, 0.25, 0.125]], dtype=np.float32)
    w = {"fmt": "fp8", "codes": np.full((n, k), 0x38, dtype=np.uint8), "scales": s, "g": None}
    d = oracle.dequant(w)
    for r in range(n):
        want = np.concatenate([np.full(128, s[r, 0]), np.full(128, s[r, 1]), np.full(64, s[r, 2])])
        assert np.array_equal(d[r], want)


def test_row_independence_and_boundary_chunks():
    """hipfire PR, Scalar-Q8 boundary matrix: widths 64/65/70/76/256 split in
    contiguous chunks of 64 give the same rows, bit for bit."""
    fx = FACTS["boundary_widths"]
    n, k = 64, 256
    w = synth.gen_weights("q8_0", n, k, seed=0)
    for bw in fx["value"]:
        x = synth.gen_x_f32(bw, k, seed=0)
        full = oracle.gemm(w, x)
        chunks = fx["chunks_of_64"].get(str(bw), [bw])
        assert sum(chunks) == bw
        parts, r0 = [], 0
        for c in chunks:
            parts.append(oracle.gemm(w, x[r0:r0 + c]))
            r0 += c
        assert np.array_equal(full, np.concatenate(parts, axis=0))


def test_sampled_matches_full():
    rng = np.random.default_rng(1)
    w = _rand_weights("nvfp4", 40, 96, rng, ntensors=2)
    x = _rand_x("bf16", 9, 96, rng)
    full = oracle.gemm(w, x)
    bi = rng.integers(0, 9, 100)
    ni = rng.integers(0, 40, 100)
    assert np.array_equal(oracle.gemm_at(w, x, bi, ni), full[bi, ni])


def test_tensor_scale_applied_per_half():
    """Powers of two for g scale each half's outputs exactly."""
    rng = np.random.default_rng(2)
    w = _rand_weights("nvfp4", 16, 64, rng, ntensors=2)
    x = _rand_x("bf16", 3, 64, rng)
    w1 = dict(w, g=np.array([1.0, 1.0], dtype=np.float32))
    w2 = dict(w, g=np.array([8.0, 0.125], dtype=np.float32))
    y1, y2 = oracle.gemm(w1, x), oracle.gemm(w2, x)
    assert np.array_equal(y2[:, :8], 8.0 * y1[:, :8])
    assert np.array_equal(y2[:, 8:], 0.125 * y1[:, 8:])


def test_silu_identities_and_scipy():
    from scipy.special import expit

    for t in (-30.0, -3.5, -1.0, -1e-3, 0.0, 1e-3, 0.7, 2.0, 9.0, 40.0):
        s = oracle.silu(t)
        assert s == pytest.approx(t * expit(t), rel=1e-15, abs=1e-300)
        assert oracle.silu(t) - oracle.silu(-t) == pytest.approx(t, rel=1e-14, abs=1e-300)
    assert oracle.silu(0.0) == 0.0


def test_swiglu_equals_two_gemms_and_elementwise():
    from scipy.special import expit

    rng = np.random.default_rng(4)
    nh, k, b = 12, 64, 5
    w = _rand_weights("nvfp4", 2 * nh, k, rng, ntensors=2)
    x = _rand_x("bf16", b, k, rng)
    y = oracle.gemm(w, x)
    G, U = y[:, :nh], y[:, nh:]
    ref = G * expit(G) * U
    out = oracle.swiglu(w, x)
    assert np.allclose(out, ref, rtol=1e-14, atol=0)
    bi = rng.integers(0, b, 30)
    ji = rng.integers(0, nh, 30)
    assert np.array_equal(oracle.swiglu_at(w, x, bi, ji), out[bi, ji])


def test_swiglu_gate_zero_gives_zero():
    rng = np.random.default_rng(6)
    nh, k = 4, 32
    w = _rand_weights("nvfp4", 2 * nh, k, rng, ntensors=2)
    w["codes"][:nh] = 0
    x = _rand_x("bf16", 2, k, rng)
    assert np.all(oracle.swiglu(w, x) == 0.0)


# ------------------------------------------------------------ routed experts

@pytest.mark.parametrize("fmt,act,epi", [("nvfp4", "bf16", True), ("mxfp4", "bf16", False),
                                         ("fp8", "f32", False)])
def test_grouped_equals_per_expert_matmul(fmt, act, epi):
    """Each expert's rows against numpy float64 matmul on that expert's
    library-decoded weights (an off-by-one row offset or a wrong expert
    index fails here); empty experts produce no rows."""
    rng = np.random.default_rng(21)
    E, n, k = 5, 32, 256
    offsets = np.array([0, 3, 3, 20, 21, 29], dtype=np.int32)   # expert 1 empty
    ws = [_rand_weights(fmt, n, k, rng, ntensors=2 if fmt == "nvfp4" else 1) for _ in range(E)]
    x = _rand_x(act, int(offsets[-1]), k, rng)
    got = oracle.gemm_grouped(ws, offsets, x, swiglu_epi=epi)
    X = _lib_x(x)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        ref = X[r0:r1] @ _lib_decode(ws[e]).T
        if epi:
            G, U = ref[:, : n // 2], ref[:, n // 2:]
            ref = G / (1.0 + np.exp(-G)) * U
        assert np.allclose(got[r0:r1], ref, rtol=1e-12, atol=1e-300)


# ------------------------------------------------ the parity metric itself

def test_rel_fro_hand_computed():
    """rel_fro against values worked out by hand: a 3-4-5 triangle, one wrong
    element in a block of ones, zero error, a zero reference, NaN."""
    assert oracle.rel_fro([3.0, 4.0], [3.0, 4.0]) == 0.0
    # error (0.3, 0.4) has norm 0.5, the reference (3, 4) norm 5
    assert oracle.rel_fro([3.3, 4.4], [3.0, 4.0]) == pytest.approx(0.1, rel=1e-14)
    ref = np.ones((4, 4))
    y = ref.copy()
    y[1, 2] = 3.0                       # one element off by 2; ||ref|| = 4
    assert oracle.rel_fro(y, ref) == 0.5
    assert oracle.rel_fro(-ref, ref) == 2.0      # sign flip: ||2 ref|| / ||ref||
    assert oracle.rel_fro(np.zeros(5), np.zeros(5)) == 0.0
    assert oracle.rel_fro([0.0, 1e-300], [0.0, 0.0]) == math.inf
    # magnitudes whose squares under- or overflow fp64 still give the ratio
    assert oracle.rel_fro([3e-200, 4.4e-200], [3e-200, 4e-200]) == pytest.approx(0.4 / 5, rel=1e-12)
    assert oracle.rel_fro([3e200, 4.4e200], [3e200, 4e200]) == pytest.approx(0.4 / 5, rel=1e-12)
    assert oracle.rel_fro([math.inf, 1.0], [1.0, 1.0]) == math.inf
    e = oracle.rel_fro([1.0, math.nan], [1.0, 2.0])
    assert math.isnan(e) and not (e <= 1.0)
    with pytest.raises(ValueError):
        oracle.rel_fro(np.ones(3), np.ones(4))


def test_rel_fro_groups_finds_one_wrong_tile():
    """A 64 x 64 output cut into 16 x 16 tiles: one tile scaled by 1.02 is
    2 % off while the global figure over all 16 tiles is only 0.5 %; the
    per-tile errors are zero elsewhere, and a group with no element is NaN."""
    rng = np.random.default_rng(8)
    ref = rng.standard_normal((64, 64))
    y = ref.copy()
    y[16:32, 48:64] *= 1.02
    tiles = (np.arange(64)[:, None] // 16) * 4 + np.arange(64)[None, :] // 16
    per = oracle.rel_fro_groups(y, ref, tiles, 17)
    assert per[1 * 4 + 3] == pytest.approx(0.02, rel=1e-12)
    assert np.all(np.delete(per[:16], 7) == 0.0)
    assert math.isnan(per[16])
    glob = oracle.rel_fro(y, ref)
    assert glob < 0.006 and per.max(initial=0, where=~np.isnan(per)) > 0.019


def test_gamma_closed_form():
    u = 2.0 ** -24
    assert oracle.gamma(0, u) == 0.0
    assert oracle.gamma(1, u) == u / (1 - u)
    assert oracle.gamma(5120, u) == pytest.approx(5120 * u, rel=1e-3)
    assert oracle.gamma(2 ** 24, u) == math.inf


@pytest.mark.parametrize("fmt,act", CASES)
def test_gemm_abs_at_vs_library_and_bruteforce(fmt, act):
    """The magnitude sum sum_k |x||w| (times |g|) against numpy's float64
    matmul of |library-decoded operands|, and against an exact rational sum
    on a few outputs; NVFP4 with two tensors and a negative tensor scale."""
    rng = np.random.default_rng(31)
    n, k, b = 24, 256, 7
    w = _rand_weights(fmt, n, k, rng, ntensors=2 if fmt == "nvfp4" else 1)
    if fmt == "nvfp4":
        w["g"] = np.array([0.003, -0.02], dtype=np.float32)
    x = _rand_x(act, b, k, rng)
    X, W = _lib_x(x), _lib_decode(w)
    ref = np.abs(X) @ np.abs(W).T
    bi = np.repeat(np.arange(b), n)
    ni = np.tile(np.arange(n), b)
    got = oracle.gemm_abs_at(w, x, bi, ni).reshape(b, n)
    assert np.all(got >= 0)
    assert oracle.rel_fro(got, ref) < 1e-14
    for i in range(4):
        bb, nn = int(bi[i * 37 % bi.size]), int(ni[i * 37 % ni.size])
        exact = sum(abs(Fraction(X[bb, kk]) * Fraction(W[nn, kk])) for kk in range(k))
        assert abs(Fraction(got[bb, nn]) - exact) <= exact * Fraction(k * 2.0 ** -52)


def test_dequant_apply_g_vs_library_two_tensors():
    """dequant(apply_g=True) for NVFP4 with two tensor scales (the fused
    gate+up matrix): every row's decoded weights times its own tensor's g,
    against the library decode (torch float8, transformers' FP4 table), and
    apply_g=False leaves g out."""
    rng = np.random.default_rng(41)
    w = _rand_weights("nvfp4", 32, 96, rng, ntensors=2)
    w["g"] = np.array([0.75, 3e-5], dtype=np.float32)
    got = oracle.dequant(w, apply_g=True)
    assert np.array_equal(got, _lib_decode(w))
    plain = oracle.dequant(w, apply_g=False)
    assert np.array_equal(got[:16], plain[:16] * np.float64(np.float32(0.75)))
    assert np.array_equal(got[16:], plain[16:] * np.float64(np.float32(3e-5)))
    # the other formats have no tensor scale: apply_g changes nothing
    for fmt in ("q8_0", "mxfp4", "fp8"):
        wf = _rand_weights(fmt, 8, 128, rng)
        assert np.array_equal(oracle.dequant(wf, apply_g=True), oracle.dequant(wf))


def test_rel_fro_groups_equals_rel_fro_per_group():
    """The vectorised per-group figure equals rel_fro over each group's
    elements, NaN, inf, zero and tiny groups included."""
    rng = np.random.default_rng(9)
    n, G = 5000, 40
    gi = rng.integers(0, G, n)
    ref = rng.standard_normal(n) * 10.0 ** rng.integers(-150, 150, n)
    y = ref * (1 + 1e-3 * rng.standard_normal(n))
    ref[gi == 3] = 0.0
    y[gi == 3] = 0.0
    ref[gi == 4] = 0.0
    y[(gi == 5)] = np.nan
    y[(gi == 6)] = np.inf
    gi[gi == 7] = 8                                  # group 7 empty
    per = oracle.rel_fro_groups(y, ref, gi, G)
    for g in range(G):
        sel = gi == g
        want = oracle.rel_fro(y[sel], ref[sel]) if sel.any() else math.nan
        assert _same(per[g], want) or per[g] == pytest.approx(want, rel=1e-12), g


def test_thread_count_does_not_change_results():
    """The one-thread timing leg computes the same outputs as all cores."""
    rng = np.random.default_rng(13)
    w = _rand_weights("q8_0", 64, 256, rng)
    x = _rand_x("f32", 5, 256, rng)
    n0 = oracle.threads()
    full = oracle.gemm(w, x)
    oracle.set_threads(1)
    try:
        assert oracle.threads() == 1
        assert np.array_equal(oracle.gemm(w, x), full)
    finally:
        oracle.set_threads(n0)
    assert oracle.threads() == n0
