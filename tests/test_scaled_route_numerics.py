"""What the hardware block-scaled MFMA route would cost in accuracy (CPU).

gfx950's block-scaled matrix instruction multiplies fp8 / fp6 / fp4 operands
that carry one E8M0 scale per row and 32-wide block.  MXFP4 weights fit it as
they are; the activations would have to become MX blocks too.  This module
quantizes N(0, 1) activation rows the way the OCP MX format defines (shared
scale 2^(floor(log2 max|x|) - emax), elements rounded to nearest even,
saturating) and measures the relative Frobenius error of x·Wᵀ against the
exact product, next to plain bf16 rounding of x (the bf16-math tier's only
activation error).  The figures back the design choice recorded with the
matrix-core rates (bench key `mx_scaled_mfma_rates`): one E4M3 term misses the
1e-2 bound of the bf16/fp8-activation path, two terms (hi + residual) meet it
at twice the fp8 instruction count, and E2M1 activations are far off.

Not a parity test and not part of the oracle: a numerical study of a route
that is not built.
"""
import numpy as np
import pytest
import torch


def _round_minifloat(v, mant_bits, emin, vmax):
    """Round float64 values to a minifloat with `mant_bits` stored mantissa
    bits, smallest normal exponent `emin` (subnormals below it) and largest
    finite magnitude `vmax`: nearest, ties to even, saturating."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    ulp = np.exp2(e - mant_bits)
    q = np.rint(a / ulp) * ulp
    return np.sign(v) * np.minimum(q, vmax)


E4M3 = dict(mant_bits=3, emin=-6, vmax=448.0, emax=8)
E2M1 = dict(mant_bits=1, emin=0, vmax=6.0, emax=2)


def _mx_quantize(x, fmt):
    """OCP MX block quantization along the last axis in blocks of 32:
    returns the dequantized values (scale x element)."""
    B, K = x.shape
    blk = x.reshape(B, K // 32, 32)
    m = np.abs(blk).max(axis=2, keepdims=True)
    e = np.floor(np.log2(np.where(m > 0, m, 1.0))) - fmt["emax"]
    s = np.exp2(e)
    q = _round_minifloat(blk / s, fmt["mant_bits"], fmt["emin"], fmt["vmax"])
    return (q * s).reshape(B, K)


def _rel_fro(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_minifloat_rounding_matches_known_values():
    # E4M3: 1 + 2^-3 is representable, 1 + 2^-4 ties to even (1.0), 1 + 3*2^-4
    # ties up to 1.25; 2^-9 is the smallest subnormal; 500 saturates to 448
    v = np.array([1.125, 1.0625, 1.1875, 2.0 ** -9, 2.0 ** -10 * 1.5, 500.0, -3.3])
    got = _round_minifloat(v, 3, -6, 448.0)
    assert got.tolist() == [1.125, 1.0, 1.25, 2.0 ** -9, 2.0 ** -9, 448.0, -3.25]
    # E2M1 holds exactly 0, 0.5, 1, 1.5, 2, 3, 4, 6
    v = np.array([0.25, 0.75, 1.25, 2.5, 3.5, 5.0, 7.0])
    assert _round_minifloat(v, 1, 0, 6.0).tolist() == [0.0, 1.0, 1.0, 2.0, 4.0, 4.0, 6.0]


def test_mx_quantize_keeps_the_block_max_in_range():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((8, 256)) * np.exp2(rng.integers(-20, 20, (8, 1)))
    for fmt in (E4M3, E2M1):
        d = _mx_quantize(x, fmt)
        blk_x = np.abs(x.reshape(8, -1, 32)).max(axis=2)
        blk_d = np.abs(d.reshape(8, -1, 32)).max(axis=2)
        # the largest element keeps its binade: relative error at most half an ulp
        # of the format, or saturation at vmax (at most 2^(emax+1)/vmax - 1 off)
        assert np.all(np.abs(blk_d - blk_x) <= blk_x * max(2.0 ** -(fmt["mant_bits"] + 1),
                                                         1 - fmt["vmax"] / 2.0 ** (fmt["emax"] + 1)))


@pytest.fixture(scope="module")
def products():
    rng = np.random.default_rng(7)
    B, K, N = 64, 4096, 256
    x = rng.standard_normal((B, K))
    w = rng.standard_normal((N, K)) * 0.02
    exact = x @ w.T
    return x, w, exact


def test_activation_error_of_each_route(products):
    x, w, exact = products
    bf16 = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    one = _mx_quantize(x, E4M3)
    hi = one
    two = hi + _mx_quantize(x - hi, E4M3)
    fp4 = _mx_quantize(x, E2M1)
    err = {name: _rel_fro(v @ w.T, exact)
           for name, v in (("bf16", bf16), ("e4m3", one), ("e4m3 x2", two), ("e2m1", fp4))}
    # bf16 rounding: about 2^-9 / sqrt(3) relative per element
    assert 5e-4 < err["bf16"] < 3e-3, err
    # one E4M3 term: past the 1e-2 bound of the bf16/fp8-activation path
    assert err["e4m3"] > 1e-2, err
    # two terms: within it, and within a few times the bf16 error
    assert err["e4m3 x2"] < 1e-2 and err["e4m3 x2"] < 4 * err["bf16"], err
    # E2M1 activations: tens of percent
    assert err["e2m1"] > 0.1, err
