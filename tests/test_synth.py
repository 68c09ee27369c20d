"""Host-side checks of the seeded input generator and the quantizers (CPU)."""

import numpy as np
import torch

import synth


def test_splitmix64_reference_values():
    # SplitMix64 seeded with state 0: the first outputs of the published
    # generator are 0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F.
    base = np.uint64(0)
    idx = np.arange(1, 4, dtype=np.uint64)
    with np.errstate(over="ignore"):
        got = synth._mix64(base + idx * synth.GOLDEN)
    assert [int(v) for v in got] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_form_is_random_access():
    a = synth.normal(0, 1, 0, 1001)
    b = synth.normal(0, 1, 37, 500)
    assert np.array_equal(a[37:537], b)
    c = synth.normal_f32(0, 1, 5, 64, row0=3)
    d = synth.normal_f32(0, 1, 8, 64)
    assert np.array_equal(c[:5], d[3:8])


def test_normal_moments():
    z = synth.normal(0, 2, 0, 400_000)
    assert abs(z.mean()) < 0.01
    assert abs(z.std() - 1.0) < 0.01
    assert np.all(np.isfinite(z))


def test_bf16_rounding_matches_torch():
    x = synth.normal_f32(0, 9, 64, 257)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(x), ref)


def test_q8_0_quantizer_error_bound():
    w = synth.normal_f32(0, 1, 64, 512, std=0.02)
    q, d = synth.quantize_q8_0(w)
    dv = d.view(np.float16).astype(np.float64)
    rec = np.repeat(dv, 32, axis=1) * q.astype(np.float64)
    d32 = np.max(np.abs(w.reshape(64, 16, 32)), axis=2) / 127.0
    # half a step of the fp32 scale plus the fp16 rounding of the scale
    bound = np.repeat(d32 * 0.5 + np.abs(dv - d32) * 127 + 1e-12, 32, axis=1)
    assert np.all(np.abs(rec - w) <= bound)
    assert np.abs(q).max() <= 127


def test_e2m1_encoder_ties_and_saturation():
    r = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.9, -0.1, -5.01, 0.0])
    # ties go to the even (mantissa-0) neighbour; values above 6 saturate
    want_mag = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 0.0, 6.0, 0.0]
    table = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    c = synth._e2m1_encode(r)
    for ci, ri, m in zip(c, r, want_mag):
        assert table[ci & 7] == m
        assert bool(ci >> 3) == bool(np.signbit(ri))


def test_mxfp4_scale_rule():
    w = synth.normal_f32(0, 3, 32, 256, std=0.02)
    codes, e = synth.quantize_mxfp4(w)
    amax = np.max(np.abs(w.reshape(32, 8, 32)), axis=2).astype(np.float64)
    ratio = amax / np.ldexp(1.0, e.astype(np.int64) - 127)
    assert np.all((ratio >= 4.0) & (ratio < 8.0))
    assert codes.max() < 16


def test_nvfp4_scales_in_range():
    w = synth.normal_f32(0, 4, 32, 256, std=0.02)
    codes, s, g = synth.quantize_nvfp4(w)
    sv = torch.from_numpy(s.copy()).view(torch.float8_e4m3fn).float().numpy()
    assert np.all(np.isfinite(sv)) and sv.max() <= 448.0
    assert g == np.float32(np.max(np.abs(w)) / np.float32(2688.0))
    assert codes.max() < 16


def test_outlier_mask_rate():
    w_plain = synth.gen_weights("q8_0", 64, 1024, seed=0)
    w_out = synth.gen_weights("q8_0", 64, 1024, seed=0, outlier_p=0.001)
    assert not np.array_equal(w_plain["scales"], w_out["scales"])
    u = synth.uniform(0, synth.SID_W + 100, 0, 64 * 1024)
    assert 20 < int((u < 0.001).sum()) < 120


def test_fp8_quantizer_error_bound():
    """E4M3 keeps 3 mantissa bits: each weight is within half a step of its
    E4M3 grid point (relative 2^-4 above 2^-6 * s, absolute 2^-10 * s below)."""
    w = synth.normal_f32(0, 6, 32, 320, std=0.02)
    c, s = synth.quantize_fp8(w)
    assert c.shape == (32, 320) and s.shape == (32, 3)
    v = torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.all(np.isfinite(v)) and np.abs(v).max() <= 448.0
    sv = np.repeat(s.astype(np.float64), 128, axis=1)[:, :320]
    rec = v * sv
    err = np.abs(rec - w.astype(np.float64))
    bound = np.maximum(np.abs(w) * 2.0 ** -4, sv * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)
    amax = np.max(np.abs(np.pad(w, ((0, 0), (0, 64))).reshape(32, 3, 128)), axis=2)
    assert np.array_equal(s, (amax / np.float32(448.0)).astype(np.float32))


def test_routing_is_topk_distinct_and_sorted():
    tok, off = synth.gen_routing(50, 4, 12, seed=0)
    assert off[0] == 0 and off[-1] == 50 * 4 and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.bincount(tok, minlength=50), np.full(50, 4))
    exp = np.repeat(np.arange(12), np.diff(off))
    for t in range(50):
        assert len(set(exp[tok == t])) == 4          # distinct experts per token
    for e in range(12):                              # token order inside an expert
        r = tok[off[e]:off[e + 1]]
        assert np.all(np.diff(r) > 0)
