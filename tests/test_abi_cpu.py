"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, validates arguments before any HIP call, and packs the documented
layout.  No compute call is made here."""

import ctypes
import json
import os
import re

import numpy as np
import pytest

import prefill_q8_mxfp4_amd as q
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemm.h")
FACTS = json.load(open(os.path.join(ROOT, "tests", "golden", "page_facts.json")))


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qgemm_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = q.lib()
    names = _declared()
    assert set(names) == set(q.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert q.version() == (1, 0)


def _has_device():
    import torch
    return torch.cuda.device_count() > 0


def _create(*args):
    h = ctypes.c_void_p()
    st = q.lib().qgemm_create(ctypes.byref(h), *args)
    return st, h


@pytest.mark.parametrize("args,status", [
    ((0, 0, 0, 0, 0, 256, 512, 0), q.OK),
    ((0, 0, 0, 0, 0, 0, 512, 0), q.EINVAL),          # N = 0
    ((0, 0, 0, 0, 0, 256, -32, 0), q.EINVAL),        # K < 0
    ((0, 0, 0, 0, 0, 256, 48, 0), q.EINVAL),         # K % 32
    ((0, 0, 0, 0, 0, 256, 1 << 20, 0), q.OK),        # largest K
    ((0, 0, 0, 0, 0, 256, (1 << 20) + 32, 0), q.EINVAL),  # K above 2^20
    ((0, 0, 0, 0, 0, (1 << 30) + 16, 512, 0), q.EINVAL),  # N above 2^30
    ((2, 1, 0, 0, 1, 256, 48, 0), q.OK),             # NVFP4: 16-wide blocks
    ((1, 1, 0, 0, 1, 256, 48, 0), q.EINVAL),         # MXFP4: K % 32
    ((4, 0, 0, 0, 0, 256, 512, 0), q.EINVAL),        # unknown format
    ((3, 0, 0, 0, 0, 256, 512, 0), q.OK),            # FP8
    ((0, 2, 0, 0, 0, 256, 512, 0), q.EINVAL),        # unknown dtype
    ((0, 0, 0, 2, 0, 256, 512, 0), q.EINVAL),        # unknown epilogue
    ((0, 0, 0, 0, 2, 256, 512, 0), q.EINVAL),        # unknown math
    ((0, 1, 0, 0, 0, 256, 512, 0), q.EINVAL),        # fp32 math with bf16 activations
    ((2, 1, 1, 1, 1, 255, 512, 0), q.EINVAL),        # SwiGLU with odd N
    ((2, 1, 1, 1, 1, 40, 512, 0), q.ENOTSUP),        # SwiGLU with N/2 % 16
    ((0, 0, 0, 0, 0, 256, 512, 3), q.EINVAL),        # both tiers forced
    ((0, 0, 0, 0, 0, 256, 512, 0x10), q.EINVAL),     # unknown flag
    ((0, 0, 0, 0, 0, 256, 512, 2), q.OK),            # fp32 math in the tiled tier
    ((0, 0, 0, 0, 0, 256, 512, 4), q.OK),            # the GEMV tier
    ((0, 0, 0, 0, 0, 256, 512, 5), q.EINVAL),        # two tiers forced
    ((2, 1, 1, 1, 1, 64, 512, 1), q.OK),             # SwiGLU in the skinny tier (B <= 16)
    ((2, 0, 0, 1, 0, 64, 512, 0), q.ENOTSUP),        # SwiGLU with fp32 math
])
def test_create_validation(args, status):
    st, h = _create(*args)
    assert st == status, q.lib().qgemm_last_error()
    if st == q.OK:
        assert h.value
        assert q.lib().qgemm_destroy(h) == q.OK
    else:
        assert not h.value
        assert q.lib().qgemm_last_error()


def test_create_is_host_only():
    """qgemm_create makes no HIP call: in a process that sees no GPU (every
    device hidden) plans are created and destroyed, nothing is probed, and
    the calls that do need a device fail cleanly with QGEMM_EHIP."""
    import subprocess
    import sys
    code = r"""
import ctypes, prefill_q8_mxfp4_amd as q
L = q.lib()
for args in ((0, 0, 0, 0, 0, 5120, 5120, 0), (2, 1, 1, 1, 1, 2 * 17408, 5120, 0), (3, 1, 0, 0, 1, 256, 512, 2)):
    h = ctypes.c_void_p()
    assert L.qgemm_create(ctypes.byref(h), *args) == q.OK, L.qgemm_last_error()
    assert h.value and L.qgemm_plan_tier(h, 16) in (1, 2)
    assert L.qgemm_workspace_bytes(h, 16) > 0
    assert L.qgemm_destroy(h) == q.OK
assert L.qgemm_xcd_local() == -1
assert L.qgemm_init_device() == q.EHIP and L.qgemm_last_error()
bits = ctypes.c_uint32(7)
assert L.qgemm_device_status(ctypes.byref(bits), 0, None) == q.EHIP and bits.value == 0
assert L.qgemm_device_status(None, 0, None) == q.EINVAL
print("ok")
"""
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1", CUDA_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120,
                       env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:] + r.stderr[-2000:]


def test_destroy_null_and_strerror():
    assert q.lib().qgemm_destroy(None) == q.OK
    for s in (q.OK, q.EINVAL, q.ENOTSUP, q.EHIP, q.ENOMEM):
        assert q.lib().qgemm_strerror(s)
    assert q.lib().qgemm_create(None, 0, 0, 0, 0, 0, 16, 32, 0) == q.EINVAL


def test_run_validation_before_any_hip_call():
    L = q.lib()
    st, h = _create(0, 0, 0, 0, 0, 256, 512, 0)
    assert st == q.OK
    buf = ctypes.create_string_buffer(64)
    p16 = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16
    assert L.qgemm_run(h, 0, None, None, None, None) == q.OK          # B = 0: no-op
    assert L.qgemm_run(h, -1, p16, p16, p16, None) == q.EINVAL
    assert L.qgemm_run(h, 4, None, p16, p16, None) == q.EINVAL
    assert L.qgemm_run(h, 4, p16 + 4, p16, p16, None) == q.EINVAL       # misaligned
    assert L.qgemm_run(None, 4, p16, p16, p16, None) == q.EINVAL
    assert L.qgemm_run(h, 1 << 31, p16, p16, p16, None) == q.EINVAL
    assert L.qgemm_plan_tier(h, 16) == 1
    assert L.qgemm_plan_tier(h, 17) == 1      # fp32 math up to 80 rows: the verify kernel
    assert L.qgemm_plan_tier(h, 80) == 1
    assert L.qgemm_plan_tier(h, 81) == 2      # above: the faithful variant of the large-batch tier
    assert L.qgemm_plan_tier(h, 256) == 2
    assert L.qgemm_plan_tier(h, 2048) == 2
    assert L.qgemm_plan_tier(h, -1) == 0
    if not _has_device():
        assert L.qgemm_xcd_local() == -1      # no device: nothing probed
    assert L.qgemm_destroy(h) == q.OK


def test_tier_choice():
    p = q.Plan("mxfp4", 5120, 17408, act="bf16")
    assert p.tier(1) == "skinny" and p.tier(16) == "skinny" and p.tier(2048) == "tiled"
    # bf16 math: the verify kernel up to 80 rows (K a whole number of slabs), tiled above
    assert p.tier(32) == "skinny" and p.tier(80) == "skinny" and p.tier(81) == "tiled"
    assert q.Plan("mxfp4", 5120, 17408 - 32, act="bf16").tier(33) == "tiled"  # skinny kernel to 32
    p = q.Plan("nvfp4", 2 * 17408, 5120, act="bf16", out="bf16", epilogue="swiglu")
    # fused gate+up: the verify kernel to 48 rows, then the tiled tier
    assert p.tier(2048) == "tiled" and p.tier(17) == "skinny" and p.tier(48) == "skinny"
    assert p.tier(49) == "tiled"
    assert p.tier(1) == "gemv" and p.tier(2) == "skinny" and p.tier(16) == "skinny"
    p = q.Plan("q8_0", 5120, 5120, act="f32", tier="skinny")
    assert p.tier(1) == "skinny" and p.tier(256) == "skinny"
    p = q.Plan("q8_0", 5120, 5120, act="f32", tier="gemv")
    assert p.tier(1) == "gemv" and p.tier(300) == "gemv" and p.workspace_bytes(2) == 0
    # automatic: the GEMV kernel for B = 1 when one activation row fits in
    # 32 KB of LDS (K <= 8192), the streaming kernel from B = 2
    for fmt, act in (("q8_0", "f32"), ("fp8", "bf16"), ("mxfp4", "bf16"), ("nvfp4", "f32")):
        p = q.Plan(fmt, 5120, 8192, act=act)
        assert p.tier(1) == "gemv" and p.tier(2) == "skinny" and p.workspace_bytes(1) == 0
        p = q.Plan(fmt, 5120, 8448, act=act)
        assert p.tier(1) == "skinny"


def _split_part_bytes(plan, B, N):
    """Partial-tile bytes of the large-batch split: the workspace minus the
    counters (small-batch counters for ceil(N/16) row tiles, then 1 KB)."""
    rt = -(-N // 16)
    cnt = -(-(8 * ((rt + 3) // 4) * 4) // 256) * 256 + 1024
    return plan.workspace_bytes(B) - cnt


@pytest.mark.parametrize("fmt,N,K,act,B,bm,s,rem", [
    # FP8 5120^2 at B = 2048: 320 128-row tiles (256 whole, the last 64 in 4 pieces)
    # beat 160 256-row tiles split in three (126 MB of partials)
    ("fp8", 5120, 5120, "bf16", 2048, 128, 4, 64),
    ("fp8", 5120, 5120, "bf16", 1024, 256, 3, 80),    # 80 256-row tiles in 3 pieces
    ("fp8", 5120, 5120, "bf16", 256, 128, 6, 40),
    ("mxfp4", 5120, 17408, "bf16", 2048, 256, 3, 160),
    ("mxfp4", 5120, 17408, "bf16", 384, 128, 4, 60),
    ("q8_0", 17408, 5120, "bf16", 2048, 256, 8, 32),  # 544 tiles: 512 whole, 32 in 8 pieces
    ("q8_0", 5120, 5120, "f32", 70, 96, 12, 20),      # fp32-faithful, 96-row tiles
    ("q8_0", 5120, 5120, "f32", 256, 64, 3, 80),
])
def test_large_batch_shape_choices(fmt, N, K, act, B, bm, s, rem):
    """The large-batch cost model's row-tile height and split count on the
    measured shapes (each the fastest of the forced choices on MI355X),
    read back through the workspace size: rem tiles x s pieces x bm x 256
    fp32 partials."""
    # fp32-faithful math at B <= 80 runs the verify kernel by default; the
    # tiled tier is forced there to read its cost model
    faithful_small = act == "f32" and B <= 80
    plan = q.Plan(fmt, N, K, act=act, out="f32", tier="tiled" if faithful_small else None)
    assert plan.tier(B) == "tiled"
    assert _split_part_bytes(plan, B, N) == rem * s * bm * 256 * 4


@pytest.mark.parametrize("fmt,K", [("q8_0", 5120), ("fp8", 5120), ("mxfp4", 17408), ("nvfp4", 5120)])
def test_verify_kernel_choice_and_workspace(fmt, K):
    """fp32-faithful math at 16 < B <= 80 takes the verify kernel (small-batch
    tier): the streaming kernel's row groups of 8 row tiles and K splits,
    partial tiles for every 16-row batch group.  Below 17 rows the streaming
    kernel, above 80 the faithful tiled variant; bf16 math takes it over the
    same widths; the fused epilogue and K not a whole number of slabs never
    take it."""
    N = 5120
    p = q.Plan(fmt, N, K, act="f32", out="f32", math="fp32")
    rt = N // 16
    cnt = -(-(8 * ((rt + 3) // 4) * 4) // 256) * 256 + 1024
    stream_part = p.workspace_bytes(16) - cnt        # ksplit x groups x 8 KB
    assert stream_part > 0 and stream_part % (-(-rt // 8) * 8 * 1024) == 0
    for B in (17, 32, 33, 64, 65, 70, 76, 80):
        assert p.tier(B) == "skinny", B
        mb = -(-B // 16)
        assert p.workspace_bytes(B) - cnt == stream_part * mb, B
    assert p.tier(81) == "tiled"
    assert q.Plan(fmt, N, K, act="f32", out="f32", math="bf16").tier(64) == "skinny"  # bf16 math too
    assert q.Plan(fmt, N, K, act="f32", out="f32", math="bf16").tier(81) == "tiled"
    slab = 64 if fmt in ("q8_0", "fp8") else 128
    assert q.Plan(fmt, N, K + 32 if K % slab else K - 32, act="f32", math="fp32").tier(64) == "tiled"


def test_weight_bytes_match_format_density():
    # N, K multiples of the tile: exactly the algorithmic bytes per weight
    assert q.weight_bytes("q8_0", 5120, 5120) == 5120 * 5120 * 17 // 16
    assert q.weight_bytes("mxfp4", 5120, 17408) == 5120 * 17408 * 17 // 32
    assert q.weight_bytes("nvfp4", 34816, 5120) == 34816 * 5120 * 9 // 16 + 256
    assert q.weight_bytes("q8_0", 16, 48) == 0
    assert q.weight_bytes("nvfp4", 0, 16) == 0


def test_mxfp4_density_matches_page():
    """HF model card, 'What's 4-bit': 22.7B MXFP4 parameters in 12.05B bytes."""
    f = FACTS["mxfp4_density"]
    per_weight = q.weight_bytes("mxfp4", 5120, 17408) / (5120 * 17408)
    assert abs(per_weight - f["packed_bytes"] / f["params"]) < 0.002


def _unpack(fmt, buf, n, k):
    """Read logical arrays back out of a packed buffer, following the layout
    the header documents (row tiles of 16, slabs, lane chunks, scale rows)."""
    ks = 64 if fmt in ("q8_0", "fp8") else 128
    kp = -(-k // ks) * ks
    np_ = -(-n // 16) * 16
    S = kp // ks
    codes = np.zeros((n, k), dtype=np.int16)
    for row in range(n):
        rt, r = divmod(row, 16)
        for kk in range(k):
            s, o = divmod(kk, ks)
            u, rem = divmod(o, 32)
            g, j = divmod(rem, 8)
            base = (rt * S + s) * 1024 + (g * 16 + r) * 16
            if fmt == "q8_0":
                codes[row, kk] = np.int8(buf[base + 8 * u + j].view(np.int8))
            elif fmt == "fp8":
                codes[row, kk] = buf[base + 8 * u + j]
            else:
                byte = int(buf[base + 4 * u + j // 2])
                codes[row, kk] = (byte >> (4 * (j & 1))) & 15
    soff = -(-(np_ // 16) * S * 1024 // 256) * 256
    if fmt == "fp8":
        # one fp32 per row and slab: the scale of the 128-wide block holding it
        nb = -(-k // 128)
        sc = np.zeros((n, nb), dtype=np.float32)
        for row in range(n):
            rt, r = divmod(row, 16)
            for s_ in range(S):
                off = soff + ((rt * S + s_) * 16 + r) * 4
                v = buf[off:off + 4].view(np.float32)[0]
                if s_ * 64 < k:
                    if s_ % 2:
                        assert v == sc[row, s_ // 2]  # both slabs of a block agree
                    sc[row, s_ // 2] = v
        return codes, sc, soff + (np_ // 16) * S * 16 * 4
    blk = 16 if fmt == "nvfp4" else 32
    esz = 2 if fmt == "q8_0" else 1
    per_slab = ks // blk
    rec = 8 if fmt == "nvfp4" else 4                 # scale bytes per row and slab
    nsc = k // blk
    sc = np.zeros((n, nsc * esz), dtype=np.uint8)
    for row in range(n):
        rt, r = divmod(row, 16)
        for j in range(nsc):
            s, i = divmod(j, per_slab)
            off = soff + ((rt * S + s) * 16 + r) * rec + i * esz
            sc[row, j * esz:(j + 1) * esz] = buf[off:off + esz]
    if fmt == "q8_0":
        sc = sc.view(np.uint16)
    return codes, sc, soff + (np_ // 16) * S * 16 * rec


@pytest.mark.parametrize("fmt,n,k", [("q8_0", 37, 96), ("mxfp4", 21, 160), ("nvfp4", 18, 144),
                                     ("fp8", 19, 352)])
def test_pack_layout_roundtrip(fmt, n, k):
    rng = np.random.default_rng(0)
    if fmt == "fp8":
        codes = rng.integers(0, 256, (n, k)).astype(np.uint8)
        scales = rng.standard_normal((n, -(-k // 128))).astype(np.float32)
        g = None
    elif fmt == "q8_0":
        codes = rng.integers(-128, 128, (n, k)).astype(np.int8)
        scales = rng.integers(0, 65536, (n, k // 32)).astype(np.uint16)
        g = None
    else:
        codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
        scales = rng.integers(0, 256, (n, k // (16 if fmt == "nvfp4" else 32))).astype(np.uint8)
        g = np.array([0.5, 2.0], dtype=np.float32) if fmt == "nvfp4" else None
    buf = q.pack(fmt, n, k, codes, scales, g)
    assert buf.size == q.weight_bytes(fmt, n, k)
    c2, s2, meta = _unpack(fmt, buf, n, k)
    assert np.array_equal(c2, codes.astype(np.int16))
    assert np.array_equal(s2, scales)
    if fmt == "nvfp4":
        meta = -(-meta // 256) * 256
        hdr = buf[meta:meta + 16].view(np.int32)
        assert list(hdr) == [2, n // 2, 0, 0]
        assert np.array_equal(buf[meta + 16:meta + 24].view(np.float32), g)


def test_pack_rejects_bad_input():
    codes = np.zeros((16, 32), dtype=np.uint8)
    codes[3, 4] = 16
    with pytest.raises(q.QgemmError):
        q.pack("mxfp4", 16, 32, codes, np.zeros((16, 1), np.uint8))
    with pytest.raises(q.QgemmError):   # NVFP4 without tensor scales
        q.pack("nvfp4", 16, 32, np.zeros((16, 32), np.uint8), np.zeros((16, 2), np.uint8))
    with pytest.raises(q.QgemmError):   # tensor count must divide N
        q.pack("nvfp4", 16, 32, np.zeros((16, 32), np.uint8), np.zeros((16, 2), np.uint8),
               np.ones(3, np.float32))


def test_plan_errors_raise():
    with pytest.raises(q.QgemmError) as e:
        q.Plan("q8_0", 256, 48, act="f32")
    assert e.value.status == q.EINVAL


def test_synth_configs_pack():
    w = synth.gen_config_weights("q8_0_256x512")
    buf = q.pack_logical(w)
    assert buf.size == q.weight_bytes("q8_0", 256, 512)


def test_grouped_argument_checks():
    """qgemm_run_grouped validates on the host before touching the device."""
    L = q.lib()
    h = ctypes.c_void_p()
    assert L.qgemm_create(ctypes.byref(h), 2, 1, 0, 0, 1, 256, 512, 0) == q.OK
    fake = ctypes.c_void_p(0x1000)
    assert L.qgemm_run_grouped(h, 0, 10, fake, fake, fake, fake, None) == q.EINVAL    # E = 0
    assert L.qgemm_run_grouped(h, 4, -1, fake, fake, fake, fake, None) == q.EINVAL    # T < 0
    assert L.qgemm_run_grouped(h, 4, 0, None, None, None, None, None) == q.OK        # T = 0: no-op
    assert L.qgemm_run_grouped(h, 4, 10, None, fake, fake, fake, None) == q.EINVAL   # null table
    assert L.qgemm_run_grouped(h, 4, 10, fake, fake, ctypes.c_void_p(0x1008), fake, None) == q.EINVAL
    L.qgemm_destroy(h)
    assert L.qgemm_create(ctypes.byref(h), 0, 0, 0, 0, 0, 256, 512, 0) == q.OK        # fp32 math
    assert L.qgemm_run_grouped(h, 4, 0, None, None, None, None, None) == q.OK
    assert L.qgemm_run_grouped(h, 4, 10, fake, None, fake, fake, None) == q.EINVAL   # null offsets
    L.qgemm_destroy(h)
    assert L.qgemm_create(ctypes.byref(h), 2, 0, 0, 0, 0, 256, 512, 1) == q.OK        # skinny, fp32 math
    assert L.qgemm_run_grouped(h, 4, 10, fake, fake, fake, fake, None) == q.ENOTSUP
    L.qgemm_destroy(h)
    assert L.qgemm_create(ctypes.byref(h), 2, 1, 0, 0, 1, 256, 512, 4) == q.OK        # forced GEMV
    assert L.qgemm_run_grouped(h, 4, 10, fake, fake, fake, fake, None) == q.ENOTSUP
    L.qgemm_destroy(h)


def test_grouped_route_choice():
    """qgemm_grouped_tier (host only): bf16 math with fewer than 64 rows per
    expert on average streams the experts (small-batch route), otherwise the
    large-batch kernel; forced tiers and fp32 math as documented."""
    cases = [  # (act, math, flags, E, T) -> tier
        ((1, 1, 0, 512, 20480), "skinny"),   # the benchmark's routed MoE: 40 rows per expert
        ((1, 1, 0, 4, 255), "skinny"),
        ((1, 1, 0, 4, 256), "tiled"),        # 64 rows per expert
        ((0, 1, 0, 4, 10), "skinny"),        # fp32 activations, bf16 math
        ((0, 0, 0, 4, 10), "tiled"),         # fp32-faithful math
        ((1, 1, 2, 4, 10), "tiled"),         # forced large-batch
        ((1, 1, 1, 4, 1000), "skinny"),      # forced small-batch, bf16 math
        ((0, 0, 1, 4, 10), "invalid"),       # forced small-batch, fp32 math
        ((1, 1, 4, 4, 10), "invalid"),       # forced GEMV
        ((1, 1, 0, 0, 10), "invalid"),       # E = 0
    ]
    for (act, math, flags, E, T), want in cases:
        plan = q.Plan("nvfp4", 256, 512, act="f32" if act == 0 else "bf16",
                      math="fp32" if math == 0 else "bf16",
                      tier={0: None, 1: "skinny", 2: "tiled", 4: "gemv"}[flags])
        assert plan.grouped_tier(E, T) == want, (act, math, flags, E, T)
