"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.  Tolerances (relative Frobenius error against the
unrounded fp64 oracle): 1e-5 for fp32 math, 1e-2 for bf16 math.  Decoded
weights, exact closed forms, one-hot read-outs and batch chunking are
compared bit for bit."""

import os

import numpy as np
import pytest
import torch

import oracle
import prefill_q8_mxfp4_amd as q
import synth

pytestmark = pytest.mark.gpu

TOL_FP32 = 1e-5
TOL_BF16 = 1e-2


def _dev():
    return torch.device("cuda:0")


def w_dev(w):
    return torch.from_numpy(q.pack_logical(w)).to(_dev())


def x_dev(x):
    if x.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(x)).to(_dev())
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(_dev())


def y_new(plan, B, fill=float("nan")):
    dt = torch.float32 if plan.out == "f32" else torch.bfloat16
    return torch.full((B, plan.out_cols), fill, dtype=dt, device=_dev())


def host(y):
    return y.float().cpu().numpy().astype(np.float64)


def run(plan, x, wd, B=None, workspace="auto"):
    B = x.shape[0] if B is None else B
    xd = x_dev(x)
    y = y_new(plan, B)
    plan.run(xd, wd, y, B=B, workspace=workspace)
    torch.cuda.synchronize()
    return host(y)


# ----------------------------------------------------------- dequantize

def _edge_weights(fmt, n, k, rng):
    if fmt == "fp8":
        # every E4M3 byte (NaN, subnormals, signed zero) and edge block scales
        codes = (np.arange(n * k) % 256).astype(np.uint8).reshape(n, k)
        rng.shuffle(codes.reshape(-1))
        s = (rng.standard_normal((n, -(-k // 128))) * 0.01).astype(np.float32)
        s.flat[:6] = [0.0, -0.0, 1e-40, 3e36, -2.0 ** -126, 1.0]  # subnormal, overflowing
        return {"fmt": fmt, "codes": codes, "scales": s, "g": None}
    if fmt == "q8_0":
        codes = rng.integers(-128, 128, (n, k)).astype(np.int8)
        d = rng.standard_normal((n, k // 32)).astype(np.float16).view(np.uint16)
        d.flat[:6] = [0x0001, 0x03FF, 0x7BFF, 0xFBFF, 0x8000, 0x0400]  # subnormal, max, -0
        return {"fmt": fmt, "codes": codes, "scales": d, "g": None}
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    if fmt == "mxfp4":
        e = rng.integers(100, 150, (n, k // 32)).astype(np.uint8)
        e.flat[:6] = [0, 1, 2, 127, 253, 255]
        return {"fmt": fmt, "codes": codes, "scales": e, "g": None}
    s = rng.integers(0, 256, (n, k // 16)).astype(np.uint8)
    s.flat[:6] = [0x00, 0x01, 0x07, 0x7E, 0x7F, 0xFF]
    return {"fmt": fmt, "codes": codes, "scales": s,
            "g": np.array([0.75, 3.0e-5], dtype=np.float32)}


@pytest.mark.parametrize("fmt,n,k", [("q8_0", 100, 96), ("mxfp4", 98, 160), ("nvfp4", 98, 144),
                                     ("q8_0", 256, 512), ("mxfp4", 64, 17408 // 8),
                                     ("fp8", 100, 320), ("fp8", 64, 96)])
def test_dequantize_bit_exact(fmt, n, k):
    rng = np.random.default_rng(n + k)
    w = _edge_weights(fmt, n, k, rng)
    got = q.dequantize(fmt, w_dev(w), n, k).cpu().numpy()
    with np.errstate(over="ignore", invalid="ignore"):
        ref = oracle.dequant(w, apply_g=True).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# ------------------------------------------------ small workload (Q8_0 256 x 512)

def test_q8_0_256x512_b70_fp32():
    c = synth.CONFIGS["q8_0_256x512"]
    w = synth.gen_config_weights("q8_0_256x512")
    x = synth.gen_config_x("q8_0_256x512", 70)
    plan = q.Plan("q8_0", c["N"], c["K"], act="f32", out="f32", math="fp32")
    y = run(plan, x, w_dev(w))
    ref = oracle.gemm(w, x)
    err = oracle.rel_fro(y, ref)
    print(f"q8_0 256x512 B=70 rel_fro={err:.3e}")
    assert err <= TOL_FP32
    bi = np.repeat(np.arange(70), 256)
    ni = np.tile(np.arange(256), 70)
    mag = oracle.gemm_abs_at(w, x, bi, ni).reshape(70, 256)
    _assert_componentwise(y, ref, 1.01 * mag, _nadds(512, 3), "q8_0 256x512 B=70 every output")


# ------------------------------------------- attention projection sweep

@pytest.fixture(scope="module")
def q8_attn():
    w = synth.gen_config_weights("q8_0_5120x5120")
    x = synth.gen_config_x("q8_0_5120x5120", 256)
    ref = oracle.gemm(w, x)  # rows are independent: prefixes serve every B
    return w, x, ref, w_dev(w)


@pytest.mark.parametrize("B", synth.CONFIGS["q8_0_5120x5120"]["Bs"])
def test_q8_0_5120_sweep_fp32(q8_attn, B):
    w, x, ref, wd = q8_attn
    plan = q.Plan("q8_0", 5120, 5120, act="f32", out="f32", math="fp32")
    y = run(plan, x[:B], wd)
    err = oracle.rel_fro(y, ref[:B])
    print(f"q8_0 5120x5120 B={B} tier={plan.tier(B)} rel_fro={err:.3e}")
    assert err <= TOL_FP32
    tid, nt = _full_tiles(B, 5120, tb=64)
    _assert_tiles(y.ravel(), ref[:B].ravel(), tid, nt, TOL_FP32, f"q8_0 5120 B={B} per tile")
    # three exact bf16 terms per activation, exact int8 codes: exact products
    bi, ni, _, _ = _tile_samples(B, 5120, 60 + B, tb=64)
    _assert_componentwise(y[bi, ni], ref[:B][bi, ni], 1.01 * oracle.gemm_abs_at(w, x[:B], bi, ni),
                          _nadds(5120, 3), f"q8_0 5120 B={B}")


@pytest.mark.parametrize("fmt,n,k", [("q8_0", 272, 2560), ("fp8", 208, 1536), ("mxfp4", 144, 2560),
                                     ("nvfp4", 200, 1536)])
def test_verify_kernel_rows_match_streaming_and_oracle(fmt, n, k):
    """fp32-faithful math at 16 < B <= 80 (the verify kernel, the MTP verify
    widths of the hipfire issue): every 16-row slice of a call is bitwise the
    streaming kernel's result on those rows alone (same row groups, K splits
    and summation order), with the K split and without a workspace, and every
    output meets the component-wise bound of exact products against the
    oracle.  Ragged row groups (N not a multiple of 128) included."""
    w = synth.gen_weights(fmt, n, k, seed=41)
    wd = w_dev(w)
    plan = q.Plan(fmt, n, k, act="f32", out="f32", math="fp32")
    xf = synth.gen_x_f32(80, k, seed=42)
    ref = oracle.gemm(w, xf)
    stream = {}
    for r0 in range(0, 80, 16):
        for wsp in ("auto", None):
            stream[r0, wsp] = run(plan, xf[r0:r0 + 16], wd, workspace=wsp)
    for B in (17, 31, 48, 64, 65, 76, 80):
        assert plan.tier(B) == "skinny"
        for wsp in ("auto", None):
            y = run(plan, xf[:B], wd, workspace=wsp)
            for r0 in range(0, B, 16):
                rows = min(16, B - r0)
                assert np.array_equal(y[r0:r0 + rows], stream[r0, wsp][:rows]), (B, wsp, r0)
        bi = np.repeat(np.arange(B), n)
        ni = np.tile(np.arange(n), B)
        mag = oracle.gemm_abs_at(w, xf[:B], bi, ni).reshape(B, n)
        _assert_componentwise(y, ref[:B], 1.01 * mag, _nadds(k, 3), f"{fmt} {n}x{k} B={B} verify")
        assert oracle.rel_fro(y, ref[:B]) <= TOL_FP32


@pytest.mark.parametrize("fmt,n,k,act", [("q8_0", 272, 2560, "f32"), ("fp8", 208, 1536, "bf16"),
                                         ("mxfp4", 144, 2560, "bf16"), ("nvfp4", 200, 1536, "f32")])
def test_verify_kernel_bf16_math_rows_match_streaming(fmt, n, k, act):
    """bf16 math at 16 < B <= 80 through the verify kernel (bf16 activations
    as they are, fp32 ones rounded to bf16 once): every 16-row slice bitwise
    the streaming kernel's result on those rows alone, with and without the
    K split, and within the bf16 tolerance of the oracle."""
    w = synth.gen_weights(fmt, n, k, seed=43)
    wd = w_dev(w)
    plan = q.Plan(fmt, n, k, act=act, out="f32", math="bf16")
    xf = synth.gen_x_f32(80, k, seed=44)
    x = xf if act == "f32" else synth.f32_to_bf16_bits(xf)
    ref = oracle.gemm(w, x)
    stream = {}
    for r0 in range(0, 80, 16):
        for wsp in ("auto", None):
            stream[r0, wsp] = run(plan, x[r0:r0 + 16], wd, workspace=wsp)
    for B in (17, 40, 64, 70, 80):
        if plan.tier(B) != "skinny":
            continue  # widths the default route sends to the tiled tier
        for wsp in ("auto", None):
            y = run(plan, x[:B], wd, workspace=wsp)
            for r0 in range(0, B, 16):
                rows = min(16, B - r0)
                assert np.array_equal(y[r0:r0 + rows], stream[r0, wsp][:rows]), (B, wsp, r0)
            assert oracle.rel_fro(y, ref[:B]) <= TOL_BF16, (B, wsp)


@pytest.mark.parametrize("fmt,nh,k,act", [("nvfp4", 1040, 2048, "bf16"), ("mxfp4", 528, 1536, "f32"),
                                          ("q8_0", 272, 1024, "bf16")])
def test_verify_kernel_swiglu_rows_match_streaming(fmt, nh, k, act):
    """The fused gate+up epilogue at 16 < B <= 48 through the verify kernel:
    every 16-row slice of SiLU(G)*U bitwise the streaming kernel's on those
    rows alone (ragged gate-tile groups included), with and without the K
    split, and within the SwiGLU tolerance of the oracle."""
    w = _gate_up(fmt, nh, k, 45)
    wd = w_dev(w)
    plan = q.Plan(fmt, 2 * nh, k, act=act, out="f32", epilogue="swiglu", math="bf16")
    xf = synth.gen_x_f32(80, k, seed=46)
    x = xf if act == "f32" else synth.f32_to_bf16_bits(xf)
    ref = oracle.swiglu(w, x)
    stream = {}
    for r0 in range(0, 80, 16):
        for wsp in ("auto", None):
            stream[r0, wsp] = run(plan, x[r0:r0 + 16], wd, workspace=wsp)
    for B in (17, 33, 48):  # above 48 rows the fused epilogue takes the tiled tier
        assert plan.tier(B) == "skinny"
        for wsp in ("auto", None):
            y = run(plan, x[:B], wd, workspace=wsp)
            for r0 in range(0, B, 16):
                rows = min(16, B - r0)
                assert np.array_equal(y[r0:r0 + rows], stream[r0, wsp][:rows]), (B, wsp, r0)
            # bf16 x: exact products, fp32 sums only; fp32 x: rounded to bf16 once
            assert oracle.rel_fro(y, ref[:B]) <= (1e-4 if act == "bf16" else TOL_BF16), (B, wsp)


@pytest.mark.parametrize("tier", ["skinny", "tiled"])
def test_boundary_matrix_chunked_is_bitwise(q8_attn, tier):
    """hipfire PR 'fix(mtp): chunk scalar Q8 batched GEMM above 64 rows',
    Scalar-Q8 boundary matrix: one call at B = 64/65/70/76/256 equals the
    same rows computed in contiguous chunks of 64, bit for bit.  The
    large-batch tier is compared on its unsplit route: its K split depends on
    the tile count, hence on B."""
    w, x, ref, wd = q8_attn
    math = "fp32" if tier == "skinny" else "bf16"
    plan = q.Plan("q8_0", 5120, 5120, act="f32", out="f32", math=math, tier=tier)
    wsp = "auto" if tier == "skinny" else None
    for B in (64, 65, 70, 76, 256):
        whole = run(plan, x[:B], wd, workspace=wsp)
        parts = [run(plan, x[r0:min(B, r0 + 64)], wd, workspace=wsp) for r0 in range(0, B, 64)]
        assert np.array_equal(whole, np.concatenate(parts, axis=0)), B
        tol = TOL_FP32 if math == "fp32" else TOL_BF16
        assert oracle.rel_fro(whole, ref[:B]) <= tol


def test_deterministic_and_row_independent(q8_attn):
    """Repeated calls agree bit for bit, and within the small-batch tier a
    row's result does not depend on how many other rows share the call (the
    summation order is fixed by N and K alone; the streaming kernel for
    B <= 16 and the skinny kernel above it share it up to 8 batch groups).
    The GEMV tier has an order of its own, equally independent of B."""
    w, x, ref, wd = q8_attn
    plan = q.Plan("q8_0", 5120, 5120, act="f32", out="f32", math="fp32", tier="skinny")
    y16 = run(plan, x[:16], wd)
    assert np.array_equal(y16, run(plan, x[:16], wd))
    for B in (1, 5, 33, 256):
        yb = run(plan, x[:B], wd)
        n = min(B, 16)
        assert np.array_equal(yb[:n], y16[:n]), B
    gv = q.Plan("q8_0", 5120, 5120, act="f32", out="f32", math="fp32", tier="gemv")
    y2 = run(gv, x[:2], wd)
    assert np.array_equal(y2, run(gv, x[:2], wd))
    assert np.array_equal(run(gv, x[:1], wd), y2[:1])


@pytest.mark.parametrize("B", (3, 16, 65, 256))
def test_split_k_and_unsplit_agree(q8_attn, B):
    """The K-split route (with a workspace) and the unsplit route both meet
    the fp32 bound, and the tile counters are re-armed after every call."""
    w, x, ref, wd = q8_attn
    plan = q.Plan("q8_0", 5120, 5120, act="f32", out="f32", math="fp32")
    assert plan.workspace_bytes(B) > 0
    ws = torch.zeros(plan.workspace_bytes(256) + (1 << 20), dtype=torch.uint8, device=_dev())
    for _ in range(3):
        assert oracle.rel_fro(run(plan, x[:B], wd, workspace=ws), ref[:B]) <= TOL_FP32
    assert oracle.rel_fro(run(plan, x[:B], wd, workspace=None), ref[:B]) <= TOL_FP32
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws[:128]) == 0  # tile counters re-armed


def test_dispatch_probe_finds_xcd_round_robin():
    """On the MI355X the dispatcher deals workgroup ids to the XCDs
    round-robin, so qgemm_init_device's probe enables the XCD-local exchange."""
    q.init_device()
    assert q.xcd_local() == 1


def test_dispatch_probe_during_graph_capture():
    """A fresh process whose first launch (the binding initialises the device
    then) is captured into a graph: the probe runs on a stream of its own in
    relaxed capture mode, the capture stays valid, and its replays match an
    eager call."""
    import subprocess
    import sys
    code = r"""
import numpy as np, torch, synth, prefill_q8_mxfp4_amd as q
w = synth.quantize("q8_0", synth.normal_f32(5, synth.SID_W, 1024, 2048, 0.02))
wd = torch.from_numpy(q.pack_logical(w)).cuda()
x = torch.from_numpy(synth.gen_x_f32(8, 2048, seed=3)).cuda()
y = torch.zeros((8, 1024), dtype=torch.float32, device="cuda")
st = torch.cuda.Stream()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g, stream=st):
    plan = q.Plan("q8_0", 1024, 2048, act="f32", out="f32")
    plan.run(x, wd, y, workspace=None)  # first launch: the binding's init_device probes here
assert q.xcd_local() == 1, q.xcd_local()
for _ in range(3):
    y.zero_()
    g.replay()
    torch.cuda.synchronize()
    ye = torch.zeros_like(y)
    plan.run(x, wd, ye, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(y, ye)
print("ok")
"""
    root = __file__.rsplit("/tests/", 1)[0]
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=180)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("fmt,n,k,act,epi", [
    ("q8_0", 5120, 5120, "f32", "none"),      # 40 row groups, 6 K splits: one round
    ("q8_0", 1664, 5120, "bf16", "none"),     # 13 groups: XCDs with one group more than others
    ("mxfp4", 6272, 8192, "f32", "none"),     # 49 groups, several rounds of workgroups
    ("nvfp4", 2 * 1040, 4096, "bf16", "swiglu"),  # 17 groups of 4 gate + 4 up tiles
])
def test_stream_split_exchange_modes_agree(fmt, n, k, act, epi, monkeypatch):
    """The streaming kernel's K splits meet through device-coherent memory or,
    with every split of a row group on one XCD, through that XCD's L2.  Both
    exchanges give bitwise the same output (same partials, same split order),
    it meets the oracle's bound, and the tile counters are re-armed."""
    if epi == "swiglu":
        w = _gate_up(fmt, n // 2, k, 41)
    else:
        w = synth.quantize(fmt, synth.normal_f32(41, synth.SID_W, n, k, 0.02))
    wd = w_dev(w)
    math = "fp32" if act == "f32" else "bf16"
    q.init_device()
    assert q.xcd_local() == 1
    plan = q.Plan(fmt, n, k, act=act, out="f32", math=math, epilogue=epi)  # XCD-local
    monkeypatch.setenv("QGEMM_ST_XLOCAL", "0")   # read at plan creation
    coh = q.Plan(fmt, n, k, act=act, out="f32", math=math, epilogue=epi)   # device-coherent
    monkeypatch.delenv("QGEMM_ST_XLOCAL")
    q.device_status(clear=True)
    for B in (3, 16) + ((70,) if math == "fp32" else ()):  # 70: the verify kernel
        assert plan.tier(B) == "skinny"
        x = synth.gen_x_f32(B, k, seed=B) if act == "f32" else synth.gen_x_bf16(B, k, seed=B)
        ws = torch.zeros(plan.workspace_bytes(B), dtype=torch.uint8, device=_dev())
        outs = []
        for p in (coh, plan, coh, plan):
            outs.append(run(p, x, wd, workspace=ws))
        for o in outs[1:]:
            assert np.array_equal(o, outs[0]), (B, fmt)
        assert torch.count_nonzero(ws[:4 * -(-n // 128)]) == 0  # row-group counters re-armed
        ref = oracle.swiglu(w, x) if epi == "swiglu" else oracle.gemm(w, x)
        err = oracle.rel_fro(outs[0], ref)
        tol = TOL_FP32 if math == "fp32" else (1e-4 if epi == "swiglu" else TOL_BF16)
        assert err <= tol, (B, fmt, err)
    assert q.device_status() == 0  # no workgroup ran off its probed XCD


def test_xcd_mismatch_is_detected():
    """The per-launch placement check of the XCD-local exchange, exercised in
    a fresh process on the debug build of the library: with QGEMM_XCC_FAKE=1
    the odd K splits of every row group report the next XCC, so the splits
    look spread over two XCDs and the launch sets QGEMM_DEV_XCD_MISMATCH
    (they really ran on one XCD, so the output is still bitwise that of the
    unperturbed plan); the unperturbed plan sets nothing."""
    import subprocess
    import sys
    code = r"""
import os, numpy as np, torch, synth, prefill_q8_mxfp4_amd as q
assert q.LIB_PATH.endswith("libqgemm_debug.so"), q.LIB_PATH
w = synth.gen_config_weights("q8_0_5120x5120")
wd = torch.from_numpy(q.pack_logical(w)).cuda()
q.init_device()
assert q.xcd_local() == 1
good = q.Plan("q8_0", 5120, 5120, act="f32", out="f32")
os.environ["QGEMM_XCC_FAKE"] = "1"
bad = q.Plan("q8_0", 5120, 5120, act="f32", out="f32")
q.device_status(clear=True)
for B in (3, 16, 70):
    x = torch.from_numpy(synth.gen_config_x("q8_0_5120x5120", B)).cuda()
    y0 = torch.full((B, 5120), float("nan"), device="cuda")
    y1 = torch.full((B, 5120), float("nan"), device="cuda")
    good.run(x, wd, y0)
    assert q.device_status() == 0
    bad.run(x, wd, y1)
    assert q.device_status(clear=True) == q.DEV_XCD_MISMATCH
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), B
    good.run(x, wd, y1)
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), B
assert q.device_status() == 0
print("ok")
"""
    root = __file__.rsplit("/tests/", 1)[0]
    env = dict(os.environ, QGEMM_LIB_PATH=os.path.join(root, "prefill_q8_mxfp4_amd", "libqgemm_debug.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=180,
                       env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:] + r.stderr[-2000:]


def test_workspace_reused_across_batch_widths(q8_attn):
    """One workspace, calls of alternating widths: every output is written and
    correct (the counters of one width are never hit by another width's
    partial tiles).  Outputs start as NaN so a skipped tile shows up."""
    w, x, ref, wd = q8_attn
    plan = q.Plan("q8_0", 5120, 5120, act="f32", out="f32", math="fp32")
    ws = torch.zeros(plan.workspace_bytes(256), dtype=torch.uint8, device=_dev())
    for B in (70, 6, 70, 64, 1, 256, 16, 70, 6):
        y = run(plan, x[:B], wd, workspace=ws)
        assert np.all(np.isfinite(y)), B
        assert oracle.rel_fro(y, ref[:B]) <= TOL_FP32, B


def test_workspace_shared_by_both_tiers(q8_attn):
    """One workspace for small- and large-batch calls of a bf16 plan: the
    large-batch pieces (left as written) must not land where the small-batch
    kernels look for published partial tiles.  Every call must match, bit for
    bit, the same call on a fresh zeroed workspace."""
    w, x, ref, wd = q8_attn
    plan = q.Plan("q8_0", 5120, 5120, act="bf16", out="f32")
    xb = np.tile(torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy(), (8, 1))  # 2048 rows
    need = max(plan.workspace_bytes(b) for b in (2048, 300, 16, 1))
    ws = torch.zeros(need, dtype=torch.uint8, device=_dev())
    for B in (2048, 16, 300, 1, 2048, 7, 16):
        xs = xb[:B]
        y = run(plan, xs, wd, workspace=ws)
        fresh = torch.zeros(plan.workspace_bytes(B), dtype=torch.uint8, device=_dev())
        y0 = run(plan, xs, wd, workspace=fresh if fresh.numel() else None)
        assert np.array_equal(y.view(np.uint32), y0.view(np.uint32)), B


# ------------------------------------------------- exact read-outs

@pytest.mark.parametrize("fmt,act,tier", [("q8_0", "f32", "skinny"), ("mxfp4", "bf16", "skinny"),
                                          ("nvfp4", "bf16", "skinny"), ("mxfp4", "bf16", "tiled"),
                                          ("nvfp4", "bf16", "tiled"), ("fp8", "f32", "skinny"),
                                          ("fp8", "bf16", "skinny"), ("q8_0", "f32", "tiled"),
                                          ("mxfp4", "f32", "tiled"), ("nvfp4", "f32", "tiled"),
                                          ("fp8", "f32", "tiled")])
def test_one_hot_reads_out_decoded_weights(fmt, act, tier):
    """x = e_j makes y[b][n] = w[n][j]: the decoded weights, read through the
    whole GEMM path, must be exact (fp32 activations run fp32-faithful math,
    in the large-batch tier too)."""
    n, k = 80, 512
    rng = np.random.default_rng(9)
    w = _edge_weights(fmt, n, k, rng)
    # keep scales in a normal range so every product stays exact
    if fmt == "q8_0":
        w["scales"] = rng.standard_normal((n, k // 32)).astype(np.float16).view(np.uint16)
    elif fmt == "mxfp4":
        w["scales"] = rng.integers(110, 140, (n, k // 32)).astype(np.uint8)
    elif fmt == "fp8":
        w["scales"] = (rng.random((n, k // 128)) + 0.5).astype(np.float32)
        w["codes"][(w["codes"] & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    else:
        w["scales"] = rng.integers(1, 0x7E, (n, k // 16)).astype(np.uint8)
        w["g"] = np.array([1.0, 1.0], dtype=np.float32)
    cols = [0, 1, 7, 8, 31, 32, 63, 64, 100, 127, 128, 255, 300, 511]
    xf = np.zeros((len(cols), k), dtype=np.float32)
    for i, j in enumerate(cols):
        xf[i, j] = 1.0
    x = xf if act == "f32" else synth.f32_to_bf16_bits(xf)
    plan = q.Plan(fmt, n, k, act=act, out="f32", tier=tier)
    y = run(plan, x, w_dev(w))
    dq = oracle.dequant(w, apply_g=True)
    assert np.array_equal(y, dq[:, cols].T.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("fmt", ["q8_0", "fp8"])
def test_one_hot_tiled_rounds_decoded_weights_once(fmt):
    """The large-batch tier folds the block scale into a bf16 operand: the
    one-hot read-out is the decoded weight rounded (fp32, then bf16) once."""
    n, k = 80, 512
    rng = np.random.default_rng(10)
    w = _edge_weights(fmt, n, k, rng)
    if fmt == "q8_0":
        w["scales"] = rng.standard_normal((n, k // 32)).astype(np.float16).view(np.uint16)
    else:
        w["scales"] = (rng.random((n, k // 128)) + 0.5).astype(np.float32)
        w["codes"][(w["codes"] & 0x7F) == 0x7F] = 0x3C
    cols = [0, 1, 31, 32, 63, 64, 127, 128, 300, 511]
    x = np.zeros((len(cols), k), dtype=np.float32)
    for i, j in enumerate(cols):
        x[i, j] = 1.0
    plan = q.Plan(fmt, n, k, act="bf16", out="f32", tier="tiled")
    y = run(plan, synth.f32_to_bf16_bits(x), w_dev(w))
    ref = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(oracle.dequant(w)[:, cols].T.astype(np.float32)))
    assert np.array_equal(y, ref.astype(np.float64))


@pytest.mark.parametrize("fmt,epi,n,k,B", [
    ("q8_0", "none", 768, 1056, 300),      # K tail, 3 x 3 tiles: a split partial round
    ("mxfp4", "none", 512, 2048, 2048),    # 256-row tiles, whole rounds
    ("nvfp4", "swiglu", 2 * 384, 1024, 200),
    ("fp8", "none", 640, 1024, 77),        # ragged weight tile and batch tile
])
def test_tiled_four_wave_form_is_bitwise_the_eight_wave_form(fmt, epi, n, k, B, monkeypatch):
    """The large-batch kernel with one wave per SIMD (QGEMM_TI_WAVES=4: 2 x 2
    waves, accumulators in AGPRs) runs the same tiles, K steps and split
    pieces in the same order as the default 8-wave form, so its output is
    bitwise the same; both meet the oracle's bf16-math bound."""
    if epi == "swiglu":
        w = _gate_up(fmt, n // 2, k, 43)
    else:
        w = synth.quantize(fmt, synth.normal_f32(43, synth.SID_W, n, k, 0.02))
    wd = w_dev(w)
    x = synth.gen_x_bf16(B, k, seed=5)
    out = "bf16" if epi == "swiglu" else "f32"
    p8 = q.Plan(fmt, n, k, act="bf16", out=out, math="bf16", epilogue=epi, tier="tiled")
    monkeypatch.setenv("QGEMM_TI_WAVES", "4")   # read at plan creation
    p4 = q.Plan(fmt, n, k, act="bf16", out=out, math="bf16", epilogue=epi, tier="tiled")
    monkeypatch.delenv("QGEMM_TI_WAVES")
    y8 = run(p8, x, wd)
    y4 = run(p4, x, wd)
    assert np.array_equal(y4, y8), (fmt, np.nanmax(np.abs(y4 - y8)))
    ref = oracle.swiglu(w, x) if epi == "swiglu" else oracle.gemm(w, x)
    assert oracle.rel_fro(y8, ref) <= TOL_BF16


@pytest.mark.parametrize("tier,math", [("skinny", "fp32"), ("tiled", "bf16"), ("tiled", "fp32")])
def test_closed_form_constant_is_exact(tier, math):
    """Constant q = 3, d = 2^-7, x = 0.5 over K = 5120: every output is
    K*d*q*x = 60 exactly and each row sums to N*K*d*q*x."""
    n, k, b = 96, 5120, 20
    w = {"fmt": "q8_0", "codes": np.full((n, k), 3, np.int8),
         "scales": np.full((n, k // 32), np.float16(2.0 ** -7).view(np.uint16), np.uint16),
         "g": None}
    x = np.full((b, k), 0.5, np.float32)
    plan = q.Plan("q8_0", n, k, act="f32", out="f32", math=math, tier=tier)
    y = run(plan, x, w_dev(w))
    assert np.all(y == 60.0)
    assert np.all(y.sum(axis=1) == n * k * 2.0 ** -7 * 3 * 0.5)


# ------------------------------------------------------ ragged shapes

@pytest.mark.parametrize("fmt,act,math,out", [
    ("q8_0", "f32", "fp32", "f32"), ("q8_0", "f32", "bf16", "f32"), ("q8_0", "bf16", "bf16", "bf16"),
    ("mxfp4", "bf16", "bf16", "f32"), ("mxfp4", "f32", "fp32", "f32"),
    ("nvfp4", "bf16", "bf16", "f32"), ("nvfp4", "f32", "fp32", "bf16"),
    ("fp8", "bf16", "bf16", "f32"), ("fp8", "f32", "fp32", "f32")])
@pytest.mark.parametrize("tier", ["skinny", "tiled"])
def test_ragged_shapes(fmt, act, math, out, tier):
    n = 100
    k = {"q8_0": 96, "mxfp4": 160, "nvfp4": 144, "fp8": 160}[fmt]
    w = synth.gen_weights(fmt, n, k, seed=1)
    for B in (1, 3, 17, 33, 65, 130):
        xf = synth.gen_x_f32(B, k, seed=2)
        x = xf if act == "f32" else synth.f32_to_bf16_bits(xf)
        plan = q.Plan(fmt, n, k, act=act, out=out, math=math, tier=tier)
        y = run(plan, x, w_dev(w))
        tol = TOL_FP32 if (math == "fp32" and out == "f32") else TOL_BF16
        err = oracle.rel_fro(y, oracle.gemm(w, x))
        assert err <= tol, (B, err)


@pytest.mark.parametrize("fmt", ["q8_0", "mxfp4", "fp8"])
def test_fp32_activations_rounded_once_in_the_workspace(fmt):
    """fp32 activations with bf16 math in the large-batch tier: with a
    workspace, x is rounded to bf16 once (nearest even) and the bf16 kernel
    runs, so the result equals, bit for bit, a bf16-activation call on the
    host-rounded rows with the same workspace; without one, the kernel rounds
    while staging and meets the same bound."""
    n, k, B = 1024, 512, 300
    w = synth.gen_weights(fmt, n, k, seed=21)
    xf = synth.gen_x_f32(B, k, seed=22)
    wd = w_dev(w)
    p32 = q.Plan(fmt, n, k, act="f32", out="f32", math="bf16")
    p16 = q.Plan(fmt, n, k, act="bf16", out="f32")
    assert p32.tier(B) == "tiled"
    need = p32.workspace_bytes(B)
    assert need >= p16.workspace_bytes(B) + B * k * 2
    ws = torch.zeros(need, dtype=torch.uint8, device=_dev())
    y32 = run(p32, xf, wd, workspace=ws)
    y16 = run(p16, synth.f32_to_bf16_bits(xf), wd, workspace=ws)
    assert np.array_equal(y32.view(np.uint64), y16.view(np.uint64))
    ref = oracle.gemm(w, xf)
    assert oracle.rel_fro(y32, ref) <= TOL_BF16
    assert oracle.rel_fro(run(p32, xf, wd, workspace=None), ref) <= TOL_BF16


@pytest.mark.parametrize("fmt,act,math,B", [("q8_0", "f32", "fp32", 16),     # streaming, K split
                                           ("q8_0", "f32", "fp32", 70),     # verify kernel, K split
                                           ("mxfp4", "bf16", "bf16", 40),   # skinny
                                           ("q8_0", "f32", "fp32", 100),    # fp32-faithful tiled
                                           ("nvfp4", "bf16", "bf16", 300),  # tiled, K split + reduce
                                           ("q8_0", "f32", "bf16", 300)])   # x rounded in the workspace
def test_graph_capture_replays(fmt, act, math, B):
    """qgemm_run captured in a HIP graph: every replay, with other work on
    the GPU between replays, reproduces the eager result bit for bit (the
    split counters are re-armed by the kernels; nothing is memset)."""
    n, k = 2048, 1024
    w = synth.gen_weights(fmt, n, k, seed=31)
    xf = synth.gen_x_f32(B, k, seed=32)
    x = xf if act == "f32" else synth.f32_to_bf16_bits(xf)
    wd, xd = w_dev(w), x_dev(x)
    plan = q.Plan(fmt, n, k, act=act, out="f32", math=math)
    ws = torch.zeros(max(plan.workspace_bytes(B), 256), dtype=torch.uint8, device=_dev())
    y0 = y_new(plan, B)
    plan.run(xd, wd, y0, workspace=ws)
    torch.cuda.synchronize()
    ref = host(y0)
    assert oracle.rel_fro(ref, oracle.gemm(w, x)) <= (TOL_FP32 if math == "fp32" else TOL_BF16)
    other = q.Plan(fmt, n, k, act=act, out="f32", math=math)
    yo = y_new(other, 7)
    st = torch.cuda.Stream()
    yg = y_new(plan, B)
    with torch.cuda.stream(st):
        plan.run(xd, wd, yg, workspace=ws)  # warm-up on the capture stream
    st.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        plan.run(xd, wd, yg, workspace=ws)
    for rep in range(3):
        yg.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(yg).view(np.uint64), ref.view(np.uint64)), rep
        other.run(xd[:7], wd, yo, workspace=None)  # unrelated eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("fmt,act,math,B,tier", [("q8_0", "f32", "fp32", 5, "skinny"),    # streaming
                                                ("mxfp4", "f32", "fp32", 100, "tiled"),   # fp32-faithful tiled
                                                ("fp8", "f32", "fp32", 40, "tiled"),
                                                ("nvfp4", "bf16", "bf16", 40, "skinny"),
                                                ("q8_0", "f32", "bf16", 300, "tiled")])
def test_activation_dynamic_range(fmt, act, math, B, tier):
    """Rows of one call scaled from 1e-20 to 1e20 (the pages' adversarial
    large-activation case, and its mirror): every row meets the bound on its
    own, so no row's accuracy depends on the others' magnitude."""
    n, k = 512, 1024
    w = synth.gen_weights(fmt, n, k, seed=41)
    xf = synth.gen_x_f32(B, k, seed=42)
    scale = (10.0 ** np.linspace(-20, 20, B)).astype(np.float32)
    xf = (xf * scale[:, None]).astype(np.float32)
    x = xf if act == "f32" else synth.f32_to_bf16_bits(xf)
    plan = q.Plan(fmt, n, k, act=act, out="f32", math=math, tier=tier)
    y = run(plan, x, w_dev(w))
    ref = oracle.gemm(w, x)
    tol = TOL_FP32 if math == "fp32" else TOL_BF16
    worst = max(oracle.rel_fro(y[b], ref[b]) for b in range(B))
    print(f"{fmt} {tier} {math} dynamic range: worst row rel_fro={worst:.3e}")
    assert np.all(np.isfinite(y))
    assert worst <= tol


def test_b_zero_is_a_noop():
    w = synth.gen_weights("q8_0", 32, 64, seed=1)
    plan = q.Plan("q8_0", 32, 64, act="f32")
    y = torch.full((1, 32), 7.0, device=_dev())
    plan.run(torch.zeros((1, 64), device=_dev()), w_dev(w), y, B=0)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


# ------------------------------------- prefill workloads, sampled outputs

def _samples(B, ncols, count, seed):
    rng = np.random.default_rng(seed)
    bi = rng.integers(0, B, count)
    ni = rng.integers(0, ncols, count)
    # always include the corners and the ragged edges
    bi[:4] = [0, B - 1, 0, B - 1]
    ni[:4] = [0, 0, ncols - 1, ncols - 1]
    return bi, ni


# Output tiles for the per-tile checks: 128 x 128 is no larger than any
# kernel's output tile in both directions (the large-batch tiles are 64-256
# batch rows x 256 weight rows, or 128 with the fused epilogue; a streaming
# workgroup owns 128 weight rows), so one wrong kernel tile makes at least
# one check tile wrong.
TB, TN = 128, 128
PER_TILE = 64
# Unit roundoff for the component-wise bounds: twice fp32's 2^-24, so that a
# matrix-core adder that truncates instead of rounding to nearest is covered.
U_ACC = 2.0 ** -23


def _tile_samples(B, ncols, seed, tb=TB, tn=TN, per_tile=PER_TILE):
    """per_tile random outputs inside every tb x tn tile of a [B][ncols]
    output (ragged edge tiles included) plus the four corners; returns row
    and column indices, each sample's tile id and the tile count."""
    rng = np.random.default_rng(seed)
    mt, nt = -(-B // tb), -(-ncols // tn)
    t = np.repeat(np.arange(mt * nt), per_tile)
    r0, c0 = (t // nt) * tb, (t % nt) * tn
    bi = r0 + (rng.random(t.size) * np.minimum(tb, B - r0)).astype(np.int64)
    ni = c0 + (rng.random(t.size) * np.minimum(tn, ncols - c0)).astype(np.int64)
    bi[:4] = [0, B - 1, 0, B - 1]
    ni[:4] = [0, 0, ncols - 1, ncols - 1]
    return bi, ni, (bi // tb) * nt + ni // tn, mt * nt


def _full_tiles(B, ncols, tb=TB, tn=TN):
    nt = -(-ncols // tn)
    return ((np.arange(B)[:, None] // tb) * nt + np.arange(ncols)[None, :] // tn).ravel(), \
        -(-B // tb) * nt


def _assert_tiles(y, ref, tid, ntiles, tol, label):
    """Every tile's relative Frobenius error within tol (NaN fails)."""
    per = oracle.rel_fro_groups(y, ref, tid, ntiles)
    assert not np.isnan(per).any(), f"{label}: NaN or empty tile"
    worst = int(np.argmax(per))
    print(f"{label}: {ntiles} tiles, median {np.median(per):.3e}, worst {per[worst]:.3e} "
          f"(tile {worst})")
    assert per[worst] <= tol, (label, worst, per[worst])


def _assert_componentwise(y, ref, mag, nadds, label):
    """|y - ref| <= gamma(nadds, U_ACC) * mag element by element: the
    forward error bound of a sum of exact products rounded nadds times (mag
    is sum |x||w|, slightly enlarged for split activations)."""
    y = np.asarray(y, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    bound = oracle.gamma(nadds, U_ACC) * np.asarray(mag, dtype=np.float64).ravel()
    excess = np.abs(y - ref) - bound
    assert not np.isnan(excess).any(), f"{label}: NaN"
    i = int(np.argmax(excess))
    print(f"{label}: component-wise max |err|/bound = "
          f"{np.max(np.abs(y - ref) / np.maximum(bound, 1e-300)):.3e} (n={nadds})")
    assert excess[i] <= 0, (label, i, float(y[i]), float(ref[i]), float(bound[i]))


def _nadds(K, terms):
    """Roundings per output of the exact-product paths: the K*terms products
    of a split activation summed in fp32, one block-scale FMA per 16 or 32
    columns, and the partial tiles of slabs and K splits (a generous 64)."""
    return terms * K + K // 16 + 64


def test_q8_0_ffn_prefill_2048_bf16():
    c = synth.CONFIGS["q8_0_ffn_17408x5120"]
    w = synth.gen_config_weights("q8_0_ffn_17408x5120")
    x = synth.gen_config_x("q8_0_ffn_17408x5120", 2048)
    plan = q.Plan("q8_0", c["N"], c["K"], act="f32", out="f32", math="bf16")
    assert plan.tier(2048) == "tiled"
    y = run(plan, x, w_dev(w))
    assert np.all(np.isfinite(y))
    bi, ni, tid, nt = _tile_samples(2048, c["N"], 3)
    ref = oracle.gemm_at(w, x, bi, ni)
    err = oracle.rel_fro(y[bi, ni], ref)
    print(f"q8_0 ffn rel_fro(sampled)={err:.3e}")
    assert err <= TOL_BF16
    _assert_tiles(y[bi, ni], ref, tid, nt, TOL_BF16, "q8_0 ffn B=2048 per tile (oracle samples)")


# -------------------------------------- full outputs against a library GEMM

def _library_ref(w, x, swiglu=False, magnitude=False):
    """Every output at full size: the oracle's decoded weights (fp64, tensor
    scales applied) times the activations as given, through torch's float64
    GEMM on the GPU (rocBLAS dgemm: every operand exact, error ~1e-16 of
    sum |x||w|), then SiLU(G) * U in fp64 for the fused epilogue.  With
    magnitude=True also |x| @ |w|^T, the magnitude sum of every output."""
    xf = (x if x.dtype == np.float32 else synth.bf16_bits_to_f32(x)).astype(np.float64)
    W = torch.from_numpy(oracle.dequant(w, apply_g=True)).to(_dev())
    X = torch.from_numpy(np.ascontiguousarray(xf)).to(_dev())
    y = torch.mm(X, W.t().contiguous())
    mag = torch.mm(X.abs(), W.abs().t().contiguous()).cpu().numpy() if magnitude else None
    del W, X
    if swiglu:
        nh = y.shape[1] // 2
        G, U = y[:, :nh], y[:, nh:]
        y = G * torch.sigmoid(G) * U
    out = y.cpu().numpy()
    del y
    torch.cuda.empty_cache()
    return (out, mag) if magnitude else out


@pytest.mark.parametrize("act,math,B", [("f32", "fp32", 4),     # streaming
                                         ("f32", "fp32", 70),    # verify kernel, hundreds of K splits
                                         ("bf16", "bf16", 48),   # verify kernel, bf16 math
                                         ("f32", "fp32", 100),   # fp32-faithful tiled, 96-row tiles
                                         ("bf16", "bf16", 300)])  # tiled, 128-row tiles
def test_largest_k(act, math, B):
    """K = 2^20, the largest K a plan accepts: every per-workgroup offset
    stays in range (against the dequantize-then-fp32-GEMM reduction)."""
    n, k = 256, 1 << 20
    w = synth.gen_weights("q8_0", n, k, seed=51)
    xf = synth.gen_x_f32(B, k, seed=52)
    x = xf if act == "f32" else synth.f32_to_bf16_bits(xf)
    plan = q.Plan("q8_0", n, k, act=act, out="f32", math=math)
    y = run(plan, x, w_dev(w))
    bi, ni = _samples(B, n, 200, 53)
    err = oracle.rel_fro(y[bi, ni], oracle.gemm_at(w, x, bi, ni))
    ref, mag = _library_ref(w, x, magnitude=True)
    lib = oracle.rel_fro(y, ref)
    print(f"K=2^20 B={B} {math} rel_fro(oracle samples)={err:.3e} (vs fp64 library GEMM {lib:.3e})")
    assert np.all(np.isfinite(y))
    tol = TOL_FP32 if math == "fp32" else TOL_BF16
    assert err <= tol
    assert lib <= tol
    tid, nt = _full_tiles(B, n, tn=64)
    _assert_tiles(y.ravel(), ref.ravel(), tid, nt, tol, f"K=2^20 B={B} per tile")
    if math == "fp32":
        _assert_componentwise(y, ref, mag * 1.01, _nadds(k, 3), f"K=2^20 B={B}")


@pytest.mark.parametrize("name,B", [("q8_0_ffn_17408x5120", 2048), ("mxfp4_down_5120x17408", 256), ("mxfp4_down_5120x17408", 2048), ("nvfp4_gate_up_34816x5120", 2048),
                                    ("fp8_5120x5120", 2048), ("q8_0_5120x5120", 256)])
def test_full_output_against_library_gemm(name, B):
    """Every output of the prefill-size workloads (not only the oracle's
    samples): against the dequantize-then-GEMM textbook reduction, within
    the path's bound (1e-5 fp32-faithful, 1e-2 bf16)."""
    c = synth.CONFIGS[name]
    w = synth.gen_config_weights(name)
    x = synth.gen_config_x(name, B)
    swiglu = c["epi"] == "swiglu"
    plan = q.Plan(c["fmt"], c["N"], c["K"], act=c["act"], out=c["out"],
                  epilogue="swiglu" if swiglu else "none", math=c["math"])
    y = run(plan, x, w_dev(w))
    # products are exact where the weights are exact in bf16 and the
    # activations are bf16 (MXFP4, NVFP4) or split into exact bf16 terms
    # (fp32-faithful math); Q8_0 and FP8 weights are rounded to bf16 with bf16 math
    exact = c["math"] == "fp32" or c["fmt"] in ("mxfp4", "nvfp4")
    want_mag = exact and not swiglu
    ref = _library_ref(w, x, swiglu, magnitude=want_mag)
    ref, mag = ref if want_mag else (ref, None)
    err = oracle.rel_fro(y, ref)
    tol = TOL_FP32 if (c["math"] == "fp32" and c["out"] == "f32") else TOL_BF16
    print(f"{name} B={B} full output vs library GEMM rel_fro={err:.3e}")
    assert np.all(np.isfinite(y))
    assert err <= tol
    tid, nt = _full_tiles(B, y.shape[1])
    _assert_tiles(y.ravel(), ref.ravel(), tid, nt, tol, f"{name} B={B} per tile (every output)")
    if want_mag:
        terms = 3 if c["math"] == "fp32" else 1
        _assert_componentwise(y, ref, mag * (1.01 if terms == 3 else 1.0), _nadds(c["K"], terms),
                              f"{name} B={B}")


@pytest.fixture(scope="module")
def mx_down():
    w = synth.gen_config_weights("mxfp4_down_5120x17408")
    x = synth.gen_config_x("mxfp4_down_5120x17408", 2048)
    return w, x, w_dev(w)


@pytest.mark.parametrize("B", synth.CONFIGS["mxfp4_down_5120x17408"]["Bs"])
def test_mxfp4_down_projection(mx_down, B):
    w, x, wd = mx_down
    plan = q.Plan("mxfp4", 5120, 17408, act="bf16", out="f32")
    y = run(plan, x[:B], wd)
    assert np.all(np.isfinite(y))
    bi, ni, tid, nt = _tile_samples(B, 5120, B)
    ref = oracle.gemm_at(w, x[:B], bi, ni)
    err = oracle.rel_fro(y[bi, ni], ref)
    print(f"mxfp4 down B={B} tier={plan.tier(B)} rel_fro(sampled)={err:.3e}")
    assert err <= TOL_BF16
    _assert_tiles(y[bi, ni], ref, tid, nt, TOL_BF16, f"mxfp4 down B={B} per tile")
    # E2M1 x E8M0 weights and bf16 activations: exact products
    _assert_componentwise(y[bi, ni], ref, oracle.gemm_abs_at(w, x[:B], bi, ni), _nadds(17408, 1),
                          f"mxfp4 down B={B}")


@pytest.fixture(scope="module")
def fp8_attn():
    w = synth.gen_config_weights("fp8_5120x5120")
    x = synth.gen_config_x("fp8_5120x5120", 2048)
    return w, x, w_dev(w)


@pytest.mark.parametrize("B", synth.CONFIGS["fp8_5120x5120"]["Bs"])
def test_fp8_attention_projection(fp8_attn, B):
    """FP8 E4M3 weights (128-wide block scales) x bf16 activations at the
    K = N = 5120 projection shape, every tier by B."""
    w, x, wd = fp8_attn
    plan = q.Plan("fp8", 5120, 5120, act="bf16", out="f32")
    y = run(plan, x[:B], wd)
    assert np.all(np.isfinite(y))
    bi, ni, tid, nt = _tile_samples(B, 5120, B + 7)
    ref = oracle.gemm_at(w, x[:B], bi, ni)
    err = oracle.rel_fro(y[bi, ni], ref)
    print(f"fp8 B={B} tier={plan.tier(B)} rel_fro(sampled)={err:.3e}")
    assert err <= TOL_BF16
    _assert_tiles(y[bi, ni], ref, tid, nt, TOL_BF16, f"fp8 B={B} per tile")


@pytest.mark.parametrize("B", [1, 16, 70])
def test_fp8_fp32_math(fp8_attn, B):
    """FP8 weights with fp32 activations in fp32-faithful math: 1e-5."""
    w, _, wd = fp8_attn
    x = synth.gen_x_f32(B, 5120, seed=3)
    plan = q.Plan("fp8", 5120, 5120, act="f32", out="f32", math="fp32")
    y = run(plan, x, wd)
    bi, ni, tid, nt = _tile_samples(B, 5120, B + 11)
    ref = oracle.gemm_at(w, x, bi, ni)
    err = oracle.rel_fro(y[bi, ni], ref)
    print(f"fp8 fp32-math B={B} rel_fro(sampled)={err:.3e}")
    assert err <= TOL_FP32
    _assert_tiles(y[bi, ni], ref, tid, nt, TOL_FP32, f"fp8 fp32-math B={B} per tile")
    _assert_componentwise(y[bi, ni], ref, 1.01 * oracle.gemm_abs_at(w, x, bi, ni), _nadds(5120, 3),
                          f"fp8 fp32-math B={B}")


def test_nvfp4_fused_gate_up_swiglu_2048():
    c = synth.CONFIGS["nvfp4_gate_up_34816x5120"]
    w = synth.gen_config_weights("nvfp4_gate_up_34816x5120")
    x = synth.gen_config_x("nvfp4_gate_up_34816x5120", 2048)
    plan = q.Plan("nvfp4", c["N"], c["K"], act="bf16", out="bf16", epilogue="swiglu")
    y = run(plan, x, w_dev(w))
    assert y.shape == (2048, c["N"] // 2)
    assert np.all(np.isfinite(y))
    bi, ji, tid, nt = _tile_samples(2048, c["N"] // 2, 5)
    ref = oracle.swiglu_at(w, x, bi, ji)
    err = oracle.rel_fro(y[bi, ji], ref)
    print(f"nvfp4 gate+up rel_fro(sampled)={err:.3e}")
    assert err <= TOL_BF16
    _assert_tiles(y[bi, ji], ref, tid, nt, TOL_BF16, "nvfp4 gate+up B=2048 per tile")


def test_swiglu_small_exhaustive():
    rng = np.random.default_rng(12)
    nh, k = 48, 160
    w = _edge_weights("nvfp4", 2 * nh, k, rng)
    w["scales"] = rng.integers(0x20, 0x50, (2 * nh, k // 16)).astype(np.uint8)
    w["g"] = np.array([0.01, 0.02], dtype=np.float32)
    for B in (1, 5, 130):
        x = synth.gen_x_bf16(B, k, seed=B)
        plan = q.Plan("nvfp4", 2 * nh, k, act="bf16", out="f32", epilogue="swiglu")
        y = run(plan, x, w_dev(w))
        assert oracle.rel_fro(y, oracle.swiglu(w, x)) <= 1e-3


@pytest.mark.parametrize("tier,math", [("skinny", "bf16"), ("tiled", "bf16"), ("tiled", "fp32")])
def test_mxfp4_extreme_scales_one_hot(tier, math):
    """E8M0 scale bytes at both ends of the range (subnormal and near-overflow
    products) read out exactly through the GEMM path."""
    n, k = 32, 256
    rng = np.random.default_rng(21)
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    e = rng.choice(np.array([1, 2, 3, 4, 126, 127, 250, 251, 252], dtype=np.uint8), (n, k // 32))
    w = {"fmt": "mxfp4", "codes": codes, "scales": e, "g": None}
    cols = [0, 9, 33, 70, 127, 128, 200, 255]
    xf = np.zeros((len(cols), k), dtype=np.float32)
    for i, j in enumerate(cols):
        xf[i, j] = 1.0
    if math == "fp32":
        plan = q.Plan("mxfp4", n, k, act="f32", out="f32", math="fp32", tier=tier)
        y = run(plan, xf, w_dev(w))
    else:
        plan = q.Plan("mxfp4", n, k, act="bf16", out="f32", tier=tier)
        y = run(plan, synth.f32_to_bf16_bits(xf), w_dev(w))
    ref = oracle.dequant(w)[:, cols].T.astype(np.float32).astype(np.float64)
    bad = np.argwhere(y != ref)
    assert bad.size == 0, [(int(i), int(j), y[i, j], ref[i, j]) for i, j in bad[:8]]


# ------------------------------------------- fused gate+up, small batch

def _gate_up(fmt, nh, k, seed):
    """Gate and up halves quantized as two tensors (own tensor scale each)."""
    parts = [synth.quantize(fmt, synth.normal_f32(seed, synth.SID_W + h, nh, k, 0.02)) for h in (0, 1)]
    w = {"fmt": fmt, "codes": np.concatenate([p["codes"] for p in parts]),
         "scales": np.concatenate([p["scales"] for p in parts]), "g": None}
    if fmt == "nvfp4":
        w["g"] = np.concatenate([p["g"] for p in parts]).astype(np.float32)
    return w


@pytest.mark.parametrize("fmt", ["q8_0", "mxfp4", "nvfp4"])
def test_swiglu_streaming_small_batch(fmt):
    """B <= 16 SwiGLU runs in the streaming kernel (gate and up tiles of a
    column in one workgroup, K split or not) and matches the fp64 oracle."""
    nh, k = 320, 1024
    w = _gate_up(fmt, nh, k, 31)
    wd = w_dev(w)
    plan = q.Plan(fmt, 2 * nh, k, act="bf16", out="f32", epilogue="swiglu", tier="skinny")
    for B in (1, 3, 7, 16):
        assert plan.tier(B) == "skinny"
        x = synth.gen_x_bf16(B, k, seed=B)
        ref = oracle.swiglu(w, x)
        for ws in ("auto", None):
            y = run(plan, x, wd, workspace=ws)
            err = oracle.rel_fro(y, ref)
            assert err <= 1e-4, (B, ws, err)


def test_swiglu_streaming_gate_up_shape_b16():
    """The NVFP4 fused gate+up shape (K = 5120, N = 2 x 17408) at B = 16,
    bf16 output, checked on sampled outputs."""
    c = synth.CONFIGS["nvfp4_gate_up_34816x5120"]
    w = synth.gen_config_weights("nvfp4_gate_up_34816x5120")
    x = synth.gen_config_x("nvfp4_gate_up_34816x5120", 16)
    plan = q.Plan("nvfp4", c["N"], c["K"], act="bf16", out="bf16", epilogue="swiglu")
    assert plan.tier(16) == "skinny"
    y = run(plan, x, w_dev(w))
    bi, ji = _samples(16, c["N"] // 2, 4000, 6)
    err = oracle.rel_fro(y[bi, ji], oracle.swiglu_at(w, x, bi, ji))
    assert err <= TOL_BF16, err


def test_swiglu_forced_skinny_limits():
    """A SwiGLU plan forced to the small-batch tier runs B <= 48 when K is a
    whole number of slabs (the verify kernel above 16 rows) and refuses wider
    calls, or B > 16 with a partial last slab, with QGEMM_ENOTSUP."""
    w = _gate_up("nvfp4", 64, 256, 3)
    plan = q.Plan("nvfp4", 128, 256, act="bf16", out="f32", epilogue="swiglu", tier="skinny")
    x = synth.gen_x_bf16(49, 256)
    y = run(plan, x[:48], w_dev(w))
    assert oracle.rel_fro(y, oracle.swiglu(w, x[:48])) <= 1e-4
    with pytest.raises(q.QgemmError) as e:
        run(plan, x, w_dev(w))
    assert e.value.status == q.ENOTSUP
    w = _gate_up("nvfp4", 64, 144, 3)
    plan = q.Plan("nvfp4", 128, 144, act="bf16", out="f32", epilogue="swiglu", tier="skinny")
    with pytest.raises(q.QgemmError) as e:
        run(plan, synth.gen_x_bf16(17, 144), w_dev(w))
    assert e.value.status == q.ENOTSUP


# ------------------------------------------------------------ routed experts

def _solo_rows(plan, tier, x_rows, buf):
    """One expert's rows as the routed call computes them: qgemm_run of that
    expert alone, without a workspace, in the route's tier (the small-batch
    route in calls of at most 16 rows: a row's result there does not depend
    on the other rows, and a SwiGLU plan forced to that tier takes B <= 16)."""
    solo = q.Plan(plan.fmt, plan.N, plan.K, act=plan.act, out=plan.out, epilogue=plan.epilogue,
                  math=plan.math, tier=tier)
    if tier == "tiled":
        return run(solo, x_rows, buf, workspace=None)
    return np.concatenate([run(solo, x_rows[i:i + 16], buf, workspace=None)
                           for i in range(0, x_rows.shape[0], 16)])


def _assert_experts_bitwise(plan, offsets, x, bufs, y, tier):
    for e in range(len(offsets) - 1):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            ye = _solo_rows(plan, tier, x[r0:r1], bufs[e])
            assert np.array_equal(ye.astype(np.float32).view(np.uint32),
                                  y[r0:r1].astype(np.float32).view(np.uint32)), (tier, e)


def _grouped_case(fmt, act, out, epi, E, n, k, offsets, seed, math="bf16", tier=None):
    ws = [synth.gen_expert_weights(fmt, n, k, e, seed=seed, swiglu=epi == "swiglu") for e in range(E)]
    T = int(offsets[-1])
    xf = synth.gen_x_f32(T, k, seed=seed + 1)
    x = xf if act == "f32" else synth.f32_to_bf16_bits(xf)
    bufs = [w_dev(w) for w in ws]
    table = torch.tensor([b.data_ptr() for b in bufs], dtype=torch.int64, device=_dev())
    off = torch.from_numpy(np.asarray(offsets, dtype=np.int32)).to(_dev())
    plan = q.Plan(fmt, n, k, act=act, out=out, epilogue=epi, math=math, tier=tier)
    y = y_new(plan, T)
    plan.run_grouped(x_dev(x), table, off, y)
    torch.cuda.synchronize()
    return ws, bufs, x, host(y), plan


@pytest.mark.parametrize("fmt,act,out,epi", [("nvfp4", "bf16", "bf16", "swiglu"),
                                             ("mxfp4", "bf16", "f32", "none"),
                                             ("q8_0", "f32", "f32", "none"),
                                             ("fp8", "bf16", "f32", "swiglu")])
@pytest.mark.parametrize("tier", ["tiled", "skinny"])
def test_grouped_matches_oracle_and_per_expert_calls(fmt, act, out, epi, tier):
    """Routed experts in one launch, on both routes (forced: the large-batch
    kernel, and the streaming kernel over (expert, row-tile group) items):
    each expert's rows match the fp64 oracle and, bit for bit, calls of that
    expert alone in the route's tier (empty experts, one-row experts, an
    expert of 300 rows, i.e. five passes of 64 rows, and ragged ones)."""
    n, k = 256, 512
    rows = [5, 0, 1, 300, 17, 0, 128, 129, 2, 40]
    offsets = np.concatenate([[0], np.cumsum(rows)])
    E = len(rows)
    ws, bufs, x, y, plan = _grouped_case(fmt, act, out, epi, E, n, k, offsets, seed=3, tier=tier)
    assert plan.grouped_tier(E, int(offsets[-1])) == tier
    ref = oracle.gemm_grouped(ws, offsets, x, swiglu_epi=epi == "swiglu")
    err = oracle.rel_fro(y, ref)
    print(f"grouped {tier} {fmt} {epi} rel_fro={err:.3e}")
    assert err <= TOL_BF16
    _assert_experts_bitwise(plan, offsets, x, bufs, y, tier)


@pytest.mark.parametrize("fmt,epi", [("nvfp4", "swiglu"), ("mxfp4", "none"), ("q8_0", "swiglu"),
                                     ("fp8", "none")])
def test_grouped_streaming_route_k_tails_and_wide_rows(fmt, epi):
    """The streaming route with K not a multiple of the slab (K = 1056: the
    last slab has padding units; NVFP4 also K = 1040, half a unit), more
    output tiles than one workgroup covers (N = 608, a partial group) and
    automatic routing (T < 64 E): oracle bound and per-expert bitwise."""
    ks = (1056, 1040) if fmt == "nvfp4" else (1056,)
    for k in ks:
        n = 608
        rows = [33, 1, 0, 64, 65, 16, 0, 7]
        offsets = np.concatenate([[0], np.cumsum(rows)])
        E = len(rows)
        ws, bufs, x, y, plan = _grouped_case(fmt, "bf16", "f32", epi, E, n, k, offsets, seed=11)
        assert plan.grouped_tier(E, int(offsets[-1])) == "skinny"
        err = oracle.rel_fro(y, oracle.gemm_grouped(ws, offsets, x, swiglu_epi=epi == "swiglu"))
        print(f"grouped streaming {fmt} {epi} K={k} rel_fro={err:.3e}")
        assert err <= TOL_BF16
        _assert_experts_bitwise(plan, offsets, x, bufs, y, "skinny")


@pytest.mark.parametrize("fmt", ["q8_0", "mxfp4", "nvfp4", "fp8"])
def test_grouped_fp32_math(fmt):
    """Routed experts with fp32-faithful math: within the fp32 bound of the
    oracle and, bit for bit, an unsplit large-batch call of each expert."""
    n, k = 256, 512
    rows = [5, 0, 1, 150, 17, 64, 65, 2]
    offsets = np.concatenate([[0], np.cumsum(rows)])
    E = len(rows)
    ws, bufs, x, y, plan = _grouped_case(fmt, "f32", "f32", "none", E, n, k, offsets, seed=4,
                                         math="fp32")
    err = oracle.rel_fro(y, oracle.gemm_grouped(ws, offsets, x))
    print(f"grouped fp32 {fmt} rel_fro={err:.3e}")
    assert err <= TOL_FP32
    assert plan.grouped_tier(E, int(offsets[-1])) == "tiled"
    _assert_experts_bitwise(plan, offsets, x, bufs, y, "tiled")


def test_grouped_graph_capture_replays():
    """qgemm_run_grouped captured in a HIP graph replays bit-identically."""
    n, k = 256, 512
    rows = [5, 0, 1, 150, 17, 64, 65, 2]
    offsets = np.concatenate([[0], np.cumsum(rows)])
    ws, bufs, x, y, plan = _grouped_case("nvfp4", "bf16", "bf16", "swiglu", len(rows), 2 * n, k, offsets,
                                         seed=6)
    table = torch.tensor([b.data_ptr() for b in bufs], dtype=torch.int64, device=_dev())
    off = torch.from_numpy(np.asarray(offsets, dtype=np.int32)).to(_dev())
    xd = x_dev(x)
    yg = y_new(plan, int(offsets[-1]))
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        plan.run_grouped(xd, table, off, yg)
    st.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        plan.run_grouped(xd, table, off, yg)
    for rep in range(3):
        yg.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(yg), y), rep


def test_grouped_many_experts_top_k_routing():
    """600 experts (more than one scan chunk of the kernel's prologue), top-4
    routing of 100 tokens: most experts get zero or one row."""
    E, n, k = 600, 256, 64
    tok, offsets = synth.gen_routing(100, 4, E, seed=1)
    ws, bufs, x, y, plan = _grouped_case("mxfp4", "bf16", "f32", "none", E, n, k, offsets, seed=5)
    ref = oracle.gemm_grouped(ws, offsets, x)
    assert oracle.rel_fro(y, ref) <= TOL_BF16


def test_grouped_single_expert_and_empty():
    n, k = 128, 256
    offsets = np.array([0, 77])
    ws, bufs, x, y, plan = _grouped_case("nvfp4", "bf16", "f32", "none", 1, n, k, offsets, seed=7)
    assert plan.grouped_tier(1, 77) == "tiled"  # 77 rows per expert: the large-batch route
    _assert_experts_bitwise(plan, offsets, x, bufs, y, "tiled")
    # T = 0: nothing enqueued, OK returned
    table = torch.tensor([bufs[0].data_ptr()], dtype=torch.int64, device=_dev())
    off = torch.zeros(2, dtype=torch.int32, device=_dev())
    xe = torch.empty((0, k), dtype=torch.bfloat16, device=_dev())
    ye = torch.empty((0, n), dtype=torch.float32, device=_dev())
    plan.run_grouped(xe, table, off, ye)


def test_grouped_benched_moe_shape():
    """The routed-expert workload the benchmark times: 512 NVFP4 experts of
    2 x 512 gate+up rows, K = 2048, top-10 routing of 2048 tokens (20,480
    rows; eight generated experts copied into 512 buffers, as the benchmark
    does).  Every (expert, 128-column) output tile within the bf16 bound on
    at least 64 oracle samples, and every expert's rows bitwise those of
    calls of that expert alone in the route's tier (the streaming route:
    40 rows per expert on average)."""
    E, topk, tokens, nh, K = 512, 10, 2048, 512, 2048
    distinct = [synth.gen_expert_weights("nvfp4", 2 * nh, K, e, swiglu=True) for e in range(8)]
    packed = [w_dev(w) for w in distinct]
    bufs = [packed[e % 8].clone() for e in range(E)]
    table = torch.tensor([b.data_ptr() for b in bufs], dtype=torch.int64, device=_dev())
    tok, offsets = synth.gen_routing(tokens, topk, E)
    T = int(offsets[-1])
    assert T == tokens * topk
    x = synth.gen_x_bf16(tokens, K)[tok]
    plan = q.Plan("nvfp4", 2 * nh, K, act="bf16", out="bf16", epilogue="swiglu")
    assert plan.grouped_tier(E, T) == "skinny"
    y = y_new(plan, T)
    plan.run_grouped(x_dev(x), table, torch.from_numpy(offsets.astype(np.int32)).to(_dev()), y)
    torch.cuda.synchronize()
    y = host(y)
    assert np.all(np.isfinite(y))
    # PER_TILE samples in every (expert with rows, 128-column) tile
    rng = np.random.default_rng(77)
    rows = np.diff(offsets)
    live = np.nonzero(rows)[0]
    ct = nh // 128
    e_s = np.repeat(live, ct * PER_TILE)
    c_s = np.tile(np.repeat(np.arange(ct), PER_TILE), live.size)
    bi = offsets[e_s] + (rng.random(e_s.size) * rows[e_s]).astype(np.int64)
    ji = c_s * 128 + rng.integers(0, 128, e_s.size)
    tid = np.repeat(np.arange(live.size * ct), PER_TILE)
    ref = np.empty(bi.size)
    for d in range(8):
        sel = e_s % 8 == d
        ref[sel] = oracle.swiglu_at(distinct[d], x, bi[sel], ji[sel])
    err = oracle.rel_fro(y[bi, ji], ref)
    print(f"routed moe 512 experts rel_fro(sampled)={err:.3e}")
    assert err <= TOL_BF16
    _assert_tiles(y[bi, ji], ref, tid, live.size * ct, TOL_BF16, "routed moe per (expert, tile)")
    for e in live:
        r0, r1 = offsets[e], offsets[e + 1]
        ye = _solo_rows(plan, "skinny", x[r0:r1], bufs[e])
        assert np.array_equal(ye.astype(np.float32).view(np.uint32),
                              y[r0:r1].astype(np.float32).view(np.uint32)), e


@pytest.mark.parametrize("case", ["decreasing", "first_not_zero", "last_not_T", "negative"])
@pytest.mark.parametrize("tier", ["tiled", "skinny"])
def test_grouped_bad_offsets_do_nothing_and_report(case, tier):
    """Offsets that break their rules (non-decreasing, offsets[0] = 0,
    offsets[E] = T): the launch writes nothing (y keeps its NaN fill) and
    sets QGEMM_DEV_BAD_OFFSETS; good offsets afterwards run normally and set
    nothing."""
    n, k = 256, 512
    rows = [5, 0, 40, 17]
    good = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    T = int(good[-1])
    bad = good.copy()
    if case == "decreasing":
        bad[2], bad[3] = bad[3], bad[2]
    elif case == "first_not_zero":
        bad[0] = 3
    elif case == "last_not_T":
        bad[-1] = T + 1000000
    else:
        bad[1] = -1000000
    ws = [synth.gen_expert_weights("mxfp4", n, k, e, seed=9) for e in range(len(rows))]
    bufs = [w_dev(w) for w in ws]
    table = torch.tensor([b.data_ptr() for b in bufs], dtype=torch.int64, device=_dev())
    x = synth.gen_x_bf16(T, k, seed=10)
    xd = x_dev(x)
    plan = q.Plan("mxfp4", n, k, act="bf16", out="f32", tier=tier)
    assert plan.grouped_tier(len(rows), T) == tier
    q.device_status(clear=True)
    y = y_new(plan, T)
    plan.run_grouped(xd, table, torch.from_numpy(bad).to(_dev()), y)
    assert q.device_status(clear=True) == q.DEV_BAD_OFFSETS
    assert torch.isnan(y).all()
    plan.run_grouped(xd, table, torch.from_numpy(good).to(_dev()), y)
    assert q.device_status() == 0
    ref = oracle.gemm_grouped(ws, good, x)
    assert oracle.rel_fro(host(y), ref) <= TOL_BF16


@pytest.mark.parametrize("fmt", ["q8_0", "mxfp4", "nvfp4", "fp8"])
@pytest.mark.parametrize("act,out", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_gemv_narrow_batches(fmt, act, out):
    """B = 1 and 2 in the GEMV tier (forced: one workgroup per row tile over
    all of K, fp32 FMA) in every format: K = 5120 (five slabs a wave) and 17408
    (nine: the register ring turns over), a ragged N; against the oracle
    element by element (component-wise bound: exact decoded weights, fp32
    FMA accumulation) and row 0 bitwise the same at B = 1 and B = 2; no
    workspace needed."""
    for n, k in ((1000, 5120), (272, 17408)):
        w = synth.gen_weights(fmt, n, k, seed=71)
        xf = synth.gen_x_f32(2, k, seed=72)
        x = xf if act == "f32" else synth.f32_to_bf16_bits(xf)
        plan = q.Plan(fmt, n, k, act=act, out=out, tier="gemv")
        ys = []
        # two fp32 rows of K = 17408 exceed the kernel's LDS budget
        for B in (1, 2) if 2 * k * 4 <= 72 * 1024 else (1,):
            assert plan.tier(B) == "gemv" and plan.workspace_bytes(B) == 0
            y = run(plan, x[:B], w_dev(w))
            ref = oracle.gemm(w, x[:B])
            bi = np.repeat(np.arange(B), n)
            ni = np.tile(np.arange(n), B)
            mag = oracle.gemm_abs_at(w, x[:B], bi, ni).reshape(B, n)
            tol = TOL_FP32 if out == "f32" else TOL_BF16
            assert oracle.rel_fro(y, ref) <= tol, (B, n, k)
            if out == "f32":
                _assert_componentwise(y, ref, mag, _nadds(k, 1), f"gemv {fmt} {act} B={B} K={k}")
            ys.append(y)
        if len(ys) == 2:
            assert np.array_equal(ys[0], ys[1][:1])


@pytest.mark.parametrize("fmt", ["q8_0", "mxfp4", "nvfp4"])
def test_gemv_swiglu_and_graph_replay(fmt):
    """Fused gate+up at B = 1 and 2 in the GEMV kernel (a workgroup owns a
    gate tile and its up tile) against the oracle, and a captured graph of
    it replayed bit-identically."""
    nh, k = 1088, 5120
    w = _gate_up(fmt, nh, k, 81)
    wd = w_dev(w)
    plan = q.Plan(fmt, 2 * nh, k, act="bf16", out="bf16", epilogue="swiglu", tier="gemv")
    for B in (1, 2):
        x = synth.gen_x_bf16(B, k, seed=82 + B)
        y = run(plan, x, wd)
        bi, ji, tid, nt = _tile_samples(B, nh, 83, tb=16, tn=16, per_tile=8)
        ref = oracle.swiglu_at(w, x, bi, ji)
        assert oracle.rel_fro(y[bi, ji], ref) <= TOL_BF16, B
        _assert_tiles(y[bi, ji], ref, tid, nt, TOL_BF16, f"gemv swiglu {fmt} B={B} per tile")
    xd = x_dev(x)
    yg = y_new(plan, 2)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        plan.run(xd, wd, yg)
    st.synchronize()
    want = host(yg)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        plan.run(xd, wd, yg)
    for rep_ in range(3):
        yg.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(yg), want), rep_


def test_gemv_tier_forced_and_refused():
    """A plan forced to the GEMV tier runs B = 1, 2 and refuses wider calls
    and activation rows past its LDS budget with QGEMM_ENOTSUP; routed
    experts refuse a plan forced to it."""
    w = synth.gen_weights("q8_0", 256, 512, seed=91)
    x = synth.gen_x_f32(3, 512, seed=92)
    plan = q.Plan("q8_0", 256, 512, act="f32", out="f32", tier="gemv")
    assert oracle.rel_fro(run(plan, x[:2], w_dev(w)), oracle.gemm(w, x[:2])) <= TOL_FP32
    with pytest.raises(q.QgemmError) as e:
        run(plan, x, w_dev(w))
    assert e.value.status == q.ENOTSUP
    big = q.Plan("mxfp4", 256, 32768, act="bf16", out="f32", tier="gemv")   # 128 KB of fp32 rows
    xb = torch.zeros((1, 32768), dtype=torch.bfloat16, device=_dev())
    wb = torch.zeros(q.weight_bytes("mxfp4", 256, 32768), dtype=torch.uint8, device=_dev())
    with pytest.raises(q.QgemmError) as e:
        big.run(xb, wb, y_new(big, 1))
    assert e.value.status == q.ENOTSUP


# ------------------------------------------------------ measurement aids

@pytest.mark.parametrize("nbytes,wgs", [(27852800, 0), (16 * 1000003, 300), (4096, 7)])
def test_read_bytes_reads_every_byte_once(nbytes, wgs):
    """The plain read kernel behind the bench's bandwidth ceiling: the XOR of
    its per-workgroup words equals the XOR of every 32-bit word of the
    buffer (each 16-byte chunk read exactly once)."""
    rng = np.random.default_rng(nbytes % 1000)
    host_words = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host_words.view(np.int32)).to(_dev())
    n = wgs or 2048
    sink = torch.zeros(n, dtype=torch.int32, device=_dev())
    q.read_bytes(buf, sink, wgs=wgs)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host_words)


def test_mfma_rate_modes_run():
    sink = torch.zeros(4096, dtype=torch.int32, device=_dev())
    for mode in q.MFMA_RATE_MODES:
        sink.zero_()
        q.mfma_rate(mode, 8, sink)
        torch.cuda.synchronize()
        assert torch.count_nonzero(sink) > 0, mode
    with pytest.raises(q.QgemmError):
        q.mfma_rate(8, 8, sink)
