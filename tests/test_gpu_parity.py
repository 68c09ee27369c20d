"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.  Tolerances (relative Frobenius error against the
unrounded fp64 oracle): 1e-5 for fp32 math, 1e-2 for bf16 math.  Decoded
weights, exact closed forms, one-hot read-outs and batch chunking are
compared bit for bit."""

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
    err = oracle.rel_fro(y, oracle.gemm(w, x))
    print(f"q8_0 256x512 B=70 rel_fro={err:.3e}")
    assert err <= TOL_FP32


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
    """Repeated calls agree bit for bit, and within the small-batch tiers a
    row's result does not depend on how many other rows share the call (the
    summation order is fixed by N and K alone)."""
    w, x, ref, wd = q8_attn
    plan = q.Plan("q8_0", 5120, 5120, act="f32", out="f32", math="fp32", tier="skinny")
    y16 = run(plan, x[:16], wd)
    assert np.array_equal(y16, run(plan, x[:16], wd))
    for B in (1, 5, 33, 256):
        yb = run(plan, x[:B], wd)
        n = min(B, 16)
        assert np.array_equal(yb[:n], y16[:n]), B


@pytest.mark.parametrize("B", (1, 16, 65, 256))
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
    round-robin, so qgemm_create's probe enables the XCD-local exchange."""
    q.Plan("q8_0", 256, 512, act="f32", out="f32")
    assert q.xcd_local() == 1


def test_dispatch_probe_during_graph_capture():
    """A fresh process whose first plan is created while a graph is being
    captured on another stream: the probe runs on a stream of its own in
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
    plan = q.Plan("q8_0", 1024, 2048, act="f32", out="f32")  # first plan: the probe runs here
    plan.run(x, wd, y, workspace=None)
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
    plan = q.Plan(fmt, n, k, act=act, out="f32", math=math, epilogue=epi)
    for B in (1, 16):
        assert plan.tier(B) == "skinny"
        x = synth.gen_x_f32(B, k, seed=B) if act == "f32" else synth.gen_x_bf16(B, k, seed=B)
        ws = torch.zeros(plan.workspace_bytes(B), dtype=torch.uint8, device=_dev())
        outs = []
        for mode in ("0", "1", "0", "1"):
            monkeypatch.setenv("QGEMM_ST_XLOCAL", mode)
            outs.append(run(plan, x, wd, workspace=ws))
        monkeypatch.delenv("QGEMM_ST_XLOCAL")
        outs.append(run(plan, x, wd, workspace=ws))  # the probed default
        for o in outs[1:]:
            assert np.array_equal(o, outs[0]), (B, fmt)
        assert torch.count_nonzero(ws[:4 * -(-n // 128)]) == 0  # row-group counters re-armed
        ref = oracle.swiglu(w, x) if epi == "swiglu" else oracle.gemm(w, x)
        err = oracle.rel_fro(outs[0], ref)
        tol = TOL_FP32 if math == "fp32" else (1e-4 if epi == "swiglu" else TOL_BF16)
        assert err <= tol, (B, fmt, err)


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


def test_q8_0_ffn_prefill_2048_bf16():
    c = synth.CONFIGS["q8_0_ffn_17408x5120"]
    w = synth.gen_config_weights("q8_0_ffn_17408x5120")
    x = synth.gen_config_x("q8_0_ffn_17408x5120", 2048)
    plan = q.Plan("q8_0", c["N"], c["K"], act="f32", out="f32", math="bf16")
    assert plan.tier(2048) == "tiled"
    y = run(plan, x, w_dev(w))
    assert np.all(np.isfinite(y))
    bi, ni = _samples(2048, c["N"], 6000, 3)
    err = oracle.rel_fro(y[bi, ni], oracle.gemm_at(w, x, bi, ni))
    print(f"q8_0 ffn rel_fro(sampled)={err:.3e}")
    assert err <= TOL_BF16


# -------------------------------------- full outputs against a library GEMM

def _library_ref(w, x, swiglu=False):
    """Every output at full size: the oracle's decoded weights (fp64 -> fp32,
    tensor scales applied) times the activations as given, through torch's
    fp32 GEMM on the GPU (rocBLAS / hipBLASLt, no reduced-precision inputs),
    then SiLU(G) * U in fp32 for the fused epilogue."""
    torch.backends.cuda.matmul.allow_tf32 = False
    xf = x if x.dtype == np.float32 else synth.bf16_bits_to_f32(x)
    W = torch.from_numpy(oracle.dequant(w, apply_g=True).astype(np.float32)).to(_dev())
    y = torch.mm(torch.from_numpy(np.ascontiguousarray(xf)).to(_dev()), W.t().contiguous())
    del W
    if swiglu:
        nh = y.shape[1] // 2
        G, U = y[:, :nh], y[:, nh:]
        y = G * torch.sigmoid(G) * U
    out = y.double().cpu().numpy()
    del y
    torch.cuda.empty_cache()
    return out


@pytest.mark.parametrize("act,math,B", [("f32", "fp32", 4),     # streaming
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
    lib = oracle.rel_fro(y, _library_ref(w, x))
    print(f"K=2^20 B={B} {math} rel_fro(oracle samples)={err:.3e} (vs fp32 library GEMM {lib:.3e})")
    assert np.all(np.isfinite(y))
    assert err <= (TOL_FP32 if math == "fp32" else TOL_BF16)


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
    ref = _library_ref(w, x, swiglu)
    err = oracle.rel_fro(y, ref)
    tol = TOL_FP32 if (c["math"] == "fp32" and c["out"] == "f32") else TOL_BF16
    print(f"{name} B={B} full output vs library GEMM rel_fro={err:.3e}")
    assert np.all(np.isfinite(y))
    assert err <= tol


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
    bi, ni = _samples(B, 5120, 3000, B)
    err = oracle.rel_fro(y[bi, ni], oracle.gemm_at(w, x[:B], bi, ni))
    print(f"mxfp4 down B={B} tier={plan.tier(B)} rel_fro(sampled)={err:.3e}")
    assert err <= TOL_BF16


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
    bi, ni = _samples(B, 5120, 3000, B + 7)
    err = oracle.rel_fro(y[bi, ni], oracle.gemm_at(w, x[:B], bi, ni))
    print(f"fp8 B={B} tier={plan.tier(B)} rel_fro(sampled)={err:.3e}")
    assert err <= TOL_BF16


@pytest.mark.parametrize("B", [1, 16, 70])
def test_fp8_fp32_math(fp8_attn, B):
    """FP8 weights with fp32 activations in fp32-faithful math: 1e-5."""
    w, _, wd = fp8_attn
    x = synth.gen_x_f32(B, 5120, seed=3)
    plan = q.Plan("fp8", 5120, 5120, act="f32", out="f32", math="fp32")
    y = run(plan, x, wd)
    bi, ni = _samples(B, 5120, 3000, B + 11)
    err = oracle.rel_fro(y[bi, ni], oracle.gemm_at(w, x, bi, ni))
    print(f"fp8 fp32-math B={B} rel_fro(sampled)={err:.3e}")
    assert err <= TOL_FP32


def test_nvfp4_fused_gate_up_swiglu_2048():
    c = synth.CONFIGS["nvfp4_gate_up_34816x5120"]
    w = synth.gen_config_weights("nvfp4_gate_up_34816x5120")
    x = synth.gen_config_x("nvfp4_gate_up_34816x5120", 2048)
    plan = q.Plan("nvfp4", c["N"], c["K"], act="bf16", out="bf16", epilogue="swiglu")
    y = run(plan, x, w_dev(w))
    assert y.shape == (2048, c["N"] // 2)
    assert np.all(np.isfinite(y))
    bi, ji = _samples(2048, c["N"] // 2, 4000, 5)
    err = oracle.rel_fro(y[bi, ji], oracle.swiglu_at(w, x, bi, ji))
    print(f"nvfp4 gate+up rel_fro(sampled)={err:.3e}")
    assert err <= TOL_BF16


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
    plan = q.Plan(fmt, 2 * nh, k, act="bf16", out="f32", epilogue="swiglu")
    for B in (1, 7, 16):
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


def test_swiglu_forced_skinny_above_16_is_not_supported():
    plan = q.Plan("nvfp4", 128, 256, act="bf16", out="f32", epilogue="swiglu", tier="skinny")
    x = synth.gen_x_bf16(17, 256)
    w = _gate_up("nvfp4", 64, 256, 3)
    with pytest.raises(q.QgemmError) as e:
        run(plan, x, w_dev(w))
    assert e.value.status == q.ENOTSUP


# ------------------------------------------------------------ routed experts

def _grouped_case(fmt, act, out, epi, E, n, k, offsets, seed, math="bf16"):
    ws = [synth.gen_expert_weights(fmt, n, k, e, seed=seed, swiglu=epi == "swiglu") for e in range(E)]
    T = int(offsets[-1])
    xf = synth.gen_x_f32(T, k, seed=seed + 1)
    x = xf if act == "f32" else synth.f32_to_bf16_bits(xf)
    bufs = [w_dev(w) for w in ws]
    table = torch.tensor([b.data_ptr() for b in bufs], dtype=torch.int64, device=_dev())
    off = torch.from_numpy(np.asarray(offsets, dtype=np.int32)).to(_dev())
    plan = q.Plan(fmt, n, k, act=act, out=out, epilogue=epi, math=math)
    y = y_new(plan, T)
    plan.run_grouped(x_dev(x), table, off, y)
    torch.cuda.synchronize()
    return ws, bufs, x, host(y), plan


@pytest.mark.parametrize("fmt,act,out,epi", [("nvfp4", "bf16", "bf16", "swiglu"),
                                             ("mxfp4", "bf16", "f32", "none"),
                                             ("q8_0", "f32", "f32", "none"),
                                             ("fp8", "bf16", "f32", "swiglu")])
def test_grouped_matches_oracle_and_per_expert_calls(fmt, act, out, epi):
    """Routed experts in one launch: each expert's rows match the fp64 oracle
    and, bit for bit, a large-batch call of that expert alone (empty experts,
    one-row experts and an expert spanning three row tiles included)."""
    n, k = 256, 512
    rows = [5, 0, 1, 300, 17, 0, 128, 129, 2, 40]
    offsets = np.concatenate([[0], np.cumsum(rows)])
    E = len(rows)
    ws, bufs, x, y, plan = _grouped_case(fmt, act, out, epi, E, n, k, offsets, seed=3)
    ref = oracle.gemm_grouped(ws, offsets, x, swiglu_epi=epi == "swiglu")
    err = oracle.rel_fro(y, ref)
    print(f"grouped {fmt} {epi} rel_fro={err:.3e}")
    assert err <= TOL_BF16
    solo = q.Plan(fmt, n, k, act=act, out=out, epilogue=epi, math="bf16", tier="tiled")
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            ye = run(solo, x[r0:r1], bufs[e], workspace=None)
            assert np.array_equal(ye.view(np.uint64), y[r0:r1].view(np.uint64)), e


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
    solo = q.Plan(fmt, n, k, act="f32", out="f32", math="fp32", tier="tiled")
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            ye = run(solo, x[r0:r1], bufs[e], workspace=None)
            assert np.array_equal(ye.view(np.uint64), y[r0:r1].view(np.uint64)), e


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
    solo = q.Plan("nvfp4", n, k, act="bf16", out="f32", tier="tiled")
    assert np.array_equal(run(solo, x, bufs[0], workspace=None), y)
    # T = 0: nothing enqueued, OK returned
    table = torch.tensor([bufs[0].data_ptr()], dtype=torch.int64, device=_dev())
    off = torch.zeros(2, dtype=torch.int32, device=_dev())
    xe = torch.empty((0, k), dtype=torch.bfloat16, device=_dev())
    ye = torch.empty((0, n), dtype=torch.float32, device=_dev())
    plan.run_grouped(xe, table, off, ye)
