"""The allocation-free entry point (qgemm_run_noalloc) through the C ABI:
its output against the workspace entry point's (qgemm_run_ws with a
workspace of qgemm_workspace_bytes) on the same inputs, bitwise (the same
route), and against the oracle's bound; two calls in a row, the second with
a smaller input; plans of different shapes sharing the one static scratch;
a call needing more scratch than the array holds is refused; a captured
graph of it replays bitwise."""

import numpy as np
import pytest
import torch

import oracle
import prefill_q8_mxfp4_amd as q
import synth

pytestmark = pytest.mark.gpu


def _dev():
    return torch.device("cuda:0")


def _x(x):
    if x.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(x)).to(_dev())
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(_dev())


def _y(plan, B):
    dt = torch.float32 if plan.out == "f32" else torch.bfloat16
    return torch.full((B, plan.out_cols), float("nan"), dtype=dt, device=_dev())


def _both(plan, wd, x, B):
    """(noalloc output, workspace output) as int32/int16 bit patterns."""
    xd = _x(x[:B])
    y0, y1 = _y(plan, B), _y(plan, B)
    plan.run_noalloc(xd, wd, y0)
    ws = torch.zeros(max(plan.workspace_bytes(B), 256), dtype=torch.uint8, device=_dev())
    plan.run(xd, wd, y1, workspace=ws)
    torch.cuda.synchronize()
    return y0, y1


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("name,Bs,tol", [
    ("q8_0_5120x5120", (16, 4), 1e-5),              # streaming kernel, K split
    ("q8_0_5120x5120", (256, 70), 1e-5),            # fp32-faithful tiled (split + reduce), then the verify kernel
    ("nvfp4_gate_up_34816x5120", (16, 1), 1e-2),    # streaming fused gate+up, 272 row groups
    ("mxfp4_down_5120x17408", (256, 33), 1e-2),     # tiled bf16, split pieces
    ("q8_0_ffn_17408x5120", (64, 17), 1e-2),        # x rounded to bf16 in the scratch
])
def test_noalloc_matches_workspace_entry(name, Bs, tol):
    c = synth.CONFIGS[name]
    w = synth.gen_config_weights(name)
    x = synth.gen_config_x(name, max(Bs))
    wd = torch.from_numpy(q.pack_logical(w)).to(_dev())
    plan = q.Plan(c["fmt"], c["N"], c["K"], act=c["act"], out=c["out"],
                  epilogue="swiglu" if c["epi"] == "swiglu" else "none", math=c["math"])
    for B in Bs:                                    # the second call is smaller
        assert plan.workspace_bytes(B) <= q.SCRATCH_BYTES
        y0, y1 = _both(plan, wd, x, B)
        assert torch.equal(_bits(y0), _bits(y1)), (name, B)
        bi = np.arange(B).repeat(8)
        ni = np.tile(np.linspace(0, plan.out_cols - 1, 8).astype(np.int64), B)
        got = y0.float().cpu().numpy()[bi, ni]
        ref = (oracle.swiglu_at(w, x[:B], bi, ni) if c["epi"] == "swiglu"
               else oracle.gemm_at(w, x[:B], bi, ni))
        assert oracle.rel_fro(got, ref) <= tol, (name, B)


def test_noalloc_plans_share_the_scratch():
    """Calls of plans with different counter layouts back to back on the one
    array: each output bitwise that of the workspace entry point."""
    shapes = [("q8_0", 5120, 5120, "f32", "f32", "fp32", 16), ("mxfp4", 1024, 8192, "bf16", "f32", "bf16", 8),
              ("q8_0", 5120, 5120, "f32", "f32", "fp32", 70), ("fp8", 2048, 4096, "bf16", "f32", "bf16", 300),
              ("q8_0", 5120, 5120, "f32", "f32", "fp32", 3)]
    for i, (fmt, n, k, act, out, math, B) in enumerate(shapes * 2):
        w = synth.gen_weights(fmt, n, k, seed=60 + i % len(shapes))
        xf = synth.gen_x_f32(B, k, seed=70 + i)
        x = xf if act == "f32" else synth.f32_to_bf16_bits(xf)
        plan = q.Plan(fmt, n, k, act=act, out=out, math=math)
        wd = torch.from_numpy(q.pack_logical(w)).to(_dev())
        y0, y1 = _both(plan, wd, x, B)
        assert torch.equal(_bits(y0), _bits(y1)), (i, fmt, B)


def test_noalloc_refuses_calls_beyond_the_scratch():
    c = synth.CONFIGS["mxfp4_down_5120x17408"]
    plan = q.Plan("mxfp4", c["N"], c["K"], act="bf16", out="f32")
    B = 2048
    assert plan.workspace_bytes(B) > q.SCRATCH_BYTES
    xd = torch.zeros((B, c["K"]), dtype=torch.bfloat16, device=_dev())
    wd = torch.zeros(q.weight_bytes("mxfp4", c["N"], c["K"]), dtype=torch.uint8, device=_dev())
    y = _y(plan, B)
    with pytest.raises(q.QgemmError) as e:
        plan.run_noalloc(xd, wd, y)
    assert e.value.status == q.EINVAL and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.isnan(y).all()            # nothing was enqueued


def test_noalloc_graph_capture_replays():
    """Captured in a HIP graph (no allocation inside the capture), replayed
    three times with eager work between: bitwise the eager result each time."""
    w = synth.gen_config_weights("q8_0_5120x5120")
    x = synth.gen_config_x("q8_0_5120x5120", 16)
    wd = torch.from_numpy(q.pack_logical(w)).to(_dev())
    plan = q.Plan("q8_0", 5120, 5120, act="f32", out="f32", math="fp32")
    xd = _x(x)
    ye = _y(plan, 16)
    plan.run_noalloc(xd, wd, ye)
    torch.cuda.synchronize()
    yg = _y(plan, 16)
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        plan.run_noalloc(xd, wd, yg, stream=st)
    other = q.Plan("q8_0", 5120, 5120, act="f32", out="f32", math="fp32")
    for rep in range(3):
        yg.fill_(float("nan"))
        y2 = _y(other, 5)
        other.run_noalloc(_x(x[:5]), wd, y2)   # eager use of the same scratch between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(yg), _bits(ye)), rep
