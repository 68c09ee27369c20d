"""bench.py's contract pieces that need no GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    """One GPU only: --gpus N > 1 (or a multi-rank launch) exits with a
    message instead of a bench line."""
    for extra_env, args in (({}, ["--gpus", "2"]), ({"WORLD_SIZE": "2"}, [])):
        env = dict(os.environ, **extra_env)
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, env=env,
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 2, (args, r.returncode, r.stderr[-500:])
        assert "one GPU" in r.stderr and r.stdout == ""


def test_pages_context_figures():
    """The pages' own figures beside the nearest measured ones: the gfx1151
    NVFP4 prefill GEMM rate, and the 27B decode rate turned into a weight
    stream (one read of the 12,618,796,032-byte MQ3 file per token, the
    hipfire issue, 'Model')."""
    import bench

    pre = {"nvfp4_gate_up_34816x5120:B=2048": {"TFLOPs": 1000.0}}
    ctx = bench.pages_context(pre, {1: {"weight_GBs": 3000.0}})
    assert ctx["nvfp4_prefill_gemm"]["pages_TFLOPs"] == 16.0
    assert ctx["nvfp4_prefill_gemm"]["here_TFLOPs"] == 1000.0
    assert ctx["ar_decode_27b"]["pages_tok_s"] == 22.8
    assert ctx["ar_decode_27b"]["pages_implied_weight_GBs"] == pytest.approx(12.618796032 * 22.8, abs=0.05)
    assert ctx["ar_decode_27b"]["here_weight_GBs"] == 3000.0
    # the sweep's keys may be ints or strings (after a JSON round trip)
    assert bench.pages_context({}, {"1": {"weight_GBs": 7.0}})["ar_decode_27b"]["here_weight_GBs"] == 7.0


def test_matrix_core_rate_modes():
    """The rate kernel's modes and the K each instruction sums (the TOPS
    figure is MFMAs x 2 x 16 x 16 x K / time)."""
    import prefill_q8_mxfp4_amd as q

    ks = {m: k for m, (_, k) in q.MFMA_RATE_MODES.items()}
    assert ks == {0: 32, 1: 32, 2: 64, 3: 32, 4: 32, 5: 128, 6: 128, 7: 128}
