#!/usr/bin/env python3
"""Throughput of the block-quantized-weight batched GEMM on one MI355X.

Headline (one JSON line on stdout): the Q8_0 attention-projection GEMM,
K = N = 5120, B = 16 fp32 activation rows, fp32 output, fp32-faithful math:
weight-stream GB/s = packed weight bytes per call / time per call.  One step
is one qgemm_run.  The packed weights rotate over enough copies (> 1 GiB in
total) that every call streams them from HBM, not from the 256 MB Infinity
Cache.  Steps are replayed from a HIP graph so host launch cost is not timed.

Extra keys carry the rest of the B sweep of that shape and the prefill
workloads (Q8_0 FFN B = 2048, MXFP4 down projection, NVFP4 fused gate+up at
B = 1 and 16 as well as 2048, FP8-weight attention projection, routed-expert
fused gate+up),
plus the roofline of the dominant kernel and the CPU oracle baseline.

    python bench.py [--steps K] [--warmup W] [--headline-only] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6       # MI355X dense bf16 MFMA
ROTATE_BYTES = 1 << 30          # weight bytes to rotate over (> Infinity Cache)
METRIC = "weight-stream GB/s (B≤16) and TFLOP/s (B≥256) vs MI355X roofline"
CSRC = os.path.join(ROOT, "prefill_q8_mxfp4_amd", "csrc")


def kernel_src_sha() -> str:
    """Hash of every library source: a stored counter record is used only
    while the kernels it was taken on are unchanged."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(CSRC, f), "rb").read())
    h.update(open(os.path.join(ROOT, "include", "qgemm.h"), "rb").read())
    return h.hexdigest()[:16]


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


# GPU work run untimed before each timed loop (the clock's ramp after host-side set-up)
WARM_MS = 20.0


class Workload:
    """Packed weights (rotating copies), activations and output on the GPU."""

    def __init__(self, name, B, copies=1, math_mode=None):
        import numpy as np
        import torch

        import prefill_q8_mxfp4_amd as q
        import synth

        c = synth.CONFIGS[name]
        self.name, self.B, self.c = name, B, c
        self.N, self.K = c["N"], c["K"]
        self.plan = q.Plan(c["fmt"], c["N"], c["K"], act=c["act"], out=c["out"],
                           epilogue="swiglu" if c["epi"] == "swiglu" else "none",
                           math=math_mode or c["math"])
        t0 = time.time()
        self.w_logical = synth.gen_config_weights(name)
        self.x_host = synth.gen_config_x(name, B)
        packed = torch.from_numpy(q.pack_logical(self.w_logical))
        dev = torch.device("cuda:0")
        self.wbytes = packed.numel()
        self.ws = [packed.to(dev) for _ in range(copies)]
        if c["act"] == "f32":
            self.x = torch.from_numpy(self.x_host).to(dev)
        else:
            self.x = torch.from_numpy(self.x_host.view(np.int16)).view(torch.bfloat16).to(dev)
        odt = torch.float32 if c["out"] == "f32" else torch.bfloat16
        self.y = torch.empty((B, self.plan.out_cols), dtype=odt, device=dev)
        torch.cuda.synchronize()
        log(f"[bench] {name} B={B} copies={copies} ready in {time.time() - t0:.1f}s "
            f"tier={self.plan.tier(B)}")

    def flops(self):
        return 2.0 * self.B * self.N * self.K

    def io_bytes(self):
        xb = self.x.numel() * self.x.element_size()
        yb = self.y.numel() * self.y.element_size()
        return self.wbytes + xb + yb

    def time_ms(self, steps, warmup, eager=False, warm_ms=WARM_MS):
        """Average ms per call over `steps` calls replayed from a HIP graph
        holding one call per weight copy (or launched one by one when
        `eager`), bracketed by events on the stream the calls run on.  Before
        the timed calls: `warmup` (at least one per weight copy) eager calls,
        then untimed replays until about `warm_ms` of GPU work has run, so the
        timed calls see the steady clock rather than the ramp after the host
        set the workload up (`self.untimed_calls` counts them all)."""
        import torch

        n = len(self.ws)
        reps = max(1, math.ceil(steps / n))
        stream = torch.cuda.Stream()
        self.untimed_calls = max(warmup, n)
        with torch.cuda.stream(stream):
            for i in range(max(warmup, n)):
                self.plan.run(self.x, self.ws[i % n], self.y)
        stream.synchronize()
        if eager:
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                start.record(stream)
                for i in range(reps * n):
                    self.plan.run(self.x, self.ws[i % n], self.y)
                end.record(stream)
            end.synchronize()
            return start.elapsed_time(end) / (reps * n), reps * n
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                self.plan.run(self.x, self.ws[i], self.y)
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            w0.record(stream)
            g.replay()
            w1.record(stream)
        w1.synchronize()
        more = math.ceil(warm_ms / max(w0.elapsed_time(w1), 1e-3)) - 1
        with torch.cuda.stream(stream):
            for _ in range(max(0, min(more, 100000))):
                g.replay()
        stream.synchronize()
        self.untimed_calls += n * (1 + max(0, min(more, 100000)))
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):  # replays and events on one stream
            start.record(stream)
            for _ in range(reps):
                g.replay()
            end.record(stream)
        end.synchronize()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / (reps * n), reps * n

    def free(self):
        self.ws = self.x = self.y = None


def copies_for(wbytes):
    return max(1, math.ceil(ROTATE_BYTES / wbytes))


def traffic_record(sha):
    p = os.path.join(ROOT, "profiles", "traffic_q8_0_5120x5120_b16.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("kernel_src_sha") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(wl, budget_s=10.0):
    """The fp64 oracle on the host cores, on whole headline calls repeated
    until about `budget_s` seconds have passed (at least one call)."""
    import oracle

    calls, t0 = 0, time.time()
    while True:
        oracle.gemm(wl.w_logical, wl.x_host)
        calls += 1
        dt = time.time() - t0
        if dt >= budget_s or dt / calls * (calls + 1) > 3 * budget_s:
            break
    per = dt / calls
    return {"value": round(wl.wbytes / per / 1e9, 6), "unit": "GB/s", "cores": oracle.threads(),
            "kind": "oracle", "seconds_per_call": round(per, 3),
            "sample": f"{calls} whole headline call(s) of the fp64 oracle: q8_0 K=N=5120, "
                      f"B={wl.B}, fp32 activations"}


def copy_calibration(mib=512, reps=5):
    """A plain device copy of known size, for scaling the HBM byte counters
    of a profiled run (FETCH_SIZE / WRITE_SIZE of this copy read mib MiB)."""
    import torch

    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} copies of {mib} MiB")


def bench_moe(steps):
    """Routed-expert NVFP4 fused gate+up at the scale of the Atlas issue's
    validation plan (512 experts, top-10, 2048 tokens).  The pages give no
    expert dimensions; K = 2048 and 2 x 512 gate/up rows stand in.  Eight
    generated experts are copied into 512 separate buffers (real memory
    traffic, repeating values) to bound the input generation time."""
    import numpy as np
    import torch

    import prefill_q8_mxfp4_amd as q
    import synth

    E, topk, tokens, nh, K = 512, 10, 2048, 512, 2048
    dev = torch.device("cuda:0")
    t0 = time.time()
    distinct = [torch.from_numpy(q.pack_logical(synth.gen_expert_weights("nvfp4", 2 * nh, K, e, swiglu=True)))
                for e in range(8)]
    bufs = [distinct[e % 8].to(dev) for e in range(E)]
    table = torch.tensor([b.data_ptr() for b in bufs], dtype=torch.int64, device=dev)
    tok, offsets = synth.gen_routing(tokens, topk, E)
    T = int(offsets[-1])
    x = torch.from_numpy(synth.gen_x_bf16(tokens, K)[tok].view(np.int16)).view(torch.bfloat16).to(dev)
    off = torch.from_numpy(offsets).to(dev)
    plan = q.Plan("nvfp4", 2 * nh, K, act="bf16", out="bf16", epilogue="swiglu")
    y = torch.empty((T, nh), dtype=torch.bfloat16, device=dev)
    log(f"[bench] moe ready in {time.time() - t0:.1f}s")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(3):
            plan.run_grouped(x, table, off, y)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        plan.run_grouped(x, table, off, y)
    with torch.cuda.stream(stream):  # untimed: about WARM_MS of work (one call is ~0.35 ms)
        for _ in range(max(1, math.ceil(WARM_MS / 0.35))):
            g.replay()
    stream.synchronize()
    reps = max(10, steps // 10)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        g.replay()
        start.record(stream)
        for _ in range(reps):
            g.replay()
        end.record(stream)
    end.synchronize()
    ms = start.elapsed_time(end) / reps
    flops = 2.0 * T * 2 * nh * K
    wbytes = sum(b.numel() for b in bufs)
    rec = {"us": round(ms * 1e3, 2), "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
           "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "weight_GBs": round(wbytes / (ms * 1e-3) / 1e9, 1), "rows": T, "experts": E, "top_k": topk}
    log(f"[bench] moe {rec}")
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch calls one by one instead of replaying a HIP graph (profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 512 MiB copy (scales profiler byte counters)")
    ap.add_argument("--calls-of", nargs=2, metavar=("CONFIG", "B"),
                    help="only launch CONFIG at batch B eagerly --steps times, print nothing "
                         "else (a short program for counter passes)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import prefill_q8_mxfp4_amd as q
    import synth

    q.lib()  # fails loudly without the HIP library
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    sha = kernel_src_sha()
    if args.copy_calibration:
        copy_calibration()
    if args.calls_of:
        w = Workload(args.calls_of[0], int(args.calls_of[1]))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        w.plan.run(w.x, w.ws[0], w.y)
        e1.record()
        e1.synchronize()
        # about WARM_MS of calls first, so most profiled dispatches run at the steady clock
        for _ in range(math.ceil(WARM_MS / max(e0.elapsed_time(e1), 1e-3)) + args.steps):
            w.plan.run(w.x, w.ws[0], w.y)
        torch.cuda.synchronize()
        log(f"[bench] {args.steps} calls of {args.calls_of[0]} B={args.calls_of[1]} done")
        return

    # ---- headline: q8_0 5120x5120, B = 16, fp32 activations
    B = 16
    probe = q.weight_bytes("q8_0", 5120, 5120)
    wl = Workload("q8_0_5120x5120", B, copies=copies_for(probe))
    ms, steps_done = wl.time_ms(args.steps, args.warmup, eager=args.eager)
    value = wl.wbytes / (ms * 1e-3) / 1e9
    achieved = wl.io_bytes() / (ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps_done,
        "warmup": args.warmup,
        "untimed_calls": wl.untimed_calls,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "Q8_0 batched GEMM K=5120 N=5120 B=16, fp32 activations "
                               "~N(0,1), weights ~N(0,0.02), fp32 out, fp32-faithful math",
                   "B": B, "N": 5120, "K": 5120, "weight_copies": len(wl.ws),
                   "tier": wl.plan.tier(B), "xcd_local_exchange": q.xcd_local()},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_record(sha), "algorithmic_bytes": wl.io_bytes(),
                     "kernel_src_sha": sha},
    }
    log(f"[bench] headline {ms * 1e3:.2f} us/call  {value:.1f} GB/s weights")
    # spread: 7 more trials of the same loop (the value above stays the timed K steps)
    trials = sorted(wl.time_ms(max(50, args.steps // 8), 0, eager=args.eager)[0] * 1e3 for _ in range(7))
    line["headline_trials_us"] = {"n": 7, "min": round(trials[0], 3), "median": round(trials[3], 3),
                                  "max": round(trials[-1], 3)}

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)
    wl.free()

    if not args.headline_only:
        sweep = {}
        for b in (1, 4, 8, 16, 64, 65, 70, 76, 256):
            w = Workload("q8_0_5120x5120", b, copies=copies_for(probe) if b <= 16 else 4)
            t, _ = w.time_ms(max(40, args.steps // 4), 5)
            sweep[str(b)] = {"us": round(t * 1e3, 2),
                             "weight_GBs": round(w.wbytes / (t * 1e-3) / 1e9, 1),
                             "hbm_frac": round(w.io_bytes() / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "TFLOPs": round(w.flops() / (t * 1e-3) / 1e12, 2),
                             "tier": w.plan.tier(b)}
            w.free()
        line["sweep_q8_0_5120x5120_fp32"] = sweep
        pre = {}
        for name, bs in (("q8_0_ffn_17408x5120", (2048,)), ("mxfp4_down_5120x17408", (1, 16, 256, 2048)), ("nvfp4_gate_up_34816x5120", (1, 16, 2048)),
                         ("fp8_5120x5120", (1, 16, 256, 2048))):
            for b in bs:
                c = synth.CONFIGS[name]
                nb = q.weight_bytes(c["fmt"], c["N"], c["K"])
                # several calls per graph replay (distinct weight copies) so the
                # replay overhead is spread as in the B sweep
                w = Workload(name, b, copies=copies_for(nb) if b <= 16 else 4)
                t, _ = w.time_ms(max(20, args.steps // 10) if b > 16 else max(40, args.steps // 4),
                                 3)
                c = w.c
                key = f"{name}:B={b}"
                rec = {"us": round(t * 1e3, 2), "TFLOPs": round(w.flops() / (t * 1e-3) / 1e12, 2),
                       "mfma_frac": round(w.flops() / (t * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                       "weight_GBs": round(w.wbytes / (t * 1e-3) / 1e9, 1),
                       "hbm_frac": round(w.io_bytes() / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "tier": w.plan.tier(b)}
                pre[key] = rec
                log(f"[bench] {key} {rec}")
                w.free()
                torch.cuda.empty_cache()
        line["prefill"] = pre
        line["routed_moe:nvfp4:512x(2x512)x2048:top10:tokens2048"] = bench_moe(args.steps)

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
