#!/usr/bin/env python3
"""Throughput of the block-quantized-weight batched GEMM on one MI355X.

Headline (one JSON line on stdout): the Q8_0 attention-projection GEMM,
K = N = 5120, B = 16 fp32 activation rows, fp32 output, fp32-faithful math:
weight-stream GB/s = packed weight bytes per call / time per call.  One step
is one qgemm_run.  The packed weights rotate over enough copies (> 1 GiB in
total) that every call streams them from HBM, not from the 256 MB Infinity
Cache.  Steps are replayed from a HIP graph so host launch cost is not timed.
value is the median of 7 timed loops of at least max(--steps, 200) calls.
The same loop over a plain read kernel of the same bytes gives the achieved
bandwidth ceiling (roofline.ceiling_GBs, frac_of_ceiling), and the same call
without a workspace (qgemm_run's unsplit route) is timed too.

Extra keys carry the rest of the B sweep of that shape and the prefill
workloads (Q8_0 FFN B = 2048, MXFP4 down projection, NVFP4 fused gate+up at
B = 1 and 16 as well as 2048, FP8-weight attention projection, routed-expert
fused gate+up), the matrix-core roofline of the B = 2048 workloads
(roofline_mfma), and the CPU oracle baseline on all cores and on one.

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
TRIALS = 7            # timed loops of the headline; value is their median
MIN_LAUNCHES = 200    # calls per timed loop, at least


class GraphTimer:
    """Launches replayed from one HIP graph on a stream of their own, timed
    with HIP events recorded on that stream.  `launches` is a list of
    closures, each enqueueing one call on the current stream; the graph
    holds them all (one per weight copy)."""

    def __init__(self, launches, eager_first=1):
        import torch

        self.n = len(launches)
        self.stream = torch.cuda.Stream()
        self.untimed = 0
        with torch.cuda.stream(self.stream):
            for i in range(max(eager_first, self.n)):
                launches[i % self.n]()
        self.untimed += max(eager_first, self.n)
        self.stream.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g, stream=self.stream):
            for f in launches:
                f()
        self.warm()

    def warm(self, warm_ms=WARM_MS):
        """Untimed replays until about warm_ms of GPU work has run: the timed
        loops then see the steady clock, not the ramp after host set-up."""
        import torch

        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):
            w0.record(self.stream)
            self.g.replay()
            w1.record(self.stream)
        w1.synchronize()
        more = max(0, min(math.ceil(warm_ms / max(w0.elapsed_time(w1), 1e-3)) - 1, 100000))
        with torch.cuda.stream(self.stream):
            for _ in range(more):
                self.g.replay()
        self.stream.synchronize()
        self.untimed += self.n * (1 + more)

    def timed(self, launches):
        """ms per call over at least `launches` calls (whole replays)."""
        import torch

        reps = max(1, math.ceil(launches / self.n))
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            start.record(self.stream)
            for _ in range(reps):
                self.g.replay()
            end.record(self.stream)
        end.synchronize()
        return start.elapsed_time(end) / (reps * self.n), reps * self.n

    def trials(self, ntrials, launches):
        """Per-call ms of `ntrials` timed loops (sorted) and calls per loop."""
        out = [self.timed(launches) for _ in range(ntrials)]
        return sorted(t for t, _ in out), out[0][1]


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

    def launches(self, workspace="auto"):
        return [(lambda w=w: self.plan.run(self.x, w, self.y, workspace=workspace)) for w in self.ws]

    def timer(self, warmup=1, workspace="auto"):
        t = GraphTimer(self.launches(workspace), eager_first=warmup)
        self.untimed_calls = t.untimed
        return t

    def time_ms(self, steps, warmup, eager=False):
        """ms per call over at least `steps` calls (whole replays of the
        graph holding one call per weight copy, or eager launches)."""
        import torch

        if eager:
            n = len(self.ws)
            reps = max(1, math.ceil(steps / n))
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for i in range(max(warmup, n)):
                    self.plan.run(self.x, self.ws[i % n], self.y)
            stream.synchronize()
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                start.record(stream)
                for i in range(reps * n):
                    self.plan.run(self.x, self.ws[i % n], self.y)
                end.record(stream)
            end.synchronize()
            self.untimed_calls = max(warmup, n)
            return start.elapsed_time(end) / (reps * n), reps * n
        return self.timer(warmup).timed(steps)

    def flops(self):
        return 2.0 * self.B * self.N * self.K

    def io_bytes(self):
        xb = self.x.numel() * self.x.element_size()
        yb = self.y.numel() * self.y.element_size()
        return self.wbytes + xb + yb

    def free(self):
        self.ws = self.x = self.y = None


def read_ceiling(wl, ntrials, launches):
    """The plain read kernel over the same packed weight copies in the same
    rotation (one launch per copy): per-call ms of each trial."""
    import torch

    import prefill_q8_mxfp4_amd as q

    sink = torch.zeros(2048, dtype=torch.int32, device="cuda:0")
    t = GraphTimer([(lambda w=w: q.read_bytes(w, sink)) for w in wl.ws])
    return t.trials(ntrials, launches)


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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s=10.0, one_thread_calls=1):
    """The fp64 oracle on the host: whole headline calls on all the cores it
    uses, repeated until about `budget_s` seconds have passed, then
    `one_thread_calls` whole calls on one thread."""
    import oracle

    calls, t0 = 0, time.time()
    while True:
        oracle.gemm(wl.w_logical, wl.x_host)
        calls += 1
        dt = time.time() - t0
        if dt >= budget_s or dt / calls * (calls + 1) > 3 * budget_s:
            break
    per = dt / calls
    cores = oracle.threads()
    oracle.set_threads(1)
    try:
        t1 = time.time()
        for _ in range(one_thread_calls):
            oracle.gemm(wl.w_logical, wl.x_host)
        per1 = (time.time() - t1) / one_thread_calls
    finally:
        oracle.set_threads(cores)
    return {"value": round(wl.wbytes / per / 1e9, 6), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "seconds_per_call": round(per, 3),
            "one_thread": {"value": round(wl.wbytes / per1 / 1e9, 6), "unit": "GB/s", "cores": 1,
                           "seconds_per_call": round(per1, 3), "calls": one_thread_calls},
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{calls} whole headline call(s) of the fp64 oracle on {cores} threads, then "
                      f"{one_thread_calls} on one thread: q8_0 K=N=5120, B={wl.B}, fp32 activations"}


def next4_mfma_rates(modes=(0, 1, 2, 3, 4), iters=4096, reps=5):
    """Dense TOPS of the matrix-core loops of qgemm_mfma_rate (median of
    `reps` launches, each after a warm-up launch): modes 0-4 answer the
    int8-activation question for Q8_0 weights, modes 5-7 time the hardware
    block-scaled route for the MX formats."""
    import torch

    import prefill_q8_mxfp4_amd as q

    sink = torch.zeros(4096, dtype=torch.int32, device="cuda:0")
    out = {}
    for mode in modes:
        name, kdeep = q.MFMA_RATE_MODES[mode]
        q.mfma_rate(mode, iters, sink)
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            q.mfma_rate(mode, iters, sink)
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        t = sorted(ts)[reps // 2]
        mfmas = 512 * 8 * iters * 8       # workgroups x waves x trips x chains
        tops = mfmas * 2.0 * 16 * 16 * kdeep / t / 1e12
        out[name] = {"TOPS": round(tops, 1), "ms": round(t * 1e3, 4)}
    log(f"[bench] matrix-core rates {out}")
    return out


def torch_bf16_gemm_rates(reps=10):
    """Context for the large-batch rates: torch's own bf16 GEMM (the vendor
    library) on the same shapes with plain bf16 weights and no decode, the
    weights stored [K][N] ("nn") and [N][K] ("nt", as this library stores
    them), timed with events after about 50 ms of untimed calls (median of
    `reps` timed calls per shape and layout)."""
    import torch

    shapes = [("2048x17408x5120", 2048, 17408, 5120), ("2048x5120x17408", 2048, 5120, 17408),
              ("2048x34816x5120", 2048, 34816, 5120), ("2048x5120x5120", 2048, 5120, 5120),
              ("256x5120x17408", 256, 5120, 17408), ("8192x8192x8192", 8192, 8192, 8192)]
    g = torch.Generator(device="cuda:0").manual_seed(0)
    out = {}
    for name, B, N, K in shapes:
        x = torch.randn(B, K, device="cuda:0", dtype=torch.bfloat16, generator=g)
        y = torch.empty(B, N, device="cuda:0", dtype=torch.bfloat16)
        flop = 2.0 * B * N * K
        n_warm = max(3, int(0.05 / (flop / 1.0e15)))
        rec = {}
        for lay in ("nn", "nt"):
            w = torch.randn((K, N) if lay == "nn" else (N, K), device="cuda:0", dtype=torch.bfloat16,
                            generator=g)
            wop = w if lay == "nn" else w.t()  # 2-D product: the transposed view is the "nt" layout
            for _ in range(n_warm):
                torch.matmul(x, wop, out=y)
            ts = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                torch.matmul(x, wop, out=y)
                e1.record()
                e1.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e-3)
            t = sorted(ts)[reps // 2]
            rec[lay] = {"us": round(t * 1e6, 2), "TFLOPs": round(flop / t / 1e12, 1)}
            del w, wop
        best = max(rec.values(), key=lambda r: r["TFLOPs"])
        out[name] = dict(rec, best_frac_bf16_peak=round(best["TFLOPs"] / BF16_PEAK_TFLOPS, 4))
        del x, y
        torch.cuda.empty_cache()
    log(f"[bench] torch bf16 GEMM {out}")
    return out


def pages_context(pre, sweep):
    """The pages' own figures for this path, on their own hardware, next to
    the nearest figure measured here (context, not a target)."""
    nv = pre.get("nvfp4_gate_up_34816x5120:B=2048", {}).get("TFLOPs")
    b1 = sweep.get(1, sweep.get("1", {})).get("weight_GBs")
    # hipfire issue, "Model": the 27B MQ3 trunk file is 12,618,796,032 bytes;
    # at one token per full read of it, 22.8 tok/s streams about 288 GB/s
    mq3_bytes = 12_618_796_032
    return {
        "nvfp4_prefill_gemm": {
            "pages_TFLOPs": 16.0, "pages_hw": "gfx1151 (Strix Halo iGPU), w4a16 GEMM, 27B FFN, 2048-token chunks",
            "source": "Atlas issue, 'Kernel ranking: Strix long prefill is GEMM-efficiency-bound'",
            "here_TFLOPs": nv, "here": "NVFP4 fused gate+up 2x17408x5120, B=2048"},
        "ar_decode_27b": {
            "pages_tok_s": 22.8, "pages_hw": "RX 9060 XT (gfx1200), 27B MQ3 trunk, single stream",
            "source": "hipfire issue, 'Baseline: AR is healthy' and 'Model'",
            "pages_implied_weight_GBs": round(mq3_bytes * 22.8 / 1e9, 1),
            "here_weight_GBs": b1, "here": "Q8_0 5120x5120, B=1 weight stream"},
    }


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


MOE_SHAPE = (512, 10, 2048, 512, 2048)  # experts, top-k, tokens, gate (= up) rows, K


def moe_inputs():
    """Routed-expert NVFP4 fused gate+up at the scale of the Atlas issue's
    validation plan (512 experts, top-10, 2048 tokens).  The pages give no
    expert dimensions; K = 2048 and 2 x 512 gate/up rows stand in.  Eight
    generated experts are copied into 512 separate buffers (real memory
    traffic, repeating values) to bound the input generation time."""
    import numpy as np
    import torch

    import prefill_q8_mxfp4_amd as q
    import synth

    E, topk, tokens, nh, K = MOE_SHAPE
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
    return plan, x, table, off, y, bufs, T


def bench_moe(steps):
    """The routed-expert workload of moe_inputs(), graph-replayed."""
    import torch

    E, topk, tokens, nh, K = MOE_SHAPE
    plan, x, table, off, y, bufs, T = moe_inputs()
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
           "weight_GBs": round(wbytes / (ms * 1e-3) / 1e9, 1),
           "hbm_frac": round(wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "route": plan.grouped_tier(E, T), "rows": T, "experts": E, "top_k": topk}
    log(f"[bench] moe {rec}")
    return rec


# The verify kernel (16 < B <= 80) against the routes it replaced (the
# skinny kernel to B = 32 with bf16 math, the tiled tier above; QGEMM_VF=0,
# read when a plan is created), alternating on one box: (config, math, widths).
VERIFY_COMPARE = (
    ("q8_0_5120x5120", None, (17, 32, 48, 64, 65, 70, 76, 80)),   # fp32-faithful
    ("q8_0_5120x5120", "bf16", (17, 24, 32, 40, 48, 64, 80)),      # fp32 x, bf16 math
    ("fp8_5120x5120", None, (17, 24, 32, 40, 48, 64, 80)),
    ("mxfp4_down_5120x17408", None, (17, 24, 32, 40, 48, 64, 80)),
    ("nvfp4_gate_up_34816x5120", None, (17, 32, 48, 64, 80)),      # fused gate+up
)


def verify_compare():
    """µs per call of each VERIFY_COMPARE width with the verify kernel and
    with QGEMM_VF=0 (graph-replayed, rotating weight copies, median of 5
    loops of at least 200 calls), one JSON line."""
    import statistics

    import torch

    import prefill_q8_mxfp4_amd as q
    import synth

    out = {}
    for name, mm, widths in VERIFY_COMPARE:
        key = name + (":" + mm if mm else "")
        c = synth.CONFIGS[name]
        copies = copies_for(q.weight_bytes(c["fmt"], c["N"], c["K"]))
        out[key] = {}
        for B in widths:
            rec = {}
            for vf in ("1", "0"):
                os.environ["QGEMM_VF"] = vf
                wl = Workload(name, B, copies=copies, math_mode=mm)
                t = wl.timer()
                tr, _ = t.trials(5, MIN_LAUNCHES)
                rec["verify" if vf == "1" else "before"] = {"us": round(statistics.median(tr) * 1e3, 2),
                                                            "tier": wl.plan.tier(B)}
                wl.free()
                del t
                torch.cuda.empty_cache()
            os.environ.pop("QGEMM_VF", None)
            out[key][B] = rec
            log(f"[bench] verify compare {key} B={B} {rec}")
    print(json.dumps({"verify_compare_us": out}), flush=True)


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
    ap.add_argument("--profile-headline", action="store_true",
                    help="time only the headline GEMM loop (no read ceiling, no no-workspace "
                         "route, no CPU baseline): the program under the kernel-trace profile")
    ap.add_argument("--calls-of", nargs=2, metavar=("CONFIG", "B"),
                    help="only launch CONFIG at batch B eagerly --steps times, print nothing "
                         "else (a short program for counter passes); CONFIG routed_moe (B "
                         "ignored) launches the routed-expert workload, mfma_rate the "
                         "matrix-core rate kernel")
    ap.add_argument("--verify-compare", action="store_true",
                    help="only time the verify kernel's widths against the routes it replaced "
                         "(QGEMM_VF=0) and print that table as one JSON line")
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
    if args.verify_compare:
        verify_compare()
        return
    if args.calls_of and args.calls_of[0] == "mfma_rate":
        sink = torch.zeros(4096, dtype=torch.int32, device="cuda:0")
        for _ in range(3 + args.steps):  # mode 0: chained bf16 MFMAs, the matrix cores' own rate
            q.mfma_rate(0, 4096, sink)
        torch.cuda.synchronize()
        log(f"[bench] {args.steps} calls of the MFMA rate kernel done")
        return
    if args.calls_of and args.calls_of[0] == "routed_moe":
        plan, x, table, off, y, bufs, T = moe_inputs()
        for _ in range(20 + args.steps):  # the first 20 warm the clock
            plan.run_grouped(x, table, off, y)
        torch.cuda.synchronize()
        log(f"[bench] {args.steps} calls of routed_moe done")
        return
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

    # ---- headline: q8_0 5120x5120, B = 16, fp32 activations.  value is the
    # median of TRIALS timed loops of at least max(--steps, MIN_LAUNCHES)
    # graph-replayed calls each (whole rotations of the weight copies).
    B = 16
    probe = q.weight_bytes("q8_0", 5120, 5120)
    wl = Workload("q8_0_5120x5120", B, copies=copies_for(probe))
    launches = max(args.steps, MIN_LAUNCHES)
    if args.eager:
        per = sorted(wl.time_ms(launches, args.warmup, eager=True)[0] for _ in range(TRIALS))
        steps_done = math.ceil(launches / len(wl.ws)) * len(wl.ws)
    else:
        timer = wl.timer(args.warmup)
        per, steps_done = timer.trials(TRIALS, launches)
    ms = per[TRIALS // 2]
    untimed = wl.untimed_calls
    value = wl.wbytes / (ms * 1e-3) / 1e9
    achieved = wl.io_bytes() / (ms * 1e-3) / 1e9
    if args.profile_headline:
        print(json.dumps({"profile_headline_us": round(ms * 1e3, 3), "calls_per_trial": steps_done,
                          "trials": TRIALS, "untimed_calls": untimed,
                          "weight_GBs": round(value, 2), "kernel_src_sha": sha}), flush=True)
        return
    # the plain read of the same bytes in the same rotation: the achieved ceiling
    rc, _ = read_ceiling(wl, TRIALS, launches)
    ceil_ms = rc[TRIALS // 2]
    ceiling = wl.wbytes / (ceil_ms * 1e-3) / 1e9
    # the same call without a workspace (qgemm_run: the unsplit route)
    nws, _ = GraphTimer(wl.launches(workspace=None)).trials(3, launches)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps_done,
        "trials": TRIALS,
        "warmup": args.warmup,
        "untimed_calls": untimed,
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
                     "ceiling_GBs": round(ceiling, 1),
                     "frac_of_ceiling": round(value / ceiling, 4),
                     "ceiling_kernel": "read_bytes_kernel (plain 16-byte-load read of the same "
                                       "packed weight copies, same rotation)",
                     "kernel_src_sha": sha},
        "headline_trials_us": {"n": TRIALS, "calls_per_trial": steps_done,
                               "min": round(per[0] * 1e3, 3), "median": round(ms * 1e3, 3),
                               "max": round(per[-1] * 1e3, 3)},
        "read_ceiling_trials_us": {"n": TRIALS, "min": round(rc[0] * 1e3, 3),
                                   "median": round(ceil_ms * 1e3, 3), "max": round(rc[-1] * 1e3, 3)},
        "headline_no_workspace": {"us": round(nws[1] * 1e3, 3),
                                  "weight_GBs": round(wl.wbytes / (nws[1] * 1e-3) / 1e9, 1),
                                  "route": "qgemm_run without a workspace (no K split)"},
    }
    log(f"[bench] headline {ms * 1e3:.2f} us/call  {value:.1f} GB/s weights; plain read "
        f"{ceil_ms * 1e3:.2f} us ({ceiling:.0f} GB/s); no workspace {nws[1] * 1e3:.2f} us")

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)
    wl.free()

    if not args.headline_only:
        sweep = {}
        for b in (1, 4, 8, 16, 64, 65, 70, 76, 256):
            w = Workload("q8_0_5120x5120", b, copies=copies_for(probe) if b <= 16 else 4)
            t, _ = w.time_ms(max(80, args.steps // 2), 5)
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
                t, _ = w.time_ms(max(20, args.steps // 10) if b > 16 else max(80, args.steps // 2),
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
        # the matrix-core side of the metric: every B = 2048 workload against
        # the dense bf16 peak (the largest, NVFP4 fused gate+up, as the object)
        big = {k: v for k, v in pre.items() if k.endswith(":B=2048")}
        key = "nvfp4_gate_up_34816x5120:B=2048"
        if key in big:
            r = big[key]
            line["roofline_mfma"] = {"bound": "mfma", "achieved": r["TFLOPs"], "peak": BF16_PEAK_TFLOPS,
                                     "unit": "TFLOP/s", "frac": r["mfma_frac"], "traffic": None,
                                     "workload": key, "dtype": "bf16",
                                     "all_B2048": {k: v["mfma_frac"] for k, v in big.items()}}
        line["routed_moe:nvfp4:512x(2x512)x2048:top10:tokens2048"] = bench_moe(args.steps)
        line["next4_int8_vs_bf16_mfma"] = next4_mfma_rates()
        line["mx_scaled_mfma_rates"] = next4_mfma_rates((0, 5, 6, 7))
        line["pages_context"] = pages_context(pre, sweep)
        line["context_torch_bf16_gemm"] = torch_bf16_gemm_rates()

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
