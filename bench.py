"""Benchmark of the tiled GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one GEMM (one launch of the library's kernel) over inputs already
resident in HBM.  The timed steps run as replays of a HIP graph that captured
consecutive steps, so no host work sits between kernels (--launch eager: one
library call per step).  Prints ONE JSON line with the throughput, the
roofline of the kernel (achieved vs peak, from HIP events around the timed
steps) and the oracle's CPU throughput on a bounded sample of the same
workload, whose output also cross-checks the sampled GPU rows.

Workloads (seeded synthetic inputs, see synth/):
  square4096  4096^3 bf16 -> bf16            (default; metric workload)
  gate_up     x[4096,4096] @ W_gate, W_up [4096,11008] -> bf16
  gate_up_swiglu  the same with silu(G) * U fused into the epilogue (one output)
  skinny      16 x 28672 x 8192 bf16 -> fp32 (HBM-bound; two B buffers rotate)
  skinny_kmajor, skinny_f8  the same with B stored [28672, 8192] (bf16, E4M3)
  skinny_split  32 x 4096 x 14336 bf16 -> fp32, B stored [4096, 14336], K split (gemm_run_split)
  prefill_384   384 x 11008 x 4096 bf16 -> bf16 (128-row tiles of the 256-wide kernel)
  square4096_f32, square4096_f8, gate_up_f8  binary32 and one-byte inputs
  square256, ragged
  rms_norm       row normalisation of 2^20 f32 rows of 256 (HBM-bound)
  rms_norm_bf16  row normalisation of 65536 bf16 rows of 4096 (HBM-bound)
  attention      softmax attention, 64 entries x 4096 queries x 4096 keys, d = 128, bf16
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

# MI355X dense MFMA: bf16/f16 256 CU x 4096 FLOP/clk x 2.4 GHz; fp32 256 CU x 256 FLOP/clk x 2.4 GHz;
# 8-bit E4M3 / E5M2 256 CU x 8192 FLOP/clk x 2.4 GHz
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3, "f8e4m3": 5033.2, "f8e5m2": 5033.2}
IN_BYTES = {"bf16": 2, "f16": 2, "f32": 4, "f8e4m3": 1, "f8e5m2": 1}
PEAK_HBM_GBS = 8000.0                            # MI355X HBM3E
METRIC = "TFLOP/s and % of MI355X dense BF16 MFMA peak, 4096^3 GEMM"


SHARED_SOURCES = ("kernel_common.hpp", "launch.hpp")
NORM_SOURCES = ("rms_norm.hip", "norm.hpp")
ATTN_SOURCES = ("attention.hip", "attention.hpp")
# GEMM kernel families by the prefix of the planned kernel's name
GEMM_SOURCES = {"fast_f8": ("gemm_fast_f8.hip", "gemm_fast.hpp"), "fast_gate_up_f8": ("gemm_fast_f8.hip", "gemm_fast.hpp"),
                "fast_": ("gemm_fast.hip", "gemm_fast_gu.hip", "gemm_fast_128.hip", "gemm_fast.hpp"),
                "tiled_f32": ("gemm_f32.hip",),
                "tiled_": ("gemm_tiled.hpp", "gemm_tiled_64.hip", "gemm_tiled_128.hip", "gemm_tiled_p3.hip"),
                "skinny_": ("gemm_skinny.hip",)}


# host code that decides which instantiation a GEMM plan launches, and with which grid
PLANNER_SOURCES = ("planner.cpp", "kernels.cpp", "kernel_table.hpp")
# the split form's range sum and the host code that launches both kernels
SPLIT_SOURCES = ("split_sum.hip", "capi.cpp")


def gemm_plan_summary(workload):
    """The planned kernel of a GEMM workload: its name, grid and K blocks in flight."""
    import layout_algebra_amd as la
    w = synth.WORKLOADS[workload]
    d = la.gemm_plan(w.M, w.N, w.K, type_code(w.in_kind), type_code(w.out_kind), gate_up=w.gate_up,
                     b_kmajor=w.b_kmajor).describe()
    if w.split:
        return "%s grid=%s split=%d" % (d["split_kernel"], d["split_grid"], d["split_k"])
    return "%s grid=%d prefetch=%d" % (d["kernel"], d["grid"], d["prefetch_blocks"])


def type_code(kind):
    import layout_algebra_amd as la
    return {"bf16": la.BF16, "f16": la.F16, "f32": la.F32, "f8e4m3": la.F8E4M3, "f8e5m2": la.F8E5M2}[kind]


def workload_sources(workload):
    """Source files (csrc/) of what a workload runs: the row normalisation's, the attention's, or
    those of the GEMM kernel family its plan selects plus the planner that selects it, and the
    shared headers."""
    if workload in synth.NORM_WORKLOADS:
        own = NORM_SOURCES
    elif workload in synth.ATTN_WORKLOADS:
        own = ATTN_SOURCES
    else:
        kernel = gemm_plan_summary(workload).split()[0]
        own = next(v for k, v in GEMM_SOURCES.items() if kernel.startswith(k)) + PLANNER_SOURCES
        if synth.WORKLOADS[workload].split:
            own += SPLIT_SOURCES
    return tuple(sorted(own + SHARED_SOURCES))


def kernel_source_hash(workload):
    """sha1 (first 16 hex) over the sources of what a workload runs (workload_sources) and, for a
    GEMM, its plan summary (kernel, grid, K blocks in flight).  Identifies the kernels the traffic
    figures belong to: a planner change that moves a workload to another instantiation changes it."""
    import hashlib
    csrc = os.path.join(ROOT, "layout_algebra_amd", "csrc")
    h = hashlib.sha1()
    for name in workload_sources(workload):
        h.update(name.encode())
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    if workload in synth.WORKLOADS:
        h.update(gemm_plan_summary(workload).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per launch from profiles/traffic.md, or None when the
    workload's kernels changed since the counters were taken (or none were taken for it)."""
    path = os.path.join(ROOT, "profiles", "traffic.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            parts = line.split()
            # "traffic <workload>: <bytes> <source hash>"
            if len(parts) == 4 and parts[0] == "traffic" and parts[1] == workload + ":":
                return int(parts[2]) if parts[3] == kernel_source_hash(workload) else None
    return None


def algorithmic_bytes(w):
    """Compulsory HBM bytes of one step: every operand read once, C written (and read if beta != 0)."""
    eb = IN_BYTES[w.in_kind]
    ob = 4 if w.out_kind == "f32" else 2
    nb = 2 if w.gate_up else 1
    nout = 1 if w.act == "swiglu" else nb
    b = w.M * w.K * eb + nb * w.K * w.N * eb + nout * w.M * w.N * ob
    if w.beta != 0.0:
        b += w.M * w.N * ob
    return b


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The chip's clock keeps ramping for tens of milliseconds of sustained load: 200 untimed steps
    # reach the steady state (1100 -> 1250 TFLOP/s at 4096^3 against 10), and 1000 timed steps
    # (about 0.1 s at 4096^3) average over the power manager's fluctuations.
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="square4096", choices=sorted(synth.WORKLOADS) + sorted(synth.NORM_WORKLOADS) + sorted(synth.ATTN_WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--b-kmajor", action="store_true",
                    help="hand B (or the gate/up weights) to the library as [N,K] (K contiguous)")
    ap.add_argument("--a-transposed", action="store_true",
                    help="hand A (or x) to the library as [K,M] (M contiguous)")
    ap.add_argument("--gate-up-as-two-gemms", action="store_true",
                    help="gate_up workload only: run each step as two separate GEMM launches (x W_gate, then x W_up) "
                         "instead of the fused launch, for comparing their HBM traffic")
    ap.add_argument("--launch", choices=("graph", "eager"), default="graph",
                    help="timed steps as replays of a captured HIP graph (default), or one library call each")
    ap.add_argument("--preroll-seconds", type=float, default=0.5,
                    help="after the warm-up steps, replay the timed steps untimed for at least this long, "
                         "whatever --warmup is, so the timed region starts at the clock the chip settles to")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the clock/power reading (amd-smi during untimed replays after the timed region)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed region, run a plain elementwise copy of 256 MiB (reads 256 MiB, writes "
                         "256 MiB) three times: the reference dispatch for scaling HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (every output tile is "
              "independent, so the work would shard by output columns without communication). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.workload in synth.NORM_WORKLOADS:
        return bench_norm(args, synth.NORM_WORKLOADS[args.workload])
    if args.workload in synth.ATTN_WORKLOADS:
        return bench_attention(args, synth.ATTN_WORKLOADS[args.workload])

    import layout_algebra_amd as la
    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    b_kmajor = args.b_kmajor or w.b_kmajor
    torch.cuda.set_device(dev)

    x = synth.make_inputs(w)
    two = args.gate_up_as_two_gemms
    if two and (not w.gate_up or w.act):
        print("--gate-up-as-two-gemms applies to the gate_up workload only", file=sys.stderr)
        sys.exit(2)
    plan = la.gemm_plan(w.M, w.N, w.K, type_code(w.in_kind), type_code(w.out_kind), gate_up=w.gate_up and not two,
                        b_kmajor=b_kmajor, a_transposed=args.a_transposed)
    dev_b = (lambda t: t.t().contiguous().to(dev)) if b_kmajor else (lambda t: t.to(dev))
    A = x["A"].t().contiguous().to(dev) if args.a_transposed else x["A"].to(dev)
    out_dt = synth.torch_dtype(w.out_kind)
    if w.gate_up:
        Wg, Wu = dev_b(x["Wg"]), dev_b(x["Wu"])
        G = torch.empty((w.M, w.N), dtype=out_dt, device=dev)
        if w.act == "swiglu":
            def step(i):
                la.gemm_gate_up_swiglu_run(plan, A, Wg, Wu, G)
        elif two:
            U = torch.empty_like(G)

            def step(i):
                la.gemm_run(plan, A, Wg, G)
                la.gemm_run(plan, A, Wu, U)
        else:
            U = torch.empty_like(G)

            def step(i):
                la.gemm_gate_up_run(plan, A, Wg, Wu, G, U)
        result = G
        b_cpu = x["Wg"]
    else:
        Bs = [dev_b(x["B"])]
        if w.name.startswith("skinny"):
            # a second B buffer so consecutive steps do not hit B in the 256 MB last-level cache
            Bs.append(dev_b(w.dist_b.sample((w.K, w.N), w.seeds[2], synth.torch_dtype(w.in_kind))))
        C0 = x["C"].to(dev) if "C" in x else None
        C = torch.empty((w.M, w.N), dtype=out_dt, device=dev) if C0 is None else C0.clone()
        if w.split:
            # K cut into the plan's ranges: partial products into a workspace allocated here, once
            ws = torch.empty(la.gemm_plan_workspace_bytes(plan), dtype=torch.uint8, device=dev)

            def step(i):
                la.gemm_run_split(plan, A, Bs[i % len(Bs)], C, w.alpha, w.beta, ws)
        else:
            def step(i):
                la.gemm_run(plan, A, Bs[i % len(Bs)], C, w.alpha, w.beta)
        result = C
        b_cpu = x["B"]

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # parity of the timed launch configuration: run once on the first B, keep the result
    check_u = None
    if w.beta == 0.0 and not w.act:
        step(0)
        torch.cuda.synchronize()
        check = result.detach().clone()
        if w.gate_up:
            check_u = U.detach().clone()
    else:
        check = None

    # Timed region: K steps back to back on the current stream (as replays of a
    # captured HIP graph unless --launch eager), bracketed by a synchronize and
    # a pair of HIP events.  Each step is one launch of the GEMM kernel, so the
    # kernel's average duration is the region's time / K.
    run = steps_runner(step, args.steps, args.launch)
    pre = preroll(run, args.preroll_seconds)
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_all0.record(stream)
    run()
    t_all1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_all0.elapsed_time(t_all1)
    ms_per_step = total_ms / args.steps

    # Untimed: the timed launches left the output of their last step; one eager call of that
    # same step must reproduce it bit for bit (only with beta = 0: otherwise every step
    # rewrites C from its previous value).
    replay_equal = None
    if check is not None:
        last = (graph_chunk(args.steps) if args.launch == "graph" else args.steps) - 1
        replayed = result.detach().clone()
        step(last)
        torch.cuda.synchronize()
        replay_equal = bool(torch.equal(replayed, result))
        del replayed

    # Untimed: per-launch event pairs, for the spread of single-launch durations.
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(min(args.steps, 20))]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(len(starts))]
    for i in range(len(starts)):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    per_launch = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    clock = clock_sample(run) if not args.no_clock else None

    if args.copy_probe:
        copy_probe(dev)

    flops = w.flops()
    value_tflops = flops / (ms_per_step * 1e-3) / 1e12
    kern_ms = ms_per_step
    if w.name.startswith("skinny"):
        metric, unit = "achieved HBM GB/s, %s %dx%dx%d GEMM" % (w.name, w.M, w.N, w.K), "GB/s"
        bytes_ = algorithmic_bytes(w)
        value = bytes_ / (ms_per_step * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": bytes_ / (kern_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        metric, unit = (METRIC, "TFLOP/s") if w.name == "square4096" else ("TFLOP/s, %s GEMM" % w.name, "TFLOP/s")
        value = value_tflops
        roof = {"bound": "mfma", "achieved": flops / (kern_ms * 1e-3) / 1e12, "peak": PEAK_TFLOPS[w.in_kind],
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if roof["bound"] == "mfma" and w.flops() >= 1e11:
        roof["mfma_ceiling"] = mfma_ceiling(dev, A, flops, roof["achieved"])
    roof["traffic"] = measured_traffic(w.name)
    roof["kernel_avg_ms"] = kern_ms
    roof["single_launch_ms"] = {"min": float(per_launch.min()), "median": float(np.median(per_launch))}

    line = {
        "metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "strong",
        "vs_baseline": None, "dtype": w.in_kind, "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "in": w.in_kind, "out": w.out_kind,
                   "launch": args.launch,
                   "b_order": "nk" if b_kmajor else "kn",
                   "a_order": "km" if args.a_transposed else "mk",
                   "alpha": w.alpha, "beta": w.beta, "gate_up": w.gate_up,
                   "gate_up_as_two_gemms": two,
                   "kernel": plan.describe()["kernel"], "grid": plan.describe()["grid"]},
        "roofline": roof,
        "wall_s_timed": wall,
        "preroll": pre,
        "tflops": value_tflops,
        "pct_of_bf16_peak": 100.0 * value_tflops / PEAK_TFLOPS[w.in_kind],
    }

    if w.split:
        d = plan.describe()
        line["config"].update({"kernel": d["split_kernel"], "grid": d["split_grid"], "split_k": d["split_k"],
                               "workspace_bytes": d["workspace_bytes"]})
    line["clock"] = clock
    if roof["bound"] == "mfma":
        roof["at_measured_clock"] = at_clock(clock, roof["peak"], roof["achieved"])
    if replay_equal is not None:
        line["timed_output_equals_eager"] = replay_equal
    if not args.no_cpu_baseline:
        line["cpu_baseline"], line["parity_sample"] = cpu_baseline(w, x, b_cpu, check, args.cpu_seconds, value, unit,
                                                                   check_u)
    print(json.dumps(line), flush=True)


def mfma_ceiling(dev, operands, flops, achieved):
    """The matrix-core rate the chip sustains at this workload's size: the library's probe issues
    the same number of MFMAs per SIMD as the workload (32x32x16 for 16-bit inputs, 32x32x2 for
    binary32, 32x32x64 for E4M3; one wave per SIMD, 16 independent
    chains, no memory traffic) on 16-byte fragments of the workload's own input values, then on
    zeros (the multipliers' power, and so the clock the chip settles to, depends on the bits).
    Context for roofline.frac, which stays relative to the nominal peak."""
    import layout_algebra_amd as la
    depth = {torch.float32: 2, torch.float8_e4m3fn: 64}.get(operands.dtype, 16)
    per_mfma = 32 * 32 * depth * 2
    per_wave = max(16, int(round(flops / per_mfma / (256 * 4) / 16)) * 16)
    sink = torch.empty(256 * 256, dtype=torch.float32, device=dev)
    ops = operands.reshape(-1)[: 1 << 19]
    res = {}
    for name, src in (("tflops", ops), ("tflops_zero_operands", torch.zeros_like(ops))):
        ms, _, _, _ = timed_steps(lambda i: la.la_probe_mfma(src, sink, 256, per_wave), 10, 3, preroll_s=0.3)
        res[name] = 256 * 4 * per_wave * per_mfma / (ms * 1e-3) / 1e12
    res["operands"] = "first %d KiB of the workload's first input" % (ops.numel() * ops.element_size() // 1024)
    res["mfma_per_wave"] = per_wave
    res["frac"] = achieved / res["tflops"]
    return res


def copy_probe(dev):
    """A plain elementwise copy of 256 MiB (reads 256 MiB, writes 256 MiB), three times: the
    reference dispatch for scaling HBM byte counters."""
    src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def settled_clock(readings):
    """Median of the clock readings after the first (the first can still show the idle state)."""
    import statistics
    return statistics.median(readings[1:] if len(readings) > 1 else readings)


def clock_sample(run, seconds=1.5):
    """GPU clock and power while the workload runs: `run` (a whole timed region's worth of steps)
    is replayed, untimed, until amd-smi has been read three times from a child process (about
    `seconds`).  Returns the median gfx clock over the chip's XCDs per reading, the socket power,
    the maximum clock, and `settled_mhz`: the median of the readings after the first (amd-smi's
    first reading can still show the idle state from before the load began), or None when amd-smi
    is not there or reports nothing."""
    import shutil
    import subprocess
    import threading
    if shutil.which("amd-smi") is None:
        return None
    readings = []

    def sample():
        time.sleep(seconds / 3)
        for _ in range(3):
            try:
                out = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--power", "--json"],
                                     capture_output=True, text=True, timeout=30).stdout
                readings.append(json.loads(out[out.index("{"):]))
            except Exception:
                pass
            time.sleep(seconds / 3)

    t = threading.Thread(target=sample)
    t.start()
    while t.is_alive():
        run()
        torch.cuda.synchronize()
    t.join()
    clk, power, cmax = [], [], None
    for r in readings:
        try:
            gpu = r["gpu_data"][0] if "gpu_data" in r else r[0]
            gfx = [v for k, v in gpu["clock"].items() if k.startswith("gfx")]
            vals = sorted(float(v["clk"]["value"]) for v in gfx if isinstance(v.get("clk", {}).get("value"), (int, float)))
            if vals:
                clk.append(vals[len(vals) // 2])
            cmax = float(gfx[0]["max_clk"]["value"])
            pw = gpu["power"]["socket_power"]["value"]
            if isinstance(pw, (int, float)):
                power.append(float(pw))
        except Exception:
            continue
    if not clk:
        return None
    return {"gfx_mhz": clk, "settled_mhz": settled_clock(clk), "max_mhz": cmax, "socket_power_w": power,
            "method": "amd-smi metric during untimed replays of the timed steps, after the timed region"}


def at_clock(clock, peak, achieved):
    """For an MFMA-bound kernel: the nominal peak scaled to the clock measured while it ran, and
    the achieved rate as a fraction of that (context beside roofline.frac, which stays nominal)."""
    if not clock or not clock.get("max_mhz"):
        return None
    mhz = clock["settled_mhz"]
    p = peak * mhz / clock["max_mhz"]
    return {"peak_tflops": p, "frac": achieved / p, "gfx_mhz": mhz}


def preroll(run, seconds):
    """Untimed: call `run` (a whole timed region's worth of steps) until at least `seconds` have
    passed.  The chip's clock ramps for tens of milliseconds of sustained load and then settles at
    what its power limit allows; this makes the timed region start there whatever --warmup is."""
    t0 = time.perf_counter()
    n = 0
    while True:
        run()
        torch.cuda.synchronize()
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    return {"seconds": time.perf_counter() - t0, "replays_of_the_timed_steps": n}


def graph_chunk(steps):
    """Steps per captured graph: the largest divisor of `steps` up to 50, an even one where there
    is one (the skinny workload alternates two B buffers from step to step)."""
    divs = [d for d in range(1, min(steps, 50) + 1) if steps % d == 0]
    even = [d for d in divs if d % 2 == 0]
    return max(even) if even else max(divs)


def steps_runner(step, steps, launch):
    """A function that runs `steps` consecutive steps on the current stream: one library call each
    ("eager"), or steps / S replays of a HIP graph that captured S consecutive steps ("graph": no
    host work between kernels, so short kernels run back to back).  Capture runs no kernel."""
    if launch == "eager":
        def run():
            for i in range(steps):
                step(i)
        return run
    chunk = graph_chunk(steps)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(chunk):
            step(i)
    torch.cuda.synchronize()

    def run():
        for _ in range(steps // chunk):
            graph.replay()
    return run


def timed_steps(step, steps, warmup, launch="eager", clock=False, preroll_s=0.0):
    """Warm-up (eager), an untimed pre-roll of at least preroll_s seconds, then `steps`
    back-to-back steps (steps_runner) between two HIP events on the current stream (synchronised on
    both sides); then up to 20 single steps each between its own event pair.  Returns (ms per step,
    wall seconds, per-launch ms, clock_sample or None)."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    run = steps_runner(step, steps, launch)
    if preroll_s > 0:
        preroll(run, preroll_s)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = e0.elapsed_time(e1) / steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(min(steps, 20))]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(len(starts))]
    for i in range(len(starts)):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    per_launch = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    return ms, wall, per_launch, clock_sample(run) if clock else None


def bench_norm(args, w):
    """Row normalisation: one launch per step over inputs resident in HBM."""
    import layout_algebra_amd as la
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.make_norm_inputs(w)
    X, G = inp["X"].to(dev), inp["G"].to(dev)
    Y = torch.empty((w.M, w.D), dtype=synth.torch_dtype(w.out_kind), device=dev)

    def step(i):
        la.la_rms_norm_run(X, G, Y, w.eps)

    ms, wall, per_launch, clock = timed_steps(step, args.steps, args.warmup, args.launch, clock=not args.no_clock,
                                              preroll_s=args.preroll_seconds)
    if args.copy_probe:
        copy_probe(dev)
    bytes_ = w.bytes()
    gbs = bytes_ / (ms * 1e-3) / 1e9
    line = {
        "metric": "achieved HBM GB/s, row normalisation %d x %d %s" % (w.M, w.D, w.in_kind),
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "strong", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "D": w.D, "in": w.in_kind, "out": w.out_kind, "eps": w.eps,
                   "launch": args.launch},
        "clock": clock,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                     "traffic": measured_traffic(w.name), "kernel_avg_ms": ms,
                     "single_launch_ms": {"min": float(per_launch.min()), "median": float(np.median(per_launch))}},
        "wall_s_timed": wall,
        "preroll": {"seconds_min": args.preroll_seconds},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"], line["parity_sample"] = cpu_baseline_norm(w, inp, Y, args.cpu_seconds, gbs)
    print(json.dumps(line), flush=True)


def bench_attention(args, w):
    """Softmax attention: one launch per step over Q, K, V resident in HBM."""
    import layout_algebra_amd as la
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = synth.make_attn_inputs(w)
    Q, K, V = x["Q"].to(dev), x["K"].to(dev), x["V"].to(dev)
    O = torch.empty((w.batch, w.sq, w.d), dtype=synth.torch_dtype(w.out_kind), device=dev)

    def step(i):
        la.la_attention_run(Q, K, V, O, w.scale)

    ms, wall, per_launch, clock = timed_steps(step, args.steps, args.warmup, args.launch, clock=not args.no_clock,
                                              preroll_s=args.preroll_seconds)
    if args.copy_probe:
        copy_probe(dev)
    tflops = w.flops() / (ms * 1e-3) / 1e12
    line = {
        "metric": "TFLOP/s, softmax attention %d x %d x %d, d=%d" % (w.batch, w.sq, w.sk, w.d),
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "strong", "vs_baseline": None,
        "dtype": w.in_kind, "data": "synthetic",
        "clock": clock,
        "config": {"workload": w.name, "launch": args.launch, "batch": w.batch, "sq": w.sq, "sk": w.sk, "d": w.d, "in": w.in_kind,
                   "out": w.out_kind, "scale": w.scale},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_TFLOPS[w.in_kind], "unit": "TFLOP/s",
                     "frac": tflops / PEAK_TFLOPS[w.in_kind],
                     "mfma_ceiling": mfma_ceiling(dev, Q, w.flops(), tflops),
                     "at_measured_clock": at_clock(clock, PEAK_TFLOPS[w.in_kind], tflops),
                     "traffic": measured_traffic(w.name), "kernel_avg_ms": ms,
                     "single_launch_ms": {"min": float(per_launch.min()), "median": float(np.median(per_launch))}},
        "wall_s_timed": wall,
        "preroll": {"seconds_min": args.preroll_seconds},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"], line["parity_sample"] = cpu_baseline_attention(w, x, O, args.cpu_seconds, tflops)
    print(json.dumps(line), flush=True)


def host_cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where there is none)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def blas_threads():
    """Threads numpy's BLAS runs its matrix products on."""
    try:
        from threadpoolctl import threadpool_info
        n = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return 1


def cpu_baseline_attention(w, x, O, budget_s, gpu_value):
    """Time the oracle (numpy, binary64) on the first R queries of batch entry 0 (all keys),
    R sized to about budget_s seconds, and compare those GPU output rows with it."""
    import oracle

    def exact(t):
        return oracle.decode(synth.bits(t), w.in_kind)

    k, v = exact(x["K"][0]), exact(x["V"][0])
    probe = min(w.sq, 64)
    t0 = time.perf_counter()
    oracle.attention_f64(exact(x["Q"][0, :probe]), k, v, w.scale)
    per_row = (time.perf_counter() - t0) / probe
    R = int(max(probe, min(w.sq, budget_s / max(per_row, 1e-12))))
    q = exact(x["Q"][0, :R])
    t0 = time.perf_counter()
    ref = oracle.attention_f64(q, k, v, w.scale)
    dt = time.perf_counter() - t0
    value = 4.0 * R * w.sk * w.d / dt / 1e12
    base = {"value": value, "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle", "cpu_model": host_cpu_model(),
            "sample": "queries 0..%d of batch entry 0 against all %d keys, numpy binary64 (BLAS matmul), %.2f s"
                      % (R - 1, w.sk, dt),
            "seconds": dt, "gpu_over_cpu": gpu_value / value if value > 0 else None}
    # parity of the timed output on the first rows of the sample, against the per-row bound
    # built from the oracle's own softmax weights
    from oracle.tolerance import attention_bound
    P = min(R, 64)
    ref_p, tol = attention_bound(q[:P], k, v, w.scale, w.in_kind, w.out_kind)
    got = O[0, :P].to("cpu", torch.float64).numpy()
    err = np.abs(got - ref_p)
    return base, {"rows": P, "max_abs_err": float(err.max()), "ok": bool(np.all(err <= tol)),
                  "bound": "per row, from the oracle's softmax weights"}


def cpu_baseline_norm(w, inp, Y, budget_s, gpu_value):
    """Time the oracle (numpy, binary64) on the first R rows, R sized to about budget_s seconds,
    and compare those rows of the GPU output with it."""
    import oracle

    def exact(t):
        return t.double().numpy() if t.dtype == torch.float32 else oracle.decode(synth.bits(t), w.in_kind)

    x, g = inp["X"], exact(inp["G"])
    probe = min(w.M, 4096)
    t0 = time.perf_counter()
    oracle.rms_norm_f64(exact(x[:probe]), g, w.eps)
    per_row = (time.perf_counter() - t0) / probe
    R = int(max(probe, min(w.M, budget_s / max(per_row, 1e-12))))
    reps = max(1, int(budget_s / max(per_row * R, 1e-9))) if R == w.M else 1
    xs = exact(x[:R])
    t0 = time.perf_counter()
    for _ in range(reps):
        ref, _ = oracle.rms_norm_f64(xs, g, w.eps)
    dt = (time.perf_counter() - t0) / reps
    isz = 4 if w.in_kind == "f32" else 2
    osz = 4 if w.out_kind == "f32" else 2
    value = (R * w.D * (isz + osz) + w.D * isz) / dt / 1e9
    base = {"value": value, "unit": "GB/s", "cores": 1, "kind": "oracle", "cpu_model": host_cpu_model(),
            "sample": "rows 0..%d of %d (D=%d), numpy binary64, %.2f s per run, %d run(s)" % (R - 1, w.M, w.D, dt, reps),
            "seconds": dt, "gpu_over_cpu": gpu_value / value if value > 0 else None}
    got = Y[:R].to("cpu", torch.float64).numpy()
    rel = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -22}[w.out_kind]
    tol = ((w.D + 8) * 2.0 ** -24 + rel) * np.abs(ref) + (2.0 ** -25 if w.out_kind == "f16" else 0.0)
    err = np.abs(got - ref)
    return base, {"rows": R, "max_abs_err": float(err.max()), "ok": bool(np.all(err <= tol))}


def gemm_tolerance(w, a, b, ref):
    """Agreement bound of a GEMM output: 2^-20 K max|A| max|B| (FP32 accumulation; 2^-14 for
    one-byte inputs, whose 64-deep products the matrix core adds with less than binary32
    precision) plus the output's own rounding for 16-bit outputs (for fp32 outputs only where the
    result carries beta * C_old or K = 0, whose final fp32 rounding no accumulation term covers)."""
    e = -14 if IN_BYTES[w.in_kind] == 1 else -20     # one-byte products: the matrix core's own precision
    acc = 2.0 ** e * w.K * float(a.float().abs().max()) * float(b.float().abs().max())
    f32_rel = 2.0 ** -22 if (w.K == 0 or w.beta != 0.0) else 0.0
    rel = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": f32_rel}[w.out_kind]
    return acc + rel * np.abs(ref)


def cpu_baseline(w, x, b_cpu, check, budget_s, gpu_value, unit, check_u=None):
    """Time the oracle (as it is) on the first R output rows, R sized to about budget_s seconds;
    when the whole workload takes less than that, repeat it.  The timed GPU output is compared with
    those rows; for gate/up the second output (U = x W_up) is compared on the first 64 rows as well
    (an untimed oracle run)."""
    import oracle
    threads = oracle.max_threads()
    a = x["A"]
    probe_rows = list(range(min(w.M, 2 * threads)))
    t0 = time.perf_counter()
    oracle.gemm_f64(synth.bits(a[probe_rows]), w.in_kind, synth.bits(b_cpu), w.in_kind)
    per_row = (time.perf_counter() - t0) / len(probe_rows)
    R = int(max(len(probe_rows), min(w.M, budget_s / max(per_row, 1e-9))))
    reps = max(1, int(budget_s / max(per_row * R, 1e-9))) if R == w.M else 1
    rows = list(range(R))
    c_in = x["C"][rows].numpy() if "C" in x else None
    a_bits, b_bits = synth.bits(a[rows]), synth.bits(b_cpu)
    t0 = time.perf_counter()
    for _ in range(reps):
        ref = oracle.gemm_f64(a_bits, w.in_kind, b_bits, w.in_kind, w.alpha, w.beta, c_in)
    dt = (time.perf_counter() - t0) / reps
    flops = 2.0 * R * w.N * w.K
    if unit == "GB/s":
        bytes_ = (R * w.K + w.K * w.N) * IN_BYTES[w.in_kind] + R * w.N * 4
        value = bytes_ / dt / 1e9
    else:
        value = flops / dt / 1e12
    base = {"value": value, "unit": unit, "cores": threads, "kind": "oracle", "cpu_model": host_cpu_model(),
            "sample": "output rows 0..%d of %d (%d x %d outputs, K=%d%s), FP64 triple loop, %.2f s per run, %d run(s)"
                      % (R - 1, w.M, R, w.N, w.K, ", W_gate product only" if w.gate_up else "", dt, reps),
            "seconds": dt, "gpu_over_cpu": gpu_value / value if value > 0 else None}
    parity = None
    if check is not None:
        got = check[:R].to("cpu", torch.float64).numpy()
        err = np.abs(got - ref)
        parity = {"rows": R, "max_abs_err": float(err.max()), "ok": bool(np.all(err <= gemm_tolerance(w, a, b_cpu, ref)))}
        if check_u is not None:
            ru = list(range(min(R, 64)))
            ref_u = oracle.gemm_f64(synth.bits(a[ru]), w.in_kind, synth.bits(x["Wu"]), w.in_kind)
            err_u = np.abs(check_u[:len(ru)].to("cpu", torch.float64).numpy() - ref_u)
            ok_u = bool(np.all(err_u <= gemm_tolerance(w, a, x["Wu"], ref_u)))
            parity.update({"U_rows": len(ru), "U_max_abs_err": float(err_u.max()), "ok": parity["ok"] and ok_u})
    return base, parity


if __name__ == "__main__":
    main()
