#!/usr/bin/env python3
"""Benchmark: full Muon + AdamW optimizer steps per second on one MI355X.

One step = ``ma_muon_step`` over every weight matrix of the parameter set
(momentum, Frobenius / MuonEq normalisation, quintic Newton-Schulz, cautious
decay and update) plus ``ma_adamw_step`` over the embedding buffers, on
synthetic seeded inputs already resident in HBM. Default workload: the
12-layer d=1024 parameter set (48 x 1024^2, 12 x 4096x1024, 12 x 1024x4096
Muon matrices in bf16; wte and lm_head 50304x1024 AdamW in fp32).

Prints one JSON line (rank 0). The ``roofline`` object reports the dominant
kernel (by time) against its roofline, from HIP events recorded around each
launch on the launch stream during the timed steps; ``cpu_baseline`` times
the oracle on a bounded sample of the same workload on the host cores.
``lion`` times ``ma_lion_step`` separately, outside the Muon + AdamW step,
over fp32 buffers of the AdamW parameters' sizes (20 bytes per element).
``practical_peaks`` measures what the part sustains with the simplest
kernels (an MFMA loop with no memory traffic, a plain copy), beside the spec
peaks the roofline uses.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c3_12L_d1024")
    ap.add_argument("--ns-steps", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    ap.add_argument("--no-profile", action="store_true", help="time without per-kernel events")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay timing (one captured step replayed --steps times)")
    ap.add_argument("--no-lion", action="store_true", help="skip the separate Lion step timing")
    ap.add_argument("--no-overlap", action="store_true",
                    help="run AdamW after the Muon step on the same stream instead of beside it on a second one")
    ap.add_argument("--adamw-workgroups", type=int, default=256,
                    help="workgroups of the AdamW update when it runs beside the Muon step")
    ap.add_argument("--no-practical", action="store_true", help="skip the practical-peak calibration kernels")
    ap.add_argument("--no-latency", action="store_true",
                    help="skip the latency lines of the single 256x1024 matrix and the 4-layer d=256 set")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the timed steps, run 3 plain device copies of MIB MiB (read MIB, write MIB) "
                         "as the known-size reference that scales HBM byte counters")
    return ap.parse_args()


def elem_bytes(dt):
    return 2 if dt == "bf16" else 4


def work_model(wl, ns_steps, row_pass=None):
    """Algorithmic work per launch of each kernel kind (per step for the rest).
    row_pass[i]: group i reads G and M once (momentum, row sums and X0 in one
    pass, counted under "pre"); otherwise the row sums read them first."""
    ex = elem_bytes(wl.ns_precision)
    ep, eg, em = elem_bytes(wl.param_dtype), elem_bytes(wl.grad_dtype), elem_bytes(wl.mom_dtype)
    gram = poly = axpy = 0.0
    gram_b = poly_b = axpy_b = 0.0
    pre = rown = post = 0.0
    upd_b = 0.0
    for gi, g in enumerate(wl.muon_groups):
        m, n = min(g.rows, g.cols), max(g.rows, g.cols)
        gram += g.count * m * m * n          # A = X X^T, symmetric: m^2 n
        poly += g.count * m * m * m          # A A, symmetric: m^3
        axpy += g.count * 2.0 * m * m * n    # B X: 2 m^2 n
        # operands read once, outputs written once: GRAM reads X, writes A;
        # POLY reads A, writes B; AXPY reads B and X, writes X'
        gram_b += g.count * (m * n + m * m) * ex
        poly_b += g.count * (2.0 * m * m) * ex
        axpy_b += g.count * (m * m + 2.0 * m * n) * ex
        e = g.rows * g.cols * g.count
        if not (row_pass and row_pass[gi]):
            rown += e * (eg + em)            # read G, M
        pre += e * (eg + 2 * em + ex)        # read G, M; write M, X0
        post += e * (2 * ep + ex)            # read W, U; write W
        upd_b += e * 2 * ep                  # fused into the last AXPY: read W, write W
    adam = 28.0 * wl.adamw_numel
    return {
        "gram": ("TFLOP/s", gram), "poly": ("TFLOP/s", poly), "axpy": ("TFLOP/s", axpy),
        # the last AXPY of a step with the update in its epilogue (every group
        # of the benchmark workloads qualifies: stacked weights, rows of a
        # multiple of 8, no row scaling after the iteration)
        "axpy_update": ("TFLOP/s", axpy),
        "gemm_bytes": {"gram": gram_b, "poly": poly_b, "axpy": axpy_b, "axpy_update": axpy_b + upd_b},
        "rownorm": ("GB/s", rown), "pre": ("GB/s", pre), "post": ("GB/s", post), "adamw": ("GB/s", adam),
        "ns_total_flops_per_step": ns_steps * (gram + poly + axpy),
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs the optimizer step on one GPU; "
                                   f"--gpus {args.gpus} (WORLD_SIZE {world}) is not supported"}))
        sys.exit(2)

    import numpy as np
    import torch

    import adamw_optimizer_step_amd as M
    from adamw_optimizer_step_amd import _lib as L
    from workloads import materialize, workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workload(args.config)
    T = args.ns_steps if args.ns_steps is not None else wl.ns_steps
    t0 = time.time()
    data = materialize(wl, device=dev, seed=0)
    torch.cuda.synchronize()
    print(f"[bench] inputs for {wl.name} built in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    groups = [M.MuonGroup(d["W"], d["G"], d["M"]) for d in data["muon"]]
    hp = M.MuonHParams(lr=wl.lr, momentum=wl.momentum, weight_decay=wl.weight_decay, nesterov=wl.nesterov,
                       ns_steps=T, coeffs=M.KELLER_JORDAN, cautious=wl.cautious, equilibrate=wl.equilibrate,
                       ns_precision=wl.ns_precision, lr_scale=wl.lr_scale)
    ws = torch.empty(max(1, M.muon_workspace_size(groups, hp)), dtype=torch.uint8, device=dev)
    segs = []
    for a in data["adamw"]:
        s = a["spec"]
        segs.append(dict(param=a["p"], grad=a["g"], exp_avg=a["m"], exp_avg_sq=a["v"], step=a["step"],
                         lr=s.lr, beta1=s.beta1, beta2=s.beta2, eps=s.eps, weight_decay=s.weight_decay))

    def step(i):
        for s in segs:
            s["step"] = wl.adamw_step + i
        # AdamW on a second stream beside the Muon step unless --no-overlap
        M.optimizer_step(groups, hp, segs, workspace=ws, overlap=not args.no_overlap,
                         background_workgroups=args.adamw_workgroups)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    if args.copy_calibration:
        n = args.copy_calibration << 18          # fp32 elements in MIB MiB
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)              # one elementwise kernel: 4n bytes read, 4n written
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 3 x {4 * n} bytes read + {4 * n} written", file=sys.stderr, flush=True)
        del src, dst

    lib = L.lib()
    profile = not args.no_profile
    if profile:
        L.check(lib.ma_profile_begin(args.steps * 64 + 64))
    stream = torch.cuda.current_stream(dev)
    # an event at every step boundary: the whole-run mean and the per-step spread
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    if profile:
        L.check(lib.ma_profile_end())
    ms_eager = marks[0].elapsed_time(marks[-1]) / args.steps
    eager_q = quantiles([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])
    print(f"[bench] timed {args.steps} steps: {ms_eager:.3f} ms/step", file=sys.stderr, flush=True)

    # The same step captured once in a HIP graph and replayed: the kernels
    # and their arguments are those of one eager step (the AdamW step count,
    # a host scalar, stays at its captured value), with the launch gaps gone.
    ms_graph = None
    graph_q = None
    if not args.no_graph:
        ms_graph, per_replay = graph_timing(torch, dev, lambda: step(args.warmup + args.steps), args.steps)
        graph_q = quantiles(per_replay)
        print(f"[bench] graph replay: {ms_graph:.3f} ms/step (median {graph_q[1]:.3f})", file=sys.stderr, flush=True)

    # per-kernel durations from the events recorded around each launch
    import ctypes as C
    model = work_model(wl, T, [M.muon_row_pass(groups, hp, i) for i in range(len(groups))])
    kernels = {}
    if profile:
        for kind, name in enumerate(L.KERNEL_KINDS):
            tot, n = C.c_double(), C.c_int64()
            L.check(lib.ma_profile_read(kind, C.byref(tot), C.byref(n)))
            if n.value == 0:
                continue
            avg_ms = tot.value / n.value
            rec = {"ms_per_launch": round(avg_ms, 5), "launches_per_step": n.value / args.steps,
                   "ms_per_step": round(tot.value / args.steps, 4)}
            if name in model:
                unit, work = model[name]
                # elementwise kinds launch once per group chunk: spread the step's work
                per_launch = work * (args.steps / n.value) if unit == "GB/s" else work
                if unit == "TFLOP/s":
                    rec.update(achieved=round(per_launch / (avg_ms * 1e-3) / 1e12, 2), unit=unit)
                    b = model["gemm_bytes"][name]
                    rec.update(achieved_hbm=round(b / (avg_ms * 1e-3) / 1e9, 1),
                               algorithmic_bytes_per_launch=round(b),
                               algorithmic_flops_per_launch=round(per_launch))
                else:
                    rec.update(achieved=round(per_launch / (avg_ms * 1e-3) / 1e9, 1), unit=unit)
            kernels[name] = rec

    # every Newton-Schulz product, the last AXPY with the update fused into it included
    ns_ms = sum(kernels[k]["ms_per_step"] for k in ("gram", "poly", "axpy", "axpy_update") if k in kernels)
    peak_f = PEAK_BF16_TFLOPS if wl.ns_precision == "bf16" else PEAK_F32_TFLOPS
    roofline = None
    if kernels:
        dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
        r = kernels[dom]
        if r.get("unit") == "TFLOP/s":
            # the binding roofline of a GEMM: its flops at the MFMA peak or its
            # algorithmic bytes at the HBM peak, whichever takes longer
            t_f = model[dom][1] / (peak_f * 1e12)
            t_b = model["gemm_bytes"][dom] / (PEAK_HBM_GBS * 1e9)
            bound = "mfma" if t_f >= t_b else "hbm"
        else:
            bound = "hbm"
        if bound == "mfma" or r.get("unit") != "TFLOP/s":
            achieved, unit = r.get("achieved"), r.get("unit")
        else:
            achieved, unit = r.get("achieved_hbm"), "GB/s"
        peak = peak_f if bound == "mfma" else PEAK_HBM_GBS
        roofline = {"kernel": dom, "bound": bound, "achieved": achieved, "peak": peak,
                    "unit": unit, "frac": round((achieved or 0) / peak, 4),
                    "traffic": traffic_for(dom, wl.name)}
        if r.get("unit") == "TFLOP/s":
            roofline.update(mfma_frac=round(r["achieved"] / peak_f, 4),
                            hbm_frac=round(r["achieved_hbm"] / PEAK_HBM_GBS, 4))

    lion = None if args.no_lion else lion_timing(M, wl, dev, args.steps)
    practical = None if args.no_practical else practical_peaks(L, lib, dev)
    if roofline is not None and practical:
        # the practical ceiling for a product of real data: MFMAs on changing operands
        key = "mfma_bf16_changing_operands" if roofline["bound"] == "mfma" else "copy"
        if roofline["unit"] == practical[key]["unit"] and roofline.get("achieved"):
            roofline["frac_of_practical_peak"] = round(roofline["achieved"] / practical[key]["achieved"], 4)
    # the reported step time: the median step of the faster timing mode
    use_graph = graph_q is not None and graph_q[1] < eager_q[1]
    q = graph_q if use_graph else eager_q
    ms = q[1]
    latency = None if args.no_latency else latency_lines(M, torch, dev, args.steps)
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, T, args.cpu_budget_s)
    out = {
        "metric": "Muon+AdamW full steps/sec at 12L d=1024; NS-GEMM MFMA util %; HBM GB/s",
        "value": round(1000.0 / ms, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.ns_precision == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "ns_steps": T,
                   "coefficients": "Keller Jordan (3.4445, -4.7750, 2.0315) each step",
                   "muon_matrices": sum(g.count for g in wl.muon_groups),
                   "muon_elements": wl.muon_numel, "adamw_elements": wl.adamw_numel,
                   "parallelism": "single GPU",
                   "streams": ("AdamW on a second stream beside the Muon step" if (data["adamw"] and not args.no_overlap)
                               else "one stream"),
                   "timing": ("median of HIP-graph replays of one captured step" if use_graph
                              else "median of eager steps"),
                   "step_ms_p10_median_p90": [round(v, 4) for v in q],
                   "ms_per_step_eager_mean": round(ms_eager, 4),
                   "eager_step_ms_p10_median_p90": [round(v, 4) for v in eager_q],
                   "ms_per_step_graph_mean": round(ms_graph, 4) if ms_graph is not None else None,
                   "graph_step_ms_p10_median_p90": [round(v, 4) for v in graph_q] if graph_q else None,
                   "kernel_timing": "per-kernel HIP events inside the eager timed steps" if profile
                   else "no per-kernel events"},
        "roofline": roofline,
        "ns_gemm": {"tflops_per_step": round(model["ns_total_flops_per_step"] / 1e12, 4),
                    "ms_per_step": round(ns_ms, 4),
                    "achieved_tflops": round(model["ns_total_flops_per_step"] / (ns_ms * 1e-3) / 1e12, 1) if ns_ms else None,
                    "mfma_util": round(model["ns_total_flops_per_step"] / (ns_ms * 1e-3) / 1e12 / peak_f, 4) if ns_ms else None},
        "kernels": kernels,
        "lion": lion,
        "latency": latency,
        "practical_peaks": practical,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def quantiles(xs):
    """(p10, median, p90) of a list of step times."""
    v = sorted(xs)
    at = lambda q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]
    return at(0.1), at(0.5), at(0.9)


def graph_timing(torch, dev, step, n):
    """One call of ``step`` captured in a HIP graph (after a warm-up call on the
    capture stream), replayed ``n`` times with an event pair around each replay.
    Returns (whole-run mean ms, per-replay ms)."""
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(cap):
        step()
    torch.cuda.current_stream(dev).wait_stream(cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record(stream)
    for i in range(n):
        g.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
    mean = ev[0].elapsed_time(ev[-1]) / n
    del g
    return mean, per


def _step_latency(M, torch, dev, wl, n, **hp_kw):
    """Eager and graph-replay p10/median/p90 of one whole optimizer step of
    workload ``wl`` (hyperparameters overridden by ``hp_kw``), in
    microseconds."""
    from workloads import materialize
    data = materialize(wl, device=dev, seed=0)
    groups = [M.MuonGroup(d["W"], d["G"], d["M"]) for d in data["muon"]]
    kw = dict(lr=wl.lr, momentum=wl.momentum, weight_decay=wl.weight_decay, nesterov=wl.nesterov,
              ns_steps=wl.ns_steps, coeffs=M.KELLER_JORDAN, cautious=wl.cautious, equilibrate=wl.equilibrate,
              ns_precision=wl.ns_precision, lr_scale=wl.lr_scale)
    kw.update(hp_kw)
    hp = M.MuonHParams(**kw)
    ws = torch.empty(max(1, M.muon_workspace_size(groups, hp)), dtype=torch.uint8, device=dev)
    segs = [dict(param=a["p"], grad=a["g"], exp_avg=a["m"], exp_avg_sq=a["v"], step=a["step"], lr=a["spec"].lr,
                 beta1=a["spec"].beta1, beta2=a["spec"].beta2, eps=a["spec"].eps,
                 weight_decay=a["spec"].weight_decay) for a in data["adamw"]]
    step = lambda: M.optimizer_step(groups, hp, segs, workspace=ws, overlap=bool(segs))
    for _ in range(10):
        step()
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    eager = quantiles([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])
    _, per = graph_timing(torch, dev, step, n)
    graph = quantiles(per)
    del data, groups, ws, segs
    torch.cuda.empty_cache()
    return ([round(1e3 * v, 1) for v in eager], [round(1e3 * v, 1) for v in graph])


def latency_lines(M, torch, dev, n):
    """Latency of one whole optimizer step on the two small configurations,
    which are launch and latency bound (they cannot fill 256 CUs): the single
    fp32 256 x 1024 matrix (5 steps of the fp32 iteration; also swept over 1,
    3 and 5 steps in fp32 and bf16 iteration) and the 4-layer d=256 set (bf16
    Muon with AdamW beside it). Median and p10/p90 over ``n`` steps, eager and
    as graph replays, in microseconds."""
    from workloads import workload
    out = {}
    for name in ("c1_256x1024_f32", "c2_4L_d256"):
        wl = workload(name)
        eager, graph = _step_latency(M, torch, dev, wl, n)
        out[name] = {"description": wl.description, "unit": "us",
                     "eager_p10_median_p90": eager, "graph_p10_median_p90": graph,
                     "ns_gflop": round(wl.ns_steps * sum(g.count * (3 * min(g.rows, g.cols) ** 2 * max(g.rows, g.cols)
                                                                   + min(g.rows, g.cols) ** 3)
                                                          for g in wl.muon_groups) / 1e9, 3)}
        print(f"[bench] latency {name}: eager {eager[1]} us, graph {graph[1]} us", file=sys.stderr, flush=True)
        if name.startswith("c1_"):
            # the ns_steps sweep {1, 3, 5} of the same matrix, in both iteration precisions
            sweep = {}
            for prec in ("f32", "bf16"):
                for t in (1, 3, 5):
                    e, g = _step_latency(M, torch, dev, wl, n, ns_steps=t, ns_precision=prec)
                    sweep[f"{prec}_T{t}"] = {"eager_p10_median_p90": e, "graph_p10_median_p90": g}
            out[name]["sweep"] = sweep
            print("[bench] latency c1 sweep (graph median, us): " +
                  ", ".join(f"{k} {v['graph_p10_median_p90'][1]}" for k, v in sweep.items()), file=sys.stderr,
                  flush=True)
    return out


def practical_peaks(L, lib, dev):
    """What this part sustains with the simplest kernels, beside the spec peaks:
    bf16 MFMA with no memory traffic (ma_calib_mfma: 1024 workgroups of 4
    waves, each wave 16 independent 32x32x16 MFMAs per round) on near-constant
    operands and on random operands that change every MFMA (the part is power
    limited: the second draws more power and runs at a lower clock, which is
    the ceiling for products of real data), and a plain 1 GiB fp32 copy
    (torch.neg: 1 GiB read, 1 GiB written). Each MFMA figure is the steady
    state: about 0.25 s of launches to let the clock settle (a few launches
    straight from idle read 6-10% low), then 100 launches (about 0.25 s)
    timed."""
    import ctypes as C
    import torch
    stream = torch.cuda.current_stream(dev)
    blocks, iters, timed = 1024, 2048, 100
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    mfma = {}
    for changing in (0, 1):
        for _ in range(timed):
            L.check(lib.ma_calib_mfma(blocks, iters, changing, C.c_void_p(sink.data_ptr()),
                                      C.c_void_p(stream.cuda_stream)))
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(timed):
            L.check(lib.ma_calib_mfma(blocks, iters, changing, C.c_void_p(sink.data_ptr()),
                                      C.c_void_p(stream.cuda_stream)))
        e1.record(stream)
        torch.cuda.synchronize()
        mfma[changing] = timed * blocks * 4 * iters * 16 * 32768 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(10):
        torch.neg(src, out=dst)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 10 * 8 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst, sink
    torch.cuda.empty_cache()
    return {"mfma_bf16": {"achieved": round(mfma[0], 1), "unit": "TFLOP/s", "kernel": "ma_calib_mfma (constant operands)",
                          "frac_of_spec": round(mfma[0] / PEAK_BF16_TFLOPS, 4)},
            "mfma_bf16_changing_operands": {"achieved": round(mfma[1], 1), "unit": "TFLOP/s",
                                            "kernel": "ma_calib_mfma (random operands, new every MFMA)",
                                            "frac_of_spec": round(mfma[1] / PEAK_BF16_TFLOPS, 4)},
            "copy": {"achieved": round(copy_gbs, 1), "unit": "GB/s", "kernel": "torch.neg over 1 GiB fp32",
                     "frac_of_spec": round(copy_gbs / PEAK_HBM_GBS, 4)}}


def lion_timing(M, wl, dev, steps):
    """ma_lion_step over fp32 buffers of the AdamW parameters' sizes (one
    segment each), timed on its own: warm-up, then ``steps`` launches between
    two events on the launch stream."""
    import torch
    sizes = [a.numel for a in wl.adamw_segments] or [1 << 26]
    g = torch.Generator(device=dev).manual_seed(5)
    segs = []
    for n in sizes:
        segs.append(dict(param=torch.randn(n, device=dev, generator=g) * 0.02,
                         grad=torch.randn(n, device=dev, generator=g) * 1e-3,
                         exp_avg=torch.randn(n, device=dev, generator=g) * 1e-3,
                         lr=1e-4, beta1=0.95, beta2=0.98, weight_decay=1.0))
    for _ in range(3):
        M.lion_step(segs)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        M.lion_step(segs)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    n = sum(sizes)
    gbs = 20.0 * n / (ms * 1e-3) / 1e9
    del segs
    torch.cuda.empty_cache()
    return {"elements": n, "segments": len(sizes), "ms_per_step": round(ms, 4),
            "bytes_per_element": 20, "achieved": round(gbs, 1), "unit": "GB/s", "peak": PEAK_HBM_GBS,
            "frac": round(gbs / PEAK_HBM_GBS, 4)}


def traffic_for(kernel, workload_name):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's reading), if every
    source it was taken on is unchanged; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload_name}.json")
    if not os.path.exists(path):
        return None
    try:
        import hashlib
        rec = json.load(open(path))
        for src, digest in rec["sources"].items():
            if hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest() != digest:
                return None
        return rec["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(wl, T, budget_s):
    """The oracle, as it stands, on a bounded sample of the workload, scaled to
    whole steps per second."""
    import numpy as np
    import torch

    import oracle as O
    from workloads import materialize

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    # rounds over the shape groups, one more matrix of each group per round,
    # until the time budget is spent (at least one round)
    rounds = 16
    sample = materialize(wl.scaled(adamw_segments=()), device="cpu", seed=0, max_count=rounds)
    spent = 0.0
    times = [[] for _ in wl.muon_groups]
    for r in range(rounds):
        for gi, d in enumerate(sample["muon"]):
            if r >= d["W"].shape[0]:
                continue
            W, G, Mo = (d[k][r].float().numpy() for k in ("W", "G", "M"))
            t0 = time.perf_counter()
            O.muon_step(W, G, Mo, lr=wl.lr, momentum=wl.momentum, nesterov=wl.nesterov,
                        coeffs=O.KELLER_JORDAN, ns_steps=T, weight_decay=wl.weight_decay, cautious=wl.cautious,
                        equilibrate=wl.equilibrate, precision="bf16" if wl.ns_precision == "bf16" else "f64",
                        param_dtype=wl.param_dtype, mom_dtype=wl.mom_dtype)
            dt = time.perf_counter() - t0
            spent += dt
            times[gi].append(dt)
        if spent >= budget_s:
            break
    del sample
    per_group = [(g, sum(t) / len(t)) for g, t in zip(wl.muon_groups, times)]
    n_sampled = sum(len(t) for t in times)
    adam_n = min(wl.adamw_numel, 1 << 24)
    adam_s = 0.0
    if adam_n:
        rng = np.random.default_rng(0)
        p = (rng.standard_normal(adam_n) * 0.02).astype(np.float32)
        g = (rng.standard_normal(adam_n) * 1e-3).astype(np.float32)
        m = (rng.standard_normal(adam_n) * 3e-4).astype(np.float32)
        v = (g * g).astype(np.float32)
        t0 = time.perf_counter()
        O.adamw_step(p, g, m, v, 10, lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0)
        adam_s = time.perf_counter() - t0
    est = sum(g.count * dt for g, dt in per_group) + adam_s * (wl.adamw_numel / max(adam_n, 1))
    return {"value": round(1.0 / est, 6) if est > 0 else None, "unit": "steps/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{n_sampled} matrices ({', '.join(str(len(t)) for t in times)} of the "
                       f"{len(per_group)} shape groups) through the oracle's full Muon step "
                       f"({'bf16 rounding points' if wl.ns_precision == 'bf16' else 'float64'}, numpy BLAS) "
                       f"and {adam_n} AdamW elements; per-group mean times scaled by matrix and element counts "
                       f"to one whole step ({spent + adam_s:.1f} s of CPU time measured)")}


if __name__ == "__main__":
    main()
