#!/usr/bin/env python3
"""One-GPU benchmark of the per-matrix Muon update.

A step is one muon_step over the workload's whole matrix list (momentum, normalisation,
Newton-Schulz in the dispatcher's form per shape, fused weight update), inputs resident
in HBM. Prints one JSON line:
  value / ms_per_step  event-timed optimizer-step latency (lower is better)
  roofline             the dominant kernel's algorithmic FLOP rate against the bf16 dense
                       MFMA peak, from per-launch hipEvents recorded by the library on the
                       launch stream during a second timed pass
  cpu_baseline         the fp64 oracle on the host cores, on a bounded sample
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {"bf16": 2500.0, "f32": 157.3}       # dense MFMA TFLOP/s (MI355X public figures)
HBM_PEAK_GBS = 8000.0
GEMM_STAGES = ("syrk", "square", "apply", "apply_update")
HBM_STAGES = ("momentum_norm", "norm_finalize", "momentum")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dense_7b_28layers",
                    help="the 196-matrix 7B shape set (the largest workload, the default), or any "
                         "other workload of matrix_orthogonalising_optimizer_muon_amd.workloads")
    ap.add_argument("--also", default="single_bf16_2560x9728",
                    help="comma-separated further workloads timed in the same run (reported under "
                         "\"also\": ms per step, GEMM rate, dominant kernel); empty for none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=30.0)
    ap.add_argument("--details", action="store_true", help="also print the per-stage table to stderr")
    ap.add_argument("--mode", default="auto", choices=["auto", "gram", "plain", "auto_schedule"],
                    help="NS form: auto (plain or Gram 2+2+1 per shape, the default), gram, plain, or "
                         "auto_schedule (plain or Gram with the cheapest segment count per shape)")
    ap.add_argument("--also-modes", default="auto_schedule",
                    help="comma-separated further NS forms timed on the primary workload in the same run "
                         "(reported under \"modes\": ms per step, plan, GEMM rate); empty for none")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one muon_step captured in a HIP graph (after the warm-up "
                         "has measured the tiles) instead of eager calls")
    ap.add_argument("--adamw", action="store_true",
                    help="also time the AdamW step over the 7B shape set's non-matrix parameters "
                         "(embedding, head, biases, norms; fp32 W / m / v, bf16 G)")
    ap.add_argument("--tune-cache", default=None,
                    help="tile-choice file: loaded before the warmup when it exists, written after "
                         "it (so that separate profiling runs use the same kernels)")
    ap.add_argument("--one-stream", action="store_true",
                    help="run every shape group on the launch stream (MUON_FLAG_ONE_STREAM) instead of "
                         "up to four concurrent streams")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before warmup, copy this many MiB device-to-device once (a plain copy "
                         "kernel of known size, for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    return ap.parse_args()


def make_inputs(w, torch):
    from matrix_orthogonalising_optimizer_muon_amd import workloads as wl
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    host = w.elements <= 64 * 1024 * 1024
    Ws, Gs, Ms = [], [], []
    for i, spec in enumerate(w.matrices):
        if host:
            Ws.append(torch.from_numpy(wl.weight_np(w, i)).to("cuda").to(tdt[w.w_dtype]))
            Gs.append(torch.from_numpy(wl.gradient_np(w, 0, i)).to("cuda").to(tdt[w.g_dtype]))
        else:
            Ws.append(wl.weight_torch(w, i, "cuda"))
            Gs.append(wl.gradient_torch(w, 0, i, "cuda"))
        Ms.append(torch.zeros(spec.rows, spec.cols, dtype=tdt[w.m_dtype], device="cuda"))
    return Ws, Gs, Ms, ("seeded numpy draw" if host else "seeded torch device draw")


def cpu_baseline(w, budget_s):
    """The oracle as it stands, timed on the host: whole matrices in list order until the
    time budget is spent, scaled to the full workload by the sampled share of the
    dispatcher-model FLOPs (exact when the whole list fits)."""
    from matrix_orthogonalising_optimizer_muon_amd import workloads as wl
    from oracle import flop_model
    from oracle import muon as om
    try:
        from threadpoolctl import threadpool_info
        cores = max(int(i.get("num_threads", 1)) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))

    def mode_of(s):
        g = flop_model.dense_flops(s.rows, s.cols, "gram")
        p = flop_model.dense_flops(s.rows, s.cols, "plain")
        return "gram" if g < p else "plain"

    total_flops = sum(flop_model.dense_flops(s.rows, s.cols, mode_of(s)) for s in w.matrices)
    done_flops, t_used, n_done = 0.0, 0.0, 0
    for i, s in enumerate(w.matrices):
        W = wl.weight_np(w, i).astype(np.float64)
        G = wl.gradient_np(w, 0, i).astype(np.float64)
        M = np.zeros_like(G)
        t0 = time.perf_counter()
        om.muon_step(W, G, M, lr=w.lr, mu=w.mu, wd=w.wd, mode=mode_of(s))
        t_used += time.perf_counter() - t0
        done_flops += flop_model.dense_flops(s.rows, s.cols, mode_of(s))
        n_done += 1
        if t_used >= budget_s:
            break
    scale = total_flops / done_flops
    sample = (f"{n_done} of {len(w.matrices)} matrices, one full oracle step each (fp64 NumPy, "
              f"{t_used:.1f} s)" + ("" if n_done == len(w.matrices) else
                                    f"; scaled x{scale:.2f} by model FLOPs to the whole list"))
    return {"value": round(t_used * scale * 1e3, 3), "unit": "ms", "cores": cores, "kind": "oracle",
            "sample": sample, "cpu": cpu_model(), "blas": blas_vendor()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_vendor():
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', '')}, "
                f"{i.get('num_threads')} threads)" for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            return "; ".join(libs)
    except Exception:  # pragma: no cover
        pass
    return "unknown"


TRAFFIC_SOURCES = ("matrix_orthogonalising_optimizer_muon_amd/csrc/gemm.hip",
                   "matrix_orthogonalising_optimizer_muon_amd/csrc/elementwise.hip",
                   "matrix_orthogonalising_optimizer_muon_amd/csrc/internal.hpp")


def traffic_record(workload):
    """HBM bytes per launch measured by rocprofv3 (FETCH_SIZE and WRITE_SIZE passes, scaled by
    a copy of known size), per stage, tile configuration and shape group, as recorded in
    profiles/muon_step_<workload>.md; None when there is no record or the kernel sources
    changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"muon_step_{workload}.md")
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("<!-- traffic-record "):
                rec = json.loads(line[len("<!-- traffic-record "):].rsplit("-->", 1)[0])
    if rec is None:
        return None
    h = hashlib.sha256()
    for src in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if rec.get("source_sha256") != h.hexdigest():
        return None
    return rec


def adamw_bench(B, ctx, torch, args):
    """muon_adamw_step over the non-matrix parameters of the 7B shape set, inputs resident
    in HBM; algorithmic bytes 26 per element (W and m, v fp32 read + written, G bf16 read)."""
    from matrix_orthogonalising_optimizer_muon_amd import workloads as wl
    sizes = [n for _, n in wl.ADAMW_SETS["dense_7b_nonmatrix"]]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    ts = []
    for n in sizes:
        W = 0.02 * torch.randn(n, generator=gen, device="cuda")
        G = (1e-3 * torch.randn(n, generator=gen, device="cuda")).to(torch.bfloat16)
        ts.append((W, G, torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")))
    arr = B.adamw_tensor_list(ts)
    stream = torch.cuda.current_stream()
    elems = sum(sizes)
    for t in range(1, args.warmup + 1):
        B.check(B.muon_adamw_step(ctx, arr, B.make_adamw_hparams(step=t), stream.cuda_stream, len(ts)), "adamw")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for t in range(args.steps):
        B.check(B.muon_adamw_step(ctx, arr, B.make_adamw_hparams(step=args.warmup + 1 + t), stream.cuda_stream,
                                  len(ts)), "adamw")
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = 26.0 * elems / (ms * 1e-3) / 1e9
    print(f"[bench] adamw companion: {len(ts)} tensors, {elems / 1e6:.1f} M elements, {ms:.3f} ms/step, "
          f"{gbs:.0f} GB/s", file=sys.stderr, flush=True)
    return {"set": "dense_7b_nonmatrix", "tensors": len(ts), "elements": elems, "ms_per_step": round(ms, 4),
            "bytes_per_element": 26, "achieved_gbs": round(gbs, 1), "peak_gbs": HBM_PEAK_GBS,
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


NS_DESC = {"auto": "auto: plain NS (5 rounds) or Gram NS 2+2+1 per shape, by measured stage cost",
           "gram": "Gram 2+2+1", "plain": "plain 5 rounds",
           "auto_schedule": "auto_schedule: plain NS or Gram NS with k balanced segments (5 rounds), "
                            "per shape by measured stage cost"}


def run_workload(w, args, B, torch, ctx, pctx, primary, mode=None):
    """Inputs resident in HBM, warm-up (measures the tiles), K event-timed steps, then K
    steps with per-launch events for the stage table. Frees its buffers on return."""
    print(f"[bench] workload {w.name}: {len(w.matrices)} matrices, {w.elements / 1e6:.1f} M elements",
          file=sys.stderr, flush=True)
    Ws, Gs, Ms, data = make_inputs(w, torch)
    mats = list(zip(Ws, Gs, Ms))
    hp = B.make_hparams(lr=w.lr, momentum=w.mu, weight_decay=w.wd, mode=mode or args.mode,
                        w_dtype=w.w_dtype, g_dtype=w.g_dtype, m_dtype=w.m_dtype, ns_dtype=w.ns_dtype)
    arr = B.matrix_list(mats, hp, 0)
    nbytes = B.muon_workspace_size(ctx, mats, hp)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(c):
        B.check(B.muon_step(c, arr, hp, ws.data_ptr(), nbytes, sp, count=len(mats)), "muon_step")

    if primary and args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: {args.calibrate_copy_mib} MiB read + written", file=sys.stderr,
              flush=True)
        del src, dst

    if primary and args.tune_cache and os.path.exists(args.tune_cache):
        n = B.muon_tune_load(ctx, args.tune_cache)
        print(f"[bench] {n} tile choices loaded from {args.tune_cache}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(ctx)
    torch.cuda.synchronize()
    if primary and args.tune_cache:
        B.muon_tune_save(ctx, args.tune_cache)
    print(f"[bench] warmup done ({args.warmup} steps), workspace {nbytes / 2**30:.2f} GiB",
          file=sys.stderr, flush=True)

    graph = None
    if args.graph:
        # one step captured on a side stream; replays run on the launch stream
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                B.check(B.muon_step(ctx, arr, hp, ws.data_ptr(), nbytes, side.cuda_stream, count=len(mats)),
                        "muon_step (capture)")
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()

    # Timed region: exactly K steps between two events on the launch stream.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # One event between consecutive steps as well (recording adds no synchronisation), for
    # the per-step distribution.
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps - 1)]
    e0.record(stream)
    for i in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step(ctx)
        if i < args.steps - 1:
            marks[i].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    edges = [e0] + marks + [e1]
    per_step = sorted(edges[i].elapsed_time(edges[i + 1]) for i in range(args.steps))
    pct = lambda q: per_step[min(len(per_step) - 1, int(round(q * (len(per_step) - 1))))]
    print(f"[bench] {w.name}: timed {args.steps} steps: {ms:.4f} ms/step (wall {wall * 1e3 / args.steps:.4f})",
          file=sys.stderr, flush=True)

    # Second pass with per-launch events (library profiler) for the per-kernel roofline.
    step(pctx)  # warm-up of the profiling context (tile choices are already cached)
    torch.cuda.synchronize()
    B.muon_profile_read(pctx, 4096)
    for _ in range(args.steps):
        step(pctx)
    torch.cuda.synchronize()
    prof = B.muon_profile_read(pctx, 4096)
    plans = {}
    for i, spec in enumerate(w.matrices):
        key = f"{min(spec.rows, spec.cols)}x{max(spec.rows, spec.cols)}"
        if key in plans:
            continue
        e = B.muon_plan_info(ctx, mats, hp, i)
        plans[key] = {"mode": {1: "plain", 2: "gram"}[e.mode], "tile_sym": e.tile_sym,
                      "tile_apply": e.tile_apply, "segments": list(e.segments[:e.n_segments])}
    del Ws, Gs, Ms, mats, arr, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"ms": ms, "pct": (pct(0.1), pct(0.5), pct(0.9)), "prof": prof, "plans": plans, "data": data}


def summarise(w, r, args):
    """Dominant GEMM kernel, GEMM and HBM-phase rates and the stage table of a run."""
    prof = r["prof"]
    gemm = [e for e in prof if e["stage"] in GEMM_STAGES]
    dom = max(gemm, key=lambda e: e["total_ms"])
    avg_ms = dom["total_ms"] / dom["launches"]
    per_launch_flops = dom["flops"] / dom["launches"]
    achieved = per_launch_flops / (avg_ms * 1e-3) / 1e12
    peak = PEAK[w.ns_dtype]
    gemm_flops = sum(e["flops"] for e in gemm) / args.steps
    gemm_ms = sum(e["total_ms"] for e in gemm) / args.steps
    hbm = [e for e in prof if e["stage"] in HBM_STAGES]
    hbm_gbs = (sum(e["bytes"] for e in hbm) / (sum(e["total_ms"] for e in hbm) * 1e-3) / 1e9) if hbm else None
    mom = [e for e in prof if e["stage"] == "momentum"]
    mom_gbs = (sum(e["bytes"] for e in mom) / (sum(e["total_ms"] for e in mom) * 1e-3) / 1e9) if mom else None
    if args.details:
        for e in prof:
            rate = (e["flops"] / (e["total_ms"] * 1e-3) / 1e12) if e["flops"] else 0.0
            print(f"[stage] {w.name} {e['stage']:14s} m'={e['m']:6d} n'={e['n']:6d} x{e['count']:4d} "
                  f"launches={e['launches']:5d} avg={e['total_ms'] / e['launches'] * 1e3:9.2f} us "
                  f"{rate:8.1f} TFLOP/s", file=sys.stderr)
    return {
        "dom": dom,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": f"{dom['stage']} m'={dom['m']} n'={dom['n']} x{dom['count']} tile {dom['tile']}",
                     "avg_launch_us": round(avg_ms * 1e3, 2),
                     "flops_per_launch": per_launch_flops},
        "gemm_tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 1),
        "gemm_frac_of_peak": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / peak, 4),
        "momentum_gbs": None if mom_gbs is None else round(mom_gbs, 1),
        "momentum_frac_of_hbm": None if mom_gbs is None else round(mom_gbs / HBM_PEAK_GBS, 4),
        "hbm_phase_gbs": None if hbm_gbs is None else round(hbm_gbs, 1),
        "hbm_phase_frac_of_hbm": None if hbm_gbs is None else round(hbm_gbs / HBM_PEAK_GBS, 4),
        "profiled_ms_per_step": round(sum(e["total_ms"] for e in prof) / args.steps, 4),
        # per stage and shape group, from the profiled pass: launches per step, average
        # launch time (us, hipEvents on the launch stream), achieved TFLOP/s or GB/s
        "stages": [{"stage": e["stage"], "group": f"{e['m']}x{e['n']}x{e['count']}", "tile": e["tile"],
                    "launches_per_step": round(e["launches"] / args.steps, 2),
                    "avg_us": round(e["total_ms"] / e["launches"] * 1e3, 2),
                    **({"tflops": round(e["flops"] / (e["total_ms"] * 1e-3) / 1e12, 1)} if e["flops"] else {}),
                    **({"gbs": round(e["bytes"] / (e["total_ms"] * 1e-3) / 1e9, 1)}
                       if e["bytes"] and not e["flops"] else {})}
                   for e in prof],
    }


def add_traffic(roofline, workload, dom):
    """roofline["traffic"]: HBM bytes per launch of the dominant kernel from the committed
    counter record of the workload (null when there is none for this stage, tile and group,
    or the kernel sources changed since it was taken)."""
    rec = traffic_record(workload)
    st = rec["kernels"].get(f"{dom['stage']}/{dom['tile']}/{dom['m']}x{dom['n']}x{dom['count']}") if rec else None
    if st is not None:
        roofline["traffic"] = st["fetch_bytes"] + st["write_bytes"]
        roofline["traffic_unit"] = "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)"
        roofline["traffic_kernel"] = st["kernel"]
        if "trace_avg_us" in st:
            roofline["rocprof_avg_us"] = st["trace_avg_us"]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "exchange of the update is not built here", file=sys.stderr)
        sys.exit(2)

    import torch
    from matrix_orthogonalising_optimizer_muon_amd import binding as B
    from matrix_orthogonalising_optimizer_muon_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    ctx = B.muon_init(0, B.MUON_FLAG_ONE_STREAM if args.one_stream else 0)
    pctx = B.muon_init(0, B.MUON_FLAG_PROFILE)
    r = run_workload(w, args, B, torch, ctx, pctx, primary=True)
    sm = summarise(w, r, args)
    ms = r["ms"]
    dom = sm.pop("dom")
    out = {
        "metric": "Muon optimizer-step ms per shape set; GEMM TFLOP/s as % of bf16 MFMA peak",
        "value": round(ms, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms_p10_p50_p90": [round(x, 4) for x in r["pct"]],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.ns_dtype == "bf16" else "f32",
        "data": f"synthetic ({r['data']})",
        "config": {"workload": w.name, "matrices": len(w.matrices), "elements": w.elements,
                   "launch": "hip graph replay" if args.graph else "eager",
                   "shapes": sorted({f"{s.rows}x{s.cols}" for s in w.matrices}),
                   "ns": NS_DESC[args.mode],
                   "precision": ("G, M bf16 storage; W fp32; NS iterate and m'xm' recurrence in fp16 "
                                 "(power-of-two prescaled) on fp16 MFMA with fp32 accumulation"
                                 if w.ns_dtype == "bf16" else "fp32 throughout (fp32 MFMA)"),
                   "storage": {"W": w.w_dtype, "G": w.g_dtype, "M": w.m_dtype},
                   "plan": r["plans"]},
        **sm,
    }
    add_traffic(out["roofline"], w.name, dom)
    also = [x for x in args.also.split(",") if x and x != w.name] if args.also else []
    if also:
        out["also"] = {}
        for name in also:
            wa = wl.WORKLOADS[name]
            ra = run_workload(wa, args, B, torch, ctx, pctx, primary=False)
            sa = summarise(wa, ra, args)
            add_traffic(sa["roofline"], wa.name, sa.pop("dom"))
            out["also"][name] = {"ms_per_step": round(ra["ms"], 4),
                                 "step_ms_p10_p50_p90": [round(x, 4) for x in ra["pct"]],
                                 "plan": ra["plans"],
                                 **{k: sa[k] for k in ("roofline", "gemm_tflops", "gemm_frac_of_peak",
                                                       "momentum_gbs", "momentum_frac_of_hbm", "hbm_phase_gbs",
                                                       "hbm_phase_frac_of_hbm", "profiled_ms_per_step",
                                                       "stages")}}
    modes = [x for x in args.also_modes.split(",") if x and x != args.mode] if args.also_modes else []
    if modes:
        # the same workload with another Newton-Schulz form (same 5 rounds); the headline value
        # stays the form selected by --mode
        out["modes"] = {}
        for mname in modes:
            rm = run_workload(w, args, B, torch, ctx, pctx, primary=False, mode=mname)
            smm = summarise(w, rm, args)
            smm.pop("dom")
            out["modes"][mname] = {"ns": NS_DESC[mname], "ms_per_step": round(rm["ms"], 4),
                                   "step_ms_p10_p50_p90": [round(x, 4) for x in rm["pct"]],
                                   "plan": rm["plans"],
                                   **{k: smm[k] for k in ("gemm_tflops", "gemm_frac_of_peak", "profiled_ms_per_step")}}
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget_s)
    if args.adamw:
        out["adamw_companion"] = adamw_bench(B, ctx, torch, args)
    B.muon_destroy(ctx)
    B.muon_destroy(pctx)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
