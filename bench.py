#!/usr/bin/env python3
"""Benchmark of the fused depthwise->pointwise module on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload down_f16_64x56x56_c256_k512_s2] [--no-per-config]

A step is one invocation of the fused DW->PW kernel (one layer) on one batch of the
downsampling block: DW 3x3 s2 p1 over C=256 + scale/bias/ReLU6, PW 256->512 +
scale/bias/ReLU6, fp16 NHWC, N=64, 56x56 -> 28x28 (synthetic seeded inputs), the
largest of the benchmark workloads.  Inputs sit in HBM before the timed region.  The timed launches rotate over enough input/output
buffer sets (footprint > the 256 MB Infinity Cache) that every step streams its
input from HBM rather than from a cache.  The K steps are captured once in a HIP
graph and replayed, so the host's launch cost does not enter the measurement;
timing uses HIP events on the stream the kernels run on, bracketed by device
synchronisation.  The layer-by-layer pair (DW kernel writing the intermediate to
HBM + PW kernel reading it back) is timed the same way for comparison.  The same
protocol then times every benchmark workload (fp32 16x16, MobileNetV1 112x112,
CIFAR 32x32, the downsampling and late-stage layers, the 3x3 -> 1x1 back-to-back
pair) into the `per_config` object of the same line.

Prints ONE JSON line on stdout.  Diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MALL_BYTES = 256 * 1024 * 1024   # Infinity Cache
COPY_BYTES = 256 * 1024 * 1024   # plain copy used to calibrate the byte counters
COPY_STEPS = 5                   # copies a calibration run makes (--mode copy --steps 5)
PROFILES = os.path.join(ROOT, "profiles")
KDIR = "depthwise_pointwise_convolution_amd/csrc/kernels/"
# source file of each fused kernel family (by variant-name prefix) and the headers they share
KERNEL_FILES = [("dwpw_i8_", "dwpw_i8.hip"), ("wsl_", "dwpw_wsl.hip"), ("ws_", "dwpw_ws.hip"), ("pwdwpw_", "pwdwpw_mm.hip"),
                ("mmw_", "dwpw_mmw.hip"), ("mmwd_", "dwpw_mmw.hip"), ("mmm_", "dwpw_mm.hip"), ("mmf_", "dwpw_mm.hip"), ("mm_", "dwpw_mm.hip"), ("b2bmm_", "b2b_mm.hip"),
                ("dwpw_", "dwpw.hip"), ("b2b_", "b2b.hip"), ("pwdw_", "pwdw_mm.hip"),
                ("pwpw_", "pwpw_mm.hip"), ("gen_", "dwpw_gen.hip")]
SHARED_SOURCES = ["mm_common.h", "stages.h", "common.h"]
HEADLINE = "down_f16_64x56x56_c256_k512_s2"
# every benchmark workload, timed into per_config
PER_CONFIG = ["tiny_f32_1x16x16_c32", "mbv1_f16_8x112x112_c64_k128", "cifar_bf16_256x32x32_c128",
              "down_f16_64x56x56_c256_k512_s2", "late_f16_64x7x7_c1024", "b2b_f16_32x56x56_c64"]
# workloads the oracle is also timed on one thread
CPU_SINGLE_THREAD = ["tiny_f32_1x16x16_c32", "mbv1_f16_8x112x112_c64_k128"]
# dense matrix peaks (flop/s) by storage type; fp32 uses the fp32 peak (vector and matrix
# fp32 rates are the same, 157.3 TFLOP/s)
MATRIX_PEAK = {"f16": 2.5e15, "bf16": 2.5e15, "f32": 157.3e12, "i8": 5.0e15}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(variant: str) -> str:
    """Hash of the sources a variant's kernel is compiled from: a change there makes its
    stored counter figures stale."""
    own = next(f for prefix, f in KERNEL_FILES if variant.startswith(prefix))
    h = hashlib.sha256()
    for p in [own] + SHARED_SOURCES:
        with open(os.path.join(ROOT, KDIR, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, variant: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(PROFILES, f"traffic_{variant}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_hash(variant):
        return None
    return t.get("hbm_bytes_per_launch")


def summarize_pmc(workload: str, kernel: str, last: int, fetch_csv: str, write_csv: str,
                  copy_fetch_csv: str, copy_write_csv: str, copy_bytes: int) -> dict:
    """HBM bytes per launch of `kernel` from two rocprofv3 --pmc runs (FETCH_SIZE,
    WRITE_SIZE; KiB per dispatch), each scaled by what the same counter reads for a
    plain copy of copy_bytes (read and written once).  Uses the last `last`
    dispatches of the kernel (the timed ones)."""
    import csv
    import statistics as st

    def rows(path, match):
        out = []
        with open(path) as f:
            for r in csv.DictReader(f):
                if match in r["Kernel_Name"]:
                    out.append((int(r["Dispatch_Id"]), r["Counter_Name"],
                                float(r["Counter_Value"]), r["Kernel_Name"]))
        out.sort()
        return out

    def per_dispatch(path, match, counter, tail):
        rs = [r for r in rows(path, match) if r[1] == counter]
        rs = rs[-tail:] if tail else rs
        if not rs:
            raise SystemExit(f"no {counter} rows for {match!r} in {path}")
        return st.median(v for _, _, v, _ in rs), rs[-1][3], len(rs)

    fetch, kname, nf = per_dispatch(fetch_csv, kernel, "FETCH_SIZE", last)
    write, _, nw = per_dispatch(write_csv, kernel, "WRITE_SIZE", last)
    # the plain copies are the last COPY_STEPS copy dispatches of a --mode copy run
    # (earlier ones are the smaller set-up copies)
    cf, _, _ = per_dispatch(copy_fetch_csv, "copyBuffer", "FETCH_SIZE", COPY_STEPS)
    cw, _, _ = per_dispatch(copy_write_csv, "copyBuffer", "WRITE_SIZE", COPY_STEPS)
    k_fetch = copy_bytes / (cf * 1024.0)
    k_write = copy_bytes / (cw * 1024.0)
    read_b = fetch * 1024.0 * k_fetch
    write_b = write * 1024.0 * k_write
    return {"workload": workload, "kernel": kname, "dispatches": [nf, nw],
            "fetch_kib": fetch, "write_kib": write, "copy_fetch_kib": cf, "copy_write_kib": cw,
            "copy_bytes": copy_bytes, "scale_fetch": k_fetch, "scale_write": k_write,
            "hbm_read_bytes_per_launch": int(read_b), "hbm_write_bytes_per_launch": int(write_b),
            "hbm_bytes_per_launch": int(read_b + write_b)}


def time_graph(fn_list, steps, warmup, torch, stream):
    """Run fn_list[i % n] for warmup steps eagerly, capture `steps` calls in a HIP
    graph, replay it once untimed and once timed.  Returns ms per step."""
    n = len(fn_list)
    with torch.cuda.stream(stream):
        for i in range(warmup):
            fn_list[i % n]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            fn_list[i % n]()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        start.record(stream)
        g.replay()
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_eager(fn_list, steps, warmup, torch, stream):
    n = len(fn_list)
    with torch.cuda.stream(stream):
        for i in range(warmup):
            fn_list[i % n]()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        for i in range(steps):
            fn_list[i % n]()
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def _oracle_call(wl):
    import oracle
    import fcm_inputs
    inp = fcm_inputs.make_inputs(wl)
    kw = dict(stride=(wl.stride,) * 2, pad=(wl.pad,) * 2, scale1=inp["scale1"],
              bias1=inp["bias1"], act1=wl.act1, scale2=inp["scale2"], bias2=inp["bias2"],
              act2=wl.act2, dtype=wl.dtype)
    if wl.kind == "pwdwpw":
        kw.update(scale3=inp["scale3"], bias3=inp["bias3"], act3=wl.act3, residual=wl.residual)
        return lambda: oracle.pwdwpw(inp["x"], inp["w1"], inp["w2"], inp["w3"], **kw)
    fn = {"dwpw": oracle.dwpw, "b2b": oracle.b2b, "pwdw": oracle.pwdw,
          "pwpw": oracle.pwpw}[wl.kind]
    if wl.kind == "dwpw" and (wl.R != 3 or wl.S != 3 or wl.dil != 1 or wl.mult != 1):
        fn = oracle.dwpw_gen  # generalised depthwise layer
        kw["dilation"] = (wl.dil, wl.dil)
    return lambda: fn(inp["x"], inp["w1"], inp["w2"], **kw)


def _time_oracle(wl, budget_s: float, max_runs: int = 50):
    call = _oracle_call(wl)
    times = []
    t_all = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        call()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all >= budget_s or len(times) >= max_runs:
            break
    return statistics.median(times), len(times)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s: float):
    """The CPU oracle, as it stands, on the same workload: the full layer (all N
    images) run repeatedly until `budget_s` of wall time is spent; median time.  Then
    the small workloads once more on a single thread."""
    import oracle
    import fcm_inputs
    med, n = _time_oracle(wl, budget_s)
    cores = oracle.threads()
    single = {}
    oracle.set_threads(1)
    try:
        for name in CPU_SINGLE_THREAD:
            m1, n1 = _time_oracle(fcm_inputs.WORKLOADS[name], budget_s / 2, max_runs=200)
            single[name] = {"value": round(m1 * 1e6, 1), "unit": "us/layer", "runs": n1}
    finally:
        oracle.set_threads(cores)
    return {"value": round(med * 1e6, 1), "unit": "us/layer", "cores": cores,
            "kind": "oracle",
            "sample": f"full layer (N={wl.N}) evaluated {n} times, median; "
                      f"C/OpenMP double-precision direct loops on {cores} threads",
            "cpu_model": cpu_model(), "single_thread": single}


def roof(plan, wl, us: float) -> dict:
    """Roofline of a measured launch: the larger of the HBM floor (compulsory bytes at
    8 TB/s) and the matrix floor (flops at the storage type's dense peak) binds."""
    t_hbm = plan.alg_bytes_fused / (HBM_PEAK_GBS * 1e9) * 1e6
    t_mat = plan.flops / MATRIX_PEAK[wl.dtype] * 1e6
    if t_mat > t_hbm:
        ach = plan.flops / (us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 1),
                "peak": MATRIX_PEAK[wl.dtype] / 1e12, "unit": "TFLOP/s",
                "frac": round(t_mat / us, 4), "floor_us": round(t_mat, 3)}
    ach = plan.alg_bytes_fused / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(t_hbm / us, 4), "floor_us": round(t_hbm, 3)}


def measure(name, args, steps, warmup, torch, dev, stream, with_unfused=True):
    """Plan (and, with --tune, measure-choose) the fused kernel of one workload,
    then time the fused and the layer-by-layer paths over a buffer rotation that
    exceeds the Infinity Cache.  Returns the figures and the module."""
    import fcm_inputs
    from depthwise_pointwise_convolution_amd import fcm_variant_name
    from depthwise_pointwise_convolution_amd.module import TORCH_DTYPES, from_workload

    wl = fcm_inputs.WORKLOADS[name]
    inp = fcm_inputs.make_inputs(wl)
    variant = args.variant if name == args.workload else None
    mod = from_workload(wl, inp, device=dev, variant=variant)
    tdt = TORCH_DTYPES[wl.dtype]
    x0 = torch.from_numpy(inp["x"]).to(tdt).to(dev)
    set_bytes = mod.plan.alg_bytes_fused + mod.plan.workspace_bytes
    nsets = args.sets if args.sets > 0 else max(2, -(-2 * MALL_BYTES // set_bytes))
    xs = [x0] + [x0.clone() for _ in range(nsets - 1)]
    ys = [mod.new_output(dev) for _ in range(nsets)]
    ts = [torch.empty(mod.t_shape, dtype=tdt, device=dev) for _ in range(nsets)]
    torch.cuda.synchronize()
    if variant is None and args.tune and args.mode != "variants":
        # measured choice of variant and grid (untimed, before the timing proper)
        with torch.cuda.stream(stream):
            mod.tune(xs, ys, iters=2 * nsets, stream=stream)
        torch.cuda.synchronize()
    plan = mod.plan
    vname = fcm_variant_name(plan.variant)
    log(f"workload {wl.name}: {wl.description}")
    log(f"  variant {plan.variant} {vname}, grid {plan.grid}"
        + (f" (tuned: {plan.tuned_us:.2f} us)" if plan.tuned_us > 0 else " (analytic plan)")
        + f", {nsets} buffer sets ({nsets * set_bytes / 2**20:.0f} MiB rotation)")
    fused = [lambda i=i: mod.fused(xs[i], ys[i]) for i in range(nsets)]
    unfused = [lambda i=i: mod.unfused(xs[i], ts[i], ys[i]) for i in range(nsets)]
    res = {"wl": wl, "mod": mod, "plan": plan, "vname": vname, "nsets": nsets,
           "fused": fused, "unfused": unfused, "xs": xs, "ys": ys}
    if args.mode != "bench":
        return res
    timer = time_eager if args.eager else time_graph
    res["ms_fused"] = timer(fused, steps, warmup, torch, stream)
    log(f"  fused: {res['ms_fused'] * 1e3:.2f} us/layer")
    # the replayed launches wrote what an eager call of the same plan writes
    ref = mod.fused(xs[0]).double()
    torch.cuda.synchronize()
    assert torch.equal(ys[0].double(), ref), f"{name}: graph replay output differs from eager"
    res["ms_unfused"] = None
    if with_unfused:
        res["ms_unfused"] = timer(unfused, steps, warmup, torch, stream)
        log(f"  unfused (DW + PW kernels): {res['ms_unfused'] * 1e3:.2f} us/layer")
    return res


def config_entry(r) -> dict:
    """One workload's figures for the per_config object."""
    wl, plan = r["wl"], r["plan"]
    us = r["ms_fused"] * 1e3
    e = {"fused_us": round(us, 3),
         "fused_gbs": round(plan.alg_bytes_fused / (us * 1e-6) / 1e9, 1),
         "alg_bytes_fused": plan.alg_bytes_fused, "alg_bytes_unfused": plan.alg_bytes_unfused,
         "roofline": roof(plan, wl, us), "traffic": measured_traffic(wl.name, r["vname"]),
         "kernel_variant": r["vname"], "grid": plan.grid, "dtype": wl.dtype}
    if r.get("ms_unfused") is not None:
        uu = r["ms_unfused"] * 1e3
        e["unfused_us"] = round(uu, 3)
        e["unfused_gbs"] = round(plan.alg_bytes_unfused / (uu * 1e-6) / 1e9, 1)
        e["speedup_fused_over_unfused"] = round(uu / us, 3)
    return e


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--variant", type=int, default=None, help="force a fused kernel variant")
    ap.add_argument("--tune", action="store_true",
                    help="replace the planner's analytic plan by the measured choice (fcm_tune); "
                         "the default analytic plan makes every run, profiled or not, use the "
                         "same kernel")
    ap.add_argument("--no-tune", dest="tune", action="store_false",
                    help="the analytic plan (the default)")
    ap.add_argument("--eager", action="store_true", help="time eager launches, no graph")
    ap.add_argument("--sets", type=int, default=0,
                    help="input/output buffer sets in rotation (0 = enough to exceed the "
                         "Infinity Cache, so inputs stream from HBM)")
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="time only the headline workload")
    ap.add_argument("--per-config-steps", type=int, default=200)
    ap.add_argument("--cpu-budget", type=float, default=8.0,
                    help="seconds of oracle time for the cpu_baseline leg (0 = skip)")
    ap.add_argument("--mode", default="bench", choices=["bench", "fused-only", "unfused-only",
                                                        "copy", "variants"],
                    help="profiling helpers: run only one path (or a plain copy) K times")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH",
                                                          "COPY_WRITE"),
                    help="write profiles/traffic_<variant>_<workload>.json from rocprofv3 "
                         "--pmc FETCH_SIZE / WRITE_SIZE csv files of --mode fused-only and "
                         "--mode copy runs (no GPU needed)")
    ap.add_argument("--kernel", default="dwpw_mm_kernel", help="kernel name for --summarize-pmc")
    ap.add_argument("--variant-name", default=None, help="variant name for --summarize-pmc")
    args = ap.parse_args(argv)

    if args.summarize_pmc:
        t = summarize_pmc(args.workload, args.kernel, args.steps, *args.summarize_pmc,
                          copy_bytes=COPY_BYTES)
        t["variant"] = args.variant_name
        t["kernel_source_sha"] = kernel_source_hash(args.variant_name)
        path = os.path.join(PROFILES, f"traffic_{args.variant_name}_{args.workload}.json")
        with open(path, "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t))
        return 0

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the module would "
              "shard over the batch with no exchange between GPUs, so the one-GPU figure is "
              "the per-GPU rate", file=sys.stderr)
        return 2

    import torch

    assert torch.cuda.is_available(), "bench.py needs the MI355X"
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)

    if args.mode == "copy":
        # plain copy of known size for counter calibration
        a = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copied {args.steps} x {a.numel()} bytes")
        return 0

    if args.mode == "variants":
        # every variant able to run the workload at its analytic plan's grid, timed like the
        # benchmark; one JSON line per variant (a stored table the planner is checked against)
        import depthwise_pointwise_convolution_amd as F
        base = measure(args.workload, args, 0, 0, torch, dev, stream, with_unfused=False)
        analytic = F.fcm_plan(base["mod"].prob)
        for v in range(F.fcm_num_variants()):
            try:
                pv = F.fcm_plan_variant(base["mod"].prob, v)
            except F.FcmError:
                continue
            base["mod"].plan = pv
            ms = time_graph(base["fused"], args.steps, args.warmup, torch, stream)
            print(json.dumps({"workload": args.workload, "variant": F.fcm_variant_name(v),
                              "grid": pv.grid, "us": round(ms * 1e3, 3),
                              "pred_us": round(pv.pred_us_fused, 3),
                              "analytic_choice": v == analytic.variant}), flush=True)
        return 0

    r = measure(args.workload, args, args.steps, args.warmup, torch, dev, stream,
                with_unfused=not args.no_unfused)
    if args.mode in ("fused-only", "unfused-only"):
        fl = r["fused"] if args.mode == "fused-only" else r["unfused"]
        with torch.cuda.stream(stream):
            for i in range(args.warmup + args.steps):
                fl[i % r["nsets"]]()
        torch.cuda.synchronize()
        log(f"{args.mode}: {args.warmup + args.steps} launches done")
        return 0

    wl, plan, vname = r["wl"], r["plan"], r["vname"]
    ms_fused, ms_unfused = r["ms_fused"], r["ms_unfused"]
    us = ms_fused * 1e3
    alg = plan.alg_bytes_fused
    achieved = alg / (us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(wl.name, vname)}
    head_entry = config_entry(r)
    nsets = r["nsets"]
    del r
    torch.cuda.empty_cache()

    per_config = {}
    if not args.no_per_config:
        for name in PER_CONFIG:
            if name == wl.name:
                per_config[name] = head_entry
                continue
            rc = measure(name, args, args.per_config_steps, min(args.warmup, 20), torch, dev,
                         stream)
            per_config[name] = config_entry(rc)
            del rc
            torch.cuda.empty_cache()

    out = {
        "metric": "fused DW+PW us/layer and achieved HBM GB/s (% of peak) vs unfused, 1 MI355X",
        "value": round(us, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_fused, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.description}", "N": wl.N, "H": wl.H,
                   "W": wl.W, "C": wl.C, "K": wl.K, "stride": wl.stride,
                   "filter": [wl.R, wl.S], "dilation": wl.dil, "depth_multiplier": wl.mult,
                   "kernel_variant": vname, "grid": plan.grid,
                   "selection": "measured (fcm_tune)" if plan.tuned_us > 0 else "analytic plan",
                   "timing": "eager" if args.eager else "hip-graph",
                   "buffer_sets": nsets},
        "roofline": roofline,
        "hbm_gbs": round(achieved, 1),
        "hbm_pct_of_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "alg_bytes_fused": alg,
        "alg_bytes_unfused": plan.alg_bytes_unfused,
    }
    if ms_unfused is not None:
        uu = ms_unfused * 1e3
        out["unfused"] = {"value": round(uu, 3), "unit": "us/layer",
                          "hbm_gbs": round(plan.alg_bytes_unfused / (uu * 1e-6) / 1e9, 1),
                          "speedup_fused_over_unfused": round(uu / us, 3)}
    if per_config:
        out["per_config"] = per_config
    if args.cpu_budget > 0:
        cb = cpu_baseline(wl, args.cpu_budget)
        out["cpu_baseline"] = cb
        log(f"cpu oracle: {cb['value']} us/layer on {cb['cores']} threads ({cb['cpu_model']})")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
