#!/usr/bin/env python3
"""Benchmark of the W4A16 group-quantized GEMM on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME[,NAME]|all]
                    [--path auto|gemv|tile|split|packed|swiglu|repacked|small-packed[,...]]
                    [--no-cpu]

A step is one call of the chosen entry point (the whole hot path: validate,
launch, unpack + dequant + contraction + reduction + store) on one batch of
synthetic input: w4a16_gemm / w4a16_gemm_path for auto, gemv and tile;
w4a16_gemm_split (activation prep, fp16-MFMA contraction, split-K reduce) for
split; w4a16_gemm_split_packed for packed, whose one-time weight repack runs
before the timed region and is reported on its own (repack_ms_one_time);
w4a16_gemm_swiglu for swiglu (the workload's W read as gate rows then up rows,
Y = silu(gate) * up, [M][N/2]); w4a16_gemm_repacked (no workspace) for
repacked, on weights repacked once by w4a16_repack, and
w4a16_gemm_small_packed (M <= 64; contraction and split-K reduce) for
small-packed, on weights repacked once by w4a16_grouped_pack
(repack_ms_one_time).  Inputs are resident in HBM before the timed region starts.
Copies of {X, qweight, scales, Y} rotate so that every step reads cold HBM
(the copies together are at least twice the 256 MB Infinity Cache).  The K
timed steps are captured once in a HIP graph and replayed, so the host's
launch cost does not starve the GPU; HIP events bracket the replay on the
stream the kernels run on.

One JSON line is printed per workload (by default only the decode gate+up
GEMV, M=1 K=7168 N=4096, which the headline metric is quoted on).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "W4A16 GEMM effective HBM GB/s (M≤64) and TFLOP/s (M=4096), % of roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
FP32_PEAK_TFLOPS = 157.3     # MI355X dense fp32 matrix, published
FP16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 matrix, published
MALL_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = "int4_weight_only_03_amd/csrc/"
PATH_NAMES = {"auto": 0, "gemv": 1, "tile": 2, "split": 3, "packed": 4, "swiglu": 5,
              "repacked": 6, "small-packed": 7}
SPLIT_PATHS = ("split", "packed")
# paths whose products are fp16 matrix instructions on two activation limbs
LIMB_PATHS = ("split", "packed", "repacked", "small-packed")
# the sources whose kernels a path runs (the C-ABI layer dispatches every path)
PATH_SOURCES = {"gemv": ["gemv.hip", "gemv_mfma.hip", "gemv_common.h", "limbs.h"], "tile": ["tile.hip"],
                "split": ["split.hip", "limbs.h"], "packed": ["split.hip", "limbs.h"],
                "swiglu": ["gemv.hip", "gemv_mfma.hip", "gemv_common.h", "limbs.h"],
                "grouped": ["grouped.hip", "gemv_common.h", "limbs.h"],
                "grouped-packed": ["grouped.hip", "gemv_common.h", "limbs.h"],
                "repacked": ["packed_gemv.hip", "small_packed.hip", "gemv_common.h", "limbs.h"],
                "small-packed": ["small_packed.hip", "gemv_common.h", "limbs.h"]}


def source_hash(path: str) -> str:
    """Hash of the sources behind a (resolved) path; counter data older than it is void."""
    h = hashlib.sha256()
    for rel in PATH_SOURCES[path] + ["w4a16_api.cpp"]:
        with open(os.path.join(ROOT, CSRC, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, path: str):
    """HBM bytes per call from the committed counter runs, if those kernels are unchanged."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    entry = rec.get("entries", {}).get(f"{workload}/{path}")
    if entry is None or entry.get("source_hash") != source_hash(path):
        return None
    return entry.get("bytes_per_launch")


def metric_in_gbs(wl) -> bool:
    """The metric is effective HBM GB/s for M <= 64 and TFLOP/s above."""
    return wl.M <= 64


def time_steps(step, steps: int, stream):
    """(ms per step of a graph replay of `steps` steps, eager per-launch ms, graphed)."""
    import torch
    # per-launch durations with events around each launch (eager), for the
    # kernel-time cross-check against rocprofv3
    n_ev = min(steps, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_ev)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    per_launch_ms = [a.elapsed_time(b) for a, b in evs]

    graphed = True
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                step(i)
        g.replay()                                  # warm replay
        torch.cuda.synchronize()
    except Exception as e:                          # capture refused: time eager launches
        graphed = False
        print(f"# graph capture failed ({e}); timing eager launches", file=sys.stderr)

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    if graphed:
        g.replay()
    else:
        for i in range(steps):
            step(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, per_launch_ms, graphed


def gpu_leg_moe(name: str, steps: int, warmup: int, packed: bool = False):
    """The grouped (MoE) GEMM on a synthetic routed decode batch; with `packed`
    the weights are first repacked (w4a16_grouped_pack, timed on its own)."""
    import torch
    import int4_weight_only_03_amd as pkg

    wl = workloads.MOE_WORKLOADS[name]
    dev = torch.device("cuda:0")
    X, W, ti, off = workloads.make_moe(name)
    quantized = [pkg.w4a16_quantize(W[e]) for e in range(wl.E)]   # the library's host quantizer
    qw = np.stack([q for q, _ in quantized])
    sc = np.stack([s for _, s in quantized])
    del quantized
    B = wl.algorithmic_bytes(off)
    copies = max(1, -(-2 * MALL_BYTES // B))
    Xd, Qd, Sd = (torch.from_numpy(a).to(dev) for a in (X, qw, sc))
    Id, Od = torch.from_numpy(ti).to(dev), torch.from_numpy(off).to(dev)
    sets = [(Xd.clone(), Qd.clone(), Sd.clone(),
             torch.empty((wl.R, wl.N), dtype=torch.float32, device=dev)) for _ in range(copies)]
    del Xd, Qd, Sd
    stream = torch.cuda.current_stream(dev)
    repack_ms = None
    if packed:  # one-time repack of every copy; its time is reported, not in the steps
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        bufs = []
        a.record(stream)
        for x, q, s, y in sets:
            bufs.append(pkg.w4a16_grouped_pack(q, s))
        b.record(stream)
        torch.cuda.synchronize()
        repack_ms = a.elapsed_time(b) / len(sets)
        sets = [(x, pb, None, y) for (x, q, s, y), pb in zip(sets, bufs)]

    def step(i):
        x, q, s, y = sets[i % copies]
        if packed:
            pkg.w4a16_gemm_grouped_packed(x, Id, Od, q, wl.E, wl.N, y)
        else:
            pkg.w4a16_gemm_grouped(x, Id, Od, q, s, y)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ms_per_step, per_launch_ms, graphed = time_steps(step, steps, stream)
    gbs = B / (ms_per_step * 1e-3) / 1e9
    tfs = wl.flops() / (ms_per_step * 1e-3) / 1e12
    path = "grouped-packed" if packed else "grouped"
    roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic(name, path)}
    med = statistics.median(per_launch_ms)
    active = int(np.count_nonzero(np.diff(off)))
    extra = {"graph_replay": graphed, "rotation_copies": copies, "algorithmic_bytes": B,
             "flops": wl.flops(), "per_launch_event_us_median": med * 1e3,
             "hbm_GBs_at_event_median": B / (med * 1e-3) / 1e9, "path": path,
             "active_experts": active, "hbm_frac": gbs / HBM_PEAK_GBS,
             "fp32_frac": tfs / FP32_PEAK_TFLOPS}
    if repack_ms is not None:
        extra["repack_ms_one_time"] = repack_ms
    y0 = sets[0][3].cpu().numpy()
    return gbs, "GB/s", ms_per_step, roof, extra, (X, qw, sc, ti, off, y0)


def cpu_leg_moe(name: str, gpu_out, budget_s: float = 12.0):
    """The oracle on a bounded sample of the grouped GEMM: the slots of the first experts."""
    import oracle
    wl = workloads.MOE_WORKLOADS[name]
    X, qw, sc, ti, off, Y = gpu_out
    cores = len(os.sched_getaffinity(0))
    # sample: every slot of the first experts, up to 8 slots
    e_end = 1
    while e_end < wl.E and off[e_end + 1] <= 8:
        e_end += 1
    r_end = int(off[e_end])
    sub_off = off[:e_end + 1]
    times, Yref = [], None
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end or not times:
        t0 = time.perf_counter()
        Yref = oracle.grouped_gemm(X, ti[:r_end], sub_off, qw[:e_end], sc[:e_end])
        times.append(time.perf_counter() - t0)
        if len(times) >= 50:
            break
    t = statistics.median(times)
    active = int(np.count_nonzero(np.diff(sub_off)))
    sample_bytes = active * (wl.N * wl.K // 2 + 4 * wl.N * (wl.K // 32)) + 4 * r_end * (wl.K + wl.N)
    v = oracle.compare_grouped(Y[:r_end], X, ti[:r_end], sub_off, qw[:e_end], sc[:e_end])
    return {"value": sample_bytes / t / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"slots 0..{r_end - 1} (experts 0..{e_end - 1}, {active} active), "
                      f"median of {len(times)} runs, {t * 1e3:.1f} ms each",
            "gpu_parity_on_sample_max_err_over_bound": v["max_ratio"]}


def gpu_leg(name: str, steps: int, warmup: int, path: str = "auto"):
    import torch
    import int4_weight_only_03_amd as pkg

    wl = workloads.WORKLOADS[name]
    dev = torch.device("cuda:0")
    X, W = workloads.make(name)
    qw, sc = pkg.w4a16_quantize(W)            # the library's own host quantizer
    B = wl.algorithmic_bytes()
    if path == "swiglu":  # Y is [M][N/2]: the gate/up outputs never reach memory
        B -= 4 * wl.M * (wl.N // 2)
    copies = 1 if B * 2 > 4 * MALL_BYTES else max(1, -(-2 * MALL_BYTES // B))
    if name == "tiny":
        copies = 1                             # cache-resident by nature
    Xd = torch.from_numpy(X).to(dev)
    Qd = torch.from_numpy(qw).to(dev)
    Sd = torch.from_numpy(sc).to(dev)
    sets = [(Xd.clone(), Qd.clone(), Sd.clone(),
             torch.empty((wl.M, wl.N), dtype=torch.float32, device=dev)) for _ in range(copies)]
    del Xd, Qd, Sd
    stream = torch.cuda.current_stream(dev)
    code = PATH_NAMES[path]
    repack_ms = None
    if path in SPLIT_PATHS:
        # one caller-owned workspace, reused by every (stream-ordered) step
        ws = torch.empty(pkg.w4a16_split_workspace_bytes(wl.M, wl.N, wl.K), dtype=torch.uint8,
                         device=dev)
    if path == "split":
        def step(i):
            x, q, s, y = sets[i % copies]
            pkg.w4a16_gemm_split(x, q, s, y, workspace=ws)
    elif path == "packed":
        # the one-time repack (outside the timed region, timed on its own)
        packs = [pkg.w4a16_split_pack(q, s) for (_, q, s, _) in sets]
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        pkg.w4a16_split_pack(sets[0][1], sets[0][2], packs[0])
        ev1.record(stream)
        torch.cuda.synchronize()
        repack_ms = ev0.elapsed_time(ev1)

        def step(i):
            x, _, _, y = sets[i % copies]
            pkg.w4a16_gemm_split_packed(x, packs[i % copies], wl.N, y, workspace=ws)
    elif path == "repacked":
        # the one-time repack (w4a16_repack), timed on its own
        packs = [pkg.w4a16_repack(q, s) for (_, q, s, _) in sets]
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        pkg.w4a16_repack(sets[0][1], sets[0][2], packs[0])
        ev1.record(stream)
        torch.cuda.synchronize()
        repack_ms = ev0.elapsed_time(ev1)

        def step(i):
            x, _, _, y = sets[i % copies]
            pkg.w4a16_gemm_repacked(x, packs[i % copies], wl.N, y)
    elif path == "small-packed":
        # the one-time repack into the grouped layout (one expert), timed on its own
        packs = [pkg.w4a16_grouped_pack(q[None], s[None]) for (_, q, s, _) in sets]
        need = pkg.w4a16_small_packed_workspace_bytes(wl.M, wl.N, wl.K)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        pkg.w4a16_grouped_pack(sets[0][1][None], sets[0][2][None], packs[0])
        ev1.record(stream)
        torch.cuda.synchronize()
        repack_ms = ev0.elapsed_time(ev1)

        def step(i):
            x, _, _, y = sets[i % copies]
            pkg.w4a16_gemm_small_packed(x, packs[i % copies], wl.N, y, workspace=ws)
    elif path == "swiglu":
        ys = [torch.empty((wl.M, wl.N // 2), dtype=torch.float32, device=dev)
              for _ in range(copies)]

        def step(i):
            x, q, s, _ = sets[i % copies]
            pkg.w4a16_gemm_swiglu(x, q, s, ys[i % copies])
    else:
        def step(i):
            x, q, s, y = sets[i % copies]
            pkg.w4a16_gemm_path(x, q, s, y, path=code)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    ms_per_step, per_launch_ms, graphed = time_steps(step, steps, stream)

    gbs = B / (ms_per_step * 1e-3) / 1e9
    tfs = wl.flops() / (ms_per_step * 1e-3) / 1e12
    value, unit = (gbs, "GB/s") if metric_in_gbs(wl) else (tfs, "TFLOP/s")
    resolved = path if path != "auto" else \
        {1: "gemv", 2: "tile"}[pkg.w4a16_select_path(wl.M, wl.N, wl.K)]
    # the limb paths issue fp16 matrix instructions (so does the GEMV path's
    # matrix-core kernel): their compute roof is the fp16 peak
    split = path in LIMB_PATHS or (
        resolved in ("gemv", "swiglu")
        and pkg.w4a16_gemv_kernel(wl.M, wl.N, wl.K) == pkg.W4A16_GEMV_MFMA)
    peak_tf = FP16_PEAK_TFLOPS if split else FP32_PEAK_TFLOPS
    if wl.flops() / (peak_tf * 1e12) < B / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS}
    else:
        roof = {"bound": "mfma", "achieved": tfs, "peak": peak_tf, "unit": "TFLOP/s",
                "frac": tfs / peak_tf}
    roof["traffic"] = measured_traffic(name, resolved)
    med = statistics.median(per_launch_ms)
    extra = {
        "graph_replay": graphed,
        "rotation_copies": copies,
        "algorithmic_bytes": B,
        "flops": wl.flops(),
        "per_launch_event_us_median": med * 1e3,
        "per_launch_event_us_p10": float(np.percentile(per_launch_ms, 10)) * 1e3,
        "per_launch_event_us_p90": float(np.percentile(per_launch_ms, 90)) * 1e3,
        "hbm_GBs_at_event_median": B / (med * 1e-3) / 1e9,
        "tflops_at_event_median": wl.flops() / (med * 1e-3) / 1e12,
        "path": resolved,
        "hbm_frac": gbs / HBM_PEAK_GBS,
        "repack_ms_one_time": repack_ms,
        "fp32_frac": tfs / FP32_PEAK_TFLOPS,
        "limb_arithmetic": split,
    }
    y0 = (ys[0] if path == "swiglu" else sets[0][3]).cpu().numpy()
    return value, unit, ms_per_step, roof, extra, (X, W, y0)


def cpu_leg(name: str, gpu_out, budget_s: float = 12.0, path: str = "auto"):
    """The oracle, as it stands, timed on the host cores over a bounded sample."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                               # pragma: no cover
        threadpool_limits = None
    wl = workloads.WORKLOADS[name]
    X, W, Y = gpu_out
    cores = len(os.sched_getaffinity(0))
    qw, sc = oracle.quantize(W)
    # sample: all N outputs of up to 8 rows of X (the whole job when M <= 8)
    rows = min(wl.M, 8)
    Xs = np.ascontiguousarray(X[:rows])
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        times = []
        t_end = time.perf_counter() + budget_s
        Yref = None
        while time.perf_counter() < t_end or not times:
            t0 = time.perf_counter()
            if path == "swiglu":
                Yref = oracle.swiglu(Xs, qw, sc)      # dequant + fp64 product + epilogue
            else:
                Yref = oracle.gemm(Xs, qw, sc)        # dequant + fp64 product
            times.append(time.perf_counter() - t0)
            if len(times) >= 50:
                break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    t = statistics.median(times)
    # the sample's share of the workload's algorithmic bytes / flops
    sample_bytes = wl.N * wl.K // 2 + 4 * wl.N * (wl.K // 32) + 4 * rows * wl.K + 4 * rows * wl.N
    sample_flops = 2 * rows * wl.N * wl.K
    if metric_in_gbs(wl):
        value, unit = sample_bytes / t / 1e9, "GB/s"
    else:
        value, unit = sample_flops / t / 1e12, "TFLOP/s"
    if path == "swiglu":
        sample_bytes -= 4 * rows * (wl.N // 2)
        err = np.abs(Y[:rows].astype(np.float64) - Yref) / oracle.swiglu_bound(Xs, qw, sc)
    else:
        T = oracle.abs_gemm(Xs, qw, sc)
        err = np.abs(Y[:rows].astype(np.float64) - Yref) / oracle.bound(T)
    return {"value": value, "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of X against all {wl.N} weight rows "
                      f"(dequant + fp64 product), median of {len(times)} runs, "
                      f"{t * 1e3:.1f} ms each",
            "gpu_parity_on_sample_max_err_over_bound": float(err.max())}


def copy_probe(nbytes: int, reps: int = 20) -> None:
    """Plain device copy of a known size, for calibrating HBM byte counters."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_gate_up",
                    help="comma-separated names from %s, or 'all'" % ", ".join(
                        workloads.ORDER + list(workloads.MOE_WORKLOADS)))
    ap.add_argument("--path", default="auto",
                    help="kernel path(s), comma-separated: auto, gemv, tile, split, packed, "
                         "swiglu, repacked, small-packed; grouped-MoE workloads run the grouped kernel on the "
                         "public layout, or with 'packed' on the repacked weights")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(sharding is described in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    names = (workloads.ORDER + list(workloads.MOE_WORKLOADS) if args.workload == "all"
             else args.workload.split(","))
    paths = args.path.split(",")
    for p in paths:
        if p not in PATH_NAMES:
            ap.error(f"unknown path {p!r}")
    for name in names:
        if name in workloads.MOE_WORKLOADS:
            # "packed": the repacked grouped weights; any other path: the public layout
            if any(p != "packed" for p in paths):
                run_moe(name, args)
            if "packed" in paths:
                run_moe(name, args, packed=True)
    names = [n for n in names if n not in workloads.MOE_WORKLOADS]
    for name, path in [(n, p) for n in names for p in paths]:
        wl = workloads.WORKLOADS[name]
        steps = args.steps if wl.M < 1024 else max(5, min(args.steps, 20))
        print(f"# {name}: M={wl.M} K={wl.K} N={wl.N} steps={steps} path={path}",
              file=sys.stderr, flush=True)
        value, unit, ms, roof, extra, out = gpu_leg(name, steps, args.warmup, path)
        # arithmetic type: fp32 FMA/MFMA, or fp16 matrix products of two fp16
        # activation limbs and exact weight codes with fp32 accumulation
        dtype = "f16x2-limb/f32-acc" if extra["limb_arithmetic"] else "f32"
        line = {
            "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
            "config": {"workload": name, "M": wl.M, "K": wl.K, "N": wl.N, "group": 32,
                       "note": wl.note, "parallelism": "none (1 GPU)"},
            "roofline": roof,
        }
        line.update(extra)
        if not args.no_cpu:
            line["cpu_baseline"] = cpu_leg(name, out, path=path)
        print(json.dumps(line), flush=True)


def moe_dtype(wl) -> str:
    """Arithmetic of the grouped kernel the library picks for this workload."""
    from int4_weight_only_03_amd import binding
    k = binding.w4a16_grouped_kernel(wl.T, wl.R, wl.E, wl.N, wl.K)
    return "f16x2-limb/f32-acc" if k == binding.W4A16_GROUPED_MFMA else "f32"


def run_moe(name, args, packed=False):
    wl = workloads.MOE_WORKLOADS[name]
    print(f"# {name}: T={wl.T} E={wl.E} top-{wl.topk} K={wl.K} N={wl.N} steps={args.steps} "
          f"path={'grouped-packed' if packed else 'grouped'}", file=sys.stderr, flush=True)
    value, unit, ms, roof, extra, out = gpu_leg_moe(name, args.steps, args.warmup, packed)
    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": moe_dtype(wl), "data": "synthetic",
        "config": {"workload": name, "T": wl.T, "experts": wl.E, "topk": wl.topk, "K": wl.K,
                   "N": wl.N, "group": 32, "note": wl.note, "parallelism": "none (1 GPU)"},
        "roofline": roof,
    }
    line.update(extra)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_leg_moe(name, out)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
