#!/usr/bin/env python3
"""Benchmark of the W4A16 group-quantized GEMM on one MI355X.

    python bench.py [--steps K] [--warmup W] [--no-cpu]
    python bench.py --workload NAME[,NAME]|all [--path P[,P]] [--steps K] [--no-cpu]

Default (no --workload): ONE JSON line.  Its `value` is the decode gate+up
GEMV (M=1, K=7168, N=4096: effective HBM GB/s of w4a16_gemm), and its
`configs` object holds every workload the metric names, each timed the same
way through the entry point w4a16_gemm runs (auto path):

  tiny (1x256x512), decode_gate_up (1x7168x4096), decode_down (1x2048x7168),
  verify_tree (64x7168x4096), prefill (4096x7168x4096)

with ms per step, GB/s, TFLOP/s, the kernel path and arithmetic, the fraction
of the roof that binds it (HBM when the FLOPs are under the ridge of the
path's arithmetic, otherwise that arithmetic's matrix peak), the
streaming-read floor of the same bytes (a plain read of X, qweight and scales
over the same rotating buffers, `w4a16_read_floor`, best of six launch
shapes), the fp32-FMA GEMV beside the matrix-core GEMV for the M=1 decodes,
the fp32 tiled path beside the matrix-core tile for the prefill, and the other
entry points (repacked weights for the decodes; repacked, small-packed and
split on packed weights for the two larger shapes; their one-time repack is
timed apart).

With --workload, one JSON line per (workload, path) instead (for profiling):
paths auto, gemv, gemv-fma, tile, tile-mx, split, packed, swiglu, repacked,
small-packed, read-floor (the plain read of the same inputs, 256 threads x 4
loads); grouped-MoE workloads take the public layout, or `packed` for the
repacked grouped weights.

A step is one call of the entry point (validate, launch, unpack + dequant +
contraction + reduction + store) on one batch of synthetic input, with inputs
already resident in HBM.  Every timed step reads its own copy of {X, qweight,
scales} (no copy is read twice in the timed steps, and the copies together
hold at least 512 MB, twice the 256 MB Infinity Cache), and 1 GiB is streamed
through the caches right before the timed steps, so every timed step reads
cold HBM.  The K steps are captured once in a HIP graph and replayed between
HIP events on the stream the kernels run on; ms_per_step is the replay time /
K.  A bounded spin kernel runs just before the start event, so that the host's
submission of the replay is not counted as GPU time.  Eager per-launch event
times (median, p10, p90) are reported beside it.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import subprocess
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
ROTATION_MIN_BYTES = 2 * MALL_BYTES
ROTATION_MAX_BYTES = 16 << 30
FLUSH_BYTES = 1 << 30
SPIN_CYCLES = 1_000_000      # GPU clock cycles of the spin before the timed region
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = "int4_weight_only_03_amd/csrc/"
PATHS = ("auto", "gemv", "gemv-fma", "tile", "tile-mx", "split", "packed", "swiglu", "repacked",
         "small-packed", "read-floor")
# paths whose products are fp16 matrix instructions on two activation limbs
LIMB_PATHS = ("tile-mx", "split", "packed", "repacked", "small-packed")
# the sources whose kernels a path runs (the C-ABI layer dispatches every path)
PATH_SOURCES = {"gemv": ["gemv.hip", "gemv_mfma.hip", "skinny.hip", "gemv_common.h", "limbs.h"],
                "gemv-fma": ["gemv.hip", "gemv_common.h"], "tile": ["tile.hip"],
                "tile-mx": ["tile_mx.hip", "limbs.h"],
                "split": ["split.hip", "limbs.h"], "packed": ["split.hip", "limbs.h"],
                "swiglu": ["gemv.hip", "gemv_mfma.hip", "skinny.hip", "gemv_common.h", "limbs.h"],
                "grouped": ["grouped.hip", "gemv_common.h", "limbs.h"],
                "grouped-packed": ["grouped.hip", "gemv_common.h", "limbs.h"],
                "repacked": ["gemv_mfma.hip", "skinny.hip", "tile_mx.hip",
                             "small_packed.hip", "gemv_common.h", "limbs.h"],
                "small-packed": ["small_packed.hip", "gemv_common.h", "limbs.h"],
                "read-floor": ["read_floor.hip", "gemv_common.h"]}
# launch shapes of the streaming-read floor: (threads per block, 16-byte loads per thread)
FLOOR_SHAPES = [(256, 1), (256, 4), (1024, 4), (512, 8), (256, 16), (1024, 16)]


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


def metric_in_gbs(M: int) -> bool:
    """The metric is effective HBM GB/s for M <= 64 and TFLOP/s above."""
    return M <= 64


_FLUSH = None


def flush_caches():
    """Stream 1 GiB (read and write) through L2 and the Infinity Cache."""
    import torch
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
    _FLUSH.add_(1.0)


def time_steps(step, steps: int, stream):
    """(ms per step of a graph replay of `steps` steps, eager per-launch ms, graphed).

    Eager launches with events around each give per-launch times; then the
    steps are captured in a graph, replayed once to warm up, the caches are
    flushed, and the timed replay runs between two events on `stream`."""
    import torch
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

    flush_caches()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # a bounded spin kernel keeps the GPU busy while the host submits the
    # replay, so the host's submission latency falls before the start event
    # and the events bracket only the K steps' GPU work
    torch.cuda._sleep(SPIN_CYCLES)
    start.record(stream)
    if graphed:
        g.replay()
    else:
        for i in range(steps):
            step(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, per_launch_ms, graphed


def timing_fields(ms, per_launch_ms, graphed):
    return {"ms_per_step": ms, "us_per_step": ms * 1e3, "graph_replay": graphed,
            "per_launch_event_us_median": statistics.median(per_launch_ms) * 1e3,
            "per_launch_event_us_p10": float(np.percentile(per_launch_ms, 10)) * 1e3,
            "per_launch_event_us_p90": float(np.percentile(per_launch_ms, 90)) * 1e3}


class Problem:
    """One workload's inputs, quantized by the library's host quantizer, in
    rotating device copies (each timed step reads its own copy)."""

    def __init__(self, name: str, steps: int):
        import torch
        import int4_weight_only_03_amd as pkg
        self.pkg = pkg
        self.name = name
        self.wl = wl = workloads.WORKLOADS[name]
        self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream(self.dev)
        self.X, self.W = workloads.make(name)
        self.qw, self.sc = pkg.w4a16_quantize(self.W)
        self.B = wl.algorithmic_bytes()
        self.flops = wl.flops()
        if name == "tiny":
            copies = 1                                # cache-resident by nature
        else:
            copies = max(-(-ROTATION_MIN_BYTES // self.B), steps)
            copies = max(1, min(copies, ROTATION_MAX_BYTES // self.B))
        self.copies = copies
        Xd = torch.from_numpy(self.X).to(self.dev)
        Qd = torch.from_numpy(self.qw).to(self.dev)
        Sd = torch.from_numpy(self.sc).to(self.dev)
        self.sets = [(Xd.clone(), Qd.clone(), Sd.clone(),
                      torch.empty((wl.M, wl.N), dtype=torch.float32, device=self.dev))
                     for _ in range(copies)]
        del Xd, Qd, Sd
        torch.cuda.synchronize()

    def input_sha256(self):
        return {"X": workloads.sha256(self.X)[:16], "W": workloads.sha256(self.W)[:16]}

    def _repack(self, fn):
        """fn(q, s) -> packed for every copy; returns (packs, ms of one repack)."""
        import torch
        packs = [fn(q, s) for (_, q, s, _) in self.sets]
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        fn(self.sets[0][1], self.sets[0][2])
        b.record(self.stream)
        torch.cuda.synchronize()
        return packs, a.elapsed_time(b)

    def measure(self, path: str, steps: int, warmup: int) -> dict:
        """Time `steps` steps of one entry point; returns timing, rates and Y of copy 0."""
        import torch
        pkg, wl, sets, C = self.pkg, self.wl, self.sets, self.copies
        B = self.B
        repack_ms = None
        y_out = [s[3] for s in sets]
        if path in ("split", "packed"):
            ws = torch.empty(pkg.w4a16_split_workspace_bytes(wl.M, wl.N, wl.K),
                             dtype=torch.uint8, device=self.dev)
        if path == "split":
            def step(i):
                x, q, s, y = sets[i % C]
                pkg.w4a16_gemm_split(x, q, s, y, workspace=ws)
        elif path == "packed":
            packs, repack_ms = self._repack(lambda q, s: pkg.w4a16_split_pack(q, s))

            def step(i):
                x, _, _, y = sets[i % C]
                pkg.w4a16_gemm_split_packed(x, packs[i % C], wl.N, y, workspace=ws)
        elif path == "repacked":
            packs, repack_ms = self._repack(lambda q, s: pkg.w4a16_repack(q, s))

            def step(i):
                x, _, _, y = sets[i % C]
                pkg.w4a16_gemm_repacked(x, packs[i % C], wl.N, y)
        elif path == "small-packed":
            packs, repack_ms = self._repack(lambda q, s: pkg.w4a16_grouped_pack(q[None], s[None]))
            need = pkg.w4a16_small_packed_workspace_bytes(wl.M, wl.N, wl.K)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=self.dev)

            def step(i):
                x, _, _, y = sets[i % C]
                pkg.w4a16_gemm_small_packed(x, packs[i % C], wl.N, y, workspace=ws)
        elif path == "read-floor":
            # the streaming read of the same X, qweight and scales (256 threads x 4 loads)
            sink = torch.zeros(4, dtype=torch.int32, device=self.dev)
            B -= 4 * wl.M * wl.N

            def step(i):
                x, q, s, _ = sets[i % C]
                pkg.w4a16_read_floor([x, q, s], sink, 256, 4)
        elif path == "swiglu":
            B -= 4 * wl.M * (wl.N // 2)   # Y is [M][N/2]: the gate/up outputs never reach memory
            y_out = [torch.empty((wl.M, wl.N // 2), dtype=torch.float32, device=self.dev)
                     for _ in range(C)]

            def step(i):
                x, q, s, _ = sets[i % C]
                pkg.w4a16_gemm_swiglu(x, q, s, y_out[i % C])
        else:
            code = {"auto": pkg.W4A16_PATH_AUTO, "gemv": pkg.W4A16_PATH_GEMV,
                    "gemv-fma": pkg.W4A16_PATH_GEMV_FMA, "tile": pkg.W4A16_PATH_TILE,
                    "tile-mx": pkg.W4A16_PATH_TILE_MX}[path]

            def step(i):
                x, q, s, y = sets[i % C]
                pkg.w4a16_gemm_path(x, q, s, y, path=code)

        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        ms, per_launch_ms, graphed = time_steps(step, steps, self.stream)
        resolved = self.resolve(path)
        limb = self.limb(resolved)
        gbs = B / (ms * 1e-3) / 1e9
        tfs = self.flops / (ms * 1e-3) / 1e12
        peak_tf = FP16_PEAK_TFLOPS if limb else FP32_PEAK_TFLOPS
        if self.flops / (peak_tf * 1e12) < B / (HBM_PEAK_GBS * 1e9):
            roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": gbs / HBM_PEAK_GBS}
        else:
            roof = {"bound": "mfma", "achieved": tfs, "peak": peak_tf, "unit": "TFLOP/s",
                    "frac": tfs / peak_tf}
        roof["traffic"] = measured_traffic(self.name, resolved)
        out = {"path": resolved, "dtype": "f16x2-limb/f32-acc" if limb else "f32",
               "algorithmic_bytes": B, "flops": self.flops, "GB_s": gbs, "TFLOP_s": tfs,
               "hbm_frac": gbs / HBM_PEAK_GBS, "fp32_frac": tfs / FP32_PEAK_TFLOPS,
               "roofline": roof, "repack_ms_one_time": repack_ms,
               "rotation_copies": self.copies,
               "timed_set_bytes": min(steps, self.copies) * B}
        out.update(timing_fields(ms, per_launch_ms, graphed))
        torch.cuda.synchronize()
        out["_y0"] = y_out[0].cpu().numpy()
        return out

    def resolve(self, path: str) -> str:
        if path != "auto":
            return path
        code = self.pkg.w4a16_select_path(self.wl.M, self.wl.N, self.wl.K)
        return {self.pkg.W4A16_PATH_GEMV: "gemv", self.pkg.W4A16_PATH_TILE_MX: "tile-mx"}.get(code, "tile")

    def limb(self, resolved: str) -> bool:
        """Whether the path's products are fp16 matrix instructions on activation limbs."""
        wl = self.wl
        return resolved in LIMB_PATHS or (
            resolved in ("gemv", "swiglu")
            and self.pkg.w4a16_gemv_kernel(wl.M, wl.N, wl.K) in (self.pkg.W4A16_GEMV_MFMA,
                                                                 self.pkg.W4A16_GEMV_SKINNY))

    def read_floor(self, steps: int, warmup: int) -> dict:
        """Best plain streaming read of the same X, qweight and scales buffers."""
        import torch
        sink = torch.zeros(4, dtype=torch.int32, device=self.dev)
        Bread = sum(t.numel() * t.element_size() for t in self.sets[0][:3])
        best, shapes = None, {}
        for threads, loads in FLOOR_SHAPES:
            def step(i, threads=threads, loads=loads):
                x, q, s, _ = self.sets[i % self.copies]
                self.pkg.w4a16_read_floor([x, q, s], sink, threads, loads)
            for i in range(warmup):
                step(i)
            ms, _, _ = time_steps(step, steps, self.stream)
            shapes[f"{threads}x{loads}"] = ms * 1e3
            if best is None or ms < best[0]:
                best = (ms, threads, loads)
        ms, threads, loads = best
        return {"read_floor_us": ms * 1e3, "read_floor_bytes": Bread,
                "read_floor_GB_s": Bread / (ms * 1e-3) / 1e9,
                "read_floor_hbm_frac": Bread / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "read_floor_shape": f"{threads} threads x {loads} loads",
                "read_floor_us_by_shape": shapes}


def steps_for(M: int, steps: int) -> int:
    return steps if M < 1024 else max(5, min(steps, 20))


def cpu_facts() -> dict:
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{b.get('name')} {b.get('version')}"
    except Exception:                                 # pragma: no cover
        pass
    return {"cpu_model": model, "blas": blas}


def cpu_leg(outputs: dict, budget_s: float = 12.0) -> dict:
    """The oracle, as it stands, timed on the host cores: a bounded sample of
    the headline workload (value), one full run of the prefill oracle, and the
    GPU parity of copy 0 of every timed workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                               # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        # the headline sample: decode_gate_up, its one row against all weight rows
        wl = workloads.WORKLOADS["decode_gate_up"]
        X, W = workloads.make("decode_gate_up")
        qw, sc = oracle.quantize(W)
        times = []
        t_end = time.perf_counter() + budget_s
        while time.perf_counter() < t_end or not times:
            t0 = time.perf_counter()
            oracle.gemm(X, qw, sc)                    # dequant + fp64 product
            times.append(time.perf_counter() - t0)
            if len(times) >= 50:
                break
        t = statistics.median(times)
        value = wl.algorithmic_bytes() / t / 1e9
        res = {"value": value, "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"decode_gate_up whole (1 row of X against all {wl.N} weight rows: "
                         f"dequant + fp64 product), median of {len(times)} runs, "
                         f"{t * 1e3:.1f} ms each"}
        res.update(cpu_facts())
        # parity of every timed workload (one copy each), and one prefill oracle run
        parity = {}
        for name, y in outputs.items():
            Xn, Wn = workloads.make(name)
            qn, sn = oracle.quantize(Wn)
            t0 = time.perf_counter()
            Yref = oracle.gemm(Xn, qn, sn)
            dt = time.perf_counter() - t0
            T = oracle.abs_gemm(Xn, qn, sn)
            parity[name] = oracle.compare_to(y, Yref, T)["max_ratio"]
            if name == "prefill":
                wlp = workloads.WORKLOADS["prefill"]
                res["prefill_oracle_s_one_rep"] = dt
                res["prefill_oracle_TFLOP_s"] = wlp.flops() / dt / 1e12
        res["gpu_parity_max_err_over_bound"] = parity
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    return res


def gpu_clocks():
    """Current shader and memory clocks (rocm-smi), if it is there."""
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        d = json.loads(r.stdout)
        card = next(iter(d.values()))
        return {k: v for k, v in card.items() if "sclk" in k or "mclk" in k or "fclk" in k}
    except Exception:
        return None


def headline(args) -> None:
    """Every configuration of the metric in one line; value = decode_gate_up."""
    import torch
    configs, outputs = {}, {}
    for name in workloads.ORDER:
        wl = workloads.WORKLOADS[name]
        steps = steps_for(wl.M, args.steps)
        print(f"# {name}: M={wl.M} K={wl.K} N={wl.N} steps={steps}", file=sys.stderr, flush=True)
        prob = Problem(name, steps)
        r = prob.measure("auto", steps, args.warmup)
        outputs[name] = r.pop("_y0")
        r.update(prob.read_floor(steps, args.warmup))
        r["us_over_read_floor"] = r["us_per_step"] / r["read_floor_us"]
        r["config"] = {"M": wl.M, "K": wl.K, "N": wl.N, "note": wl.note}
        r["input_sha256"] = prob.input_sha256()
        r["steps"] = steps
        if name in ("decode_gate_up", "decode_down"):
            f = prob.measure("gemv-fma", steps, args.warmup)
            f.pop("_y0")
            r["fp32_fma_gemv"] = {k: f[k] for k in ("us_per_step", "GB_s", "hbm_frac", "dtype",
                                                   "per_launch_event_us_median")}
        others = {"decode_gate_up": ("repacked",), "decode_down": ("repacked",),
                  "verify_tree": ("small-packed", "repacked", "packed"),
                  "prefill": ("tile", "packed", "repacked")}.get(name, ())
        if others:
            alts = {}
            for p in others:
                a = prob.measure(p, steps, args.warmup)
                a.pop("_y0")
                alts[p] = {k: a[k] for k in ("us_per_step", "GB_s", "TFLOP_s", "hbm_frac",
                                             "fp32_frac", "dtype", "repack_ms_one_time")}
                alts[p]["frac_of_fp16_peak"] = a["TFLOP_s"] / FP16_PEAK_TFLOPS
            r["other_entry_points"] = alts
        configs[name] = r
        del prob
        torch.cuda.empty_cache()

    head = configs["decode_gate_up"]
    line = {
        "metric": METRIC, "value": head["GB_s"], "unit": "GB/s", "n_gpus": 1,
        "steps": head["steps"], "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head["dtype"], "data": "synthetic",
        "config": {"workload": "decode_gate_up", "M": 1, "K": 7168, "N": 4096, "group": 32,
                   "note": workloads.WORKLOADS["decode_gate_up"].note,
                   "parallelism": "none (1 GPU)"},
        "roofline": head["roofline"],
        "path": head["path"],
        "read_floor_us": head["read_floor_us"],
        "configs": configs,
        "gpu_clocks": gpu_clocks(),
        "rotation": "each timed step reads its own copy of X, qweight and scales; 1 GiB "
                    "streamed through the caches before the timed steps",
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_leg(outputs)
    print(json.dumps(line), flush=True)


def per_path(args) -> None:
    names = (workloads.ORDER + list(workloads.MOE_WORKLOADS) if args.workload == "all"
             else args.workload.split(","))
    paths = args.path.split(",")
    for p in paths:
        if p not in PATHS:
            raise SystemExit(f"unknown path {p!r}")
    for name in names:
        if name in workloads.MOE_WORKLOADS:
            if any(p != "packed" for p in paths):
                run_moe(name, args)
            if "packed" in paths:
                run_moe(name, args, packed=True)
            continue
        wl = workloads.WORKLOADS[name]
        steps = steps_for(wl.M, args.steps)
        prob = Problem(name, steps)
        for path in paths:
            print(f"# {name}: M={wl.M} K={wl.K} N={wl.N} steps={steps} path={path}",
                  file=sys.stderr, flush=True)
            r = prob.measure(path, steps, args.warmup)
            y0 = r.pop("_y0")
            metric_gbs = metric_in_gbs(wl.M)
            line = {
                "metric": METRIC, "value": r["GB_s"] if metric_gbs else r["TFLOP_s"],
                "unit": "GB/s" if metric_gbs else "TFLOP/s", "n_gpus": 1, "steps": steps,
                "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                "dtype": r["dtype"], "data": "synthetic",
                "config": {"workload": name, "M": wl.M, "K": wl.K, "N": wl.N, "group": 32,
                           "note": wl.note, "parallelism": "none (1 GPU)"},
                "roofline": r.pop("roofline"),
            }
            line.update(r)
            if not args.no_cpu:
                line["cpu_baseline"] = cpu_leg_sample(name, y0, path)
            print(json.dumps(line), flush=True)
        del prob


def cpu_leg_sample(name: str, Y, path: str, budget_s: float = 12.0) -> dict:
    """The oracle on up to 8 rows of one workload (per-path lines)."""
    import oracle
    wl = workloads.WORKLOADS[name]
    X, W = workloads.make(name)
    qw, sc = oracle.quantize(W)
    rows = min(wl.M, 8)
    Xs = np.ascontiguousarray(X[:rows])
    times = []
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end or not times:
        t0 = time.perf_counter()
        Yref = oracle.swiglu(Xs, qw, sc) if path == "swiglu" else oracle.gemm(Xs, qw, sc)
        times.append(time.perf_counter() - t0)
        if len(times) >= 50:
            break
    t = statistics.median(times)
    sample_bytes = wl.N * wl.K // 2 + 4 * wl.N * (wl.K // 32) + 4 * rows * (wl.K + wl.N)
    if path == "swiglu":
        err = np.abs(Y[:rows].astype(np.float64) - Yref) / oracle.swiglu_bound(Xs, qw, sc)
    else:
        err = np.abs(Y[:rows].astype(np.float64) - Yref) / oracle.bound(
            oracle.abs_gemm(Xs, qw, sc))
    return {"value": sample_bytes / t / 1e9, "unit": "GB/s",
            "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of X against all {wl.N} weight rows, median of "
                      f"{len(times)} runs, {t * 1e3:.1f} ms each",
            "gpu_parity_on_sample_max_err_over_bound": float(err.max())}


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
    copies = max(-(-ROTATION_MIN_BYTES // B), steps)
    copies = max(1, min(copies, ROTATION_MAX_BYTES // B))
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
    ms, per_launch_ms, graphed = time_steps(step, steps, stream)
    gbs = B / (ms * 1e-3) / 1e9
    tfs = wl.flops() / (ms * 1e-3) / 1e12
    path = "grouped-packed" if packed else "grouped"
    roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic(name, path)}
    active = int(np.count_nonzero(np.diff(off)))
    extra = {"rotation_copies": copies, "algorithmic_bytes": B, "flops": wl.flops(),
             "path": path, "active_experts": active, "hbm_frac": gbs / HBM_PEAK_GBS,
             "fp32_frac": tfs / FP32_PEAK_TFLOPS}
    extra.update(timing_fields(ms, per_launch_ms, graphed))
    if repack_ms is not None:
        extra["repack_ms_one_time"] = repack_ms
    y0 = sets[0][3].cpu().numpy()
    return gbs, ms, roof, extra, (X, qw, sc, ti, off, y0)


def cpu_leg_moe(name: str, gpu_out, budget_s: float = 12.0):
    """The oracle on a bounded sample of the grouped GEMM: the slots of the first experts."""
    import oracle
    wl = workloads.MOE_WORKLOADS[name]
    X, qw, sc, ti, off, Y = gpu_out
    cores = len(os.sched_getaffinity(0))
    e_end = 1
    while e_end < wl.E and off[e_end + 1] <= 8:
        e_end += 1
    r_end = int(off[e_end])
    sub_off = off[:e_end + 1]
    times = []
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end or not times:
        t0 = time.perf_counter()
        oracle.grouped_gemm(X, ti[:r_end], sub_off, qw[:e_end], sc[:e_end])
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


def moe_dtype(wl) -> str:
    """Arithmetic of the grouped kernel the library picks for this workload."""
    from int4_weight_only_03_amd import binding
    k = binding.w4a16_grouped_kernel(wl.T, wl.R, wl.E, wl.N, wl.K)
    return "f16x2-limb/f32-acc" if k == binding.W4A16_GROUPED_MFMA else "f32"


def run_moe(name, args, packed=False):
    wl = workloads.MOE_WORKLOADS[name]
    print(f"# {name}: T={wl.T} E={wl.E} top-{wl.topk} K={wl.K} N={wl.N} steps={args.steps} "
          f"path={'grouped-packed' if packed else 'grouped'}", file=sys.stderr, flush=True)
    value, ms, roof, extra, out = gpu_leg_moe(name, args.steps, args.warmup, packed)
    line = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
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
    ap.add_argument("--workload", default=None,
                    help="comma-separated names from %s, or 'all' (one line per workload "
                         "and path instead of the headline line)" % ", ".join(
                             workloads.ORDER + list(workloads.MOE_WORKLOADS)))
    ap.add_argument("--path", default="auto", help="with --workload: " + ", ".join(PATHS))
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
    if args.workload is None:
        headline(args)
    else:
        per_path(args)


if __name__ == "__main__":
    main()
