#!/usr/bin/env python3
"""Throughput of the IndexGrid hot path on one MI355X.

One step = the whole path over one synthetic scene already resident in HBM: build the
IndexGrid from the shuffled coordinates (tile hash, radix sort, node registration), the
27-offset kernel map, and the 3x3x3 submanifold convolution on the automatically chosen
path. Prints one JSON line.

    python bench.py [--workload large] [--steps K] [--warmup W] [--gpus 1] [--backward | --strided S | --chain S,..]

The default workload is the largest one (50M signed coordinates -> 48.2M voxels, bf16 128 -> 256):
the headline line. The others (tiny, leaf, band, lidar, band32) are selected with --workload.

value = effective conv FLOPs (2 * pairs * cin * cout, empty MACs excluded, as the fVDB notes
define effective TFLOPS in their micro-benchmarks) per second of the whole step. The line also
carries per-phase times, the build rate in Mvox/s, the roofline of the dominant kernel (the
convolution) timed with HIP events on its launch stream, and the CPU oracle timed on the host
cores as a reference point.

With --backward a step also runs the two gradients of the convolution (input gradient, then
weight gradient, as two calls of igc_sparse_conv_backward) for a synthetic output gradient;
value is then 3 * 2 * pairs * cin * cout per second of the whole step, and the line carries
both gradients' phase times and rooflines. With --strided S a step is one strided layer on
the gather-GEMM-scatter path (bf16 workloads): build the input grid, its stride-S output grid
(igc_conv_grid), the map between them (igc_conv_map) and the convolution (igc_sparse_conv_between);
value is 2 * pairs * cin * cout of that convolution per second of the step. With --chain
S1,S2,... a step builds a chain of strided output grids with the counts kept on the device
(igc_conv_grid_chain, one synchronisation) and, for comparison, the same grids one call at a
time; value is the chain's wall-clock milliseconds. With --layer DTYPE:CIN:COUT the step runs the
workload's scene with that layer shape instead (for example --layer bf16:4:32, which no tuned
path takes and runs on the general-shape path, whose roof is the fp32 vector peak). The default
line is unchanged.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-conv effective TFLOP/s (2·pairs·Cin·Cout/s) + IndexGrid build Mvox/s"
HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}  # dense MFMA peaks of MI355X
CONV_SRC = {"leaf": "sparse_convolution_amd/csrc/igc_conv_leaf.hip",
            "ggs": "sparse_convolution_amd/csrc/igc_conv_ggs.hip"}
CONV_KERNEL = {("leaf", "f32"): "k_conv_leaf_f32", ("leaf", "bf16"): "k_conv_leaf_bf16",
               ("ggs", "bf16"): "k_conv_ggs_bf16", ("gather", "f32"): "k_conv_gather", ("gather", "bf16"): "k_conv_gather"}
DEFAULT_STEPS = {"tiny": (50, 5), "leaf": (20, 3), "band": (10, 2), "lidar": (20, 3), "large": (10, 2),
                 "band32": (10, 2)}


def _sha(path: str) -> str:
    with open(os.path.join(ROOT, path), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def _traffic(path_name: str, dtype: str, workload: str):
    """Measured HBM bytes per launch of the conv kernel, if the committed counter summary was
    taken on the current kernel source; None otherwise."""
    f = os.path.join(ROOT, "profiles", f"traffic_{CONV_KERNEL[(path_name, dtype)]}_{workload}.json")
    if not os.path.exists(f):
        return None
    with open(f) as fh:
        d = json.load(fh)
    if d.get("source_sha") != _sha(CONV_SRC[path_name]):
        return None
    return d.get("bytes_per_launch")


def _progress(msg: str) -> None:
    """Progress on stderr (stdout carries only the JSON line)."""
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _pct(a, q):
    return float(np.percentile(np.asarray(a), q)) if len(a) else None


def copy_calibration(gib: float = 2.0, reps: int = 5) -> None:
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": 4 * n, "reps": reps}))


def cpu_baseline(coords, wl, cin, cout, dtype_name, min_seconds=10.0):
    """The CPU oracle (as written, untuned) on a bounded sample of the same workload."""
    import oracle
    import workloads
    max_coords = 4_000_000
    sample = coords[:max_coords]
    t0 = time.perf_counter()
    g = oracle.OracleGrid(sample)
    t_build = time.perf_counter() - t0
    t0 = time.perf_counter()
    m = g.kernel_map()
    t_kmap = time.perf_counter() - t0
    pairs = int((m >= 0).sum())
    mean_pairs = pairs / max(g.n, 1)
    rows_max = max(1024, int(2e10 / max(mean_pairs * cin * cout, 1)))
    f = workloads.make_features(g.n, cin, 3000 + wl.index)
    w = workloads.make_weights(cin, cout, 4000 + wl.index, wl.weight_std)
    if dtype_name == "bf16":
        import torch
        f = torch.from_numpy(f).bfloat16().float().numpy()
        w = torch.from_numpy(w).bfloat16().float().numpy()
    rows = None
    if g.n > rows_max:
        rows = np.sort(np.random.default_rng(7).choice(g.n, rows_max, replace=False))
    t0 = time.perf_counter()
    oracle.conv(m, f, w, rows=rows)
    t_conv = time.perf_counter() - t0
    n_rows = g.n if rows is None else rows.shape[0]
    t_conv_all = t_conv * g.n / n_rows
    total = t_build + t_kmap + t_conv_all
    flops = 2.0 * pairs * cin * cout
    desc = (f"oracle build + kernel map on the first {sample.shape[0]} of {coords.shape[0]} input coordinates "
            f"({g.n} voxels), conv on {n_rows} of those rows")
    if rows is not None:
        desc += " (conv time scaled to all rows)"
    desc += f"; build {t_build:.2f} s, kernel map {t_kmap:.2f} s, conv {t_conv_all:.2f} s"
    return {"value": flops / total / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": desc, "build_mvox_s": sample.shape[0] / t_build / 1e6, "cpu_model": _cpu_model()}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="large", choices=["tiny", "leaf", "band", "lidar", "large", "band32"])
    ap.add_argument("--path", default="auto", choices=["auto", "leaf", "ggs", "gather"])
    ap.add_argument("--layer", default="", help="DTYPE:CIN:COUT (f32 or bf16) in place of the workload's layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--backward", action="store_true", help="add the input and weight gradients to the step")
    ap.add_argument("--strided", type=int, default=0, help="time one strided layer with this stride instead")
    ap.add_argument("--chain", default="", help="time a chain of strided output grids, e.g. 2,2,2,2, instead")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU sharding of this "
              "path is a design note, not an implemented mode.", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration()
        return 0

    import torch
    import sparse_convolution_amd as igc
    import workloads

    if args.strided:
        return strided_main(args, torch, igc, workloads)
    if args.chain:
        return chain_main(args, torch, igc, workloads)

    wl = workloads.WORKLOADS[args.workload]
    if args.layer:
        dt, ci, co = args.layer.split(":")
        if dt not in ("f32", "bf16"):
            raise SystemExit("--layer: dtype must be f32 or bf16")
        wl = dataclasses.replace(wl, dtype=dt, cin=int(ci), cout=int(co), weight_std=1.0 / np.sqrt(27 * int(ci)))
    steps, warmup = DEFAULT_STEPS[args.workload]
    steps = args.steps if args.steps is not None else steps
    warmup = args.warmup if args.warmup is not None else warmup
    tdtype = torch.float32 if wl.dtype == "f32" else torch.bfloat16

    _progress(f"workload {args.workload}: coordinates")
    coords = workloads.make_coords(args.workload)
    dev = torch.device("cuda", 0)
    coords_d = torch.from_numpy(coords).to(dev)
    g0 = igc.grid_build(coords_d)
    N = g0.n_voxels
    feats = torch.from_numpy(workloads.make_features(N, wl.cin, 3000 + wl.index)).to(dev, tdtype)
    weights = torch.from_numpy(workloads.make_weights(wl.cin, wl.cout, 4000 + wl.index, wl.weight_std)).to(dev, tdtype)
    m0 = igc.kernel_map(g0)
    pairs = int((m0 >= 0).sum().item())
    path = g0.select_path(tdtype, wl.cin, wl.cout) if args.path == "auto" else args.path
    info = dict(n_input=g0.n_input, n_voxels=N, n_leaf=g0.n_leaf, n_lower=g0.n_lower, n_upper=g0.n_upper,
                sort_passes=g0.sort_passes, leaf_occupancy=round(g0.leaf_occupancy, 4))
    out = torch.empty((N, wl.cout), dtype=tdtype, device=dev)
    dout = (torch.from_numpy(workloads.make_features(N, wl.cout, 7000 + wl.index)).to(dev, tdtype)
            if args.backward else None)
    del m0, g0
    n_ev = 6 if args.backward else 4

    stream = torch.cuda.current_stream(dev)

    def step(ev):
        ev[0].record(stream)
        g = igc.grid_build(coords_d)
        ev[1].record(stream)
        m = igc.kernel_map(g)
        ev[2].record(stream)
        igc.sparse_conv(g, feats, weights, kmap=m, path=path, out=out)
        ev[3].record(stream)
        if args.backward:
            dx, _ = igc.sparse_conv_backward(g, feats, weights, dout, m, path=path, need_dweights=False)
            ev[4].record(stream)
            _, dw = igc.sparse_conv_backward(g, feats, weights, dout, m, path=path, need_dfeats=False)
            ev[5].record(stream)
            return g, m, dx, dw
        return g, m

    _progress(f"{warmup} warm-up steps, then {steps} timed steps")
    for _ in range(warmup):
        step([torch.cuda.Event(enable_timing=True) for _ in range(n_ev)])
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    keep = None
    syncs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        keep = step(events[s])
        syncs.append(keep[0].host_syncs)  # host-side field of the grid built in this step
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del keep

    t_build = [e[0].elapsed_time(e[1]) for e in events]
    t_kmap = [e[1].elapsed_time(e[2]) for e in events]
    t_conv = [e[2].elapsed_time(e[3]) for e in events]
    ms_step = wall * 1e3 / steps
    flops = 2.0 * pairs * wl.cin * wl.cout
    value = (3.0 if args.backward else 1.0) * flops / (ms_step * 1e-3) / 1e12

    conv_ms = float(np.mean(t_conv))
    conv_tflops = flops / (conv_ms * 1e-3) / 1e12
    # The general-shape path runs fp32 FMAs on the vector ALUs: its roof is the fp32 vector peak.
    peak = PEAK_TFLOPS["f32"] if path == "gather" else PEAK_TFLOPS[wl.dtype]
    roofline = {"bound": "alu" if path == "gather" else "mfma", "achieved": round(conv_tflops, 3), "peak": peak,
                "unit": "TFLOP/s",
                "frac": round(conv_tflops / peak, 4), "traffic": _traffic(path, wl.dtype, args.workload),
                "kernel": CONV_KERNEL[(path, wl.dtype)], "flops_per_launch": flops,
                "avg_launch_ms": round(conv_ms, 4)}

    # Phase-level HBM view (algorithmic bytes; see the design notes for the per-unit figures).
    esize = 4 if wl.dtype == "f32" else 2
    kmap_bytes = 108.0 * N
    p = info["sort_passes"]
    build_bytes = (48.0 + 16.0 * p) * info["n_input"]
    conv_bytes = N * (wl.cin + wl.cout) * esize + 27 * wl.cin * wl.cout * esize + (108.0 * N if path == "ggs" else 0)
    phases = {
        "build_ms": {"mean": round(float(np.mean(t_build)), 4), "p50": _pct(t_build, 50), "p95": _pct(t_build, 95),
                     "p99": _pct(t_build, 99)},
        "kernel_map_ms": {"mean": round(float(np.mean(t_kmap)), 4), "p50": _pct(t_kmap, 50),
                          "p95": _pct(t_kmap, 95), "p99": _pct(t_kmap, 99)},
        "conv_ms": {"mean": round(conv_ms, 4), "p50": _pct(t_conv, 50), "p95": _pct(t_conv, 95),
                    "p99": _pct(t_conv, 99)},
        "build_hbm_frac": round(build_bytes / (np.mean(t_build) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_map_gbs": round(kmap_bytes / (np.mean(t_kmap) * 1e-3) / 1e9, 1),
        "kernel_map_hbm_frac": round(kmap_bytes / (np.mean(t_kmap) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "conv_hbm_frac": round(conv_bytes / (conv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "host_syncs_per_step": max(syncs),
    }

    if args.backward:
        t_dgrad = [e[3].elapsed_time(e[4]) for e in events]
        t_wgrad = [e[4].elapsed_time(e[5]) for e in events]
        for name, t in (("dgrad_ms", t_dgrad), ("wgrad_ms", t_wgrad)):
            phases[name] = {"mean": round(float(np.mean(t)), 4), "p50": _pct(t, 50), "p95": _pct(t, 95),
                            "p99": _pct(t, 99)}
        backward = {}
        for name, t in (("dgrad", t_dgrad), ("wgrad", t_wgrad)):
            tf = flops / (float(np.mean(t)) * 1e-3) / 1e12
            # The weight gradient's operands are the layer's dtype; its fp32 form runs on fp32 MFMA.
            backward[name] = {"tflops": round(tf, 3), "peak": peak, "frac": round(tf / peak, 4),
                              "avg_call_ms": round(float(np.mean(t)), 4)}
        bf16_mfma = wl.dtype == "bf16" and wl.cin % 32 == 0 and wl.cout % 64 == 0
        f32_leaf = wl.dtype == "f32" and (wl.cin, wl.cout) in {(4, 4), (4, 8), (4, 16), (4, 32), (8, 4), (8, 8), (8, 16),
                                                               (8, 32), (16, 4), (16, 8), (16, 16)}
        backward["wgrad"]["kernel"] = ("k_wgrad_bf16" if bf16_mfma else "k_wgrad_leaf_f32" if f32_leaf
                                       else "k_wgrad_gather")

    line = {
        "metric": (METRIC if not args.backward else
                   "sparse-conv training-step effective TFLOP/s (3·2·pairs·Cin·Cout/s: forward, input and weight "
                   "gradients) incl. IndexGrid build and kernel map"),
        "value": round(value, 4), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": args.workload + (f" layer {args.layer}" if args.layer else ""),
                   "description": wl.description, "cin": wl.cin, "cout": wl.cout,
                   "path": path, "pairs": pairs, "pairs_per_voxel": round(pairs / N, 3), **info},
        "build_mvox_s": round(info["n_input"] / (np.mean(t_build) * 1e-3) / 1e6, 1),
        "conv_tflops": round(conv_tflops, 3),
        "phases": phases,
        "roofline": roofline,
    }
    if args.backward:
        line["backward"] = backward
    if not args.no_cpu_baseline:
        _progress("cpu baseline (the oracle on a bounded sample)")
        line["cpu_baseline"] = cpu_baseline(coords, wl, wl.cin, wl.cout, wl.dtype)
    print(json.dumps(line), flush=True)
    return 0


def strided_main(args, torch, igc, workloads) -> int:
    wl = workloads.WORKLOADS[args.workload]
    if wl.dtype != "bf16":
        print("--strided runs on the gather-GEMM-scatter path: pick a bf16 workload (band, lidar, large)",
              file=sys.stderr)
        return 2
    steps, warmup = DEFAULT_STEPS[args.workload]
    steps = args.steps if args.steps is not None else steps
    warmup = args.warmup if args.warmup is not None else warmup
    S = args.strided
    dev = torch.device("cuda", 0)
    coords_d = torch.from_numpy(workloads.make_coords(args.workload)).to(dev)
    g0 = igc.grid_build(coords_d)
    go0 = igc.conv_grid(g0, S)
    m0 = igc.conv_map(g0, go0, S)
    pairs = int((m0 >= 0).sum().item())
    n_in, n_out = g0.n_voxels, go0.n_voxels
    feats = workloads.make_features_device(n_in, wl.cin, 3000 + wl.index, dev, torch.bfloat16)
    weights = torch.from_numpy(workloads.make_weights(wl.cin, wl.cout, 4000 + wl.index, wl.weight_std)).to(
        dev, torch.bfloat16)
    out = torch.empty((n_out, wl.cout), dtype=torch.bfloat16, device=dev)
    del m0, go0, g0
    stream = torch.cuda.current_stream(dev)

    def step(ev):
        ev[0].record(stream)
        g = igc.grid_build(coords_d)
        ev[1].record(stream)
        go = igc.conv_grid(g, S)
        ev[2].record(stream)
        m = igc.conv_map(g, go, S)
        ev[3].record(stream)
        igc.sparse_conv_between(go, feats, weights, m, out=out)
        ev[4].record(stream)
        return g, go, m

    for _ in range(warmup):
        step([torch.cuda.Event(enable_timing=True) for _ in range(5)])
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    t0 = time.perf_counter()
    for st in range(steps):
        keep = step(events[st])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del keep
    ms_step = wall * 1e3 / steps
    flops = 2.0 * pairs * wl.cin * wl.cout
    names = ["build_ms", "conv_grid_ms", "conv_map_ms", "conv_ms"]
    phases = {}
    for i, name in enumerate(names):
        t = [e[i].elapsed_time(e[i + 1]) for e in events]
        phases[name] = {"mean": round(float(np.mean(t)), 4), "p50": _pct(t, 50), "p95": _pct(t, 95), "p99": _pct(t, 99)}
    conv_ms = phases["conv_ms"]["mean"]
    conv_tflops = flops / (conv_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS["bf16"]
    line = {
        "metric": f"strided (stride {S}) sparse-conv layer effective TFLOP/s incl. IndexGrid builds and map",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 4), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "stride": S, "cin": wl.cin, "cout": wl.cout, "n_in": n_in,
                   "n_out": n_out, "pairs": pairs, "pairs_per_output": round(pairs / max(n_out, 1), 3)},
        "phases": phases,
        "conv_map_gbs": round(108.0 * n_out / (phases["conv_map_ms"]["mean"] * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(conv_tflops, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(conv_tflops / peak, 4), "traffic": None, "kernel": "k_conv_ggs_bf16",
                     "flops_per_launch": flops, "avg_launch_ms": round(conv_ms, 4)},
    }
    print(json.dumps(line), flush=True)
    return 0


def chain_main(args, torch, igc, workloads) -> int:
    """A chain of strided output grids (stage k over stage k-1's output) built with the counts on
    the device and one synchronisation (igc_conv_grid_chain), against the same grids built one
    call at a time (igc_conv_grid, one read-back each). Wall-clock per chain: the host waits
    are the point."""
    strides = [int(x) for x in args.chain.split(",")]
    steps, warmup = DEFAULT_STEPS[args.workload]
    steps = args.steps if args.steps is not None else max(steps, 5)
    warmup = args.warmup if args.warmup is not None else max(warmup, 1)
    dev = torch.device("cuda", 0)
    g = igc.grid_build(torch.from_numpy(workloads.make_coords(args.workload)).to(dev))

    def chained():
        return igc.conv_grid_chain(g, strides)

    def one_by_one():
        out, cur = [], g
        for s in strides:
            cur = igc.conv_grid(cur, s)
            out.append(cur)
        return out

    res = {}
    for name, fn in (("chain", chained), ("one_by_one", one_by_one)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(steps):
            t0 = time.perf_counter()
            grids = fn()
            torch.cuda.synchronize()
            t.append((time.perf_counter() - t0) * 1e3)
        res[name] = {"mean_ms": round(float(np.mean(t)), 4), "p50": _pct(t, 50), "p95": _pct(t, 95),
                     "n_voxels": [x.n_voxels for x in grids], "n_leaf": [x.n_leaf for x in grids]}
    line = {"metric": "strided output-grid chain, ms per chain (wall clock)", "value": res["chain"]["mean_ms"],
            "unit": "ms", "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": res["chain"]["mean_ms"],
            "higher_is_better": False, "dtype": "int32", "data": "synthetic",
            "config": {"workload": args.workload, "strides": strides, "n_input_voxels": g.n_voxels},
            "chain": res["chain"], "one_by_one": res["one_by_one"],
            "host_syncs": {"chain": 1, "one_by_one": len(strides)}}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
