"""Selects the gather-GEMM-scatter row order per layer on this GPU and writes the tuning file
that the library loads (igc_tuning_load; the package loads igconv_tuning.txt beside it).

    python -m sparse_convolution_amd.tune [--workloads lidar band large large:grad] [--out PATH]

For every workload (synthetic scenes of the bench, see workloads/) each candidate (span 256 /
1024 / 4096 rows sorted by neighbour mask, natural or class bit order, output-tile width,
input channels per chunk and rows per workgroup) is timed
on the same path that runs in deployment (igc_sparse_conv, gather-GEMM-scatter), after checking
that its output equals the default order's; the fastest is written as one rule for the layer's
channels, with the measured times as comments (DriveRT, "Measurement and reproducibility":
algorithms are selected offline on the target GPU with the deployment path, and the selection
is stored in a documented file). A workload named NAME:grad tunes the layer's input-gradient
shape (cout -> cin, the gather-GEMM-scatter call the backward pass makes) on the same scene.
"""
from __future__ import annotations

import argparse
import os
import sys
import tempfile
import time

import torch

from . import _lib
import sparse_convolution_amd as igc

SPANS = [(256, "natural"), (256, "class"), (1024, "natural"), (1024, "class"), (4096, "natural"), (4096, "class")]


def _tiles(cin: int, cout: int) -> list:
    """Output-tile shapes the layer can use (auto = the widest): the narrower widths, with cin a
    multiple of 64 also the 128- and 64-channel tiles on 32-channel chunks (NNNk32), and each
    128- or 64-channel shape on half tiles (suffix h: 128 rows per workgroup)."""
    widest = 256 if cout % 256 == 0 and cin % 64 == 0 else 128 if cout % 128 == 0 else 64
    tiles = ["auto"] + [str(b) for b in (128, 64) if b < widest and cout % b == 0]
    if cin % 64 == 0:
        tiles += [f"{b}k32" for b in (128, 64) if cout % b == 0]
    tiles += [t + "h" if t != "auto" else f"{widest}h" for t in tiles if t != "auto" or widest < 256]
    return tiles


def _time(fn, reps):
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def tune_workload(spec: str, log) -> tuple[str, list]:
    import workloads
    name, _, kind = spec.partition(":")
    wl = workloads.WORKLOADS[name]
    cin, cout = (wl.cout, wl.cin) if kind == "grad" else (wl.cin, wl.cout)
    c = torch.from_numpy(workloads.make_coords(name)).cuda()
    g = igc.grid_build(c)
    m = igc.kernel_map(g)
    f = workloads.make_features_device(g.n_voxels, cin, 3000 + wl.index, "cuda", torch.bfloat16)
    w = torch.from_numpy(workloads.make_weights(cin, cout, 4000 + wl.index, 1.0 / (27 * cin) ** 0.5)).bfloat16().cuda()
    occ = g.n_voxels / (512.0 * g.n_leaf)
    reps = 3 if g.n_voxels > 20_000_000 else 10
    results = []
    ref = None
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "rule.txt")
        for (span, order), tile in [(so, t) for so in SPANS for t in _tiles(cin, cout)]:
            with open(path, "w") as fh:
                fh.write(f"ggs {cin} {cout} 0 1e30 {span} {order} {tile}\n")
            igc.tuning_load(path)
            out = torch.empty((g.n_voxels, cout), dtype=torch.bfloat16, device="cuda")
            ms = _time(lambda: igc.sparse_conv(g, f, w, kmap=m, path="ggs", out=out), reps)
            if ref is None:
                ref = out.clone()
            elif not torch.equal(out.float().abs(), ref.float().abs()):  # signs of exact zeros may differ
                raise RuntimeError(f"{spec}: row order {span} {order} tile {tile} changed the output")
            results.append((ms, span, order, tile))
            log(f"[tune] {spec} span {span} {order} tile {tile}: {ms:.4f} ms")
    igc.tuning_load(None)
    best = min(results)
    what = " (the input-gradient shape)" if kind == "grad" else ""
    lines = [f"# {spec}: {g.n_voxels} voxels, leaf occupancy {occ:.3f}, bf16 {cin} -> {cout}{what}; ms per conv: "
             + ", ".join(f"{s}/{o}/{t} {ms:.3f}" for ms, s, o, t in results),
             f"ggs {cin} {cout} 0 1e30 {best[1]} {best[2]} {best[3]}"]
    return "\n".join(lines), results


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workloads", nargs="+", default=["lidar", "band", "large", "large:grad"])
    ap.add_argument("--out", default=_lib.TUNING_PATH)
    args = ap.parse_args()
    log = lambda s: (sys.stderr.write(s + "\n"), sys.stderr.flush())
    _lib.load()
    igc.tuning_load(None)
    blocks = [f"# gather-GEMM-scatter row order and tile width per layer, selected by python -m sparse_convolution_amd.tune on "
              f"{torch.cuda.get_device_name(0)} {getattr(torch.cuda.get_device_properties(0), 'gcnArchName', '')} "
              f"({time.strftime('%Y-%m-%d')})",
              "# ggs <cin|*> <cout|*> <occupancy_lo> <occupancy_hi> <span 256|1024|4096> <natural|class> <tile>"]
    for name in args.workloads:
        text, _ = tune_workload(name, log)
        blocks.append(text)
    with open(args.out, "w") as fh:
        fh.write("\n".join(blocks) + "\n")
    log(f"[tune] wrote {args.out}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
