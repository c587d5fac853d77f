#!/usr/bin/env python3
"""Writes tests/golden/strided_<workload>.json: the CPU oracle's stride-2 output grid of the
band and large workloads and the neighbour map from it to the input grid, used by
tests/test_gpu_strided.py to check igc_conv_grid and igc_conv_map at full size.

Calls only oracle/ and workloads/. The output grid is the oracle's build of every candidate
coordinate (oracle.conv_grid_candidates: duplicates included, the build deduplicates); the map
is oracle.conv_map_between. Stored: counts, SHA-256 digests of every topology array, of the
output voxels in linear-index order and of the full map int32[27, N_out].

    python tests/golden/make_strided_golden.py [band] [large]   # minutes, ~16 GB of host memory
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402

STRIDE = 2


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def make(name: str) -> None:
    t0 = time.time()
    c = workloads.make_coords(name)
    gi = oracle.OracleGrid(c)
    del c
    print(f"{name}: input grid N={gi.n} {time.time() - t0:.0f}s", flush=True)
    cand = oracle.conv_grid_candidates(gi.active_ijk(), STRIDE)
    go = oracle.OracleGrid(cand)
    del cand
    print(f"{name}: output grid N={go.n} {time.time() - t0:.0f}s", flush=True)
    m = oracle.conv_map_between(go, gi, STRIDE)
    print(f"{name}: map {time.time() - t0:.0f}s", flush=True)
    out = {
        "workload": name,
        "generator": f"workloads.make_coords('{name}')",
        "stride": STRIDE,
        "transposed": False,
        "n_in": gi.n,
        "counts": {"n_voxels": go.n, "n_leaf": go.n_leaf, "n_lower": go.n_lower, "n_upper": go.n_upper},
        "topology_sha256": {k: digest(v) for k, v in go.topology().items()},
        "active_ijk_sha256": digest(go.active_ijk()),
        "map_sha256": digest(m),
        "pairs": int((m >= 0).sum()),
    }
    with open(os.path.join(HERE, f"strided_{name}.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    print(f"{name}: written {time.time() - t0:.0f}s", flush=True)


if __name__ == "__main__":
    for n in sys.argv[1:] or ["band", "large"]:
        make(n)
