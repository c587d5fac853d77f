#!/usr/bin/env python3
"""Writes tests/golden/large_workload.json: the CPU oracle's results for the large workload
(50M signed coordinates, ~10% duplicates, from the narrow-band generator over [-2048,2048)^3),
used by tests/test_gpu_large.py to check the HIP path at full size.

Calls only oracle/ and workloads/. Stored: counts, SHA-256 digests of every topology array,
of the active voxels in linear-index order and of the full kernel map int32[27, N], and the
oracle's kernel-map entries of 256 seeded sample rows (plus the first and last row), from which
the test recomputes the sampled conv outputs with oracle.conv_rows.

    python tests/golden/make_large_golden.py      # ~3 minutes, ~10 GB of host memory
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


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def main() -> None:
    t0 = time.time()
    c = workloads.make_coords("large")
    print(f"coords {c.shape} {time.time() - t0:.0f}s", flush=True)
    g = oracle.OracleGrid(c)
    print(f"oracle build N={g.n} {time.time() - t0:.0f}s", flush=True)
    topo = g.topology()
    act = g.active_ijk()
    m = g.kernel_map()
    print(f"kernel map {time.time() - t0:.0f}s", flush=True)
    rows = np.sort(np.random.default_rng(5077).choice(g.n, 256, replace=False))
    rows = np.unique(np.concatenate([[0], rows, [g.n - 1]]))
    out = {
        "workload": "large",
        "generator": "workloads.make_coords('large')",
        "n_input": int(c.shape[0]),
        "counts": {"n_voxels": g.n, "n_leaf": g.n_leaf, "n_lower": g.n_lower, "n_upper": g.n_upper},
        "topology_sha256": {k: digest(v) for k, v in topo.items()},
        "active_ijk_sha256": digest(act),
        "kernel_map_sha256": digest(m),
        "sample_rows": rows.tolist(),
        "sample_map": m[:, rows].T.tolist(),
        "sample_ijk": act[rows].tolist(),
    }
    with open(os.path.join(HERE, "large_workload.json"), "w") as fh:
        json.dump(out, fh)
    print(f"written {time.time() - t0:.0f}s", flush=True)


if __name__ == "__main__":
    main()
