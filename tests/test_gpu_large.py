"""Full-size parity of the large workload (50M signed coordinates with ~10% duplicates ->
48.2M voxels, bf16 128 -> 256 conv) against the CPU oracle.

The oracle needs minutes for this workload's build, so tests/golden/make_large_golden.py ran it
once and stored SHA-256 digests of its topology arrays, active voxels and full kernel map. The
HIP results must match every digest bit for bit. The kernel map on the GPU is then the oracle's
map, so the conv is checked against oracle.conv over that map's columns at 2^20+ output rows:
4096 whole 256-row runs spread evenly over the grid (the first and the last, partial, run among
them) and the runs on both sides of the boundaries of eight equal ranges of runs, where the
launch's per-XCD tile ranges change hands - with the path and launch configuration bench.py
uses. Gate: normwise error <= 2e-2 (bf16); the elementwise error is reported.
"""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import (TOPO_KEYS, elementwise_error, normwise_error, require_gpu, say, segment_sample_rows,
                        sub_map, to_dev)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "large_workload.json")


def _digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_large_workload_full_size():
    require_gpu()
    import sparse_convolution_amd as igc
    with open(GOLDEN) as fh:
        gold = json.load(fh)
    say("large: coordinates (50M)")
    c = workloads.make_coords("large")
    assert c.shape[0] == gold["n_input"]
    say("large: build")
    g = igc.grid_build(to_dev(c))
    del c
    counts = {"n_voxels": g.n_voxels, "n_leaf": g.n_leaf, "n_lower": g.n_lower, "n_upper": g.n_upper}
    assert counts == gold["counts"]
    topo = g.export()
    for k in TOPO_KEYS:
        assert _digest(topo[k]) == gold["topology_sha256"][k], f"topology array {k} differs"
    say("large: active voxels and index queries")
    rows = np.asarray(gold["sample_rows"], dtype=np.int64)
    act = g.active_ijk().cpu().numpy()
    assert np.array_equal(act[rows], np.asarray(gold["sample_ijk"], dtype=np.int32))
    assert _digest(act) == gold["active_ijk_sha256"]
    idx = g.ijk_to_index(to_dev(act[rows])).cpu().numpy()
    assert np.array_equal(idx, rows.astype(np.int32))
    del act
    say("large: kernel map")
    m = igc.kernel_map(g)
    mh = m.cpu().numpy()
    nbrs = np.asarray(gold["sample_map"], dtype=np.int32)
    assert np.array_equal(mh[:, rows].T, nbrs)
    assert _digest(mh) == gold["kernel_map_sha256"]
    wl = workloads.WORKLOADS["large"]
    path = g.select_path(torch.bfloat16, wl.cin, wl.cout)
    say(f"large: conv bf16 {wl.cin}->{wl.cout} path={path}")
    f = workloads.make_features_device(g.n_voxels, wl.cin, 3000 + wl.index, "cuda", torch.bfloat16)
    w = torch.from_numpy(workloads.make_weights(wl.cin, wl.cout, 4000 + wl.index, wl.weight_std)).bfloat16()
    y = igc.sparse_conv(g, f, w.cuda(), kmap=m, path=path)
    torch.cuda.synchronize()
    sample = segment_sample_rows(g.n_voxels, 4096, seg=256)
    assert sample.shape[0] >= 1 << 20 and sample[0] == 0 and sample[-1] == g.n_voxels - 1
    sub, need = sub_map(mh, sample)
    del mh
    say(f"large: oracle conv on {sample.shape[0]} rows ({need.shape[0]} input rows)")
    fr = f[torch.from_numpy(need).cuda()].float().cpu().numpy()
    ref = oracle.conv(sub, fr, w.float().numpy())
    got = y[torch.from_numpy(sample).cuda()].float().cpu().numpy()
    err = normwise_error(got, ref)
    say(f"  normwise error {err:.3e}, elementwise {elementwise_error(got, ref):.3e}")
    assert np.all(np.isfinite(got))
    assert err <= 2e-2
