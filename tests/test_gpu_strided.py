"""GPU parity of the strided / transposed convolution: output grids (bit-exact topology against
the oracle's build of oracle.conv_grid_coords), the neighbour map between two grids (bit-exact
against oracle.conv_map_between) and the convolution between two grids (bf16 inputs, fp32
accumulation; normwise error <= 2e-2 against the float64 oracle reading the same bf16 values).

At full size (band: 17.3M voxels, large: 48.2M voxels, stride 2) the oracle's output grid and
map were computed once by tests/golden/make_strided_golden.py; the HIP results must match their
SHA-256 digests bit for bit, and the convolution between the grids is then checked at sampled
output rows against oracle.conv over the (oracle-identical) map's columns.
"""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import (TOPO_KEYS, assert_topology_equal, elementwise_error, normwise_error, require_gpu, say,
                        segment_sample_rows, sub_map, to_dev)

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _igc():
    import sparse_convolution_amd as igc
    return igc


def _clusters(seed, n=5, size=20, spread=200, fill=0.3):
    rng = np.random.default_rng(seed)
    parts = []
    for _ in range(n):
        c = rng.integers(-spread, spread, size=3)
        cube = np.stack(np.meshgrid(*[np.arange(size)] * 3, indexing="ij"), -1).reshape(-1, 3)
        parts.append(cube[rng.random(cube.shape[0]) < fill] + c)
    return np.concatenate(parts).astype(np.int32)


def _check_grid_and_map(coords, stride, transposed, name):
    igc = _igc()
    say(f"conv grid {name} stride={stride} transposed={transposed} n_in={coords.shape[0]}")
    gi = igc.grid_build(to_dev(coords))
    go = igc.conv_grid(gi, stride, transposed)
    m = igc.conv_map(gi, go, stride, transposed)
    torch.cuda.synchronize()
    ri = oracle.OracleGrid(coords)
    ro = oracle.OracleGrid(oracle.conv_grid_coords(ri.active_ijk(), stride, transposed))
    assert go.n_voxels == ro.n
    assert_topology_equal(go.export(), ro.topology())
    assert np.array_equal(m.cpu().numpy(), oracle.conv_map_between(ro, ri, stride, transposed))
    return gi, go, m, ri, ro


@pytest.mark.parametrize("stride,transposed", [(1, False), (2, False), (3, False), ((2, 1, 3), False),
                                               (2, True), ((1, 2, 3), True)])
def test_conv_grid_and_map(stride, transposed):
    _check_grid_and_map(_clusters(60 + (stride if isinstance(stride, int) else 7)), stride, transposed, "clusters")


def test_conv_grid_workloads():
    _check_grid_and_map(workloads.make_coords("lidar"), 2, False, "lidar")
    _check_grid_and_map(workloads.make_coords("tiny"), 2, True, "tiny")


def _conv_case(coords, stride, transposed, cin, cout, name, seed, sample_rows=None):
    igc = _igc()
    gi, go, m, ri, ro = _check_grid_and_map(coords, stride, transposed, name)
    say(f"conv between {name} {cin}->{cout} n_out={go.n_voxels}")
    f = torch.from_numpy(workloads.make_features(gi.n_voxels, cin, 8000 + seed)).bfloat16()
    w = torch.from_numpy(workloads.make_weights(cin, cout, 9000 + seed, 1.0 / np.sqrt(27 * cin))).bfloat16()
    y = igc.sparse_conv_between(go, f.cuda(), w.cuda(), m)
    torch.cuda.synchronize()
    rows = None
    if sample_rows is not None and sample_rows < go.n_voxels:
        rows = np.sort(np.random.default_rng(seed).choice(go.n_voxels, sample_rows, replace=False))
    r = oracle.conv(m.cpu().numpy(), f.float().numpy(), w.float().numpy(), rows=rows)
    yy = y.float().cpu().numpy()
    if rows is not None:
        yy = yy[rows]
    err = normwise_error(yy, r)
    say(f"  normwise error {err:.3e}")
    assert np.all(np.isfinite(yy)) and err <= BF16_TOL


@pytest.mark.parametrize("stride,transposed,cin,cout", [(2, False, 64, 64), (2, False, 128, 256), (1, False, 32, 64),
                                                        (2, True, 128, 64), ((2, 1, 2), False, 64, 128),
                                                        (2, False, 32, 128), (2, True, 96, 256)])
def test_conv_between_clusters(stride, transposed, cin, cout):
    _conv_case(_clusters(70 + cin + cout), stride, transposed, cin, cout, "clusters", seed=cin + cout)


def test_conv_between_lidar_downsample_and_upsample():
    c = workloads.make_coords("lidar")
    _conv_case(c, 2, False, 128, 128, "lidar down", seed=3)
    _conv_case(c, 2, True, 128, 128, "lidar up", seed=4, sample_rows=1 << 15)


def test_edge_cases():
    igc = _igc()
    say("conv grid edge cases")
    g0 = igc.grid_build(torch.zeros((0, 3), dtype=torch.int32, device="cuda"))
    assert igc.conv_grid(g0, 2).n_voxels == 0
    assert igc.conv_grid(g0, 2, True).n_voxels == 0
    one = igc.grid_build(to_dev(np.array([[-5, 7, 0]], np.int32)))
    down = igc.conv_grid(one, 2)
    assert {tuple(r) for r in down.active_ijk().cpu().numpy().tolist()} == \
        {tuple(r) for r in oracle.conv_grid_coords(np.array([[-5, 7, 0]]), 2).tolist()}
    up = igc.conv_grid(one, 3, True)
    assert up.n_voxels == 27
    with pytest.raises(igc.IgcError):
        igc.conv_grid(one, 4)
    big = igc.grid_build(to_dev(np.array([[2 ** 30, 0, 0]], np.int32)))
    with pytest.raises(igc.IgcError):
        igc.conv_grid(big, 3, True)  # 3 * 2^30 leaves the int32 range
    # fp32 is not a gather-GEMM-scatter dtype: it runs on the general-shape path.
    f = torch.randn(one.n_voxels, 16, device="cuda")
    w = torch.randn(27, 16, 16, device="cuda")
    mo = igc.conv_map(one, down, 2)
    y = igc.sparse_conv_between(down, f, w, mo)
    torch.cuda.synchronize()
    r = oracle.conv(mo.cpu().numpy(), f.cpu().numpy(), w.cpu().numpy())
    assert normwise_error(y.cpu().numpy(), r) <= 1e-5
    with pytest.raises(igc.IgcError):  # beyond 4096 channels
        igc.sparse_conv_between(down, torch.zeros((one.n_voxels, 4100), device="cuda"),
                                torch.zeros((27, 4100, 4), device="cuda"), mo)


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


@pytest.mark.parametrize("name", ["band", "large"])
def test_strided_workload_full_size(name):
    igc = _igc()
    with open(os.path.join(GOLDEN, f"strided_{name}.json")) as fh:
        gold = json.load(fh)
    wl = workloads.WORKLOADS[name]
    say(f"strided {name}: build input grid")
    gi = igc.grid_build(to_dev(workloads.make_coords(name)))
    assert gi.n_voxels == gold["n_in"]
    S = gold["stride"]
    say(f"strided {name}: stride-{S} output grid and map")
    go = igc.conv_grid(gi, S)
    m = igc.conv_map(gi, go, S)
    counts = {"n_voxels": go.n_voxels, "n_leaf": go.n_leaf, "n_lower": go.n_lower, "n_upper": go.n_upper}
    assert counts == gold["counts"]
    topo = go.export()
    for k in TOPO_KEYS:
        assert _digest(topo[k]) == gold["topology_sha256"][k], f"output grid topology array {k} differs"
    assert _digest(go.active_ijk().cpu().numpy()) == gold["active_ijk_sha256"]
    mh = m.cpu().numpy()
    assert _digest(mh) == gold["map_sha256"]
    say(f"strided {name}: conv between grids bf16 {wl.cin}->{wl.cout}")
    f = workloads.make_features_device(gi.n_voxels, wl.cin, 8000 + wl.index, "cuda", torch.bfloat16)
    w = torch.from_numpy(workloads.make_weights(wl.cin, wl.cout, 9000 + wl.index, wl.weight_std)).bfloat16()
    y = igc.sparse_conv_between(go, f, w.cuda(), m)
    torch.cuda.synchronize()
    rows = segment_sample_rows(go.n_voxels, 1024, seg=256, n_random=1 << 18, seed=wl.index)
    sub, need = sub_map(mh, rows)
    del mh
    say(f"strided {name}: oracle conv on {rows.shape[0]} rows")
    ref = oracle.conv(sub, f[torch.from_numpy(need).cuda()].float().cpu().numpy(), w.float().numpy())
    got = y[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    err = normwise_error(got, ref)
    say(f"  normwise error {err:.3e}, elementwise {elementwise_error(got, ref):.3e}")
    assert np.all(np.isfinite(got)) and err <= BF16_TOL
