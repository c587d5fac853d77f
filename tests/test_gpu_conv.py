"""GPU parity of the submanifold convolution (leaf path: fp32 and bf16 windows;
gather-GEMM-scatter path: bf16; both with fp32 accumulation) against the float64 CPU oracle.

Tolerances (normwise, max|y - r| / max|r| over the output): 1e-5 for fp32 and 2e-2 for bf16,
where the oracle reads exactly the bf16 values the GPU reads. Both paths must run: the
path is forced explicitly in every case.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import elementwise_error, normwise_error, require_gpu, say, segment_sample_rows, to_dev

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _igc():
    import sparse_convolution_amd as igc
    return igc


def _inputs(n, cin, cout, dtype, seed, std=None):
    f = workloads.make_features(n, cin, 3000 + seed)
    w = workloads.make_weights(cin, cout, 4000 + seed, std)
    ft = torch.from_numpy(f).to(dtype)
    wt = torch.from_numpy(w).to(dtype)
    return ft, wt


def run_conv(coords, cin, cout, dtype, path, name, seed=0, std=None, sample_rows=None):
    igc = _igc()
    say(f"conv {name} path={path} {dtype} {cin}->{cout} n_in={coords.shape[0]}")
    g = igc.grid_build(to_dev(coords))
    m = igc.kernel_map(g)
    ft, wt = _inputs(g.n_voxels, cin, cout, dtype, seed, std)
    y = igc.sparse_conv(g, ft.cuda(), wt.cuda(), kmap=m, path=path)
    torch.cuda.synchronize()
    ref_grid = oracle.OracleGrid(coords)
    mr = ref_grid.kernel_map()
    rows = None
    if sample_rows is not None and sample_rows < g.n_voxels:
        # Half in whole 256-row runs spread over the grid (first and last included), half uniform.
        rows = segment_sample_rows(g.n_voxels, sample_rows // 512, seg=256, n_random=sample_rows // 2,
                                   seed=seed + 77)
    r = oracle.conv(mr, ft.float().numpy(), wt.float().numpy(), rows=rows)
    yy = y.float().cpu().numpy()
    if rows is not None:
        yy = yy[rows]
    err = normwise_error(yy, r)
    say(f"  normwise error {err:.3e}, elementwise {elementwise_error(yy, r):.3e}"
        + (f" ({rows.shape[0]} sampled rows)" if rows is not None else ""))
    assert np.all(np.isfinite(yy))
    assert err <= TOL[dtype], f"normwise error {err} > {TOL[dtype]}"
    return g, y


def _cluster_coords(n_clusters, size, spread, seed, fill=0.35):
    rng = np.random.default_rng(seed)
    parts = []
    for _ in range(n_clusters):
        c = rng.integers(-spread, spread, size=3)
        cube = np.stack(np.meshgrid(*[np.arange(size)] * 3, indexing="ij"), -1).reshape(-1, 3)
        keep = rng.random(cube.shape[0]) < fill
        parts.append(cube[keep] + c)
    return np.concatenate(parts).astype(np.int32)


@pytest.mark.parametrize("cin,cout", [(4, 8), (8, 8), (8, 16), (8, 32), (16, 16), (4, 32)])
def test_leaf_path_shapes(cin, cout):
    c = _cluster_coords(6, 20, 200, seed=cin * 100 + cout)
    run_conv(c, cin, cout, torch.float32, "leaf", "clusters", seed=cin + cout)


@pytest.mark.parametrize("cin,cout", [(32, 64), (64, 64), (64, 128), (128, 128), (128, 256), (96, 192), (32, 128),
                                      (96, 256), (64, 256), (256, 64)])
def test_ggs_path_shapes(cin, cout):
    c = _cluster_coords(5, 24, 300, seed=cin + cout, fill=0.2)
    run_conv(c, cin, cout, torch.bfloat16, "ggs", "clusters", seed=cin * 3 + cout, std=1.0 / np.sqrt(27 * cin))


@pytest.mark.parametrize("cin,cout", [(16, 16), (16, 32), (16, 64), (32, 16), (32, 32), (32, 64), (64, 16),
                                      (64, 32), (64, 64)])
def test_leaf_path_bf16_shapes(cin, cout):
    # The bf16 leaf window (brick) path: dense clusters and a sparse shell in one grid.
    c = np.concatenate([_cluster_coords(4, 20, 200, seed=cin * 11 + cout, fill=0.6),
                        workloads.make_coords("tiny") + 700])
    run_conv(c, cin, cout, torch.bfloat16, "leaf", "clusters+shell", seed=cin * 13 + cout,
             std=1.0 / np.sqrt(27 * cin))


def test_leaf_workload_bf16_sampled():
    w = workloads.WORKLOADS["leaf"]
    run_conv(workloads.make_coords("leaf"), 32, 32, torch.bfloat16, "leaf", "leaf bf16 32->32", seed=w.index,
             std=1.0 / np.sqrt(27 * 32), sample_rows=1 << 18)


def test_tiny_workload_leaf():
    w = workloads.WORKLOADS["tiny"]
    run_conv(workloads.make_coords("tiny"), w.cin, w.cout, torch.float32, "leaf", "tiny", seed=w.index)


def test_leaf_workload_leaf():
    w = workloads.WORKLOADS["leaf"]
    run_conv(workloads.make_coords("leaf"), w.cin, w.cout, torch.float32, "leaf", "leaf", seed=w.index,
             std=w.weight_std)


def test_lidar_workload_ggs():
    w = workloads.WORKLOADS["lidar"]
    run_conv(workloads.make_coords("lidar"), w.cin, w.cout, torch.bfloat16, "ggs", "lidar", seed=w.index,
             std=w.weight_std)


@pytest.mark.parametrize("cin,cout", [(32, 64), (64, 64)])
@pytest.mark.parametrize("dense_min", [None, "1", "512"])
def test_mixed_path_per_leaf_dispatch(monkeypatch, cin, cout, dense_min):
    # Per-leaf dispatch: dense leaves (full cubes) on the bf16 leaf window, the rest (a sparse
    # shell and partly filled clusters) on gather-GEMM-scatter; thresholds that send every leaf
    # to one side or leave only full leaves on the window must give the same result.
    if dense_min is not None:
        monkeypatch.setenv("IGC_MIXED_MIN", dense_min)
    g3 = np.stack(np.meshgrid(*[np.arange(16)] * 3, indexing="ij"), -1).reshape(-1, 3)
    c = np.concatenate([_cluster_coords(3, 20, 150, seed=cin + cout, fill=0.5), g3 + 600,
                        workloads.make_coords("tiny") + 900]).astype(np.int32)
    run_conv(c, cin, cout, torch.bfloat16, "mixed", f"mixed dense_min={dense_min}", seed=cin * 7 + cout,
             std=1.0 / np.sqrt(27 * cin))


def test_band_workload_ggs_sampled():
    w = workloads.WORKLOADS["band"]
    run_conv(workloads.make_coords("band"), w.cin, w.cout, torch.bfloat16, "ggs", "band", seed=w.index,
             std=w.weight_std, sample_rows=1 << 20)


def test_band_workload_leaf_sampled():
    w = workloads.WORKLOADS["band"]
    run_conv(workloads.make_coords("band"), w.cin, w.cout, torch.bfloat16, "leaf", "band leaf window", seed=w.index,
             std=w.weight_std, sample_rows=1 << 20)


def test_identity_kernel_both_paths():
    igc = _igc()
    c = _cluster_coords(3, 16, 100, seed=3)
    g = igc.grid_build(to_dev(c))
    m = igc.kernel_map(g)
    say("identity kernels")
    f32 = torch.randn(g.n_voxels, 8, device="cuda")
    w32 = torch.zeros(27, 8, 8, device="cuda")
    w32[13] = torch.eye(8, device="cuda")
    assert torch.equal(igc.sparse_conv(g, f32, w32, path="leaf"), f32)
    f16 = torch.randn(g.n_voxels, 64, device="cuda").bfloat16()
    w16 = torch.zeros(27, 64, 64, device="cuda", dtype=torch.bfloat16)
    w16[13] = torch.eye(64, device="cuda", dtype=torch.bfloat16)
    assert torch.equal(igc.sparse_conv(g, f16, w16, kmap=m, path="ggs"), f16)
    fb = torch.randn(g.n_voxels, 32, device="cuda").bfloat16()
    wb = torch.zeros(27, 32, 32, device="cuda", dtype=torch.bfloat16)
    wb[13] = torch.eye(32, device="cuda", dtype=torch.bfloat16)
    assert torch.equal(igc.sparse_conv(g, fb, wb, path="leaf"), fb)
    assert torch.equal(igc.sparse_conv(g, f16, w16, path="leaf"), f16)  # 64 channels on the leaf window


def test_path_selection_and_errors():
    igc = _igc()
    g = igc.grid_build(to_dev(workloads.make_coords("tiny")))
    assert g.select_path(torch.float32, 8, 8) == "leaf"
    assert g.select_path(torch.bfloat16, 64, 64) == "ggs"
    assert g.select_path(torch.bfloat16, 32, 32) == "leaf"  # the only bf16 path below 64 outputs
    assert g.select_path(torch.bfloat16, 64, 32) == "leaf"
    cube = np.stack(np.meshgrid(*[np.arange(32)] * 3, indexing="ij"), -1).reshape(-1, 3).astype(np.int32)
    dense = igc.grid_build(to_dev(cube))  # 64 full leaves
    assert dense.leaf_occupancy == 1.0
    assert dense.select_path(torch.bfloat16, 64, 64) == "leaf"  # 64 input channels: leaf window above 0.5
    f = torch.randn(g.n_voxels, 8, device="cuda")
    w = torch.randn(27, 8, 8, device="cuda")
    with pytest.raises(igc.IgcError):
        igc.sparse_conv(g, f, w, path="ggs")  # fp32 is not a gather-GEMM-scatter dtype
    fb = torch.randn(g.n_voxels, 64, device="cuda").bfloat16()
    wb = torch.randn(27, 64, 64, device="cuda").bfloat16()
    with pytest.raises(igc.IgcError):
        igc.sparse_conv(g, fb, wb, path="ggs")  # no map
    with pytest.raises(igc.IgcError):
        igc.sparse_conv(g, torch.randn(g.n_voxels, 5, device="cuda"), torch.randn(27, 5, 8, device="cuda"))


def test_conv_deterministic():
    igc = _igc()
    c = workloads.make_coords("lidar")
    g = igc.grid_build(to_dev(c))
    m = igc.kernel_map(g)
    ft, wt = _inputs(g.n_voxels, 128, 128, torch.bfloat16, 4, 0.03)
    say("determinism ggs")
    a = igc.sparse_conv(g, ft.cuda(), wt.cuda(), kmap=m, path="ggs")
    b = igc.sparse_conv(g, ft.cuda(), wt.cuda(), kmap=m, path="ggs")
    assert torch.equal(a, b)


@pytest.fixture
def _restore_tuning():
    yield
    from sparse_convolution_amd import _lib as L
    import os
    _igc().tuning_load(L.TUNING_PATH if os.path.exists(L.TUNING_PATH) else None)


@pytest.mark.parametrize("span,order,tile", [(256, "class", "auto"), (1024, "natural", "64"), (4096, "natural", "auto"),
                                             (4096, "class", "64"), (256, "class", "64k32"), (1024, "class", "128k32"),
                                             (256, "class", "128h"), (4096, "natural", "64h"), (256, "natural", "64k32h"),
                                             (1024, "class", "128k32h")])
@pytest.mark.parametrize("case", ["lidar", "clusters", "mixed"])
def test_row_order_rules_keep_outputs(tmp_path, _restore_tuning, span, order, tile, case):
    # A row-order / tile rule (igc_tuning_load) changes which offsets each tile visits and how
    # many channels a workgroup computes, never an output: every rule gives the default's output
    # (up to the sign of exact zeros), and that
    # output matches the oracle on sampled rows. Spans wider than the grid and ragged last spans
    # are included (clusters: a few thousand rows).
    igc = _igc()
    if case == "lidar":
        coords, cin, cout, path = workloads.make_coords("lidar"), 128, 128, "ggs"
    elif case == "clusters":
        coords, cin, cout, path = _cluster_coords(4, 14, 200, seed=5), 64, 64, "ggs"
    else:
        g3 = np.stack(np.meshgrid(*[np.arange(16)] * 3, indexing="ij"), -1).reshape(-1, 3)
        coords = np.concatenate([_cluster_coords(3, 20, 150, seed=9, fill=0.5), g3 + 600]).astype(np.int32)
        cin, cout, path = 64, 64, "mixed"
    say(f"row order {case} span={span} order={order} n_in={coords.shape[0]}")
    g = igc.grid_build(to_dev(coords))
    m = igc.kernel_map(g)
    ft, wt = _inputs(g.n_voxels, cin, cout, torch.bfloat16, 31, 1.0 / np.sqrt(27 * cin))
    f, w = ft.cuda(), wt.cuda()
    igc.tuning_load(None)
    y0 = igc.sparse_conv(g, f, w, kmap=m, path=path)
    rule = tmp_path / "rule.txt"
    rule.write_text(f"ggs * * 0 1e30 {span} {order} {tile}\n")
    igc.tuning_load(str(rule))
    y1 = igc.sparse_conv(g, f, w, kmap=m, path=path)
    torch.cuda.synchronize()
    assert torch.equal(y1.float().abs(), y0.float().abs())
    rows = np.random.default_rng(span).choice(g.n_voxels, size=min(g.n_voxels, 2000), replace=False)
    mr = oracle.OracleGrid(coords).kernel_map()
    r = oracle.conv(mr, ft.float().numpy(), wt.float().numpy(), rows=rows)
    assert normwise_error(y1.float().cpu().numpy()[rows], r) <= TOL[torch.bfloat16]
