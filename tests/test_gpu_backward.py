"""GPU parity of the backward pass of the submanifold convolution against the float64 CPU
oracle (oracle.conv_dgrad, oracle.conv_wgrad).

Tolerances (normwise, max|y - r| / max|r|):
  - input gradient: the forward path's bars, 1e-5 for fp32 data and 2e-2 for bf16 data (the
    bf16 result is rounded to bf16 once, relative error <= 2^-8, plus fp32 accumulation);
  - weight gradient: 1e-5 for both dtypes. It is returned in fp32; bf16 inputs are exact in
    fp32, products of two bf16 values are exact in fp32, and the sum over rows is accumulated
    in fp32 within a chunk of at most a few thousand rows (random-walk rounding error about
    2^-24 * sqrt(rows) relative) and in fp64 across chunks.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import elementwise_error, normwise_error, require_gpu, say, segment_sample_rows, to_dev

pytestmark = pytest.mark.gpu

DGRAD_TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
WGRAD_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _igc():
    import sparse_convolution_amd as igc
    return igc


def _cluster_coords(n_clusters, size, spread, seed, fill=0.35):
    rng = np.random.default_rng(seed)
    parts = []
    for _ in range(n_clusters):
        c = rng.integers(-spread, spread, size=3)
        cube = np.stack(np.meshgrid(*[np.arange(size)] * 3, indexing="ij"), -1).reshape(-1, 3)
        keep = rng.random(cube.shape[0]) < fill
        parts.append(cube[keep] + c)
    return np.concatenate(parts).astype(np.int32)


def run_backward(coords, cin, cout, dtype, path, name, seed=0, std=None, need_dfeats=True, need_dweights=True):
    igc = _igc()
    say(f"backward {name} path={path} {dtype} {cin}->{cout} n_in={coords.shape[0]} "
        f"dfeats={need_dfeats} dweights={need_dweights}")
    g = igc.grid_build(to_dev(coords))
    m = igc.kernel_map(g)
    n = g.n_voxels
    f = torch.from_numpy(workloads.make_features(n, cin, 5000 + seed)).to(dtype)
    w = torch.from_numpy(workloads.make_weights(cin, cout, 6000 + seed, std)).to(dtype)
    dy = torch.from_numpy(workloads.make_features(n, cout, 7000 + seed)).to(dtype)
    dx, dw = igc.sparse_conv_backward(g, f.cuda(), w.cuda(), dy.cuda(), m, path=path,
                                      need_dfeats=need_dfeats, need_dweights=need_dweights)
    torch.cuda.synchronize()
    mr = oracle.OracleGrid(coords).kernel_map()
    assert np.array_equal(m.cpu().numpy(), mr)
    if need_dfeats:
        r = oracle.conv_dgrad(mr, dy.float().numpy(), w.float().numpy())
        got = dx.float().cpu().numpy()
        assert dx.dtype == dtype and got.shape == (n, cin)
        assert np.all(np.isfinite(got))
        err = normwise_error(got, r)
        say(f"  dfeats normwise error {err:.3e}")
        assert err <= DGRAD_TOL[dtype], f"dfeats normwise error {err} > {DGRAD_TOL[dtype]}"
    else:
        assert dx is None
    if need_dweights:
        r = oracle.conv_wgrad(mr, f.float().numpy(), dy.float().numpy())
        got = dw.cpu().numpy()
        assert dw.dtype == torch.float32 and got.shape == (27, cin, cout)
        err = normwise_error(got, r)
        say(f"  dweights normwise error {err:.3e}")
        assert err <= WGRAD_TOL, f"dweights normwise error {err} > {WGRAD_TOL}"
        # Offsets with no pair have an exactly zero gradient.
        for o in range(27):
            if not np.any(mr[o] >= 0):
                assert not np.any(got[o])
    else:
        assert dw is None
    return g, m, dx, dw


@pytest.mark.parametrize("cin,cout", [(32, 64), (64, 64), (64, 128), (128, 128), (128, 256), (96, 192)])
def test_bf16_weight_gradient_shapes(cin, cout):
    c = _cluster_coords(5, 24, 300, seed=cin + 7 * cout, fill=0.2)
    # dgrad runs cout -> cin on the gather-GEMM-scatter path, which needs cin % 64 == 0.
    run_backward(c, cin, cout, torch.bfloat16, "ggs", "clusters", seed=cin + cout, std=1.0 / np.sqrt(27 * cin),
                 need_dfeats=cin % 64 == 0)


@pytest.mark.parametrize("cin,cout", [(4, 8), (4, 16), (8, 16), (8, 8), (16, 16), (16, 8), (16, 4)])
def test_fp32_leaf_shapes(cin, cout):
    c = _cluster_coords(6, 20, 200, seed=cin * 31 + cout)
    run_backward(c, cin, cout, torch.float32, "leaf", "clusters", seed=cin * 5 + cout)


@pytest.mark.parametrize("cin,cout", [(16, 16), (16, 32), (32, 16), (32, 32), (16, 64), (32, 64), (64, 64)])
def test_bf16_leaf_input_gradient_shapes(cin, cout):
    # dgrad runs cout -> cin on the bf16 leaf window; the bf16 weight gradient needs cout >= 64.
    c = _cluster_coords(4, 20, 200, seed=cin * 41 + cout)
    run_backward(c, cin, cout, torch.bfloat16, "leaf", "clusters", seed=cin * 3 + cout, std=1.0 / np.sqrt(27 * cin),
                 need_dweights=False)


@pytest.mark.parametrize("cin,cout", [(4, 32), (8, 32), (4, 4), (8, 4)])
def test_fp32_leaf_weight_gradient_only_shapes(cin, cout):
    # The input gradient of these runs cout -> cin, not a leaf-path shape.
    c = _cluster_coords(6, 20, 200, seed=cin * 37 + cout)
    run_backward(c, cin, cout, torch.float32, "leaf", "clusters", seed=cin * 7 + cout, need_dfeats=False)


def test_fp32_weight_gradient_odd_channels():
    c = _cluster_coords(4, 18, 150, seed=11)
    run_backward(c, 5, 7, torch.float32, "leaf", "clusters-odd", seed=9, need_dfeats=False)
    run_backward(c, 64, 16, torch.float32, "leaf", "clusters-wide", seed=10, need_dfeats=False)


def test_leaf_workload():
    w = workloads.WORKLOADS["leaf"]
    run_backward(workloads.make_coords("leaf"), w.cin, w.cout, torch.float32, "leaf", "leaf", seed=w.index,
                 std=w.weight_std)


def test_lidar_workload():
    w = workloads.WORKLOADS["lidar"]
    run_backward(workloads.make_coords("lidar"), w.cin, w.cout, torch.bfloat16, "ggs", "lidar", seed=w.index,
                 std=w.weight_std)


def test_band_workload_sampled():
    # Full-size band geometry (17.3M voxels), bf16 64 -> 64 on gather-GEMM-scatter: the input
    # gradient is checked at 2^18+ sampled rows; the weight gradient for a dY that is zero outside
    # a row sample (every row still runs through the kernels) against the oracle's sum over it.
    igc = _igc()
    w = workloads.WORKLOADS["band"]
    c = workloads.make_coords("band")
    say("backward band: build and map")
    g = igc.grid_build(to_dev(c))
    m = igc.kernel_map(g)
    n = g.n_voxels
    f = workloads.make_features_device(n, w.cin, 5000 + w.index, "cuda", torch.bfloat16)
    wt = torch.from_numpy(workloads.make_weights(w.cin, w.cout, 6000 + w.index, w.weight_std)).bfloat16().cuda()
    dy = workloads.make_features_device(n, w.cout, 7000 + w.index, "cuda", torch.bfloat16)
    sel = segment_sample_rows(n, 512, seg=256, n_random=1 << 17, seed=w.index)
    keep = torch.zeros(n, dtype=torch.bool, device="cuda")
    keep[torch.from_numpy(sel).cuda()] = True
    dy_sel = torch.where(keep[:, None], dy, torch.zeros_like(dy))
    say("backward band: dgrad (full dY), wgrad (sampled dY)")
    dx, _ = igc.sparse_conv_backward(g, f, wt, dy, m, path="ggs", need_dweights=False)
    _, dw = igc.sparse_conv_backward(g, f, wt, dy_sel, m, path="ggs", need_dfeats=False)
    torch.cuda.synchronize()
    mr = oracle.OracleGrid(c).kernel_map()
    assert np.array_equal(m.cpu().numpy(), mr)
    say(f"backward band: oracle dgrad on {sel.shape[0]} rows")
    r = oracle.conv_dgrad(mr, dy.float().cpu().numpy(), wt.float().cpu().numpy(), rows=sel)
    got = dx[torch.from_numpy(sel).cuda()].float().cpu().numpy()
    err = normwise_error(got, r)
    say(f"  dfeats normwise error {err:.3e}, elementwise {elementwise_error(got, r):.3e}")
    assert np.all(np.isfinite(got)) and err <= DGRAD_TOL[torch.bfloat16]
    say("backward band: oracle wgrad")
    r = oracle.conv_wgrad(mr, f.float().cpu().numpy(), dy.float().cpu().numpy(), rows=sel)
    got = dw.cpu().numpy()
    err = normwise_error(got, r)
    say(f"  dweights normwise error {err:.3e}")
    assert err <= WGRAD_TOL


def test_single_voxel_and_sparse_offsets():
    # One voxel: only the centre offset has a pair. Isolated voxels: the same for every row.
    run_backward(np.array([[3, -4, 5]], np.int32), 8, 16, torch.float32, "leaf", "single", seed=1)
    iso = (np.arange(300, dtype=np.int32)[:, None] * np.array([[4, 0, 0]], np.int32))
    run_backward(iso, 64, 64, torch.bfloat16, "ggs", "isolated", seed=2, std=0.02)


def test_empty_grid():
    igc = _igc()
    say("backward empty grid")
    g = igc.grid_build(torch.zeros((0, 3), dtype=torch.int32, device="cuda"))
    m = igc.kernel_map(g)
    f = torch.zeros((0, 8), device="cuda")
    w = torch.randn(27, 8, 16, device="cuda")
    dy = torch.zeros((0, 16), device="cuda")
    dx, dw = igc.sparse_conv_backward(g, f, w, dy, m)
    torch.cuda.synchronize()
    assert dx.shape == (0, 8)
    assert dw.shape == (27, 8, 16) and not torch.any(dw)


def test_unsupported_shapes_raise():
    igc = _igc()
    c = _cluster_coords(2, 12, 50, seed=5)
    g = igc.grid_build(to_dev(c))
    m = igc.kernel_map(g)
    say("backward unsupported shapes")
    n = g.n_voxels
    fb = torch.randn(n, 32, device="cuda").bfloat16()
    wb = torch.randn(27, 32, 64, device="cuda").bfloat16()
    dyb = torch.randn(n, 64, device="cuda").bfloat16()
    with pytest.raises(igc.IgcError):  # dgrad 64 -> 32 is not a gather-GEMM-scatter shape
        igc.sparse_conv_backward(g, fb, wb, dyb, m, path="ggs")
    # The fp32 weight gradient beyond 64 x 64 channels runs on the general-shape kernel.
    f = torch.randn(n, 96, device="cuda")
    w = torch.randn(27, 96, 96, device="cuda")
    dy = torch.randn(n, 96, device="cuda")
    _, dw = igc.sparse_conv_backward(g, f, w, dy, m, need_dfeats=False)
    torch.cuda.synchronize()
    r = oracle.conv_wgrad(m.cpu().numpy(), f.cpu().numpy(), dy.cpu().numpy())
    assert normwise_error(dw.cpu().numpy(), r) <= WGRAD_TOL
    with pytest.raises(igc.IgcError):  # beyond the general-shape path's 4096 channels
        igc.sparse_conv_backward(g, torch.zeros((n, 4100), device="cuda"), torch.zeros((27, 4100, 4), device="cuda"),
                                 torch.zeros((n, 4), device="cuda"), m, need_dfeats=False)


def test_centre_identity_gradient():
    # W = identity at the centre offset only: dX = dY, and dW[13] = X^T dY.
    igc = _igc()
    c = _cluster_coords(3, 16, 100, seed=3)
    g = igc.grid_build(to_dev(c))
    m = igc.kernel_map(g)
    say("backward identity kernel")
    f = torch.randn(g.n_voxels, 64, device="cuda").bfloat16()
    dy = torch.randn(g.n_voxels, 64, device="cuda").bfloat16()
    w = torch.zeros(27, 64, 64, device="cuda", dtype=torch.bfloat16)
    w[13] = torch.eye(64, device="cuda", dtype=torch.bfloat16)
    dx, dw = igc.sparse_conv_backward(g, f, w, dy, m, path="ggs")
    assert torch.equal(dx, dy)
    ref = f.double().T @ dy.double()
    assert float((dw[13].double() - ref).abs().max() / ref.abs().max()) <= WGRAD_TOL


def test_backward_deterministic():
    igc = _igc()
    c = workloads.make_coords("lidar")
    g = igc.grid_build(to_dev(c))
    m = igc.kernel_map(g)
    n = g.n_voxels
    say("backward determinism")
    f = workloads.make_features_device(n, 128, 41, "cuda", torch.bfloat16)
    dy = workloads.make_features_device(n, 128, 42, "cuda", torch.bfloat16)
    w = (workloads.make_features_device(27 * 128, 128, 43, "cuda") * 0.02).bfloat16().reshape(27, 128, 128)
    a = igc.sparse_conv_backward(g, f, w, dy, m, path="ggs")
    b = igc.sparse_conv_backward(g, f, w, dy, m, path="ggs")
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    fl = workloads.make_features_device(n, 8, 44, "cuda")
    dyl = workloads.make_features_device(n, 16, 45, "cuda")
    wl = workloads.make_features_device(27 * 8, 16, 46, "cuda").reshape(27, 8, 16)
    a = igc.sparse_conv_backward(g, fl, wl, dyl, m, path="leaf")
    b = igc.sparse_conv_backward(g, fl, wl, dyl, m, path="leaf")
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
