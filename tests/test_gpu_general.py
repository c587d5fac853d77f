"""GPU parity of the general-shape path (IGC_PATH_GATHER: any fp32 / bf16 channel counts up to
4096, one wave per output row, fp32 accumulation) against the float64 CPU oracle: the forward
convolution, the convolution between two grids, and the backward pass (input gradient through
the forward with flipped weights, weight gradient on the general-shape kernel).

Tolerances (normwise, max|y - r| / max|r|): 1e-5 for fp32 outputs and gradients, 2e-2 for bf16
outputs (rounded to bf16 once after an fp32 sum), 1e-5 for weight gradients (returned in fp32;
products of bf16 values are exact in fp32, sums of at most 8192 rows in fp32 and across row
chunks in fp64).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import elementwise_error, normwise_error, require_gpu, say, to_dev

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
WGRAD_TOL = 1e-5


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


def _data(n, cin, cout, dtype, seed):
    f = torch.from_numpy(workloads.make_features(n, cin, 3100 + seed)).to(dtype)
    w = torch.from_numpy(workloads.make_weights(cin, cout, 4100 + seed, 1.0 / np.sqrt(27 * cin))).to(dtype)
    return f, w


def _check(got, ref, tol, what):
    got = got.float().cpu().numpy()
    assert np.all(np.isfinite(got)), what
    err = normwise_error(got, ref)
    say(f"  {what}: normwise error {err:.3e}, elementwise {elementwise_error(got, ref):.3e}")
    assert err <= tol, f"{what}: normwise error {err} > {tol}"


# Shapes the tuned paths do not take (ragged channel counts, cout > 256 in two slices, cin > 64
# in two broadcast rounds) and one they do (forced onto this path).
SHAPES = [(torch.float32, 3, 16), (torch.float32, 32, 32), (torch.float32, 130, 70), (torch.float32, 1, 1),
          (torch.bfloat16, 4, 32), (torch.bfloat16, 128, 32), (torch.bfloat16, 96, 200), (torch.bfloat16, 64, 300),
          (torch.bfloat16, 64, 64)]


@pytest.mark.parametrize("dtype,cin,cout", SHAPES)
def test_forward_matches_oracle(dtype, cin, cout):
    igc = _igc()
    coords = _clusters(500 + cin + cout)
    say(f"general conv {dtype} {cin}->{cout} n_in={coords.shape[0]}")
    g = igc.grid_build(to_dev(coords))
    m = igc.kernel_map(g)
    f, w = _data(g.n_voxels, cin, cout, dtype, cin + cout)
    y = igc.sparse_conv(g, f.cuda(), w.cuda(), kmap=m, path="gather")
    torch.cuda.synchronize()
    assert y.dtype == dtype and tuple(y.shape) == (g.n_voxels, cout)
    mr = oracle.OracleGrid(coords).kernel_map()
    assert np.array_equal(m.cpu().numpy(), mr)
    _check(y, oracle.conv(mr, f.float().numpy(), w.float().numpy()), TOL[dtype], "forward")
    # The automatic choice takes this path exactly when no tuned path supports the shape, and then
    # gives the same bits; a rerun is bit-identical (fixed summation order).
    tuned = (dtype == torch.bfloat16 and cin % 32 == 0 and cout % 64 == 0)
    if not tuned:
        assert g.select_path(dtype, cin, cout) == "gather"
        y2 = igc.sparse_conv(g, f.cuda(), w.cuda(), kmap=m)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)


def test_lidar_first_layer():
    # A bf16 first layer with 4 input channels on the LiDAR-like scene (auto path).
    igc = _igc()
    coords = workloads.make_coords("lidar")
    say(f"general conv lidar bf16 4->32 n_in={coords.shape[0]}")
    g = igc.grid_build(to_dev(coords))
    m = igc.kernel_map(g)
    f, w = _data(g.n_voxels, 4, 32, torch.bfloat16, 7)
    y = igc.sparse_conv(g, f.cuda(), w.cuda(), kmap=m)
    torch.cuda.synchronize()
    _check(y, oracle.conv(m.cpu().numpy(), f.float().numpy(), w.float().numpy()), TOL[torch.bfloat16], "lidar 4->32")


@pytest.mark.parametrize("dtype,cin,cout,stride,transposed", [(torch.bfloat16, 16, 16, 2, False),
                                                              (torch.float32, 8, 24, 2, True),
                                                              (torch.float32, 33, 5, (2, 1, 3), False)])
def test_between_grids(dtype, cin, cout, stride, transposed):
    igc = _igc()
    coords = _clusters(600 + cin)
    say(f"general conv between {dtype} {cin}->{cout} stride={stride} transposed={transposed}")
    gi = igc.grid_build(to_dev(coords))
    go = igc.conv_grid(gi, stride, transposed)
    m = igc.conv_map(gi, go, stride, transposed)
    f, w = _data(gi.n_voxels, cin, cout, dtype, 11 + cin)
    y = igc.sparse_conv_between(go, f.cuda(), w.cuda(), m)
    torch.cuda.synchronize()
    assert y.dtype == dtype and tuple(y.shape) == (go.n_voxels, cout)
    _check(y, oracle.conv(m.cpu().numpy(), f.float().numpy(), w.float().numpy()), TOL[dtype], "between")


@pytest.mark.parametrize("dtype,cin,cout", [(torch.float32, 32, 32), (torch.bfloat16, 4, 32), (torch.bfloat16, 128, 32),
                                            (torch.float32, 70, 130), (torch.float32, 3, 5), (torch.bfloat16, 1, 36),
                                            (torch.bfloat16, 7, 16), (torch.float32, 64, 64), (torch.bfloat16, 20, 36)])
def test_backward_matches_oracle(dtype, cin, cout):
    igc = _igc()
    coords = _clusters(700 + cin + cout, n=4)
    say(f"general backward {dtype} {cin}->{cout} n_in={coords.shape[0]}")
    g = igc.grid_build(to_dev(coords))
    m = igc.kernel_map(g)
    f, w = _data(g.n_voxels, cin, cout, dtype, 21 + cin)
    dy = torch.from_numpy(workloads.make_features(g.n_voxels, cout, 7100 + cin)).to(dtype)
    dx, dw = igc.sparse_conv_backward(g, f.cuda(), w.cuda(), dy.cuda(), m)
    torch.cuda.synchronize()
    mr = m.cpu().numpy()
    _check(dx, oracle.conv_dgrad(mr, dy.float().numpy(), w.float().numpy()), TOL[dtype], "dfeats")
    _check(dw, oracle.conv_wgrad(mr, f.float().numpy(), dy.float().numpy()), WGRAD_TOL, "dweights")


def test_errors_and_empty():
    igc = _igc()
    from sparse_convolution_amd._lib import IgcError
    g = igc.grid_build(to_dev(_clusters(801, n=2)))
    m = igc.kernel_map(g)
    f, w = _data(g.n_voxels, 8, 8, torch.float32, 3)
    with pytest.raises(IgcError) as e:
        igc.sparse_conv(g, f.cuda(), w.cuda(), path="gather")  # no map
    assert e.value.status == 1
    big = torch.zeros((g.n_voxels, 4097), dtype=torch.float32, device="cuda")
    with pytest.raises(IgcError) as e:
        igc.sparse_conv(g, big, torch.zeros((27, 4097, 8), dtype=torch.float32, device="cuda"), kmap=m)
    assert e.value.status == 2
    empty = igc.grid_build(torch.zeros((0, 3), dtype=torch.int32, device="cuda"))
    y = igc.sparse_conv(empty, torch.zeros((0, 5), device="cuda"), torch.zeros((27, 5, 7), device="cuda"),
                        kmap=torch.zeros((27, 0), dtype=torch.int32, device="cuda"))
    assert tuple(y.shape) == (0, 7)


def test_general_weight_gradient_on_tuned_shapes(monkeypatch):
    # IGC_TEST_WGRAD_FORM=general sends shapes the matrix-core kernels take to the general one.
    igc = _igc()
    monkeypatch.setenv("IGC_TEST_WGRAD_FORM", "general")
    coords = _clusters(901, n=4)
    for dtype, cin, cout in [(torch.bfloat16, 64, 128), (torch.float32, 8, 16)]:
        say(f"general wgrad forced {dtype} {cin}->{cout}")
        g = igc.grid_build(to_dev(coords))
        m = igc.kernel_map(g)
        f, w = _data(g.n_voxels, cin, cout, dtype, 31 + cin)
        dy = torch.from_numpy(workloads.make_features(g.n_voxels, cout, 7300 + cin)).to(dtype)
        _, dw = igc.sparse_conv_backward(g, f.cuda(), w.cuda(), dy.cuda(), m, need_dfeats=False)
        torch.cuda.synchronize()
        _check(dw, oracle.conv_wgrad(m.cpu().numpy(), f.float().numpy(), dy.float().numpy()), WGRAD_TOL, "dweights")
