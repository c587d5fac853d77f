"""igc_sparse_conv_noalloc (the conv entry point that allocates nothing, for callers that
cannot allocate) against igc_sparse_conv on the same inputs: bit-identical outputs on every
path (the same kernels run; only where their temporaries live differs), over two calls in a
row on one device with the second one smaller, and a host-side capacity error for a layer
whose temporaries exceed the static scratch array (nothing is launched then). The general-shape
path keeps its packed fp32 weights there."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from tests._gpu import require_gpu, say, to_dev

pytestmark = pytest.mark.gpu

PATH = {"leaf": 1, "ggs": 2, "mixed": 3, "gather": 4}


def _clusters(seed, n=4, size=20, spread=200, fill=0.35):
    rng = np.random.default_rng(seed)
    parts = []
    for _ in range(n):
        c = rng.integers(-spread, spread, size=3)
        cube = np.stack(np.meshgrid(*[np.arange(size)] * 3, indexing="ij"), -1).reshape(-1, 3)
        parts.append(cube[rng.random(cube.shape[0]) < fill] + c)
    return np.concatenate(parts).astype(np.int32)


def _noalloc(g, m, f, w, path):
    from sparse_convolution_amd import _lib as L
    out = torch.full((g.n_voxels, w.shape[2]), float("nan"), dtype=f.dtype, device="cuda")
    dt = 0 if f.dtype == torch.float32 else 1
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.load().igc_sparse_conv_noalloc(g.handle, ctypes.c_void_p(m.data_ptr()) if m is not None else None,
                                          ctypes.c_void_p(f.data_ptr()), dt, f.shape[1], ctypes.c_void_p(w.data_ptr()),
                                          w.shape[2], ctypes.c_void_p(out.data_ptr()), PATH[path], st)
    return rc, out


def _case(coords, cin, cout, dtype, path, seed):
    import sparse_convolution_amd as igc
    say(f"no-alloc {path} {dtype} {cin}->{cout} n_in={coords.shape[0]}")
    g = igc.grid_build(to_dev(coords))
    m = igc.kernel_map(g)
    f = torch.from_numpy(workloads.make_features(g.n_voxels, cin, 3100 + seed)).to("cuda", dtype)
    w = torch.from_numpy(workloads.make_weights(cin, cout, 4100 + seed, 1.0 / np.sqrt(27 * cin))).to("cuda", dtype)
    ref = igc.sparse_conv(g, f, w, kmap=m, path=path)
    rc, y = _noalloc(g, m, f, w, path)
    assert rc == 0, igc._lib.load().igc_last_error()
    torch.cuda.synchronize()
    assert torch.equal(y, ref)


@pytest.mark.parametrize("path,dtype,cin,cout,big,small", [
    ("ggs", torch.bfloat16, 128, 128, "lidar", 1),
    ("ggs", torch.bfloat16, 64, 256, "clusters", 2),
    ("leaf", torch.bfloat16, 32, 32, "clusters", 3),
    ("leaf", torch.float32, 8, 16, "leaf", 4),
    ("mixed", torch.bfloat16, 64, 64, "clusters", 5),
    ("gather", torch.bfloat16, 4, 32, "lidar", 6),
    ("gather", torch.float32, 32, 300, "clusters", 7),
])
def test_noalloc_matches_conv_twice_second_smaller(path, dtype, cin, cout, big, small):
    require_gpu()
    first = workloads.make_coords(big) if big in ("lidar", "leaf") else _clusters(40 + small, n=8, size=24)
    second = _clusters(60 + small, n=2, size=12)
    assert second.shape[0] < first.shape[0]
    _case(first, cin, cout, dtype, path, small)
    _case(second, cin, cout, dtype, path, small + 10)


def test_noalloc_rejects_layers_beyond_the_scratch():
    require_gpu()
    import sparse_convolution_amd as igc
    say("no-alloc capacity error (band, 64 -> 64)")
    g = igc.grid_build(to_dev(workloads.make_coords("band")))
    m = igc.kernel_map(g)
    f = torch.zeros((g.n_voxels, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((27, 64, 64), dtype=torch.bfloat16, device="cuda")
    rc, y = _noalloc(g, m, f, w, "ggs")
    assert rc == 6  # IGC_ERR_CAPACITY, decided on the host before any launch
    # The general-shape path's packed weights (27 * cin * cout * 4 bytes) beyond the scratch.
    gs = igc.grid_build(to_dev(_clusters(91, n=1, size=8)))
    ms = igc.kernel_map(gs)
    f = torch.zeros((gs.n_voxels, 1024), dtype=torch.float32, device="cuda")
    w = torch.zeros((27, 1024, 1024), dtype=torch.float32, device="cuda")
    rc, y = _noalloc(gs, ms, f, w, "gather")
    assert rc == 6
    assert b"igc_sparse_conv_noalloc" in igc._lib.load().igc_last_error()
    torch.cuda.synchronize()
    assert torch.isnan(y).all()  # nothing was written
