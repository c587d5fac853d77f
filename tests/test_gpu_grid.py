"""GPU parity of the IndexGrid build, the index query and the kernel map against the CPU
oracle: bit-exact topology, row order, indices and maps."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import assert_topology_equal, require_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _igc():
    import sparse_convolution_amd as igc
    return igc


def check_grid(coords: np.ndarray, name: str, offsets=None, queries: np.ndarray | None = None):
    igc = _igc()
    say(f"build {name} n_in={coords.shape[0]}")
    g = igc.grid_build(to_dev(coords))
    torch.cuda.synchronize()
    ref = oracle.OracleGrid(coords)
    assert (g.n_voxels, g.n_leaf, g.n_lower, g.n_upper) == (ref.n, ref.n_leaf, ref.n_lower, ref.n_upper)
    assert_topology_equal(g.export(), ref.topology())
    say(f"active_ijk / ijk_to_index {name}")
    act = g.active_ijk().cpu().numpy()
    assert np.array_equal(act, ref.active_ijk())
    q = coords if queries is None else np.concatenate([coords, queries])
    got = g.ijk_to_index(to_dev(q)).cpu().numpy()
    assert np.array_equal(got, ref.ijk_to_index(q))
    say(f"kernel_map {name}")
    m, nb = igc.kernel_map(g, offsets, with_mask=True) if (offsets is None or len(offsets) <= 32) else (
        igc.kernel_map(g, offsets), None)
    mr, nbr = ref.kernel_map(offsets, with_mask=True)
    assert np.array_equal(m.cpu().numpy(), mr)
    if nb is not None:
        assert np.array_equal(nb.cpu().numpy().view(np.uint32), nbr)
    return g, ref


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_signed_with_duplicates(seed):
    rng = np.random.default_rng(seed)
    # clusters straddling tile / node boundaries and the sign change, plus scattered points
    centres = np.array([[0, 0, 0], [4096, -4096, 128], [-1, 2047, -2049], [123457, -98765, 5]])
    parts = [c + rng.integers(-40, 41, size=(20000, 3)) for c in centres]
    parts.append(rng.integers(-2**20, 2**20, size=(3001, 3)))
    c = np.concatenate(parts).astype(np.int32)
    c = np.concatenate([c, c[rng.integers(0, c.shape[0], 7777)]])
    c = c[rng.permutation(c.shape[0])]
    q = rng.integers(-50, 50, size=(5000, 3)).astype(np.int32)
    check_grid(c, f"random seed {seed}", queries=q)


def test_tiny_workload():
    check_grid(workloads.make_coords("tiny"), "tiny")


def test_leaf_workload():
    check_grid(workloads.make_coords("leaf"), "leaf")


def test_lidar_workload():
    check_grid(workloads.make_coords("lidar"), "lidar")


def test_band_workload():
    check_grid(workloads.make_coords("band"), "band")


def test_all_identical():
    check_grid(np.tile(np.array([[-7, 3, 100000]], np.int32), (10000, 1)), "identical")


def test_sorted_and_reverse_sorted_inputs():
    g3 = np.stack(np.meshgrid(np.arange(40), np.arange(40), np.arange(40), indexing="ij"), -1).reshape(-1, 3)
    c = (g3 - 20).astype(np.int32)
    check_grid(c, "sorted")
    check_grid(c[::-1].copy(), "reverse")


def test_one_voxel_per_leaf_and_full_leaves():
    rng = np.random.default_rng(5)
    origins = np.unique(rng.integers(-300, 300, size=(3000, 3)) * 8, axis=0)
    one = (origins + rng.integers(0, 8, size=origins.shape)).astype(np.int32)
    check_grid(one, "one per leaf")
    g3 = np.stack(np.meshgrid(np.arange(8), np.arange(8), np.arange(8), indexing="ij"), -1).reshape(-1, 3)
    full = (origins[:200, None, :] + g3[None]).reshape(-1, 3).astype(np.int32)
    check_grid(full[rng.permutation(full.shape[0])], "full leaves")


def test_int32_extremes():
    M, m = 2**31 - 1, -2**31
    c = np.array([[M, M, M], [m, m, m], [M, 0, m], [m, M, 0], [M - 1, M, M], [m + 1, m, m], [0, 0, 0], [-1, -1, -1],
                  [M, M - 8, M], [m, m + 8, m]], np.int32)
    check_grid(c, "int32 extremes")


def test_general_offsets():
    rng = np.random.default_rng(9)
    c = (rng.integers(-30, 30, size=(20000, 3))).astype(np.int32)
    d = np.arange(-2, 3)
    off = np.stack(np.meshgrid(d, d, d, indexing="ij"), -1).reshape(-1, 3).astype(np.int32)  # 5x5x5
    check_grid(c, "5x5x5 offsets", offsets=off)
    off8 = np.array([[8, 0, 0], [-8, 8, -8], [7, -7, 1], [0, 0, 0]], np.int32)
    check_grid(c, "offsets up to 8", offsets=off8)


def test_unit_stencil_forms():
    """The standard 27-offset order takes the window kernel; a permuted or partial unit stencil
    and an output buffer that is not 16-byte aligned take the per-pair kernel. All must agree
    with the oracle."""
    igc = _igc()
    from sparse_convolution_amd import _lib, _ptr, _stream, _STD_OFFSETS_PTR
    c = workloads.make_coords("lidar")
    std = oracle.standard_offsets()
    rng = np.random.default_rng(21)
    perm = np.ascontiguousarray(std[rng.permutation(27)])
    seven = np.array([[0, 0, 0], [1, 0, 0], [-1, 0, 0], [0, 1, 0], [0, -1, 0], [0, 0, 1], [0, 0, -1]], np.int32)
    g, ref = check_grid(c, "lidar permuted stencil", offsets=perm)
    check_grid(c, "lidar 7-point stencil", offsets=seven)
    say("kernel map into a buffer offset by one element")
    N = g.n_voxels
    buf = torch.full((27 * N + 8,), 7, dtype=torch.int32, device="cuda")
    out = buf[1:1 + 27 * N].view(27, N)
    _lib.check(_lib.load().igc_kernel_map(g.handle, _STD_OFFSETS_PTR, 27, _ptr(out), None, _stream(g.device)))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref.kernel_map(None))
    assert int(buf[0]) == 7 and bool((buf[1 + 27 * N:] == 7).all())


def test_capacity_retry(monkeypatch):
    monkeypatch.setenv("IGC_TEST_INITIAL_CAPACITY", "1")
    rng = np.random.default_rng(13)
    c = rng.integers(-2**24, 2**24, size=(5000, 3)).astype(np.int32)  # ~5000 root tiles
    g, _ = check_grid(c, "root table retry")
    assert g.root_capacity >= 2 * g.n_upper


def test_many_tiles_radix_tile_sort():
    # more than 4096 distinct root tiles: the one-read-back build falls back to the build with
    # read-backs after the tile pass and the counts, whose tile keys go through the radix sort
    rng = np.random.default_rng(17)
    c = rng.integers(-2**30, 2**30, size=(60000, 3)).astype(np.int32)
    g, _ = check_grid(c, "many tiles")
    assert g.host_syncs == 4


def test_counted_build_repeats_with_exact_counts():
    # The build sizes its node arrays from the previous build's rows per coordinate and reads the
    # device state back once. A dense block (216 leaves for 110,592 coordinates) followed by 343
    # isolated voxels, each its own leaf, lower node and root tile, outgrows every estimate: the
    # build is repeated with the exact counts (a second read-back) and matches the oracle.
    igc = _igc()
    dense = np.stack(np.meshgrid(*[np.arange(48)] * 3, indexing="ij"), -1).reshape(-1, 3).astype(np.int32)
    igc.grid_build(to_dev(dense))
    g1, _ = check_grid(dense, "dense block")
    assert g1.host_syncs == 1  # the same scene again: its estimate fits
    t = np.arange(-3, 4)
    pts = np.stack(np.meshgrid(4096 * t + 7, 4096 * t + 100, 4096 * t + 1000, indexing="ij"), -1)
    pts = pts.reshape(-1, 3).astype(np.int32)
    g2, ref = check_grid(pts, "isolated voxels in 343 tiles")
    assert (g2.n_leaf, g2.n_lower, g2.n_upper) == (343, 343, 343)
    assert g2.host_syncs == 2
    g3, _ = check_grid(workloads.make_coords("lidar"), "lidar after isolated voxels")
    assert g3.host_syncs in (1, 2)


def test_empty_grid():
    igc = _igc()
    say("empty grid")
    g = igc.grid_build(torch.zeros((0, 3), dtype=torch.int32, device="cuda"))
    assert (g.n_voxels, g.n_leaf, g.n_lower, g.n_upper) == (0, 0, 0, 0)
    assert igc.kernel_map(g).shape == (27, 0)
    idx = g.ijk_to_index(torch.tensor([[0, 0, 0]], dtype=torch.int32, device="cuda"))
    assert idx.cpu().tolist() == [-1]


def test_deterministic():
    igc = _igc()
    c = workloads.make_coords("lidar")
    say("determinism lidar")
    a = igc.grid_build(to_dev(c))
    b = igc.grid_build(to_dev(c))
    ta, tb = a.export(), b.export()
    for k in ta:
        assert np.array_equal(ta[k], tb[k])
    assert torch.equal(igc.kernel_map(a), igc.kernel_map(b))


def test_errors():
    igc = _igc()
    from sparse_convolution_amd import _lib
    lib = _lib.load()
    import ctypes
    h = ctypes.c_void_p()
    assert lib.igc_grid_build(None, 5, None, None, ctypes.byref(h)) == 1
    assert b"d_ijk" in lib.igc_last_error()
    assert lib.igc_grid_build(None, -1, None, None, ctypes.byref(h)) == 1
    g = igc.grid_build(to_dev(np.array([[1, 2, 3]], np.int32)))
    off = np.array([[9, 0, 0]], np.int32)
    with pytest.raises(igc.IgcError):
        igc.kernel_map(g, off)


@pytest.mark.parametrize("form", ["pc", "window"])
def test_kernel_map_forms(monkeypatch, form):
    """Both standard-stencil kernel-map forms (producer / consumer, taken by grids of many leaves,
    and the persistent window form) agree with the oracle on every grid shape, whichever the
    grid size would select: a single voxel, sparse and full leaves, a leaf count that leaves
    workgroups without a full step, and a grid large enough for many steps per workgroup."""
    monkeypatch.setenv("IGC_TEST_KMAP_FORM", form)
    rng = np.random.default_rng(31)
    check_grid(np.array([[5, -3, 7]], np.int32), f"{form}: one voxel")
    origins = np.unique(rng.integers(-200, 200, size=(4001, 3)) * 8, axis=0)
    one = (origins + rng.integers(0, 8, size=origins.shape)).astype(np.int32)
    check_grid(one[:4001], f"{form}: one voxel per leaf")
    g3 = np.stack(np.meshgrid(np.arange(8), np.arange(8), np.arange(8), indexing="ij"), -1).reshape(-1, 3)
    full = (origins[:37, None, :] + g3[None]).reshape(-1, 3).astype(np.int32)
    check_grid(full, f"{form}: 37 full leaves")
    check_grid(workloads.make_coords("lidar"), f"{form}: lidar")
    check_grid(workloads.make_coords("leaf"), f"{form}: leaf")


def test_concurrent_builds_two_threads():
    """Two host threads building on their own streams at once (the shared workspace is busy for
    one of them, and each thread has its own pinned staging buffer for the read-backs) give
    the same grids as builds one at a time."""
    import threading
    igc = _igc()
    inputs = [workloads.make_coords("lidar"), workloads.make_coords("tiny"),
              np.random.default_rng(41).integers(-3000, 3000, size=(200000, 3)).astype(np.int32)]
    ref = [igc.grid_build(to_dev(c)).export() for c in inputs]
    torch.cuda.synchronize()
    say("concurrent builds")
    results, errors = {}, []

    def worker(tid):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for rep in range(3):
                    for i, c in enumerate(inputs):
                        g = igc.grid_build(to_dev(c))
                        stream.synchronize()
                        results[(tid, rep, i)] = g.export()
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert len(results) == 2 * 3 * len(inputs)
    for (tid, rep, i), topo in results.items():
        for k in ref[i]:
            assert np.array_equal(topo[k], ref[i][k]), (tid, rep, i, k)


class _TorchCountingAllocator:
    """PyTorch's caching allocator behind the C allocator interface, counting live blocks and
    failing the `fail_at`-th request (1-based) on purpose."""

    def __init__(self, fail_at=None):
        from sparse_convolution_amd import _lib as L
        self.fail_at = fail_at
        self.n_req = 0
        self.live = {}
        self._a = L.ALLOC_FN(self._alloc)
        self._r = L.RELEASE_FN(self._release)
        self.struct = L.Allocator(self._a, self._r, None)

    def _alloc(self, ctx, nbytes, stream):
        self.n_req += 1
        if self.fail_at is not None and self.n_req == self.fail_at:
            return None
        p = torch.cuda.caching_allocator_alloc(int(nbytes), torch.cuda.current_device(), int(stream or 0))
        self.live[p] = nbytes
        return p

    def _release(self, ctx, ptr, nbytes, stream):
        assert self.live.pop(ptr) == nbytes
        torch.cuda.caching_allocator_delete(ptr)


def test_caller_allocator_and_failure_injection():
    # Every device block of a build, a kernel map and a conv comes from the caller's allocator and
    # goes back to it; an allocation failing at any point of the build is reported as
    # IGC_ERR_OOM and every block taken before it is returned.
    from sparse_convolution_amd import _lib as L
    igc = _igc()
    lib = L.load()
    c = to_dev(workloads.make_coords("lidar"))
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    say("allocator: counting build, map and conv")
    a = _TorchCountingAllocator()
    h = ctypes.c_void_p()
    assert lib.igc_grid_build(ctypes.c_void_p(c.data_ptr()), c.shape[0], ctypes.byref(a.struct), stream,
                              ctypes.byref(h)) == 0
    n_build = a.n_req
    assert n_build >= 2 and len(a.live) == 1  # the grid's block stays, the temporaries came back
    g = igc.Grid(h, c.device)
    ref = igc.grid_build(c, memory="library")
    for k, v in g.export().items():
        assert np.array_equal(v, ref.export()[k]), k
    m = igc.kernel_map(g)
    f = torch.randn(g.n_voxels, 128, device="cuda").bfloat16()
    w = (torch.randn(27, 128, 128, device="cuda") * 0.02).bfloat16()
    y = igc.sparse_conv(g, f, w, kmap=m, path="ggs")
    assert torch.equal(y, igc.sparse_conv(ref, f, w, kmap=m, path="ggs"))
    assert a.n_req > n_build and len(a.live) == 1  # the conv's workspace came back too
    torch.cuda.synchronize()
    del g
    assert len(a.live) == 0
    for k in range(1, n_build + 1):
        say(f"allocator: request {k} of {n_build} fails")
        b = _TorchCountingAllocator(fail_at=k)
        h = ctypes.c_void_p()
        assert lib.igc_grid_build(ctypes.c_void_p(c.data_ptr()), c.shape[0], ctypes.byref(b.struct), stream,
                                  ctypes.byref(h)) == 3
        assert b"igc_grid_build" in lib.igc_last_error()
        assert not h.value and len(b.live) == 0
