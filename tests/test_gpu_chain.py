"""GPU parity of counted strided chains (igc_conv_grid_chain): every stage's grid is bit-exact
against the oracle applied stage by stage (oracle.conv_grid_coords, then the oracle's build of
those coordinates), equal to igc_conv_grid applied in turn, and usable downstream (kernel map on
the last grid and the map between consecutive grids, both bit-exact against the oracle).

Inputs whose outputs outgrow the library's capacity estimates (isolated voxels whose stride-2
outputs straddle leaf and root-tile boundaries: up to 8 output leaves and 8 output tiles per
input leaf) exercise the repeat-with-exact-counts path; a chain that needs more than 4096 root
tiles is refused with IGC_ERR_UNSUPPORTED.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import assert_topology_equal, require_gpu, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _igc():
    import sparse_convolution_amd as igc
    return igc


def _clusters(seed, n=6, size=24, spread=300, fill=0.3):
    rng = np.random.default_rng(seed)
    parts = []
    for _ in range(n):
        c = rng.integers(-spread, spread, size=3)
        cube = np.stack(np.meshgrid(*[np.arange(size)] * 3, indexing="ij"), -1).reshape(-1, 3)
        parts.append(cube[rng.random(cube.shape[0]) < fill] + c)
    return np.concatenate(parts).astype(np.int32)


def _leaf_straddlers(n_side=6):
    # x = 8 (1 + 4 q) + 7 is odd, and its stride-2 outputs (x - 1) / 2, (x + 1) / 2 lie on both
    # sides of an output-leaf boundary on every axis: 8 output leaves per (isolated) input leaf.
    x = 8 * (1 + 4 * np.arange(n_side)) + 7
    return np.stack(np.meshgrid(x, -x, x, indexing="ij"), -1).reshape(-1, 3).astype(np.int32)


def _tile_straddlers(n_side=5):
    # x = 8192 t - 1: stride-2 outputs 4096 t - 1 and 4096 t, one on each side of a root-tile
    # boundary on every axis (8 output tiles per input tile, one voxel per tile).
    t = np.arange(1, n_side + 1)
    x = 8192 * t - 1
    return np.stack(np.meshgrid(x, x, -x, indexing="ij"), -1).reshape(-1, 3).astype(np.int32)


def _oracle_chain(coords, strides, transposed):
    grids, cur = [], oracle.OracleGrid(coords)
    for s, t in zip(strides, transposed):
        cur = oracle.OracleGrid(oracle.conv_grid_coords(cur.active_ijk(), s, t))
        grids.append(cur)
    return grids


CASES = [
    ("clusters", [2, 2, 2], None),
    ("clusters", [1, 2], None),
    ("clusters", [2, 2], [False, True]),
    ("clusters", [(2, 1, 3), (1, 2, 2)], None),
    ("clusters", [3, (1, 2, 3)], [False, True]),
    ("lidar", [2, 2, 2, 2], None),
    ("leaf_straddlers", [2, 2], None),
    ("tile_straddlers", [2], None),
    ("tile_straddlers", [2, 2, 1], None),
]


@pytest.mark.parametrize("name,strides,transposed", CASES)
def test_chain_matches_oracle_and_single_stages(name, strides, transposed):
    igc = _igc()
    coords = {"clusters": lambda: _clusters(70 + len(strides)), "lidar": lambda: workloads.make_coords("lidar"),
              "leaf_straddlers": _leaf_straddlers, "tile_straddlers": _tile_straddlers}[name]()
    tr = [False] * len(strides) if transposed is None else transposed
    say(f"chain {name} strides={strides} transposed={tr} n_in={coords.shape[0]}")
    gi = igc.grid_build(to_dev(coords))
    chain = igc.conv_grid_chain(gi, strides, transposed)
    torch.cuda.synchronize()
    ref = _oracle_chain(coords, strides, tr)
    prev, rprev = gi, oracle.OracleGrid(coords)
    for k, (g, r) in enumerate(zip(chain, ref)):
        assert g.n_voxels == r.n, (k, g.n_voxels, r.n)
        assert_topology_equal(g.export(), r.topology())
        single = igc.conv_grid(prev, strides[k], tr[k])
        assert_topology_equal(single.export(), r.topology())
        m = igc.conv_map(prev, g, strides[k], tr[k])
        assert np.array_equal(m.cpu().numpy(), oracle.conv_map_between(r, rprev, strides[k], tr[k]))
        prev, rprev = g, r
    km = igc.kernel_map(chain[-1])
    assert np.array_equal(km.cpu().numpy(), ref[-1].kernel_map())


def test_chain_of_an_empty_grid():
    igc = _igc()
    gi = igc.grid_build(torch.empty((0, 3), dtype=torch.int32, device="cuda"))
    chain = igc.conv_grid_chain(gi, [2, 2], [False, True])
    assert [g.n_voxels for g in chain] == [0, 0]


def test_chain_errors():
    igc = _igc()
    gi = igc.grid_build(to_dev(_clusters(5)))
    with pytest.raises(igc.IgcError):
        igc.conv_grid_chain(gi, [2, 4])  # stride beyond 3
    with pytest.raises(igc.IgcError):
        igc.conv_grid_chain(gi, [2] * 17)  # more than 16 stages
    # More than 4096 output root tiles: refused (igc_conv_grid builds such a grid).
    t = np.arange(17)
    x = 4096 * t + 100
    pts = np.stack(np.meshgrid(x, x, x, indexing="ij"), -1).reshape(-1, 3).astype(np.int32)
    gm = igc.grid_build(to_dev(pts))
    assert gm.n_upper == 17 ** 3
    with pytest.raises(igc.IgcError, match="4096 root tiles"):
        igc.conv_grid_chain(gm, [1])
    single = igc.conv_grid(gm, 1)
    assert single.n_upper == 17 ** 3
