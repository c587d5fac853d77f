"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties the oracle to one of: a worked example derived by hand from the pages'
definitions (tests/golden), a closed form, a library routine computing the same
quantity another way (torch conv3d), brute force on tiny inputs, or an invariant the
method guarantees. Chosen so that a dropped term, a swapped axis, a wrong shift or a
wrong sign in the oracle fails at least one of them.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import OracleGrid, standard_offsets
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _popcount64(a: np.ndarray) -> np.ndarray:
    a = a.astype(np.uint64)
    return np.array([bin(int(x)).count("1") for x in a.ravel()], dtype=np.int64).reshape(a.shape)


def _single_bit(mask_row: np.ndarray) -> int:
    """Index of the only set bit of a multi-word mask."""
    nz = np.nonzero(mask_row)[0]
    assert nz.size == 1
    w = int(nz[0])
    v = int(mask_row[w])
    assert v & (v - 1) == 0
    return w * 64 + v.bit_length() - 1


# ----------------------------------------------------------------------------- worked examples

def _read_key_examples():
    rows = []
    with open(os.path.join(GOLDEN, "key_examples.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            i, j, k, key, up, lo, lf = line.split()
            rows.append(((int(i), int(j), int(k)), int(key, 16), int(up), int(lo), int(lf)))
    return rows


@pytest.mark.parametrize("row", _read_key_examples(), ids=lambda r: str(r[0]))
def test_key_worked_examples(row):
    (c, key1, up, lo, lf) = row
    g = OracleGrid(np.array([c], np.int32))
    assert (g.n, g.n_leaf, g.n_lower, g.n_upper) == (1, 1, 1, 1)
    t = g.topology()
    assert int(t["root_key"][0]) == key1
    assert _single_bit(t["upper_mask"][0]) == up
    assert _single_bit(t["lower_mask"][0]) == lo
    assert _single_bit(t["leaf_mask"][0]) == lf
    # node origins: the coordinate with the low 12 / 7 / 3 bits cleared
    c = np.array(c, np.int64)
    assert tuple(t["upper_origin"][0]) == tuple(c & ~4095)
    assert tuple(t["lower_origin"][0]) == tuple(c & ~127)
    assert tuple(t["leaf_origin"][0]) == tuple(c & ~7)


def test_leaf_encoding_worked_example():
    vox, absent, words, prefix = [], [], {}, None
    with open(os.path.join(GOLDEN, "leaf_example.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            p = line.split()
            if p[0] == "voxel":
                vox.append(((int(p[1]), int(p[2]), int(p[3])), int(p[4])))
            elif p[0] == "absent":
                absent.append((int(p[1]), int(p[2]), int(p[3])))
            elif p[0] == "word":
                words[int(p[1])] = int(p[2], 16)
            elif p[0] == "prefix":
                prefix = int(p[1], 16)
    coords = np.array([v[0] for v in vox][::-1] * 2, np.int32)  # reversed and duplicated input
    g = OracleGrid(coords)
    assert (g.n, g.n_leaf) == (5, 1)
    t = g.topology()
    assert [int(x) for x in t["leaf_mask"][0]] == [words[w] for w in range(8)]
    assert int(t["leaf_prefix"][0]) == prefix
    assert int(t["leaf_offset"][0]) == 0
    idx = g.ijk_to_index(np.array([v[0] for v in vox], np.int32))
    assert list(idx) == [v[1] for v in vox]
    assert list(g.ijk_to_index(np.array(absent, np.int32))) == [-1] * len(absent)


def test_leaf_index_record_is_80_bytes():
    # 8 mask words + one offset word + one packed-prefix word; a leaf of 512 uint64
    # values takes 4096 B, so the compression is 4096 / 80 = 51.2 > 50.
    t = OracleGrid(np.array([[0, 0, 0]], np.int32)).topology()
    rec = t["leaf_mask"][0].nbytes + t["leaf_offset"][:1].nbytes + t["leaf_prefix"][:1].nbytes
    assert rec == 80 and 512 * 8 / rec > 50


# ----------------------------------------------------------------------------- closed forms

def test_full_leaf_order_is_ijk_lexicographic():
    g3 = np.stack(np.meshgrid(np.arange(8), np.arange(8), np.arange(8), indexing="ij"), -1).reshape(-1, 3)
    g = OracleGrid((g3 + np.array([16, 8, 24])).astype(np.int32)[::-1])
    idx = g.ijk_to_index((g3 + np.array([16, 8, 24])).astype(np.int32))
    assert np.array_equal(idx, g3[:, 0] * 64 + g3[:, 1] * 8 + g3[:, 2])
    t = g.topology()
    assert np.all(t["leaf_mask"][0] == np.uint64(0xFFFFFFFFFFFFFFFF))
    # prefix of a full leaf: 64 * w for w = 1..7
    assert int(t["leaf_prefix"][0]) == sum((64 * w) << (9 * (w - 1)) for w in range(1, 8))


def test_full_block_order_is_leaf_major():
    # A full 16^3 block at the origin spans 8 leaves of one lower node; leaves are taken
    # x-major by (i>>3, j>>3, k>>3), voxels x-major inside each leaf.
    g3 = np.stack(np.meshgrid(np.arange(16), np.arange(16), np.arange(16), indexing="ij"), -1).reshape(-1, 3)
    rng = np.random.default_rng(7)
    g = OracleGrid(g3[rng.permutation(g3.shape[0])].astype(np.int32))
    leaf_rank = (g3[:, 0] >> 3) * 4 + (g3[:, 1] >> 3) * 2 + (g3[:, 2] >> 3)
    vox = (g3[:, 0] & 7) * 64 + (g3[:, 1] & 7) * 8 + (g3[:, 2] & 7)
    assert np.array_equal(g.ijk_to_index(g3.astype(np.int32)), leaf_rank * 512 + vox)
    assert (g.n_leaf, g.n_lower, g.n_upper) == (8, 1, 1)
    assert list(g.topology()["leaf_offset"]) == [512 * r for r in range(8)]


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_line_order_is_unsigned_order(axis):
    # Along one axis (others fixed) the tile / upper / lower / leaf fields are a mixed-radix
    # split of the 32-bit pattern, so the order is ascending uint32: 0, 1, ..., 2^31-1,
    # -2^31, ..., -1. Values straddle tile, node and sign boundaries.
    vals = np.array([0, 1, 7, 8, 127, 128, 4095, 4096, 4097, 123456, 2**31 - 1, -2**31, -4097, -4096,
                     -129, -128, -9, -8, -2, -1], np.int64)
    c = np.zeros((vals.size, 3), np.int32)
    c[:, axis] = vals.astype(np.int32)
    c[:, (axis + 1) % 3] = 5
    g = OracleGrid(c[::-1].copy())
    expect = np.argsort(np.argsort(vals.astype(np.int32).view(np.uint32)))
    assert np.array_equal(g.ijk_to_index(c), expect)


def test_axis_priority_between_tiles():
    # i is the most significant key field: a larger tile in i wins over any j, k.
    c = np.array([[4096, 0, 0], [0, 4096 * 5, 4096 * 7], [0, 4096, 0], [0, 0, 4096 * 9]], np.int32)
    g = OracleGrid(c)
    assert list(g.ijk_to_index(c)) == [3, 2, 1, 0]
    assert g.n_upper == 4


def test_counts_by_shifted_sets():
    # F, Lw, U = numbers of distinct c>>3, c>>7, c>>12 (arithmetic shifts partition Z the
    # same way as the logical shifts of the two's-complement pattern); sum of leaf
    # popcounts = N; consecutive leaf offsets differ by the leaf's popcount.
    c = workloads.random_coords(20000, -300, 300, seed=11)
    c = np.concatenate([c, c[:5000]])  # duplicates
    g = OracleGrid(c)
    u = np.unique(c, axis=0)
    assert g.n == u.shape[0]
    assert g.n_leaf == np.unique(u >> 3, axis=0).shape[0]
    assert g.n_lower == np.unique(u >> 7, axis=0).shape[0]
    assert g.n_upper == np.unique(u >> 12, axis=0).shape[0]
    t = g.topology()
    pc = _popcount64(t["leaf_mask"]).sum(axis=1)
    assert pc.sum() == g.n
    off = t["leaf_offset"].astype(np.int64)
    assert off[0] == 0 and np.array_equal(np.diff(off), pc[:-1])
    # child masks: one bit per child, first-child links consecutive
    assert _popcount64(t["lower_mask"]).sum() == g.n_leaf
    assert _popcount64(t["upper_mask"]).sum() == g.n_lower
    lf = t["lower_first"].astype(np.int64)
    assert lf[0] == 0 and np.array_equal(np.diff(lf), _popcount64(t["lower_mask"]).sum(axis=1)[:-1])
    uf = t["upper_first"].astype(np.int64)
    assert uf[0] == 0 and np.array_equal(np.diff(uf), _popcount64(t["upper_mask"]).sum(axis=1)[:-1])


# ----------------------------------------------------------------------------- invariants

def test_index_is_a_permutation_and_inverse_of_active_ijk():
    c = workloads.random_coords(30000, -2000, 2000, seed=3)
    c = np.concatenate([c, c[::7]])
    g = OracleGrid(c)
    idx = g.ijk_to_index(c)
    assert idx.min() >= 0
    assert np.array_equal(np.sort(np.unique(idx)), np.arange(g.n))
    act = g.active_ijk()
    assert np.array_equal(act[idx], c)  # duplicates map to the same row
    # non-members map to -1
    q = workloads.random_coords(5000, -2000, 2000, seed=4)
    s = set(map(tuple, c.tolist()))
    expect = np.array([0 if tuple(x) in s else -1 for x in q.tolist()])
    got = g.ijk_to_index(q)
    assert np.array_equal(got < 0, expect < 0)


def test_index_equals_mask_encoding():
    # The index of every voxel equals offset + prefix[w] + popcount(word & below) read from
    # the exported leaf records (the encoding carries the whole index).
    c = workloads.random_coords(4000, -40, 40, seed=5)
    g = OracleGrid(c)
    t = g.topology()
    act = g.active_ijk().astype(np.int64)
    leaf_of = {tuple(o): f for f, o in enumerate(t["leaf_origin"].tolist())}
    for r, (i, j, k) in enumerate(act.tolist()):
        f = leaf_of[(i & ~7, j & ~7, k & ~7)]
        w, b = i & 7, ((j & 7) << 3) | (k & 7)
        word = int(t["leaf_mask"][f, w])
        pre = (int(t["leaf_prefix"][f]) >> (9 * (w - 1))) & 511 if w else 0
        assert (word >> b) & 1
        assert int(t["leaf_offset"][f]) + pre + bin(word & ((1 << b) - 1)).count("1") == r


def test_empty_and_single():
    g = OracleGrid(np.zeros((0, 3), np.int32))
    assert (g.n, g.n_leaf, g.n_lower, g.n_upper) == (0, 0, 0, 0)
    assert g.kernel_map().shape == (27, 0)
    g = OracleGrid(np.array([[5, 5, 5]] * 10, np.int32))
    assert g.n == 1
    m = g.kernel_map()
    assert m[13, 0] == 0 and np.all(np.delete(m[:, 0], 13) == -1)


# ----------------------------------------------------------------------------- kernel map

def _brute_map(act: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    a = act.astype(np.int64)
    K, N = offsets.shape[0], a.shape[0]
    out = np.full((K, N), -1, np.int32)
    for o in range(K):
        tgt = a + offsets[o]
        eq = np.all(tgt[:, None, :] == a[None, :, :], axis=2)  # O(N^2)
        r, s = np.nonzero(eq)
        out[o, r] = s
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_kernel_map_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    # clustered signed points so that neighbours exist and leaves / tiles are crossed
    centres = rng.integers(-5000, 5000, size=(6, 3))
    c = np.concatenate([cc + rng.integers(-6, 7, size=(300, 3)) for cc in centres]).astype(np.int32)
    c = np.concatenate([c, np.array([[4095, 0, 0], [4096, 0, 0], [-1, -1, -1], [0, 0, 0]], np.int32)])
    g = OracleGrid(c)
    off = standard_offsets()
    assert np.array_equal(g.kernel_map(off), _brute_map(g.active_ijk(), off))
    # a non-standard offset list (5x5x5 corners and axes)
    off2 = np.array([[2, 0, 0], [-2, 0, 0], [0, 2, -2], [2, 2, 2], [-2, -2, -2], [0, 0, 0]], np.int32)
    assert np.array_equal(g.kernel_map(off2), _brute_map(g.active_ijk(), off2))


def test_kernel_map_symmetry_and_centre():
    c = workloads.shell_coords()
    g = OracleGrid(c)
    m, nb = g.kernel_map(with_mask=True)
    N = g.n
    assert np.array_equal(m[13], np.arange(N))
    for o in range(27):
        r = np.nonzero(m[o] >= 0)[0]
        assert np.array_equal(m[26 - o][m[o][r]], r)
    bits = ((m >= 0).astype(np.uint64) << np.arange(27, dtype=np.uint64)[:, None]).sum(axis=0)
    assert np.array_equal(nb.astype(np.uint64), bits)


def test_kernel_map_no_wraparound_at_int32_limits():
    c = np.array([[2**31 - 1, 0, 0], [-2**31, 0, 0], [0, 2**31 - 1, 0], [0, -2**31, 0]], np.int32)
    g = OracleGrid(c)
    m = g.kernel_map()
    assert np.all(np.delete(m, 13, axis=0) == -1)


# ----------------------------------------------------------------------------- convolution

def _dense_conv_masked(act: np.ndarray, feats: np.ndarray, w: np.ndarray) -> np.ndarray:
    """torch conv3d (float64, CPU) on a zero-filled dense volume, read at the active voxels.
    conv3d is a cross-correlation, so weight[co, ci, di+1, dj+1, dk+1] = W[o, ci, co]."""
    lo = act.min(axis=0) - 1
    ext = act.max(axis=0) - lo + 2
    cin, cout = w.shape[1], w.shape[2]
    vol = torch.zeros((1, cin, *ext.tolist()), dtype=torch.float64)
    loc = torch.from_numpy((act - lo).astype(np.int64))
    vol[0, :, loc[:, 0], loc[:, 1], loc[:, 2]] = torch.from_numpy(feats.astype(np.float64)).T
    wt = torch.from_numpy(w.astype(np.float64)).reshape(3, 3, 3, cin, cout).permute(4, 3, 0, 1, 2).contiguous()
    out = torch.nn.functional.conv3d(vol, wt, padding=1)
    return out[0, :, loc[:, 0], loc[:, 1], loc[:, 2]].T.numpy()


@pytest.mark.parametrize("case", ["random", "shell"])
def test_conv_matches_masked_dense_conv3d(case):
    if case == "random":
        c = workloads.random_coords(1500, -6, 9, seed=21)
        cin, cout = 5, 7
    else:
        c = workloads.shell_coords()  # the tiny workload at full size: 64^3, 8 -> 8
        cin, cout = 8, 8
    g = OracleGrid(c)
    rng = np.random.default_rng(22)
    f = rng.standard_normal((g.n, cin)).astype(np.float32)
    w = rng.standard_normal((27, cin, cout)).astype(np.float32)
    got = oracle.conv(g.kernel_map(), f, w)
    ref = _dense_conv_masked(g.active_ijk().astype(np.int64), f, w)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_conv_identity_shift_and_linearity():
    c = workloads.random_coords(3000, -20, 20, seed=31)
    g = OracleGrid(c)
    m = g.kernel_map()
    rng = np.random.default_rng(32)
    f = rng.standard_normal((g.n, 6)).astype(np.float32)
    eye = np.zeros((27, 6, 6), np.float32)
    eye[13] = np.eye(6)
    assert np.array_equal(oracle.conv(m, f, eye), f.astype(np.float64))
    # single-offset kernel = neighbour gather times W[o]
    o = 5
    w = np.zeros((27, 6, 4), np.float32)
    w[o] = rng.standard_normal((6, 4))
    valid = m[o] >= 0
    expect = np.zeros((g.n, 4))
    expect[valid] = f[m[o][valid]].astype(np.float64) @ w[o].astype(np.float64)
    assert np.allclose(oracle.conv(m, f, w), expect, rtol=0, atol=1e-12)
    # linear in W
    w1 = rng.standard_normal((27, 6, 4)).astype(np.float32)
    w2 = rng.standard_normal((27, 6, 4)).astype(np.float32)
    lhs = oracle.conv(m, f, w1) + oracle.conv(m, f, w2)
    rhs = oracle.conv(m, f, (w1.astype(np.float64) + w2).astype(np.float32))
    assert np.max(np.abs(lhs - rhs)) < 1e-5


def test_conv_sampled_rows_equal_full():
    c = workloads.random_coords(2000, -10, 10, seed=41)
    g = OracleGrid(c)
    m = g.kernel_map()
    rng = np.random.default_rng(42)
    f = rng.standard_normal((g.n, 3)).astype(np.float32)
    w = rng.standard_normal((27, 3, 5)).astype(np.float32)
    full = oracle.conv(m, f, w)
    rows = rng.choice(g.n, size=100, replace=False)
    assert np.array_equal(oracle.conv(m, f, w, rows=rows), full[rows])


def test_conv_rows_equals_conv():
    """conv_rows (neighbour lists of chosen rows) is the same definition as conv."""
    c = workloads.random_coords(3000, -12, 12, seed=21)
    g = oracle.OracleGrid(c)
    m = g.kernel_map()
    rng = np.random.default_rng(22)
    f = rng.standard_normal((g.n, 5)).astype(np.float32)
    w = rng.standard_normal((27, 5, 7)).astype(np.float32)
    rows = np.sort(rng.choice(g.n, 64, replace=False))
    nbrs = m[:, rows].T
    ref = oracle.conv(m, f, w, rows=rows)
    got = oracle.conv_rows(nbrs, {int(s): f[s] for s in np.unique(nbrs[nbrs >= 0])}, w)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- backward pass

def test_conv_gradients_match_autograd_of_masked_dense_conv3d():
    """dgrad and wgrad equal torch autograd (float64) of conv3d on the zero-filled dense volume,
    read at the active voxels: the loss sum(out * dY) over active outputs."""
    c = workloads.random_coords(900, -5, 7, seed=51)
    g = OracleGrid(c)
    act = g.active_ijk().astype(np.int64)
    rng = np.random.default_rng(52)
    cin, cout = 3, 4
    f = rng.standard_normal((g.n, cin)).astype(np.float32)
    w = rng.standard_normal((27, cin, cout)).astype(np.float32)
    dy = rng.standard_normal((g.n, cout)).astype(np.float32)
    lo = act.min(axis=0) - 1
    ext = act.max(axis=0) - lo + 2
    loc = torch.from_numpy(act - lo)
    x = torch.from_numpy(f.astype(np.float64)).requires_grad_(True)
    wt = torch.from_numpy(w.astype(np.float64)).requires_grad_(True)
    vol = torch.zeros((cin, *ext.tolist()), dtype=torch.float64)
    vol = vol.index_put((torch.arange(cin)[:, None], loc[:, 0][None], loc[:, 1][None], loc[:, 2][None]), x.T)
    k = wt.reshape(3, 3, 3, cin, cout).permute(4, 3, 0, 1, 2)
    out = torch.nn.functional.conv3d(vol[None], k, padding=1)[0]
    loss = (out[:, loc[:, 0], loc[:, 1], loc[:, 2]].T * torch.from_numpy(dy.astype(np.float64))).sum()
    loss.backward()
    m = g.kernel_map()
    dx = oracle.conv_dgrad(m, dy, w)
    dw = oracle.conv_wgrad(m, f, dy)
    assert np.max(np.abs(dx - x.grad.numpy())) <= 1e-12 * np.max(np.abs(dx))
    assert np.max(np.abs(dw - wt.grad.numpy())) <= 1e-12 * np.max(np.abs(dw))


def test_conv_gradients_on_row_subsets_match_autograd():
    """The row-restricted gradients: conv_dgrad(rows=R) equals the autograd input gradient at the
    rows R, and conv_wgrad(rows=R) equals the autograd weight gradient of a dY that is zero
    outside R (torch conv3d on the zero-filled dense volume, float64)."""
    c = workloads.random_coords(700, -4, 6, seed=53)
    g = OracleGrid(c)
    act = g.active_ijk().astype(np.int64)
    rng = np.random.default_rng(54)
    cin, cout = 3, 5
    f = rng.standard_normal((g.n, cin)).astype(np.float32)
    w = rng.standard_normal((27, cin, cout)).astype(np.float32)
    dy = rng.standard_normal((g.n, cout)).astype(np.float32)
    sel = np.sort(rng.choice(g.n, g.n // 3, replace=False))
    dy_sel = np.zeros_like(dy)
    dy_sel[sel] = dy[sel]
    lo = act.min(axis=0) - 1
    ext = act.max(axis=0) - lo + 2
    loc = torch.from_numpy(act - lo)

    def autograd(dy_used):
        x = torch.from_numpy(f.astype(np.float64)).requires_grad_(True)
        wt = torch.from_numpy(w.astype(np.float64)).requires_grad_(True)
        vol = torch.zeros((cin, *ext.tolist()), dtype=torch.float64)
        vol = vol.index_put((torch.arange(cin)[:, None], loc[:, 0][None], loc[:, 1][None], loc[:, 2][None]), x.T)
        k = wt.reshape(3, 3, 3, cin, cout).permute(4, 3, 0, 1, 2)
        out = torch.nn.functional.conv3d(vol[None], k, padding=1)[0]
        (out[:, loc[:, 0], loc[:, 1], loc[:, 2]].T * torch.from_numpy(dy_used.astype(np.float64))).sum().backward()
        return x.grad.numpy(), wt.grad.numpy()

    m = g.kernel_map()
    gx, _ = autograd(dy)
    _, gw_sel = autograd(dy_sel)
    dx = oracle.conv_dgrad(m, dy, w, rows=sel)
    dw = oracle.conv_wgrad(m, f, dy, rows=sel)
    assert dx.shape == (sel.shape[0], cin)
    assert np.max(np.abs(dx - gx[sel])) <= 1e-12 * np.max(np.abs(dx))
    assert np.max(np.abs(dw - gw_sel)) <= 1e-12 * np.max(np.abs(dw))


def test_conv_gradients_are_adjoints_of_the_forward():
    """<conv(x, W), dY> = <x, dgrad(dY, W)> = <W, wgrad(x, dY)>."""
    c = workloads.random_coords(4000, -15, 15, seed=61)
    g = OracleGrid(c)
    m = g.kernel_map()
    rng = np.random.default_rng(62)
    f = rng.standard_normal((g.n, 5)).astype(np.float32)
    w = rng.standard_normal((27, 5, 6)).astype(np.float32)
    dy = rng.standard_normal((g.n, 6)).astype(np.float32)
    lhs = float(np.sum(oracle.conv(m, f, w) * dy.astype(np.float64)))
    via_x = float(np.sum(f.astype(np.float64) * oracle.conv_dgrad(m, dy, w)))
    via_w = float(np.sum(w.astype(np.float64) * oracle.conv_wgrad(m, f, dy)))
    assert abs(lhs - via_x) <= 1e-10 * abs(lhs)
    assert abs(lhs - via_w) <= 1e-10 * abs(lhs)


# ----------------------------------------------------------------------------- strided / transposed grids

def _occupancy(act: np.ndarray, lo: np.ndarray, ext: np.ndarray) -> torch.Tensor:
    vol = torch.zeros((1, 1, *ext.tolist()), dtype=torch.float64)
    loc = torch.from_numpy((act - lo).astype(np.int64))
    vol[0, 0, loc[:, 0], loc[:, 1], loc[:, 2]] = 1.0
    return vol


def _coords_of(vol: torch.Tensor, shift: np.ndarray) -> set:
    nz = torch.nonzero(vol[0, 0] > 0).numpy()
    return {tuple(int(v) for v in (r + shift)) for r in nz}


@pytest.mark.parametrize("stride", [1, 2, 3])
def test_conv_grid_equals_dense_max_pool(stride):
    # Output y is active iff the 3x3x3 window centred on s*y holds an input: max_pool3d with
    # kernel 3, stride s and padding 1 over the occupancy, on coordinates >= 0.
    act = workloads.random_coords(900, 1, 17, seed=31 + stride)  # every output index is >= 0
    got = {tuple(r) for r in oracle.conv_grid_coords(act, stride).tolist()}
    ext = act.max(axis=0) + 2  # the pooled volume reaches every output
    occ = _occupancy(act, np.zeros(3, np.int64), ext)
    pooled = torch.nn.functional.max_pool3d(occ, kernel_size=3, stride=stride, padding=1)
    assert got == _coords_of(pooled, np.zeros(3, np.int64))


def test_conv_grid_brute_force_signed_and_anisotropic():
    act = workloads.random_coords(60, -9, 9, seed=35)
    s = np.array([2, 1, 3])
    got = {tuple(r) for r in oracle.conv_grid_coords(act, s).tolist()}
    inputs = {tuple(r) for r in act.tolist()}
    want = set()
    for y0 in range(-6, 7):
        for y1 in range(-11, 12):
            for y2 in range(-5, 6):
                if any((s[0] * y0 + a, s[1] * y1 + b, s[2] * y2 + c) in inputs
                       for a in (-1, 0, 1) for b in (-1, 0, 1) for c in (-1, 0, 1)):
                    want.add((y0, y1, y2))
    assert got == want


def test_conv_transpose_grid_equals_dense_transposed_conv():
    # y = 2x + d: conv_transpose3d of the occupancy with a 3^3 box of ones, stride 2, padding 1.
    act = workloads.random_coords(700, 1, 15, seed=37)
    got = {tuple(r) for r in oracle.conv_grid_coords(act, 2, transposed=True).tolist()}
    ext = act.max(axis=0) + 1
    occ = _occupancy(act, np.zeros(3, np.int64), ext)
    ones = torch.ones((1, 1, 3, 3, 3), dtype=torch.float64)
    up = torch.nn.functional.conv_transpose3d(occ, ones, stride=2, padding=1, output_padding=1)
    assert got == _coords_of(up, np.zeros(3, np.int64))


def _strided_case(seed, transposed):
    act = workloads.random_coords(800, 1, 15, seed=seed)
    gi = OracleGrid(act)
    go = OracleGrid(oracle.conv_grid_coords(gi.active_ijk(), 2, transposed=transposed))
    m = oracle.conv_map_between(go, gi, 2, transposed=transposed)
    return gi, go, m


def test_conv_map_between_brute_force():
    for transposed in (False, True):
        gi, go, m = _strided_case(41, transposed)
        xin = {tuple(r): i for i, r in enumerate(gi.active_ijk().tolist())}
        y = go.active_ijk().astype(np.int64)
        offs = standard_offsets().astype(np.int64)
        for r in range(0, y.shape[0], 7):
            for o, d in enumerate(offs):
                if transposed:
                    z = y[r] - d
                    q = tuple((z // 2).tolist()) if np.all(z % 2 == 0) else None
                else:
                    q = tuple((2 * y[r] + d).tolist())
                assert m[o, r] == (xin.get(q, -1) if q is not None else -1)


def test_strided_conv_matches_dense_conv3d():
    gi, go, m = _strided_case(43, False)
    cin, cout = 4, 6
    rng = np.random.default_rng(44)
    f = rng.standard_normal((gi.n, cin)).astype(np.float32)
    w = rng.standard_normal((27, cin, cout)).astype(np.float32)
    got = oracle.conv(m, f, w)
    xi = gi.active_ijk().astype(np.int64)
    ext = xi.max(axis=0) + 2
    vol = torch.zeros((1, cin, *ext.tolist()), dtype=torch.float64)
    vol[0, :, xi[:, 0], xi[:, 1], xi[:, 2]] = torch.from_numpy(f.astype(np.float64)).T
    wt = torch.from_numpy(w.astype(np.float64)).reshape(3, 3, 3, cin, cout).permute(4, 3, 0, 1, 2).contiguous()
    dense = torch.nn.functional.conv3d(vol, wt, stride=2, padding=1)
    y = go.active_ijk().astype(np.int64)
    want = dense[0, :, y[:, 0], y[:, 1], y[:, 2]].T.numpy()
    assert np.max(np.abs(got - want)) < 1e-9 * max(1.0, np.max(np.abs(want)))


def test_transposed_conv_matches_dense_conv_transpose3d():
    gi, go, m = _strided_case(45, True)
    cin, cout = 5, 3
    rng = np.random.default_rng(46)
    f = rng.standard_normal((gi.n, cin)).astype(np.float32)
    w = rng.standard_normal((27, cin, cout)).astype(np.float32)
    got = oracle.conv(m, f, w)
    xi = gi.active_ijk().astype(np.int64)
    ext = xi.max(axis=0) + 1
    vol = torch.zeros((1, cin, *ext.tolist()), dtype=torch.float64)
    vol[0, :, xi[:, 0], xi[:, 1], xi[:, 2]] = torch.from_numpy(f.astype(np.float64)).T
    # conv_transpose3d: out[y] += in[x] w[ci, co, k] for y = 2x - 1 + k, i.e. d = k - 1.
    wt = torch.from_numpy(w.astype(np.float64)).reshape(3, 3, 3, cin, cout).permute(3, 4, 0, 1, 2).contiguous()
    dense = torch.nn.functional.conv_transpose3d(vol, wt, stride=2, padding=1, output_padding=1)
    y = go.active_ijk().astype(np.int64)
    want = dense[0, :, y[:, 0], y[:, 1], y[:, 2]].T.numpy()
    assert np.max(np.abs(got - want)) < 1e-9 * max(1.0, np.max(np.abs(want)))


def test_transposed_conv_is_adjoint_of_strided_conv():
    # <Y, S X> = <T Y, X> where S is the stride-2 conv with W and T the transposed conv of the
    # output grid with W[o]^T, read at the input grid's voxels (T's grid contains them).
    act = workloads.random_coords(600, -8, 8, seed=47)
    gx = OracleGrid(act)
    gy = OracleGrid(oracle.conv_grid_coords(gx.active_ijk(), 2))
    gt = OracleGrid(oracle.conv_grid_coords(gy.active_ijk(), 2, transposed=True))
    cin, cout = 3, 4
    rng = np.random.default_rng(48)
    X = rng.standard_normal((gx.n, cin)).astype(np.float32)
    Y = rng.standard_normal((gy.n, cout)).astype(np.float32)
    w = rng.standard_normal((27, cin, cout)).astype(np.float32)
    SX = oracle.conv(oracle.conv_map_between(gy, gx, 2), X, w)
    TY = oracle.conv(oracle.conv_map_between(gt, gy, 2, transposed=True), Y, np.ascontiguousarray(w.transpose(0, 2, 1)))
    rows = gt.ijk_to_index(gx.active_ijk())
    assert np.all(rows >= 0)
    lhs = float(np.sum(Y.astype(np.float64) * SX))
    rhs = float(np.sum(TY[rows] * X.astype(np.float64)))
    assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(lhs))
