"""CPU oracle: ctypes wrapper over ``igc_oracle.cpp``.

TEST INFRASTRUCTURE ONLY. It may be imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library. It shares no code with the HIP path.

Each function cites the passage it follows (see ``igc_oracle.cpp`` for the definitions
and the readings taken where the pages are silent). All functions here are pinned by the
``-m "not gpu"`` tests in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "igc_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

__all__ = ["build_library", "OracleGrid", "kernel_map", "conv", "conv_rows", "conv_dgrad", "conv_wgrad",
           "conv_grid_candidates", "conv_grid_coords", "conv_map_between", "standard_offsets", "num_threads"]


def build_library(force: bool = True) -> str:
    """Compiles the oracle with g++ (-O2, OpenMP). Returns the library path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build_library(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int32
        lib.orc_build.restype = P
        lib.orc_build.argtypes = [P, i64]
        lib.orc_free.argtypes = [P]
        lib.orc_counts.argtypes = [P, P]
        lib.orc_export.argtypes = [P] * 12
        lib.orc_active_ijk.argtypes = [P, P]
        lib.orc_ijk_to_index.argtypes = [P, P, i64, P]
        lib.orc_kernel_map.argtypes = [P, P, i32, P, P]
        lib.orc_conv.argtypes = [P, i64, i32, P, i32, P, i32, P, i64, P]
        lib.orc_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def standard_offsets() -> np.ndarray:
    """The 27 offsets of a 3x3x3 kernel, o = (di+1)*9 + (dj+1)*3 + (dk+1)."""
    d = np.array([-1, 0, 1], dtype=np.int32)
    di, dj, dk = np.meshgrid(d, d, d, indexing="ij")
    return np.ascontiguousarray(np.stack([di.ravel(), dj.ravel(), dk.ravel()], axis=1))


def num_threads() -> int:
    return int(_load().orc_num_threads())


class OracleGrid:
    """IndexGrid built on the CPU from int32[n,3] coordinates (fVDB notes: "IndexGrid" and
    "GPU-accelerated IndexGrid build" sections; the order and encoding are defined in
    igc_oracle.cpp)."""

    def __init__(self, coords: np.ndarray):
        lib = _load()
        c = np.ascontiguousarray(coords, dtype=np.int32).reshape(-1, 3)
        self._keep = c
        h = lib.orc_build(_ptr(c), c.shape[0])
        if not h:
            raise ValueError("oracle build failed")
        self._h = h
        cnt = np.zeros(4, dtype=np.int64)
        lib.orc_counts(h, _ptr(cnt))
        self.n, self.n_leaf, self.n_lower, self.n_upper = (int(x) for x in cnt)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.orc_free(h)
            self._h = None

    def topology(self) -> dict:
        """Canonical topology arrays, keyed like the HIP library's export."""
        U, L, F = self.n_upper, self.n_lower, self.n_leaf
        t = {
            "root_key": np.zeros(U, np.uint64),
            "upper_origin": np.zeros((U, 3), np.int32),
            "upper_mask": np.zeros((U, 512), np.uint64),
            "upper_first": np.zeros(U, np.uint32),
            "lower_origin": np.zeros((L, 3), np.int32),
            "lower_mask": np.zeros((L, 64), np.uint64),
            "lower_first": np.zeros(L, np.uint32),
            "leaf_origin": np.zeros((F, 3), np.int32),
            "leaf_mask": np.zeros((F, 8), np.uint64),
            "leaf_offset": np.zeros(F, np.uint64),
            "leaf_prefix": np.zeros(F, np.uint64),
        }
        _load().orc_export(self._h, *[_ptr(t[k]) for k in (
            "root_key", "upper_origin", "upper_mask", "upper_first", "lower_origin", "lower_mask",
            "lower_first", "leaf_origin", "leaf_mask", "leaf_offset", "leaf_prefix")])
        return t

    def active_ijk(self) -> np.ndarray:
        out = np.zeros((self.n, 3), np.int32)
        _load().orc_active_ijk(self._h, _ptr(out))
        return out

    def ijk_to_index(self, q: np.ndarray) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.int32).reshape(-1, 3)
        out = np.zeros(q.shape[0], np.int32)
        _load().orc_ijk_to_index(self._h, _ptr(q), q.shape[0], _ptr(out))
        return out

    def kernel_map(self, offsets: np.ndarray | None = None, with_mask: bool = False):
        """Neighbour map int32[K, N] (DriveRT page, "Shared neighbour maps")."""
        off = standard_offsets() if offsets is None else np.ascontiguousarray(offsets, dtype=np.int32)
        K = off.shape[0]
        m = np.zeros((K, self.n), np.int32)
        nb = np.zeros(self.n, np.uint32) if with_mask else None
        _load().orc_kernel_map(self._h, _ptr(off), K, _ptr(m), _ptr(nb))
        return (m, nb) if with_mask else m


def kernel_map(grid: OracleGrid, offsets: np.ndarray | None = None):
    return grid.kernel_map(offsets)


def conv(kmap: np.ndarray, feats: np.ndarray, w: np.ndarray, rows: np.ndarray | None = None) -> np.ndarray:
    """Submanifold convolution in float64 over a neighbour map (fVDB notes, sparse-conv
    operators): out[r] = sum_o W[o]^T feats[map[o, r]] over map[o, r] >= 0.

    feats float32[N_in, cin] (bf16 inputs are passed as their exact float32 values; N_in = N
    for a map over one grid, the input grid's size for a map between two grids),
    w float32[K, cin, cout]; returns float64[len(rows) or N, cout].
    """
    kmap = np.ascontiguousarray(kmap, dtype=np.int32)
    K, N = kmap.shape
    f = np.ascontiguousarray(feats, dtype=np.float32)
    ww = np.ascontiguousarray(w, dtype=np.float32)
    cin, cout = ww.shape[1], ww.shape[2]
    assert f.ndim == 2 and f.shape[1] == cin and ww.shape[0] == K
    assert kmap.size == 0 or int(kmap.max()) < f.shape[0]
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = N if r is None else r.shape[0]
    out = np.zeros((R, cout), np.float64)
    _load().orc_conv(_ptr(kmap), N, K, _ptr(f), cin, _ptr(ww), cout, _ptr(r), R, _ptr(out))
    return out


def conv_rows(nbrs: np.ndarray, feats_of: dict, w: np.ndarray) -> np.ndarray:
    """The same submanifold convolution as ``conv`` for output rows given by their neighbour
    lists: out[i] = sum over o with nbrs[i, o] >= 0 of W[o]^T feats[nbrs[i, o]], in float64.

    nbrs int[R, K] (row i's entries of the kernel map), feats_of maps an input row to its
    float32[cin] features (only the rows nbrs refers to are needed), w float32[K, cin, cout].
    """
    nbrs = np.asarray(nbrs)
    ww = np.asarray(w, dtype=np.float64)
    out = np.zeros((nbrs.shape[0], ww.shape[2]), np.float64)
    for i in range(nbrs.shape[0]):
        for o in range(nbrs.shape[1]):
            s = int(nbrs[i, o])
            if s >= 0:
                out[i] += np.asarray(feats_of[s], dtype=np.float64) @ ww[o]
    return out


def conv_dgrad(kmap: np.ndarray, dout: np.ndarray, w: np.ndarray, rows: np.ndarray | None = None) -> np.ndarray:
    """Gradient of the submanifold convolution with respect to its input features, in float64:
    dX[s, ci] = sum over the pairs (o, r) with map[o, r] = s of sum_co dY[r, co] W[o, ci, co]
    (the convolution of the fVDB notes' sparse-conv operators differentiated term by term).

    kmap int32[K, N], dout float32[N, cout] (exact bf16 values for bf16 data),
    w float32[K, cin, cout]; returns float64[N, cin], or float64[len(rows), cin] for the input
    rows `rows` only (sorted, unique): then only the pairs whose input is one of them are summed."""
    kmap = np.asarray(kmap)
    dy = np.asarray(dout)
    ww = np.asarray(w, dtype=np.float64)
    if rows is None:
        dx = np.zeros((kmap.shape[1], ww.shape[1]), np.float64)
    else:
        rows = np.asarray(rows, dtype=np.int64)
        dx = np.zeros((rows.shape[0], ww.shape[1]), np.float64)
        wanted = np.zeros(kmap.shape[1], bool)
        wanted[rows] = True
    for o in range(kmap.shape[0]):
        valid = kmap[o] >= 0
        if rows is not None:
            valid[valid] = wanted[kmap[o][valid]]
        s = kmap[o][valid]
        np.add.at(dx, s if rows is None else np.searchsorted(rows, s), dy[valid].astype(np.float64) @ ww[o].T)
    return dx


def conv_wgrad(kmap: np.ndarray, feats: np.ndarray, dout: np.ndarray, rows: np.ndarray | None = None) -> np.ndarray:
    """Gradient of the submanifold convolution with respect to its weights, in float64:
    dW[o, ci, co] = sum over r with map[o, r] >= 0 of feats[map[o, r], ci] dY[r, co].

    kmap int32[K, N], feats float32[N, cin], dout float32[N, cout]; returns float64[K, cin, cout].
    With `rows` the sum runs over those output rows only (the gradient for a dY that is zero at
    every other row)."""
    kmap = np.asarray(kmap)
    f = np.asarray(feats)
    dy = np.asarray(dout)
    dw = np.zeros((kmap.shape[0], f.shape[1], dy.shape[1]), np.float64)
    r = np.arange(kmap.shape[1]) if rows is None else np.asarray(rows, dtype=np.int64)
    for o in range(kmap.shape[0]):
        src = kmap[o][r]
        valid = src >= 0
        dw[o] = f[src[valid]].astype(np.float64).T @ dy[r[valid]].astype(np.float64)
    return dw


def _stride3(stride) -> np.ndarray:
    s = np.broadcast_to(np.asarray(stride, dtype=np.int64), (3,)).copy()
    assert np.all(s >= 1)
    return s


def conv_grid_candidates(coords: np.ndarray, stride, transposed: bool = False) -> np.ndarray:
    """Every output coordinate of a 3x3x3 sparse convolution with the given stride, once per
    (input voxel, offset) that produces it, duplicates included (see conv_grid_coords for the
    definition). Offsets d run over {-1, 0, 1}^3. Returns int32[M, 3], input-major per offset;
    passing it to OracleGrid gives the output grid without a separate dedupe."""
    c = np.asarray(coords, dtype=np.int64).reshape(-1, 3)
    s = _stride3(stride)
    parts = []
    for d in standard_offsets().astype(np.int64):
        if transposed:
            parts.append((s * c + d).astype(np.int32))
        else:
            z = c - d
            ok = np.all(z % s == 0, axis=1)
            parts.append((z[ok] // s).astype(np.int32))
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, 3), np.int32)


def conv_grid_coords(coords: np.ndarray, stride, transposed: bool = False) -> np.ndarray:
    """Output coordinates of a 3x3x3 sparse convolution with the given stride (the grid-to-grid
    ops ConvGrid / ConvTransposeGrid in the op table of the "ONNX Runtime support for fVDB
    operations" proposal; the pages name them without a formula, so the plain reading is used).
    Offsets d run over {-1, 0, 1}^3.

    strided:    y is an output iff some input x has x = s * y + d (its receptive field holds
                an input voxel);
    transposed: y is an output iff y = s * x + d for some input x.
    Returns the unique coordinates, int32[M, 3], in lexicographic order."""
    cand = conv_grid_candidates(coords, stride, transposed)
    if cand.shape[0] == 0:
        return cand
    return np.unique(cand.astype(np.int64), axis=0).astype(np.int32)


def conv_map_between(out_grid: OracleGrid, in_grid: OracleGrid, stride, transposed: bool = False) -> np.ndarray:
    """Neighbour map int32[27, N_out] from the output grid's rows to the input grid's rows
    (DriveRT page, "Shared neighbour maps", for two coordinate domains):
    strided:    map[o, r] = in.index(s * y_r + d_o);
    transposed: map[o, r] = in.index((y_r - d_o) / s) where s divides y_r - d_o, else -1.
    o = (dx+1)*9 + (dy+1)*3 + (dz+1); -1 where the input voxel is absent."""
    y = out_grid.active_ijk().astype(np.int64)
    s = _stride3(stride)
    offs = standard_offsets().astype(np.int64)
    m = np.full((27, y.shape[0]), -1, np.int32)
    for o, d in enumerate(offs):
        if transposed:
            z = y - d
            ok = np.all(z % s == 0, axis=1)
            q = z // s
        else:
            q = s * y + d
            ok = np.ones(y.shape[0], bool)
        if np.any(ok):
            m[o, ok] = in_grid.ijk_to_index(q[ok].astype(np.int32))
    return m
