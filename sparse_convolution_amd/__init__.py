"""MI355X-native IndexGrid build, neighbour map and submanifold sparse convolution.

Thin Python binding over libigconv (include/igconv.h): it checks tensor shapes, dtypes and
devices, and passes raw device pointers and the current HIP stream to the C ABI. All device
work runs in the library's HIP kernels; torch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import IgcError

__all__ = [
    "Grid", "grid_build", "kernel_map", "sparse_conv", "sparse_conv_backward", "conv_grid", "conv_grid_chain", "conv_map",
    "sparse_conv_between", "standard_offsets", "release_memory", "tuning_load", "IgcError",
    "PATH_AUTO", "PATH_LEAF", "PATH_GGS", "PATH_GATHER",
]

F32, BF16 = 0, 1
PATH_AUTO, PATH_LEAF, PATH_GGS, PATH_MIXED, PATH_GATHER = 0, 1, 2, 3, 4
_PATHS = {"auto": PATH_AUTO, "leaf": PATH_LEAF, "ggs": PATH_GGS, "mixed": PATH_MIXED, "gather": PATH_GATHER}


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p | None:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _device_tensor(t: torch.Tensor, name: str, dtype: torch.dtype, cols: int | None = None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if cols is not None and (t.dim() != 2 or t.shape[1] != cols):
        raise ValueError(f"{name} must have shape [n, {cols}], got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def standard_offsets() -> np.ndarray:
    """The 27 offsets of a 3x3x3 kernel in the order o = (di+1)*9 + (dj+1)*3 + (dk+1)."""
    d = np.array([-1, 0, 1], dtype=np.int32)
    di, dj, dk = np.meshgrid(d, d, d, indexing="ij")
    return np.ascontiguousarray(np.stack([di.ravel(), dj.ravel(), dk.ravel()], axis=1))


# PyTorch's caching allocator as the library's memory provider (igc_allocator): the grid's
# block and every call's temporaries are torch allocations on the call's stream.
def _torch_alloc(ctx, nbytes, stream):
    try:
        return torch.cuda.caching_allocator_alloc(int(nbytes), torch.cuda.current_device(), int(stream or 0))
    except Exception:  # reported by the library as IGC_ERR_OOM
        return None


def _torch_release(ctx, ptr, nbytes, stream):
    try:
        torch.cuda.caching_allocator_delete(ptr)
    except Exception:
        pass


_TORCH_ALLOC_CB = _lib.ALLOC_FN(_torch_alloc)
_TORCH_RELEASE_CB = _lib.RELEASE_FN(_torch_release)
TORCH_ALLOCATOR = _lib.Allocator(_TORCH_ALLOC_CB, _TORCH_RELEASE_CB, None)


def _allocator(memory: str):
    if memory == "torch":
        return ctypes.byref(TORCH_ALLOCATOR)
    if memory == "library":
        return None
    raise ValueError("memory must be 'torch' (PyTorch's caching allocator) or 'library' (the library's pool)")


def release_memory() -> None:
    """Returns the library's own cached device memory (igc_release_memory)."""
    _lib.check(_lib.load().igc_release_memory())


class Grid:
    """An immutable IndexGrid on one GPU (igc_grid_build)."""

    def __init__(self, handle: ctypes.c_void_p, device: torch.device):
        self._h = handle
        self.device = device
        info = _lib.GridInfo()
        _lib.check(_lib.load().igc_grid_info(self._h, ctypes.byref(info)))
        self.n_input = info.n_input
        self.n_voxels = info.n_voxels
        self.n_leaf = info.n_leaf
        self.n_lower = info.n_lower
        self.n_upper = info.n_upper
        self.topology_bytes = info.topology_bytes
        self.sort_passes = info.sort_passes
        self.host_syncs = info.host_syncs
        self.root_capacity = info.root_capacity

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            try:
                _lib.load().igc_grid_destroy(h)
            except Exception:
                pass
            self._h = None

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    @property
    def leaf_occupancy(self) -> float:
        return self.n_voxels / (512.0 * self.n_leaf) if self.n_leaf else 0.0

    def active_ijk(self) -> torch.Tensor:
        out = torch.empty((self.n_voxels, 3), dtype=torch.int32, device=self.device)
        _lib.check(_lib.load().igc_grid_active_ijk(self._h, _ptr(out), _stream(self.device)))
        return out

    def ijk_to_index(self, q: torch.Tensor) -> torch.Tensor:
        q = _device_tensor(q, "q", torch.int32, 3)
        out = torch.empty(q.shape[0], dtype=torch.int32, device=self.device)
        _lib.check(_lib.load().igc_grid_ijk_to_index(self._h, _ptr(q), q.shape[0], _ptr(out),
                                                      _stream(self.device)))
        return out

    def export(self) -> dict:
        """Topology copied to host numpy arrays (igc_grid_export)."""
        U, L, F = self.n_upper, self.n_lower, self.n_leaf
        t = {
            "root_key": np.zeros(U, np.uint64), "upper_origin": np.zeros((U, 3), np.int32),
            "upper_mask": np.zeros((U, 512), np.uint64), "upper_first": np.zeros(U, np.uint32),
            "lower_origin": np.zeros((L, 3), np.int32), "lower_mask": np.zeros((L, 64), np.uint64),
            "lower_first": np.zeros(L, np.uint32), "leaf_origin": np.zeros((F, 3), np.int32),
            "leaf_mask": np.zeros((F, 8), np.uint64), "leaf_offset": np.zeros(F, np.uint64),
            "leaf_prefix": np.zeros(F, np.uint64),
        }
        th = _lib.TopologyHost(**{k: v.ctypes.data_as(ctypes.c_void_p) for k, v in t.items()})
        _lib.check(_lib.load().igc_grid_export(self._h, ctypes.byref(th)))
        return t

    def select_path(self, dtype: torch.dtype, cin: int, cout: int) -> str:
        p = ctypes.c_int32(0)
        _lib.check(_lib.load().igc_select_path(self._h, _dtype_code(dtype), cin, cout, ctypes.byref(p)))
        return {PATH_LEAF: "leaf", PATH_GGS: "ggs", PATH_GATHER: "gather"}[p.value]


def _dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return F32
    if dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {dtype}")


def grid_build(ijk: torch.Tensor, memory: str = "torch") -> Grid:
    """IndexGrid from int32[n, 3] device coordinates (any order, duplicates allowed). Its device
    memory, and that of every later call on it, comes from PyTorch's caching allocator
    (memory="torch") or from the library's own pool (memory="library")."""
    ijk = _device_tensor(ijk, "ijk", torch.int32, 3)
    h = ctypes.c_void_p()
    _lib.check(_lib.load().igc_grid_build(_ptr(ijk), ijk.shape[0], _allocator(memory), _stream(ijk.device),
                                          ctypes.byref(h)))
    return Grid(h, ijk.device)


_STD_OFFSETS = standard_offsets()
_STD_OFFSETS_PTR = _STD_OFFSETS.ctypes.data_as(ctypes.c_void_p)


def kernel_map(grid: Grid, offsets: np.ndarray | None = None, with_mask: bool = False):
    """Neighbour map int32[K, N] (and optionally the uint32[N] neighbour bit masks, stored
    in an int32 tensor)."""
    if offsets is None:
        off, off_ptr = _STD_OFFSETS, _STD_OFFSETS_PTR
    else:
        off = np.ascontiguousarray(offsets, dtype=np.int32).reshape(-1, 3)
        off_ptr = off.ctypes.data_as(ctypes.c_void_p)
    K = off.shape[0]
    m = torch.empty((K, grid.n_voxels), dtype=torch.int32, device=grid.device)
    nb = torch.empty(grid.n_voxels, dtype=torch.int32, device=grid.device) if with_mask else None
    _lib.check(_lib.load().igc_kernel_map(grid.handle, off_ptr, K, _ptr(m), _ptr(nb), _stream(grid.device)))
    return (m, nb) if with_mask else m


def sparse_conv(grid: Grid, feats: torch.Tensor, weights: torch.Tensor, kmap: torch.Tensor | None = None,
                path: str = "auto", out: torch.Tensor | None = None) -> torch.Tensor:
    """3x3x3 submanifold convolution: feats [N, cin], weights [27, cin, cout] -> [N, cout]."""
    dt = feats.dtype
    cin = feats.shape[1] if feats.dim() == 2 else -1
    feats = _device_tensor(feats, "feats", dt, cin)
    if feats.shape[0] != grid.n_voxels:
        raise ValueError(f"feats has {feats.shape[0]} rows, grid has {grid.n_voxels} voxels")
    if weights.dim() != 3 or weights.shape[0] != 27 or weights.shape[1] != cin:
        raise ValueError(f"weights must have shape [27, {cin}, cout], got {tuple(weights.shape)}")
    weights = _device_tensor(weights, "weights", dt)
    cout = weights.shape[2]
    if kmap is not None:
        kmap = _device_tensor(kmap, "kmap", torch.int32)
        if tuple(kmap.shape) != (27, grid.n_voxels):
            raise ValueError(f"kmap must have shape [27, {grid.n_voxels}]")
    if out is None:
        out = torch.empty((grid.n_voxels, cout), dtype=dt, device=grid.device)
    else:
        out = _device_tensor(out, "out", dt, cout)
    _lib.check(_lib.load().igc_sparse_conv(grid.handle, _ptr(kmap), _ptr(feats), _dtype_code(dt), cin,
                                           _ptr(weights), cout, _ptr(out), _PATHS[path], _stream(grid.device)))
    return out


def sparse_conv_backward(grid: Grid, feats: torch.Tensor, weights: torch.Tensor, dout: torch.Tensor,
                         kmap: torch.Tensor, path: str = "auto", need_dfeats: bool = True,
                         need_dweights: bool = True):
    """Gradients of sparse_conv: (dfeats [N, cin] of feats' dtype or None, dweights [27, cin, cout]
    float32 or None) for the output gradient dout [N, cout]."""
    dt = feats.dtype
    cin = feats.shape[1] if feats.dim() == 2 else -1
    feats = _device_tensor(feats, "feats", dt, cin)
    if weights.dim() != 3 or weights.shape[0] != 27 or weights.shape[1] != cin:
        raise ValueError(f"weights must have shape [27, {cin}, cout], got {tuple(weights.shape)}")
    weights = _device_tensor(weights, "weights", dt)
    cout = weights.shape[2]
    dout = _device_tensor(dout, "dout", dt, cout)
    kmap = _device_tensor(kmap, "kmap", torch.int32)
    if tuple(kmap.shape) != (27, grid.n_voxels) or feats.shape[0] != grid.n_voxels or dout.shape[0] != grid.n_voxels:
        raise ValueError("feats, dout and kmap must cover the grid's voxels")
    dx = torch.empty((grid.n_voxels, cin), dtype=dt, device=grid.device) if need_dfeats else None
    dw = torch.empty((27, cin, cout), dtype=torch.float32, device=grid.device) if need_dweights else None
    _lib.check(_lib.load().igc_sparse_conv_backward(grid.handle, _ptr(kmap), _ptr(feats), _dtype_code(dt), cin,
                                                    _ptr(weights), cout, _ptr(dout), _ptr(dx), _ptr(dw),
                                                    _PATHS[path], _stream(grid.device)))
    return dx, dw


def _stride_array(stride) -> np.ndarray:
    s = np.broadcast_to(np.asarray(stride, dtype=np.int32), (3,))
    return np.ascontiguousarray(s)


def conv_grid(grid: Grid, stride=2, transposed: bool = False, memory: str = "torch") -> Grid:
    """Output grid of a 3x3x3 convolution with the given stride (int or 3 ints, each 1..3) over
    `grid`, or of the transposed convolution (igc_conv_grid); memory as for grid_build."""
    s = _stride_array(stride)
    h = ctypes.c_void_p()
    _lib.check(_lib.load().igc_conv_grid(grid.handle, s.ctypes.data_as(ctypes.c_void_p), int(bool(transposed)),
                                         _allocator(memory), _stream(grid.device), ctypes.byref(h)))
    return Grid(h, grid.device)


def conv_grid_chain(grid: Grid, strides, transposed=None, memory: str = "torch") -> list:
    """Output grids of a chain of 3x3x3 convolutions (stage k over stage k-1's output), strides a
    list of ints or 3-int triples, transposed a list of bools (None: none), built with the
    counts on the device and one synchronisation (igc_conv_grid_chain)."""
    st = np.ascontiguousarray(np.stack([_stride_array(x) for x in strides]), dtype=np.int32)
    n = st.shape[0]
    tr = np.zeros(n, dtype=np.int32) if transposed is None else np.asarray([int(bool(t)) for t in transposed],
                                                                           dtype=np.int32)
    if tr.shape[0] != n:
        raise ValueError("transposed must have one entry per stage")
    hs = (ctypes.c_void_p * n)()
    _lib.check(_lib.load().igc_conv_grid_chain(grid.handle, n, st.ctypes.data_as(ctypes.c_void_p),
                                               tr.ctypes.data_as(ctypes.c_void_p), _allocator(memory),
                                               _stream(grid.device), hs))
    return [Grid(ctypes.c_void_p(hs[k]), grid.device) for k in range(n)]


def tuning_load(path) -> None:
    """Replaces the per-layer row-order table of the gather-GEMM-scatter path (igc_tuning_load);
    None clears it. The package's measured table (igconv_tuning.txt) is loaded with the library."""
    _lib.check(_lib.load().igc_tuning_load(None if path is None else str(path).encode()))


def conv_map(in_grid: Grid, out_grid: Grid, stride=2, transposed: bool = False) -> torch.Tensor:
    """Neighbour map int32[27, N_out] from out_grid's rows to in_grid's rows (igc_conv_map)."""
    s = _stride_array(stride)
    m = torch.empty((27, out_grid.n_voxels), dtype=torch.int32, device=out_grid.device)
    _lib.check(_lib.load().igc_conv_map(in_grid.handle, out_grid.handle, s.ctypes.data_as(ctypes.c_void_p),
                                        int(bool(transposed)), _ptr(m), _stream(out_grid.device)))
    return m


def sparse_conv_between(out_grid: Grid, feats: torch.Tensor, weights: torch.Tensor, kmap: torch.Tensor,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """Convolution from an input grid's features [N_in, cin] to out_grid's rows through kmap
    (from conv_map); weights [27, cin, cout] (igc_sparse_conv_between)."""
    dt = feats.dtype
    cin = feats.shape[1] if feats.dim() == 2 else -1
    feats = _device_tensor(feats, "feats", dt, cin)
    if weights.dim() != 3 or weights.shape[0] != 27 or weights.shape[1] != cin:
        raise ValueError(f"weights must have shape [27, {cin}, cout], got {tuple(weights.shape)}")
    weights = _device_tensor(weights, "weights", dt)
    cout = weights.shape[2]
    kmap = _device_tensor(kmap, "kmap", torch.int32)
    if tuple(kmap.shape) != (27, out_grid.n_voxels):
        raise ValueError(f"kmap must have shape [27, {out_grid.n_voxels}]")
    if out is None:
        out = torch.empty((out_grid.n_voxels, cout), dtype=dt, device=out_grid.device)
    _lib.check(_lib.load().igc_sparse_conv_between(out_grid.handle, _ptr(kmap), feats.shape[0], _ptr(feats),
                                                   _dtype_code(dt), cin, _ptr(weights), cout, _ptr(out),
                                                   _stream(out_grid.device)))
    return out
