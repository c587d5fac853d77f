"""ctypes loader for libigconv.so. Fails loudly when the library is missing: there is no
fallback implementation of any operation."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libigconv.so")
TUNING_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "igconv_tuning.txt")

EXPORTS = (
    "igc_grid_build", "igc_grid_destroy", "igc_grid_info", "igc_release_memory", "igc_grid_active_ijk",
    "igc_grid_ijk_to_index", "igc_grid_export", "igc_kernel_map", "igc_sparse_conv", "igc_sparse_conv_noalloc", "igc_tuning_load",
    "igc_sparse_conv_backward", "igc_conv_grid", "igc_conv_grid_chain", "igc_conv_map", "igc_sparse_conv_between", "igc_select_path",
    "igc_last_error",
)

STATUS = {
    0: "IGC_OK", 1: "IGC_ERR_INVALID_ARG", 2: "IGC_ERR_UNSUPPORTED", 3: "IGC_ERR_OOM",
    4: "IGC_ERR_HIP", 5: "IGC_ERR_RANGE", 6: "IGC_ERR_CAPACITY", 7: "IGC_ERR_INTERNAL",
}


class GridInfo(ctypes.Structure):
    _fields_ = [
        ("n_input", ctypes.c_int64), ("n_voxels", ctypes.c_int64), ("n_leaf", ctypes.c_int64),
        ("n_lower", ctypes.c_int64), ("n_upper", ctypes.c_int64), ("topology_bytes", ctypes.c_int64),
        ("sort_passes", ctypes.c_int32), ("root_capacity", ctypes.c_int32), ("host_syncs", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


# igc_allocator: stream-ordered device memory provider (include/igconv.h).
ALLOC_FN = ctypes.CFUNCTYPE(ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p)
RELEASE_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p)


class Allocator(ctypes.Structure):
    _fields_ = [("alloc", ALLOC_FN), ("release", RELEASE_FN), ("ctx", ctypes.c_void_p)]


class TopologyHost(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "root_key", "upper_origin", "upper_mask", "upper_first", "lower_origin", "lower_mask",
        "lower_first", "leaf_origin", "leaf_mask", "leaf_offset", "leaf_prefix")]


class IgcError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libigconv.so not found at {LIB_PATH}; build it with `python -m sparse_convolution_amd.build` "
            "(hipcc, gfx950). There is no non-HIP fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    sig = {
        "igc_grid_build": [P, i64, ctypes.POINTER(Allocator), P, ctypes.POINTER(P)],
        "igc_grid_destroy": [P],
        "igc_grid_info": [P, ctypes.POINTER(GridInfo)],
        "igc_release_memory": [],
        "igc_grid_active_ijk": [P, P, P],
        "igc_grid_ijk_to_index": [P, P, i64, P, P],
        "igc_grid_export": [P, ctypes.POINTER(TopologyHost)],
        "igc_kernel_map": [P, P, i32, P, P, P],
        "igc_sparse_conv": [P, P, P, i32, i32, P, i32, P, i32, P],
        "igc_sparse_conv_noalloc": [P, P, P, i32, i32, P, i32, P, i32, P],
        "igc_tuning_load": [ctypes.c_char_p],
        "igc_sparse_conv_backward": [P, P, P, i32, i32, P, i32, P, P, P, i32, P],
        "igc_conv_grid": [P, P, i32, ctypes.POINTER(Allocator), P, ctypes.POINTER(P)],
        "igc_conv_grid_chain": [P, i32, P, P, ctypes.POINTER(Allocator), P, ctypes.POINTER(P)],
        "igc_conv_map": [P, P, P, i32, P, P],
        "igc_sparse_conv_between": [P, P, i64, P, i32, i32, P, i32, P, P],
        "igc_select_path": [P, i32, i32, i32, ctypes.POINTER(i32)],
        "igc_last_error": [],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "igc_last_error" else ctypes.c_int
    _lib = lib
    # The measured per-layer row-order selection shipped with the package (igc_tuning_load).
    if os.path.exists(TUNING_PATH) and lib.igc_tuning_load(TUNING_PATH.encode()) != 0:
        raise IgcError(1, lib.igc_last_error().decode(errors="replace"))
    return lib


def check(status: int) -> None:
    if status != 0:
        msg = load().igc_last_error().decode(errors="replace")
        raise IgcError(status, msg)
