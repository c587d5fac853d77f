"""The C ABI library loads on the host and exports every function include/igconv.h declares;
host-side argument checks answer without touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "igconv.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(igc_\w+)\s*\(", src, flags=re.M)))


def _lib():
    from sparse_convolution_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libigconv.so is not built; run `python -m sparse_convolution_amd.build`")
    return _lib.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("igc_grid_build", "igc_kernel_map", "igc_sparse_conv", "igc_grid_destroy", "igc_last_error"):
        assert n in names
    from sparse_convolution_amd import _lib
    assert sorted(_lib.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_host_side_errors_without_gpu():
    lib = _lib()
    h = ctypes.c_void_p()
    assert lib.igc_grid_build(None, 3, None, ctypes.byref(h)) == 1
    assert b"d_ijk" in lib.igc_last_error()
    assert lib.igc_grid_build(None, -1, None, ctypes.byref(h)) == 1
    assert lib.igc_grid_build(ctypes.c_void_p(16), 1 << 40, None, ctypes.byref(h)) == 5
    assert lib.igc_grid_build(None, 0, None, None) == 1
    assert lib.igc_kernel_map(None, None, 27, None, None, None) == 1
    assert lib.igc_sparse_conv(None, None, None, 0, 8, None, 8, None, 0, None) == 1
    assert lib.igc_grid_destroy(None) == 0
    assert lib.igc_grid_get_info(None, None) == 1
    assert lib.igc_last_error() != b""
