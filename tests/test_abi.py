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
    assert lib.igc_grid_build(None, 3, None, None, ctypes.byref(h)) == 1
    assert b"d_ijk" in lib.igc_last_error()
    assert lib.igc_grid_build(None, -1, None, None, ctypes.byref(h)) == 1
    assert lib.igc_grid_build(ctypes.c_void_p(16), 1 << 40, None, None, ctypes.byref(h)) == 5
    assert lib.igc_grid_build(None, 0, None, None, None) == 1
    assert lib.igc_kernel_map(None, None, 27, None, None, None) == 1
    assert lib.igc_sparse_conv(None, None, None, 0, 8, None, 8, None, 0, None) == 1
    assert lib.igc_grid_destroy(None) == 0
    assert lib.igc_grid_info(None, None) == 1
    assert lib.igc_last_error() != b""


class _CountingAllocator:
    """A host-side stand-in for a device memory provider: hands out addresses of a host buffer
    (an empty build never touches them), fails from the `fail_at`-th request on, and records
    every request and release."""

    def __init__(self, fail_at=None):
        from sparse_convolution_amd import _lib as L
        self.buf = ctypes.create_string_buffer(1 << 16)
        self.fail_at = fail_at
        self.allocs, self.releases = [], []
        self._a = L.ALLOC_FN(self._alloc)
        self._r = L.RELEASE_FN(self._release)
        self.struct = L.Allocator(self._a, self._r, None)

    def _alloc(self, ctx, nbytes, stream):
        if self.fail_at is not None and len(self.allocs) + 1 >= self.fail_at:
            self.allocs.append(None)
            return None
        base = ctypes.addressof(self.buf)
        p = (base + 255) // 256 * 256 + 256 * len(self.allocs)
        self.allocs.append((p, nbytes))
        return p

    def _release(self, ctx, ptr, nbytes, stream):
        self.releases.append((ptr, nbytes))


def test_allocator_provides_and_takes_back_the_grid_block():
    # An empty grid does no device work, so the allocator path runs without a GPU: the grid's
    # block comes from the caller's allocator and goes back to it at destroy, once.
    lib = _lib()
    a = _CountingAllocator()
    h = ctypes.c_void_p()
    assert lib.igc_grid_build(None, 0, ctypes.byref(a.struct), None, ctypes.byref(h)) == 0
    assert len(a.allocs) == 1 and a.allocs[0][1] >= 1 and a.allocs[0][0] % 256 == 0
    from sparse_convolution_amd import _lib as L
    info = L.GridInfo()
    assert lib.igc_grid_info(h, ctypes.byref(info)) == 0
    assert info.n_voxels == 0 and info.n_input == 0 and info.topology_bytes == a.allocs[0][1]
    assert a.releases == []
    assert lib.igc_grid_destroy(h) == 0
    assert a.releases == [a.allocs[0]]


def test_allocator_failure_is_reported_and_nothing_leaks():
    lib = _lib()
    a = _CountingAllocator(fail_at=1)
    h = ctypes.c_void_p(1234)
    assert lib.igc_grid_build(None, 0, ctypes.byref(a.struct), None, ctypes.byref(h)) == 3  # IGC_ERR_OOM
    msg = lib.igc_last_error()
    assert b"igc_grid_build" in msg and b"allocator" in msg
    assert not h.value  # no grid
    assert a.releases == []  # the failed request returned nothing to give back


def test_allocator_without_both_functions_is_rejected():
    from sparse_convolution_amd import _lib as L
    lib = _lib()
    half = L.Allocator(L.ALLOC_FN(lambda c, n, s: None), ctypes.cast(None, L.RELEASE_FN), None)
    h = ctypes.c_void_p()
    assert lib.igc_grid_build(None, 0, ctypes.byref(half), None, ctypes.byref(h)) == 1
    assert b"allocator" in lib.igc_last_error()


def test_tuning_file_is_parsed_on_the_host(tmp_path):
    lib = _lib()
    good = tmp_path / "good.txt"
    good.write_text("# comment " + "x" * 3000 + "\n\nggs 128 * 0 0.1 4096 class  # lidar-like\nggs 64 64 0 1 256 class 64\n"
                    "ggs 64 128 0 1 256 class 128k32\nggs 96 64 0 1 1024 natural 64k32\n"
                    "ggs 128 128 0 1 256 class 128h\nggs 64 64 0 1 256 natural 64k32h\n"
                    "ggs * * 0 1e30 256 natural auto\n")
    assert lib.igc_tuning_load(str(good).encode()) == 0
    for bad_line in ("ggs 128 128 0 1 512 class\n", "ggs 128 128 0 1 256 sideways\n", "conv 1 1 0 1 256 natural\n",
                     "ggs 128 128 0.5 0.1 256 natural\n", "ggs 128 128 0 1\n", "ggs 128 128 0 1 256 class 32\n",
                     "ggs 128 128 0 1 256 class 256k32\n", "ggs 128 128 0 1 256 class 64k16\n",
                     "ggs 128 128 0 1 256 class k32\n", "ggs 128 128 0 1 256 class 64k32x\n",
                     "ggs 128 128 0 1 256 class 256h\n", "ggs 128 128 0 1 256 class autoh\n",
                     "ggs 128 128 0 1 256 class 64hk32\n", "ggs 128 128 0 1 256 class h\n"):
        bad = tmp_path / "bad.txt"
        bad.write_text(bad_line)
        assert lib.igc_tuning_load(str(bad).encode()) == 1, bad_line
        assert b"igc_tuning_load" in lib.igc_last_error()
    assert lib.igc_tuning_load(str(tmp_path / "missing.txt").encode()) == 1
    assert lib.igc_tuning_load(None) == 0
    from sparse_convolution_amd import _lib as L
    if os.path.exists(L.TUNING_PATH):  # the shipped table parses
        assert lib.igc_tuning_load(L.TUNING_PATH.encode()) == 0
