"""Shared helpers of the GPU tests (not collected)."""
import os
import sys

import numpy as np
import pytest
import torch

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "sparse_convolution_amd",
                   "libigconv.so")


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(LIB):
        pytest.fail("libigconv.so is not built; run `python -m sparse_convolution_amd.build`")


def say(msg: str) -> None:
    """Names the case on stdout before its GPU step (kept if the step never returns)."""
    sys.stdout.write(f"[case] {msg}\n")
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


TOPO_KEYS = ("root_key", "upper_origin", "upper_mask", "upper_first", "lower_origin", "lower_mask",
             "lower_first", "leaf_origin", "leaf_mask", "leaf_offset", "leaf_prefix")


def assert_topology_equal(got: dict, ref: dict) -> None:
    for k in TOPO_KEYS:
        a, b = got[k], ref[k]
        assert a.shape == b.shape, f"{k}: shape {a.shape} vs {b.shape}"
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            raise AssertionError(f"{k}: {bad.shape[0]} mismatches, first at {bad[0].tolist()}: "
                                 f"{a[tuple(bad[0])]} vs {b[tuple(bad[0])]}")


def normwise_error(y: np.ndarray, r: np.ndarray) -> float:
    """max |y - r| / max |r| over the whole output."""
    den = float(np.max(np.abs(r))) if r.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(y))) if y.size else 0.0
    return float(np.max(np.abs(y.astype(np.float64) - r))) / den
