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


def elementwise_error(y: np.ndarray, r: np.ndarray) -> float:
    """max over elements of |y - r| / (|r| + 1e-3 max|r|): reported next to the normwise gate
    (an elementwise relative error without the floor is unbounded at zero outputs)."""
    if not r.size:
        return 0.0
    floor = 1e-3 * float(np.max(np.abs(r)))
    if floor == 0.0:
        return float(np.max(np.abs(y)))
    return float(np.max(np.abs(y.astype(np.float64) - r) / (np.abs(r) + floor)))


def segment_sample_rows(n: int, n_segments: int, seg: int = 256, n_random: int = 0, seed: int = 0) -> np.ndarray:
    """Sorted output rows for sampled parity at full size: n_segments whole runs of `seg`
    consecutive rows aligned to `seg` (every row tile of 64, 128 or 256 rows that such a run
    covers is checked whole, sorted positions included), evenly spaced so that the first and the
    last (possibly partial) run are among them, plus the runs on both sides of the boundaries of
    eight equal ranges of runs (where a grid split over the eight XCDs changes hands), plus
    n_random rows drawn uniformly."""
    n_seg_total = (n + seg - 1) // seg
    picks = set(np.linspace(0, n_seg_total - 1, min(n_segments, n_seg_total)).round().astype(np.int64).tolist())
    q, rem = divmod(n_seg_total, 8)
    for x in range(1, 8):
        b = x * q + min(x, rem)
        picks.update(v for v in (b - 1, b) if 0 <= v < n_seg_total)
    rows = [np.arange(s * seg, min((s + 1) * seg, n), dtype=np.int64) for s in sorted(picks)]
    if n_random:
        rows.append(np.random.default_rng(seed).choice(n, min(n_random, n), replace=False).astype(np.int64))
    return np.unique(np.concatenate(rows))


def sub_map(map_host: np.ndarray, rows: np.ndarray):
    """The kernel-map columns of `rows`, renumbered onto the input rows they use: returns
    (sub, need) with sub int32[K, len(rows)], sub[o, i] = position of map[o, rows[i]] in need
    (or -1), need the sorted input rows. oracle.conv(sub, feats[need], w) is then the oracle's
    convolution at those output rows."""
    cols = map_host[:, rows]
    need = np.unique(cols[cols >= 0])
    sub = np.full(cols.shape, -1, np.int32)
    ok = cols >= 0
    sub[ok] = np.searchsorted(need, cols[ok]).astype(np.int32)
    return sub, need
