"""Seeded synthetic workloads for the IndexGrid build, the kernel map and the 3x3x3
submanifold convolution.

This module holds geometry and random numbers only: it places voxels, features and
weights. It contains none of the method's arithmetic (no keys, no ordering, no index,
no convolution), so that both the HIP path and the CPU oracle can consume the same
inputs without sharing any computation.

Every generator is deterministic in its seed. The seed scheme for workload k is
geometry 1000+k, shuffle 2000+k, features 3000+k, weights 4000+k.

The five workloads stand in for the regimes that the fVDB paper notes ("fVDB: A
Deep-Learning Framework for Sparse, Large Scale, and High Performance Spatial
Intelligence", sections on sparse-convolution operators and on micro-benchmarks)
name: a small shell, dense domains with leaf occupancy above 20%, narrow bands with
high neighbour occupancy, very sparse LiDAR-like frames, and a build at 4096^3 scale.
The datasets the pages measure on (SemanticKITTI, nuScenes, KartonCity) are not used;
the LiDAR workload simulates a spinning scanner instead.
"""
from __future__ import annotations

import dataclasses
import math
import os

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_coords",
    "make_features",
    "make_weights",
    "shell_coords",
    "boxes_coords",
    "band_coords",
    "lidar_coords",
    "large_band_coords",
    "random_coords",
    "make_features_device",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: its geometry, channel counts and arithmetic type."""

    index: int          # 1-based workload number (seed base)
    name: str
    cin: int
    cout: int
    dtype: str          # "f32" or "bf16": the type features, weights and outputs are stored in
    weight_std: float | None  # None: N(0,1); otherwise N(0, std)
    description: str


def _std(cin: int) -> float:
    return 1.0 / math.sqrt(27.0 * cin)


WORKLOADS = {
    "tiny": Workload(1, "tiny", 8, 8, "f32", None,
                     "64^3 box, 1-voxel shell of a sphere r=24 at (32,32,32), fp32 8->8"),
    "leaf": Workload(2, "leaf", 8, 16, "f32", _std(8),
                     "512^3 box, union of 40 axis-aligned solid boxes (log-uniform sides 16-96), fp32 8->16"),
    "band": Workload(3, "band", 64, 64, "bf16", _std(64),
                     "2048^3 box, |sd|<=1.5 band around 200 spheres/tori (radii 20-300), bf16 64->64"),
    "lidar": Workload(4, "lidar", 128, 128, "bf16", _std(128),
                      "64-beam x 2048-azimuth scan of ground + 150 boxes at 0.1 m, 5 frames, bf16 128->128"),
    "large": Workload(5, "large", 128, 256, "bf16", _std(128),
                      "50M signed coords (~10% duplicates) from a band generator over [-2048,2048)^3, bf16 128->256"),
    # The band geometry at feature depth 32, the regime of the pages' brick backend (depths 32-64,
    # narrow bands); coordinates are those of "band", features and weights its own.
    "band32": Workload(6, "band32", 32, 32, "bf16", _std(32),
                       "the band geometry (workload 3) at bf16 32->32, the brick-backend regime"),
}


# ----------------------------------------------------------------------------- helpers

def _shuffle(a: np.ndarray, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return a[rng.permutation(a.shape[0])]


def _pack(c: np.ndarray) -> np.ndarray:
    """Packs int32 triples with |x| < 2^20 into int64 for set operations (dedupe only)."""
    c = c.astype(np.int64) + (1 << 20)
    return (c[:, 0] << 42) | (c[:, 1] << 21) | c[:, 2]


def _unpack(p: np.ndarray) -> np.ndarray:
    out = np.empty((p.shape[0], 3), dtype=np.int32)
    m = (1 << 21) - 1
    out[:, 0] = ((p >> 42) & m) - (1 << 20)
    out[:, 1] = ((p >> 21) & m) - (1 << 20)
    out[:, 2] = (p & m) - (1 << 20)
    return out


# ----------------------------------------------------------------------------- workload 1

def shell_coords(seed_base: int = 1) -> np.ndarray:
    """Integer points p of [0,64)^3 with | |p-(32,32,32)| - 24 | < 0.5, shuffled."""
    g = np.arange(64)
    i, j, k = np.meshgrid(g, g, g, indexing="ij")
    d = np.sqrt((i - 32.0) ** 2 + (j - 32.0) ** 2 + (k - 32.0) ** 2)
    m = np.abs(d - 24.0) < 0.5
    c = np.stack([i[m], j[m], k[m]], axis=1).astype(np.int32)
    return _shuffle(c, 2000 + seed_base)


# ----------------------------------------------------------------------------- workload 2

def boxes_coords(seed_base: int = 2, n_boxes: int = 40, domain: int = 512,
                 side_lo: float = 16.0, side_hi: float = 96.0) -> np.ndarray:
    """Union of axis-aligned solid boxes in [0,domain)^3.

    Per-axis side = floor(exp(U(ln side_lo, ln side_hi))); the corner is uniform so that
    the box fits. The union is shuffled.
    """
    rng = np.random.default_rng(1000 + seed_base)
    occ = np.zeros((domain, domain, domain), dtype=bool)
    for _ in range(n_boxes):
        sides = np.floor(np.exp(rng.uniform(math.log(side_lo), math.log(side_hi), size=3))).astype(int)
        lo = [int(rng.integers(0, domain - s + 1)) for s in sides]
        occ[lo[0]:lo[0] + sides[0], lo[1]:lo[1] + sides[1], lo[2]:lo[2] + sides[2]] = True
    c = np.argwhere(occ).astype(np.int32)
    return _shuffle(c, 2000 + seed_base)


# ----------------------------------------------------------------------------- workloads 3, 5

def _column_band(I, J, a2, cz, r, band):
    """Integer k with | sqrt(a2 + (k-cz)^2) - r | <= band, per column (I,J).

    a2 is the squared in-plane distance term of the signed distance (rho^2 for a sphere,
    (rho-R)^2 for a torus around the k axis). Candidate intervals are widened by one voxel
    and filtered with the exact test.
    """
    hi = r + band
    lo = max(r - band, 0.0)
    keep = a2 <= hi * hi
    I, J, a2 = I[keep], J[keep], a2[keep]
    zhi = np.sqrt(np.maximum(hi * hi - a2, 0.0))
    zlo = np.sqrt(np.maximum(lo * lo - a2, 0.0))
    # Two candidate runs per column: [cz-zhi, cz-zlo] and [cz+zlo, cz+zhi] (merged when zlo == 0).
    a0 = np.floor(cz - zhi).astype(np.int64) - 1
    a1 = np.ceil(cz - zlo).astype(np.int64) + 1
    b0 = np.floor(cz + zlo).astype(np.int64) - 1
    b1 = np.ceil(cz + zhi).astype(np.int64) + 1
    merged = a1 >= b0
    a1 = np.where(merged, b1, a1)
    b1 = np.where(merged, b0 - 1, b1)  # empty second run
    na = np.maximum(a1 - a0 + 1, 0)
    nb = np.maximum(b1 - b0 + 1, 0)
    starts = np.concatenate([a0, b0])
    counts = np.concatenate([na, nb])
    ci = np.concatenate([I, I])
    cj = np.concatenate([J, J])
    ca2 = np.concatenate([a2, a2])
    tot = int(counts.sum())
    if tot == 0:
        return np.empty((0, 3), dtype=np.int32)
    rep = np.repeat(np.arange(counts.shape[0]), counts)
    first = np.cumsum(counts) - counts
    K = starts[rep] + (np.arange(tot) - first[rep])
    d = np.sqrt(ca2[rep] + (K - cz) ** 2)
    ok = np.abs(d - r) <= band
    return np.stack([ci[rep][ok], cj[rep][ok], K[ok]], axis=1).astype(np.int32)


def _sphere_band(c, r, band):
    cx, cy, cz = c
    hi = r + band
    I, J = np.meshgrid(np.arange(int(np.floor(cx - hi)), int(np.ceil(cx + hi)) + 1),
                       np.arange(int(np.floor(cy - hi)), int(np.ceil(cy + hi)) + 1), indexing="ij")
    I = I.ravel(); J = J.ravel()
    a2 = (I - cx) ** 2 + (J - cy) ** 2
    return _column_band(I, J, a2, cz, r, band)


def _torus_band(c, R, rm, band):
    cx, cy, cz = c
    ext = R + rm + band
    I, J = np.meshgrid(np.arange(int(np.floor(cx - ext)), int(np.ceil(cx + ext)) + 1),
                       np.arange(int(np.floor(cy - ext)), int(np.ceil(cy + ext)) + 1), indexing="ij")
    I = I.ravel(); J = J.ravel()
    q = np.sqrt((I - cx) ** 2 + (J - cy) ** 2) - R
    return _column_band(I, J, q * q, cz, rm, band)


def _draw_shape(rng, lo: float, hi: float, r_min: float, r_max: float, band: float):
    """One sphere or torus (p = 1/2) with r^-2 ~ U(r_max^-2, r_min^-2), centred uniformly
    so that the shape lies inside [lo, hi)^3."""
    is_torus = rng.uniform() < 0.5
    r = float(rng.uniform(r_max ** -2, r_min ** -2) ** -0.5)
    if is_torus:
        R, rm = r, r / 3.0
        exy = R + rm + band + 2.0
        ez = rm + band + 2.0
    else:
        exy = ez = r + band + 2.0
    cx = rng.uniform(lo + exy, hi - exy)
    cy = rng.uniform(lo + exy, hi - exy)
    cz = rng.uniform(lo + ez, hi - ez)
    if is_torus:
        return _torus_band((cx, cy, cz), R, rm, band)
    return _sphere_band((cx, cy, cz), r, band)


def band_coords(seed_base: int = 3, n_shapes: int = 200, domain: int = 2048,
                r_min: float = 20.0, r_max: float = 300.0, band: float = 1.5) -> np.ndarray:
    """Voxels within |signed distance| <= band of random spheres / tori in [0,domain)^3.

    Torus major radius R = r, minor r/3, axis k. Union of all shapes, shuffled.
    """
    rng = np.random.default_rng(1000 + seed_base)
    parts = [_draw_shape(rng, 0.0, float(domain), r_min, r_max, band) for _ in range(n_shapes)]
    p = np.unique(_pack(np.concatenate(parts)))
    return _shuffle(_unpack(p), 2000 + seed_base)


def large_band_coords(seed_base: int = 5, n_in: int = 50_000_000, n_unique: int = 45_000_000,
                      half: int = 2048, r_min: float = 40.0, r_max: float = 600.0,
                      band: float = 1.5) -> np.ndarray:
    """The band generator over the signed domain [-half, half)^3.

    Shapes are added in seeded order until the union S holds at least n_unique voxels;
    then n_in - |S| duplicates drawn uniformly from S are appended and everything is
    shuffled.
    """
    rng = np.random.default_rng(1000 + seed_base)
    packed, owner = [], []
    raw, k = 0, 0
    target_raw = int(n_unique * 1.08)
    while True:
        while raw < target_raw:
            pts = _draw_shape(rng, float(-half), float(half), r_min, r_max, band)
            packed.append(_pack(pts))
            owner.append(np.full(pts.shape[0], k, dtype=np.int32))
            raw += pts.shape[0]
            k += 1
        # First occurrence in shape order = the earliest shape that produced the voxel, so
        # |S_k| (union of the first k shapes) is a cumulative count over that owner.
        uniq, first = np.unique(np.concatenate(packed), return_index=True)
        first_owner = np.concatenate(owner)[first]
        cum = np.cumsum(np.bincount(first_owner, minlength=k))
        hit = np.nonzero(cum >= n_unique)[0]
        if hit.size:
            S = uniq[first_owner <= int(hit[0])]
            break
        target_raw = raw + int(n_unique * 0.05) + 1
    del packed, owner
    n_dup = max(n_in - S.shape[0], 0)
    dup_idx = np.random.default_rng(2000 + seed_base + 100).integers(0, S.shape[0], size=n_dup)
    allc = np.concatenate([S, S[dup_idx]])
    return _shuffle(_unpack(allc), 2000 + seed_base)


# ----------------------------------------------------------------------------- workload 4

def _lidar_frame(seed: int, n_beams: int = 64, n_az: int = 2048, elev_lo: float = -25.0,
                 elev_hi: float = 3.0, ground_z: float = -1.73, n_boxes: int = 150,
                 xy_half: float = 51.2, z_lo: float = -5.0, z_hi: float = 3.0,
                 voxel: float = 0.1) -> np.ndarray:
    """Points of one simulated sweep, voxelized to signed integer coordinates (with repeats)."""
    rng = np.random.default_rng(seed)
    # Boxes standing on the ground, centres away from the sensor.
    cx = np.empty(0); cy = np.empty(0)
    while cx.shape[0] < n_boxes:
        c = rng.uniform(-xy_half, xy_half, size=(n_boxes, 2))
        c = c[np.hypot(c[:, 0], c[:, 1]) > 4.0]
        cx = np.concatenate([cx, c[:, 0]]); cy = np.concatenate([cy, c[:, 1]])
    cx = cx[:n_boxes]; cy = cy[:n_boxes]
    sx = rng.uniform(1.0, 5.0, size=n_boxes)
    sy = rng.uniform(1.0, 5.0, size=n_boxes)
    sz = rng.uniform(1.0, 4.0, size=n_boxes)
    bmin = np.stack([cx - sx / 2, cy - sy / 2, np.full(n_boxes, ground_z)], axis=1)
    bmax = np.stack([cx + sx / 2, cy + sy / 2, ground_z + sz], axis=1)

    el = np.deg2rad(np.linspace(elev_lo, elev_hi, n_beams))
    az = np.arange(n_az) * (2.0 * math.pi / n_az)
    E, A = np.meshgrid(el, az, indexing="ij")
    d = np.stack([np.cos(E) * np.cos(A), np.cos(E) * np.sin(A), np.sin(E)], axis=-1).reshape(-1, 3)

    t_best = np.full(d.shape[0], np.inf)
    down = d[:, 2] < 0
    t_best[down] = ground_z / d[down, 2]
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = 1.0 / d
    for b in range(n_boxes):  # slab test, first hit
        t0 = bmin[b] * inv
        t1 = bmax[b] * inv
        tn = np.nanmax(np.minimum(t0, t1), axis=1)
        tf = np.nanmin(np.maximum(t0, t1), axis=1)
        hit = (tn <= tf) & (tf > 0)
        th = np.where(tn > 0, tn, tf)
        better = hit & (th < t_best)
        t_best[better] = th[better]
    ok = np.isfinite(t_best)
    p = d[ok] * t_best[ok][:, None]
    keep = ((p[:, 0] >= -xy_half) & (p[:, 0] < xy_half) & (p[:, 1] >= -xy_half)
            & (p[:, 1] < xy_half) & (p[:, 2] >= z_lo) & (p[:, 2] < z_hi))
    p = p[keep]
    return np.floor(p / voxel).astype(np.int32)


def lidar_coords(seed_base: int = 4, frames: int = 5, shift: int = 1024) -> np.ndarray:
    """frames simulated sweeps; frame f is shifted by f*shift voxels along i. Shuffled,
    with the repeated voxels of each sweep kept (the build deduplicates them)."""
    parts = []
    for f in range(frames):
        c = _lidar_frame(1000 + seed_base + 10 * f)
        c[:, 0] += f * shift
        parts.append(c)
    return _shuffle(np.concatenate(parts), 2000 + seed_base)


# ----------------------------------------------------------------------------- misc

def random_coords(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """n uniform integer coordinates in [lo, hi)^3 (duplicates possible)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, size=(n, 3), dtype=np.int64).astype(np.int32)


_CACHE = os.environ.get("IGC_WORKLOAD_CACHE", "")


def make_coords(name: str) -> np.ndarray:
    """Input coordinates int32[N_in, 3] of a named workload."""
    w = WORKLOADS[name]
    path = os.path.join(_CACHE, f"{name}_coords.npy") if _CACHE else ""
    if path and os.path.exists(path):
        return np.load(path)
    if name == "tiny":
        c = shell_coords(w.index)
    elif name == "leaf":
        c = boxes_coords(w.index)
    elif name == "band":
        c = band_coords(w.index)
    elif name == "band32":
        return make_coords("band")
    elif name == "lidar":
        c = lidar_coords(w.index)
    elif name == "large":
        c = large_band_coords(w.index)
    else:
        raise KeyError(name)
    c = np.ascontiguousarray(c, dtype=np.int32)
    if path:
        os.makedirs(_CACHE, exist_ok=True)
        np.save(path, c)
    return c


def make_features(n: int, cin: int, seed: int) -> np.ndarray:
    """float32[n, cin] ~ N(0, 1), row-major in linear-index order."""
    return np.random.default_rng(seed).standard_normal((n, cin), dtype=np.float32)


def make_weights(cin: int, cout: int, seed: int, std: float | None) -> np.ndarray:
    """float32[27, cin, cout] ~ N(0, std^2) (std None: 1)."""
    w = np.random.default_rng(seed).standard_normal((27, cin, cout), dtype=np.float32)
    if std is not None:
        w *= np.float32(std)
    return w


def make_features_device(n: int, cin: int, seed: int, device, dtype=None):
    """float32[n, cin] ~ N(0, 1) drawn on `device` by torch's seeded generator (Philox on the
    GPU), cast to `dtype` if given. For feature arrays too large to draw on the host."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f = torch.randn((n, cin), generator=g, dtype=torch.float32, device=device)
    return f if dtype is None else f.to(dtype)
