"""Seeded synthetic voxel workloads for the 3x3x3 submanifold convolution.

This module only draws inputs: active-voxel coordinates and the feature,
weight, bias and output-gradient values.  It holds none of the convolution's
arithmetic (no neighbour search, no sort keys, no products), so the CPU oracle
and the HIP path can both consume what it produces without sharing any code.

The FlexGEMM pages benchmark on unnamed "voxel data" with C = 64..1024 and
RES = 8..1024 (contributor report, section one, "what problem it solves"), and
their tests draw sphere-shaped coordinates (section three, pitfall 6).  No
dataset is named, so the five workloads below stand in for it:

  1  1 x 32^3, cells within 0.5 of a radius-12 sphere, C = 32,   fp32
  2  2 x 64^3, 26-connected shells of 3 ellipsoids,    C = 64,   fp16
  3  4 x 256^3, shells of 5 ellipsoids,                C = 256,  bf16
  4  1 x 1024^3, shells of 8 ellipsoids + 1 % noise,   C = 64,   fp16, 64-bit keys
  5  1 x 128^3, every cell active with p = 0.3,         C = 1024, bf16

Recipe (one ``numpy.random.default_rng(cfg)`` stream per workload, draws in
this order): geometry, then features X ~ N(0,1) [N, Ci], then weights
W ~ N(0,1)/sqrt(27 Ci) [27, Ci, Co], then dY ~ N(0,1) [N, Co], then (only if
asked) bias ~ N(0,1) [Co].  Values are drawn in float64 and rounded to
nearest-even into the workload dtype; both sides consume the rounded values.
Coordinates come out in lexicographic (b, x, y, z) order as int32 rows.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# (B, R, Ci=Co, dtype, key_bits, description)
CONFIGS = {
    1: dict(B=1, R=32, C=32, dtype="f32", key_bits=0,
            desc="1x32^3 sphere shell r=12, C=32, fp32"),
    2: dict(B=2, R=64, C=64, dtype="f16", key_bits=0,
            desc="2x64^3 shells of 3 ellipsoids (semi-axes U[8,28]), C=64, fp16"),
    3: dict(B=4, R=256, C=256, dtype="bf16", key_bits=0,
            desc="4x256^3 shells of 5 ellipsoids (semi-axes U[24,84]), C=256, bf16"),
    4: dict(B=1, R=1024, C=64, dtype="f16", key_bits=64,
            desc="1x1024^3 shells of 8 ellipsoids (semi-axes U[128,448]) + 1% noise, C=64, fp16, 64-bit keys"),
    5: dict(B=1, R=128, C=1024, dtype="bf16", key_bits=0,
            desc="1x128^3 iid occupancy p=0.3, C=1024, bf16"),
}

_ELLIPSOIDS = {2: (3, 8.0, 28.0), 3: (5, 24.0, 84.0), 4: (8, 128.0, 448.0)}


@dataclasses.dataclass
class Workload:
    cfg: int
    desc: str
    coords: np.ndarray            # int32 [N, 4] rows (b, x, y, z), lexicographic
    shape: tuple                  # (B, X, Y, Z)
    ci: int
    co: int
    dtype: str                    # "f32" | "f16" | "bf16"
    key_bits: int                 # 0 = chosen from the grid volume, else 32 / 64
    feats: torch.Tensor | None    # [N, Ci] CPU tensor in the workload dtype
    weight: torch.Tensor | None   # [27, Ci, Co]
    bias: torch.Tensor | None     # [Co]
    dout: torch.Tensor | None     # [N, Co]

    @property
    def n(self) -> int:
        return int(self.coords.shape[0])

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]


# ----------------------------------------------------------------------------
# geometry
# ----------------------------------------------------------------------------

def sphere_shell(R: int = 32, radius: float = 12.0, half_width: float = 0.5) -> np.ndarray:
    """Cells p of an R^3 grid with | |p - c| - radius | <= half_width, c the grid centre."""
    c = (R - 1) / 2.0
    g = np.arange(R, dtype=np.float64) - c
    d = np.sqrt(g[:, None, None] ** 2 + g[None, :, None] ** 2 + g[None, None, :] ** 2)
    return np.abs(d - radius) <= half_width


def ellipsoid_union(R: int, centres: np.ndarray, axes: np.ndarray) -> np.ndarray:
    """Boolean R^3 grid: cell p is inside when some axis-aligned ellipsoid holds it.

    For ellipsoid (c, a) and column (x, y) with u = ((x-cx)/ax)^2 + ((y-cy)/ay)^2 <= 1,
    the inside cells are the integers z in [cz - az sqrt(1-u), cz + az sqrt(1-u)].
    Columns are filled with a +1/-1 difference array and a running sum along z.
    """
    diff = np.zeros((R, R, R + 1), dtype=np.int8)
    for (cx, cy, cz), (ax, ay, az) in zip(centres, axes):
        x0, x1 = max(0, math.ceil(cx - ax)), min(R - 1, math.floor(cx + ax))
        y0, y1 = max(0, math.ceil(cy - ay)), min(R - 1, math.floor(cy + ay))
        if x0 > x1 or y0 > y1:
            continue
        xs = np.arange(x0, x1 + 1, dtype=np.float64)
        ys = np.arange(y0, y1 + 1, dtype=np.float64)
        u = ((xs[:, None] - cx) / ax) ** 2 + ((ys[None, :] - cy) / ay) ** 2
        ok = u <= 1.0
        h = az * np.sqrt(np.where(ok, 1.0 - u, 0.0))
        zlo = np.maximum(np.ceil(cz - h), 0).astype(np.int64)
        zhi = np.minimum(np.floor(cz + h), R - 1).astype(np.int64)
        ok &= zlo <= zhi
        ix, iy = np.nonzero(ok)
        gx, gy = ix + x0, iy + y0
        diff[gx, gy, zlo[ix, iy]] += 1
        diff[gx, gy, zhi[ix, iy] + 1] -= 1
    inside = np.cumsum(diff, axis=2, dtype=np.int8)[:, :, :R] > 0
    return inside


def shell_26(inside: np.ndarray) -> np.ndarray:
    """Cells that are inside and have at least one of their 26 neighbours outside or off-grid."""
    core = inside.copy()
    for axis in range(3):
        sl = [slice(None)] * 3
        out = np.zeros_like(core)
        mid = [slice(None)] * 3
        mid[axis] = slice(1, -1)
        lo = list(sl); lo[axis] = slice(0, -2)
        hi = list(sl); hi[axis] = slice(2, None)
        out[tuple(mid)] = core[tuple(lo)] & core[tuple(mid)] & core[tuple(hi)]
        core = out
    return inside & ~core


def _shell_grid(rng: np.random.Generator, R: int, E: int, lo: float, hi: float) -> np.ndarray:
    centres = rng.uniform(0.0, float(R), size=(E, 3))
    axes = rng.uniform(lo, hi, size=(E, 3))
    return shell_26(ellipsoid_union(R, centres, axes))


def _noise(rng: np.random.Generator, active_lin: np.ndarray, R: int, count: int) -> np.ndarray:
    """Draw `count` grid cells uniformly, one by one, rejecting active or already drawn ones."""
    taken: list[np.ndarray] = []
    have = 0
    seen = np.empty(0, dtype=np.int64)
    while have < count:
        cand = rng.integers(0, R, size=(max(2 * (count - have), 1024), 3), dtype=np.int64)
        lin = (cand[:, 0] * R + cand[:, 1]) * R + cand[:, 2]
        keep = ~np.isin(lin, active_lin) & ~np.isin(lin, seen)
        lin = lin[keep]
        _, first = np.unique(lin, return_index=True)
        lin = lin[np.sort(first)][: count - have]
        taken.append(lin)
        seen = np.concatenate([seen, lin])
        have += lin.size
    return np.concatenate(taken) if taken else np.empty(0, dtype=np.int64)


def _grid_to_coords(grids: list[np.ndarray]) -> np.ndarray:
    rows = []
    for b, g in enumerate(grids):
        x, y, z = np.nonzero(g)
        rows.append(np.stack([np.full_like(x, b), x, y, z], axis=1))
    return np.concatenate(rows).astype(np.int32)


def geometry(cfg: int, rng: np.random.Generator) -> np.ndarray:
    """Active-voxel coordinates of workload `cfg`, drawing from `rng` first."""
    p = CONFIGS[cfg]
    B, R = p["B"], p["R"]
    if cfg == 1:
        return _grid_to_coords([sphere_shell(R)])
    if cfg == 5:
        occ = rng.random((R, R, R)) < 0.3
        return _grid_to_coords([occ])
    E, lo, hi = _ELLIPSOIDS[cfg]
    grids = [_shell_grid(rng, R, E, lo, hi) for _ in range(B)]
    coords = _grid_to_coords(grids)
    if cfg == 4:
        x, y, z = coords[:, 1].astype(np.int64), coords[:, 2].astype(np.int64), coords[:, 3].astype(np.int64)
        lin = (x * R + y) * R + z
        extra = _noise(rng, lin, R, int(round(0.01 * coords.shape[0])))
        all_lin = np.sort(np.concatenate([lin, extra]))
        coords = np.stack([np.zeros_like(all_lin), all_lin // (R * R), (all_lin // R) % R, all_lin % R],
                          axis=1).astype(np.int32)
    return coords


# ----------------------------------------------------------------------------
# values
# ----------------------------------------------------------------------------

def normal(rng: np.random.Generator, shape, dtype: str, scale: float = 1.0,
           chunk_rows: int = 65536) -> torch.Tensor:
    """N(0, scale^2) drawn in float64 row-chunk by row-chunk, rounded to `dtype`."""
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=DTYPES[dtype])
    if len(shape) == 0 or shape[0] == 0:
        return out
    rest = shape[1:]
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        v = rng.standard_normal((r1 - r0,) + rest)
        if scale != 1.0:
            v *= scale
        out[r0:r1] = torch.from_numpy(v).to(DTYPES[dtype])
    return out


def make_workload(cfg: int, values: bool = True, random_bias: bool = False) -> Workload:
    p = CONFIGS[cfg]
    rng = np.random.default_rng(cfg)
    coords = geometry(cfg, rng)
    C, dt = p["C"], p["dtype"]
    feats = weight = bias = dout = None
    if values:
        n = coords.shape[0]
        feats = normal(rng, (n, C), dt)
        weight = normal(rng, (27, C, C), dt, scale=1.0 / math.sqrt(27 * C))
        dout = normal(rng, (n, C), dt)
        bias = normal(rng, (C,), dt) if random_bias else torch.zeros(C, dtype=DTYPES[dt])
    return Workload(cfg, p["desc"], coords, (p["B"], p["R"], p["R"], p["R"]), C, C, dt,
                    p["key_bits"], feats, weight, bias, dout)


def random_workload(seed: int, B: int, dims: tuple, p: float, ci: int, co: int, dtype: str,
                    random_bias: bool = True, shuffle: bool = False) -> Workload:
    """Small iid-occupancy workload for tests: each cell of B grids of `dims` active with prob p."""
    rng = np.random.default_rng(seed)
    grids = [rng.random(dims) < p for _ in range(B)]
    coords = _grid_to_coords(grids) if any(g.any() for g in grids) else np.zeros((0, 4), np.int32)
    if shuffle and coords.shape[0] > 1:
        coords = coords[rng.permutation(coords.shape[0])]
    n = coords.shape[0]
    feats = normal(rng, (n, ci), dtype)
    weight = normal(rng, (27, ci, co), dtype, scale=1.0 / math.sqrt(27 * ci))
    dout = normal(rng, (n, co), dtype)
    bias = normal(rng, (co,), dtype) if random_bias else torch.zeros(co, dtype=DTYPES[dtype])
    return Workload(0, f"random seed={seed} B={B} dims={dims} p={p}", coords, (B,) + tuple(dims),
                    ci, co, dtype, 0, feats, weight, bias, dout)


def values_for(coords: np.ndarray, shape: tuple, seed: int, ci: int, co: int, dtype: str,
               random_bias: bool = True) -> Workload:
    """Workload with given coordinates and seeded values (hand-made geometries in tests)."""
    rng = np.random.default_rng(seed)
    n = coords.shape[0]
    feats = normal(rng, (n, ci), dtype)
    weight = normal(rng, (27, ci, co), dtype, scale=1.0 / math.sqrt(27 * ci))
    dout = normal(rng, (n, co), dtype)
    bias = normal(rng, (co,), dtype) if random_bias else torch.zeros(co, dtype=DTYPES[dtype])
    return Workload(0, "given coords", np.ascontiguousarray(coords, dtype=np.int32), tuple(shape),
                    ci, co, dtype, 0, feats, weight, bias, dout)


def strided_values(seed: int, n_in: int, n_out: int, ks: int, ci: int, co: int, dtype: str,
                   random_bias: bool = True) -> tuple:
    """Seeded (feats [n_in, ci], weight [ks^3, ci, co], bias [co], dout [n_out, co]) for a strided
    convolution, drawn in that order; weight ~ N(0, 1 / (ks^3 ci)), the rest ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    V = ks ** 3
    feats = normal(rng, (n_in, ci), dtype)
    weight = normal(rng, (V, ci, co), dtype, scale=1.0 / math.sqrt(V * ci))
    bias = normal(rng, (co,), dtype) if random_bias else torch.zeros(co, dtype=DTYPES[dtype])
    dout = normal(rng, (n_out, co), dtype)
    return feats, weight, bias, dout


# ----------------------------------------------------------------------------
# query points for sparse grid sampling
# ----------------------------------------------------------------------------

def sample_points(coords: np.ndarray, shape: tuple, m: int, seed: int, near: float = 0.9) -> np.ndarray:
    """Seeded float32 [m, 4] query rows (b, x, y, z) for sparse grid sampling.

    A fraction `near` of the points sit within one cell of an active voxel
    (the voxel's position plus a uniform offset in [-1, 1)^3, same sample);
    the rest are uniform over the sample-and-box [0, B) x [-1, X] x [-1, Y] x
    [-1, Z], so some fall partly or wholly off the grid.  Points only: no
    lookups or weights are computed here.
    """
    rng = np.random.default_rng(seed)
    B, X, Y, Z = (int(s) for s in shape)
    out = np.empty((m, 4), np.float32)
    k = int(round(m * near)) if len(coords) else 0
    if k:
        pick = coords[rng.integers(0, len(coords), k)].astype(np.float64)
        pick[:, 1:] += rng.uniform(-1.0, 1.0, (k, 3))
        out[:k] = pick
    r = m - k
    if r:
        out[k:, 0] = rng.integers(0, B, r)
        for a, d in enumerate((X, Y, Z)):
            out[k:, 1 + a] = rng.uniform(-1.0, d, r)
    return out
