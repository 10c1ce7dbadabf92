"""CPU oracle for sparse grid sampling: trilinear weighted sums (test infrastructure).

This module is test infrastructure.  Only the test suite, the package smoke
check and the benchmark's CPU-baseline leg may import it; the HIP library and
its Python binding never do, and it shares no code with them.

What the pages fix (contributor report, page 1, section two: the module table
rows ops.grid_sample, kernels.triton.grid_sample and kernels.cuda.grid_sample,
and the key-function table row indice_weighed_sum_fwd / bwd; the extension
section, which speaks of adding interpolation modes other than trilinear):

* a sparse grid_sample operator samples the features of a sparse voxel set at
  query points;
* its forward pass is a weighted sum of voxel feature rows picked by indices,
  and its backward pass is the transposed weighted sum;
* the interpolation is trilinear.

The pages give no signature, no coordinate convention and no rule for absent
voxels.  Readings taken here:

* a query point is a float row ``[b, x, y, z]`` in voxel-index units: voxel
  ``[b, x, y, z]`` sits at the integer point (x, y, z) of sample b;
* trilinear weights: with x0 = floor(x) and t = x - x0 (same for y, z), the
  corner (x0 + dx, y0 + dy, z0 + dz), dx, dy, dz in {0, 1}, has weight
  wx * wy * wz with wx = t if dx else 1 - t; corners are taken in the order
  j = 4 dx + 2 dy + dz;
* a corner that is off the grid or not an active voxel contributes nothing
  (the weights of the others are not renormalised): the sparse tensor is zero
  away from its active sites, as a dense volume with zero padding would be;
* a point whose batch value is not an integer in [0, B), or whose
  coordinates are not finite, samples zero;
* forward: ``out[m] = sum_j w[m, j] * feats[idx[m, j]]``; backward (feature
  gradient only; the pages name no gradient with respect to the points):
  ``dfeats[i] = sum over (m, j) with idx[m, j] = i of w[m, j] * dout[m]``.

Pinned by tests/test_oracle_grid_sample.py against torch's dense
``grid_sample`` (trilinear, align_corners=True, zero padding) on the
zero-filled dense volume and its autograd, against hand-derived cases, the
adjoint identity and a planted mistake.  Floats are float64 on the exact
values of the (already rounded) inputs.

Tier A (``*_loops``) is the definition written out with a dict and loops;
Tier B restates it with numpy gathers (any size).
"""
from __future__ import annotations

import numpy as np

# corner j = 4 dx + 2 dy + dz
CORNERS = np.array([(dx, dy, dz) for dx in (0, 1) for dy in (0, 1) for dz in (0, 1)], dtype=np.int64)


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def point_batch(b: float, B: int):
    """The sample index of a point's batch value, or None when it names no sample."""
    if not np.isfinite(b) or b != np.floor(b) or not (0 <= b < B):
        return None
    return int(b)


def corners(point, shape):
    """[(cell (b, x, y, z) or None, weight)] for the 8 corners of one point, in corner order."""
    B, X, Y, Z = (int(s) for s in shape)
    b = point_batch(float(point[0]), B)
    xyz = [float(v) for v in point[1:4]]
    if b is None or not all(np.isfinite(v) for v in xyz):
        return [(None, 0.0)] * 8
    base = [int(np.floor(v)) for v in xyz]
    frac = [v - np.floor(v) for v in xyz]
    out = []
    for d in CORNERS.tolist():
        w = 1.0
        cell = [b]
        for a in range(3):
            w *= frac[a] if d[a] else 1.0 - frac[a]
            cell.append(base[a] + d[a])
        inside = all(0 <= cell[1 + a] < (X, Y, Z)[a] for a in range(3))
        out.append((tuple(cell) if inside else None, w))
    return out


def sample_fwd_loops(coords, feats, shape, points) -> np.ndarray:
    """Tier A forward: out[m] = sum over present corners of weight * feats[row]."""
    coords = np.asarray(coords, dtype=np.int64).reshape(-1, 4)
    F = _f64(feats)
    D = {tuple(c): i for i, c in enumerate(coords.tolist())}
    P = np.asarray(points, dtype=np.float64).reshape(-1, 4)
    out = np.zeros((len(P), F.shape[1]))
    for m, p in enumerate(P):
        for cell, w in corners(p, shape):
            i = D.get(cell) if cell is not None else None
            if i is not None:
                out[m] += w * F[i]
    return out


def sample_bwd_loops(coords, shape, points, dout, n=None) -> np.ndarray:
    """Tier A backward: dfeats[i] = sum over (point, corner) hitting row i of weight * dout[point]."""
    coords = np.asarray(coords, dtype=np.int64).reshape(-1, 4)
    G = _f64(dout)
    D = {tuple(c): i for i, c in enumerate(coords.tolist())}
    P = np.asarray(points, dtype=np.float64).reshape(-1, 4)
    dF = np.zeros((len(coords) if n is None else n, G.shape[1]))
    for m, p in enumerate(P):
        for cell, w in corners(p, shape):
            i = D.get(cell) if cell is not None else None
            if i is not None:
                dF[i] += w * G[m]
    return dF


# ---------------------------------------------------------------------------
# Tier B: vectorised
# ---------------------------------------------------------------------------

def corner_table(coords, shape, points):
    """idx [M, 8] int64 (-1 where absent) and weights [M, 8] float64, corner order."""
    B, X, Y, Z = (int(s) for s in shape)
    coords = np.asarray(coords, dtype=np.int64).reshape(-1, 4)
    P = np.asarray(points, dtype=np.float64).reshape(-1, 4)
    M = len(P)
    b = P[:, 0]
    ok = np.isfinite(P).all(axis=1) & (b == np.floor(np.where(np.isfinite(b), b, 0))) & (b >= 0) & (b < B)
    xyz = np.where(ok[:, None], P[:, 1:4], 0.0)
    base = np.floor(xyz)
    frac = xyz - base
    # linear keys of the active voxels, sorted, for the lookups
    lin = ((coords[:, 0] * X + coords[:, 1]) * Y + coords[:, 2]) * Z + coords[:, 3]
    order = np.argsort(lin, kind="stable")
    slin = lin[order]
    idx = np.full((M, 8), -1, dtype=np.int64)
    w = np.zeros((M, 8))
    dims = np.array([X, Y, Z], dtype=np.float64)
    for j, d in enumerate(CORNERS):
        c = base + d
        inside = ok & ((c >= 0) & (c < dims)).all(axis=1)
        wj = np.prod(np.where(d == 1, frac, 1.0 - frac), axis=1)
        ci = np.where(inside[:, None], c, 0).astype(np.int64)
        bi = np.where(inside, b, 0).astype(np.int64)
        key = ((bi * X + ci[:, 0]) * Y + ci[:, 1]) * Z + ci[:, 2]
        pos = np.searchsorted(slin, key)
        pos_c = np.minimum(pos, max(len(slin) - 1, 0))
        hit = inside & (len(slin) > 0) & (slin[pos_c] == key) if len(slin) else np.zeros(M, bool)
        idx[:, j] = np.where(hit, order[pos_c] if len(slin) else 0, -1)
        w[:, j] = np.where(ok, wj, 0.0)
    return idx, w


def sample_fwd(coords, feats, shape, points) -> np.ndarray:
    """Tier B forward (float64)."""
    F = _f64(feats)
    idx, w = corner_table(coords, shape, points)
    out = np.zeros((len(idx), F.shape[1]))
    for j in range(8):
        hit = idx[:, j] >= 0
        out[hit] += w[hit, j:j + 1] * F[idx[hit, j]]
    return out


def sample_bwd(coords, shape, points, dout) -> np.ndarray:
    """Tier B backward (float64): the transposed weighted sum."""
    G = _f64(dout)
    n = len(np.asarray(coords).reshape(-1, 4))
    idx, w = corner_table(coords, shape, points)
    dF = np.zeros((n, G.shape[1]))
    for j in range(8):
        hit = idx[:, j] >= 0
        np.add.at(dF, idx[hit, j], w[hit, j:j + 1] * G[hit])
    return dF
