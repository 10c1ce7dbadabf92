"""CPU oracle for the generalised (strided) sparse convolution (test infrastructure).

This module is test infrastructure.  Only the test suite, the package smoke
check and the benchmark's CPU-baseline leg may import it; the HIP library and
its Python binding never do, and it shares no code with them.

What the pages fix (contributor report, page 1, section two: the module
table rows ops.spconv and kernels.cuda.spconv, and the key-function table
rows sparse_conv3d, sparse_conv_implicit_gemm[_splitk],
sparse_conv_masked_implicit_gemm[_splitk] and subm_neighbor_map /
sparse_neighbor_map):

* besides the submanifold operator the library has a regular 3D sparse
  convolution, ``sparse_conv3d``, whose output sites need not be its input
  sites;
* it is computed by the same (masked) implicit GEMM, through a neighbour map
  built by its own primitive, ``sparse_neighbor_map``.

The pages give no formula, geometry or output rule.  Readings taken here:

* the kernel is a cube of side ks in {1, 2, 3}, so V = ks^3 <= 27 offsets;
  stride s >= 1 and padding 0 <= p < ks are the same on every axis; no
  dilation;
* offset k = (a ks + b) ks + c for (a, b, c) in [0, ks)^3 on axes (x, y, z);
  output site o meets the input site (o_x s - p + a, o_y s - p + b,
  o_z s - p + c) of the same sample (cross-correlation, as a dense conv3d
  with that stride and padding);
* the output grid is (B, Xo, Yo, Zo) with Xo = (X + 2p - ks) // s + 1;
* the active output sites, when the caller does not give them, are every
  output-grid site whose window holds at least one active input site (the
  sites where a dense convolution of the occupancy with an all-ones kernel is
  non-zero), in ascending lexicographic (b, x, y, z) order;
* the map is ``nmap[o][k]`` = input row, or 0xFFFFFFFF, with 27 columns;
  columns k >= V are always the sentinel;
* rows of the output are ordered for the GEMM exactly as in the submanifold
  case: ascending by (neighbour mask, z-order code of the output site over the
  output grid);
* fwd ``out[o] = bias + sum_k X[nmap[o][k]] @ W[k]`` with W of shape
  [V][Ci][Co]; input gradient ``dX[j] = sum over (o, k) with nmap[o][k] = j of
  W[k] @ dY[o]``; ``dW[k] = sum_o outer(X[nmap[o][k]], dY[o])``;
  ``dbias = sum_o dY[o]``.

With ks = 3, s = 1, p = 1 and the input sites given as the output sites, this
is the submanifold convolution.

Pinned by tests/test_oracle_sparse_conv.py against torch's dense ``conv3d``
(stride s, padding p, float64) on the zero-filled grid and its autograd, the
output-site rule against a dense all-ones convolution of the occupancy, an
all-pairs brute force, hand-derived cases and planted mistakes.  Floats are
float64 on the exact values of the (already rounded) inputs.

Tier A (``*_loops``, ``*_dict``) is the definition with dicts and loops;
Tier B restates it with numpy sorting, gathers and float64 BLAS products.
"""
from __future__ import annotations

import numpy as np

SENTINEL = np.uint32(0xFFFFFFFF)
MAP_COLS = 27


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def check_geometry(shape, ks: int, stride: int, pad: int) -> None:
    if ks not in (1, 2, 3):
        raise ValueError("kernel size must be 1, 2 or 3")
    if stride < 1:
        raise ValueError("stride must be positive")
    if pad < 0 or pad >= ks:
        raise ValueError("padding must be in [0, ks)")
    if any(int(d) < 1 for d in shape):
        raise ValueError("grid dimensions must be positive")
    if any(d < 1 for d in out_shape(shape, ks, stride, pad)[1:]):
        raise ValueError("empty output grid")


def out_shape(shape, ks: int, stride: int, pad: int) -> tuple:
    """(B, Xo, Yo, Zo) with Xo = (X + 2 pad - ks) // stride + 1."""
    B, X, Y, Z = (int(d) for d in shape)
    return (B,) + tuple((d + 2 * pad - ks) // stride + 1 for d in (X, Y, Z))


def offsets(ks: int) -> np.ndarray:
    """[V][3] window positions (a, b, c); row k = (a ks + b) ks + c."""
    r = range(ks)
    return np.array([(a, b, c) for a in r for b in r for c in r], dtype=np.int64)


def validate(coords, shape) -> None:
    coords = np.asarray(coords)
    if coords.ndim != 2 or coords.shape[1] != 4:
        raise ValueError("coords must be [N, 4]")
    lim = np.asarray(shape, dtype=np.int64)
    c = coords.astype(np.int64)
    if c.size and ((c < 0).any() or (c >= lim[None, :]).any()):
        raise ValueError("coordinate out of range")


# ============================================================================
# Tier A: the definition, with dicts and loops
# ============================================================================

def out_coords_loops(coords, shape, ks: int, stride: int, pad: int) -> np.ndarray:
    """Active output sites: every output site whose window holds an active input, lexicographic order.

    Walks every input voxel and every window position, and keeps the output
    sites o with o * stride - pad + a = the voxel's coordinate on each axis.
    """
    validate(coords, shape)
    check_geometry(shape, ks, stride, pad)
    _, Xo, Yo, Zo = out_shape(shape, ks, stride, pad)
    found = set()
    for b, x, y, z in np.asarray(coords).tolist():
        for a, bb, c in offsets(ks).tolist():
            qx, qy, qz = x + pad - a, y + pad - bb, z + pad - c
            if qx % stride or qy % stride or qz % stride:
                continue
            ox, oy, oz = qx // stride, qy // stride, qz // stride
            if 0 <= ox < Xo and 0 <= oy < Yo and 0 <= oz < Zo:
                found.add((b, ox, oy, oz))
    return np.array(sorted(found), dtype=np.int32).reshape(-1, 4)


def neighbor_map_dict(coords_in, shape, coords_out, ks: int, stride: int, pad: int) -> np.ndarray:
    """nmap[o][k] = row of the input voxel at o * stride - pad + offset_k, or the sentinel."""
    validate(coords_in, shape)
    check_geometry(shape, ks, stride, pad)
    oshape = out_shape(shape, ks, stride, pad)
    validate(coords_out, oshape)
    _, X, Y, Z = (int(d) for d in shape)
    table: dict[tuple, int] = {}
    for i, t in enumerate(np.asarray(coords_in).tolist()):
        if tuple(t) in table:
            raise ValueError("duplicate input coordinate")
        table[tuple(t)] = i
    seen = set()
    for t in np.asarray(coords_out).tolist():
        if tuple(t) in seen:
            raise ValueError("duplicate output coordinate")
        seen.add(tuple(t))
    nmap = np.full((len(coords_out), MAP_COLS), SENTINEL, dtype=np.uint32)
    for o, (b, x, y, z) in enumerate(np.asarray(coords_out).tolist()):
        for k, (a, bb, c) in enumerate(offsets(ks).tolist()):
            px, py, pz = x * stride - pad + a, y * stride - pad + bb, z * stride - pad + c
            if 0 <= px < X and 0 <= py < Y and 0 <= pz < Z:
                j = table.get((b, px, py, pz))
                if j is not None:
                    nmap[o, k] = j
    return nmap


def fwd_loops(feats, weight, bias, nmap) -> np.ndarray:
    """out[o] = bias + sum over valid k of X[nmap[o][k]] @ W[k]."""
    X, W = _f64(feats), _f64(weight)
    nout, co = nmap.shape[0], W.shape[2]
    bvec = np.zeros(co) if bias is None else _f64(bias)
    out = np.zeros((nout, co))
    for o in range(nout):
        acc = bvec.copy()
        for k in range(W.shape[0]):
            j = int(nmap[o, k])
            if j != int(SENTINEL):
                acc += X[j] @ W[k]
        out[o] = acc
    return out


def dgrad_scatter(dout, weight, nmap, n_in: int) -> np.ndarray:
    """dX[j] gets W[k] @ dY[o] from every valid (o, k) with nmap[o][k] = j."""
    dY, W = _f64(dout), _f64(weight)
    dX = np.zeros((n_in, W.shape[1]))
    for o in range(nmap.shape[0]):
        for k in range(W.shape[0]):
            j = int(nmap[o, k])
            if j != int(SENTINEL):
                dX[j] += W[k] @ dY[o]
    return dX


def wgrad_loops(feats, dout, nmap, V: int) -> np.ndarray:
    """dW[k] = sum over outputs o with a valid k of outer(X[nmap[o][k]], dY[o])."""
    X, dY = _f64(feats), _f64(dout)
    dW = np.zeros((V, X.shape[1], dY.shape[1]))
    for o in range(nmap.shape[0]):
        for k in range(V):
            j = int(nmap[o, k])
            if j != int(SENTINEL):
                dW[k] += np.outer(X[j], dY[o])
    return dW


# ============================================================================
# Tier B: the same definition, vectorised
# ============================================================================

def _linear(c: np.ndarray, shape) -> np.ndarray:
    _, X, Y, Z = (int(d) for d in shape)
    c = c.astype(np.int64)
    return ((c[:, 0] * X + c[:, 1]) * Y + c[:, 2]) * Z + c[:, 3]


def out_coords(coords, shape, ks: int, stride: int, pad: int) -> np.ndarray:
    """Tier B output sites: candidate keys of every (voxel, window position), unique and sorted."""
    validate(coords, shape)
    check_geometry(shape, ks, stride, pad)
    oshape = out_shape(shape, ks, stride, pad)
    c = np.asarray(coords).astype(np.int64).reshape(-1, 4)
    lim = np.array(oshape[1:], dtype=np.int64)
    keys = []
    for off in offsets(ks):
        q = c[:, 1:] + pad - off[None, :]
        ok = ((q % stride) == 0).all(axis=1)
        o = q // stride
        ok &= ((o >= 0) & (o < lim[None, :])).all(axis=1)
        keys.append(_linear(np.concatenate([c[ok, :1], o[ok]], axis=1), oshape))
    u = np.unique(np.concatenate(keys)) if keys else np.zeros(0, np.int64)
    _, Xo, Yo, Zo = oshape
    out = np.stack([u // (Xo * Yo * Zo), (u // (Yo * Zo)) % Xo, (u // Zo) % Yo, u % Zo], axis=1)
    return out.astype(np.int32).reshape(-1, 4)


def neighbor_map(coords_in, shape, coords_out, ks: int, stride: int, pad: int) -> np.ndarray:
    """Tier B map: sorted input keys + binary search, per-axis bounds first."""
    validate(coords_in, shape)
    check_geometry(shape, ks, stride, pad)
    oshape = out_shape(shape, ks, stride, pad)
    validate(coords_out, oshape)
    ci = np.asarray(coords_in).astype(np.int64).reshape(-1, 4)
    co = np.asarray(coords_out).astype(np.int64).reshape(-1, 4)
    keys = _linear(ci, shape)
    order = np.argsort(keys, kind="stable")
    skeys = keys[order]
    if len(skeys) > 1 and (np.diff(skeys) == 0).any():
        raise ValueError("duplicate input coordinate")
    okeys = np.sort(_linear(co, oshape))
    if len(okeys) > 1 and (np.diff(okeys) == 0).any():
        raise ValueError("duplicate output coordinate")
    nmap = np.full((len(co), MAP_COLS), SENTINEL, dtype=np.uint32)
    if len(ci) == 0 or len(co) == 0:
        return nmap
    lim = np.array(shape[1:], dtype=np.int64)
    for k, off in enumerate(offsets(ks)):
        p = co[:, 1:] * stride - pad + off[None, :]
        inb = ((p >= 0) & (p < lim[None, :])).all(axis=1)
        q = _linear(np.concatenate([co[:, :1], p], axis=1), shape)
        pos = np.minimum(np.searchsorted(skeys, q), len(skeys) - 1)
        hit = inb & (skeys[pos] == q)
        nmap[hit, k] = order[pos[hit]].astype(np.uint32)
    return nmap


def masks(nmap) -> np.ndarray:
    valid = np.asarray(nmap) != SENTINEL
    return (valid.astype(np.int64) << np.arange(MAP_COLS, dtype=np.int64)[None, :]).sum(axis=1)


def zorder_keys(coords, shape) -> np.ndarray:
    """Batch above the z-order code of (x, y, z), x most significant in each bit triplet."""
    nb = 0
    while (1 << nb) < max(int(d) for d in shape[1:]):
        nb += 1
    c = np.asarray(coords).astype(np.int64).reshape(-1, 4)
    code = np.zeros(len(c), dtype=np.int64)
    for bit in range(nb):
        code |= ((c[:, 1] >> bit) & 1) << (3 * bit + 2)
        code |= ((c[:, 2] >> bit) & 1) << (3 * bit + 1)
        code |= ((c[:, 3] >> bit) & 1) << (3 * bit)
    return (c[:, 0] << (3 * nb)) | code


def sort_perm(coords_out, nmap, oshape) -> np.ndarray:
    """GEMM row order of the outputs: ascending (mask, z-order code over the output grid)."""
    return np.lexsort((zorder_keys(coords_out, oshape), masks(nmap))).astype(np.int64)


def _pairs(nmap, k):
    col = np.asarray(nmap)[:, k]
    I = np.nonzero(col != SENTINEL)[0]
    return I, col[I].astype(np.int64)


def fwd(feats, weight, bias, nmap) -> np.ndarray:
    X, W = _f64(feats), _f64(weight)
    out = np.zeros((np.asarray(nmap).shape[0], W.shape[2]))
    if bias is not None:
        out += _f64(bias)[None, :]
    for k in range(W.shape[0]):
        I, J = _pairs(nmap, k)
        if I.size:
            out[I] += X[J] @ W[k]
    return out


def dgrad(dout, weight, nmap, n_in: int) -> np.ndarray:
    dY, W = _f64(dout), _f64(weight)
    dX = np.zeros((n_in, W.shape[1]))
    for k in range(W.shape[0]):
        I, J = _pairs(nmap, k)
        if I.size:
            dX[J] += dY[I] @ W[k].T
    return dX


def wgrad(feats, dout, nmap, V: int) -> np.ndarray:
    X, dY = _f64(feats), _f64(dout)
    dW = np.zeros((V, X.shape[1], dY.shape[1]))
    for k in range(V):
        I, J = _pairs(nmap, k)
        if I.size:
            dW[k] = X[J].T @ dY[I]
    return dW


def dbias(dout) -> np.ndarray:
    return _f64(dout).sum(axis=0)
