"""CPU oracle for the 3x3x3 submanifold sparse convolution (test infrastructure).

This module is test infrastructure.  Only the test suite, the package smoke
check and the benchmark's CPU-baseline leg may import it; the HIP library and
its Python binding never do, and it shares no code with them.

What is computed, and where the pages say so
--------------------------------------------
* The operator is the submanifold convolution of FlexGEMM's
  ``sparse_submanifold_conv3d(feats, coords, shape, weight, bias)``
  (contributor report, page 1: section one "project positioning" and the
  section two table "key types and functions").  Output sites are the input
  sites.
* Coordinates are int32 rows ``[b, x, y, z]`` and the spatial shape is passed
  explicitly (page 1, section three "minimal runnable": the serialize and
  hashmap snippets).
* The GEMM reduction dimension is V * Ci with V = 27 offsets (page 2, the
  Triton compile-cache post, section six: the autotune-cache key and the
  ``BK`` comment of the masked implicit GEMM kernel signature).
* The neighbour map is a uint32 tensor (page 2, the same cache key's dtype
  list); the missing-neighbour sentinel is 0xFFFFFFFF.
* Rows are reordered by a ``sorted_idx`` permutation (page 2, kernel
  signature); the sort key is the 27-bit valid-neighbour mask, ties broken by
  the z-order code (page 1, z_order_encode in the serialize module).
* Gradients for feats and weight come back through the backward kernels
  (page 1, section two "how one call flows").

The pages give no formula.  The readings taken here are the plain ones:
offset index k = (dx+1)*9 + (dy+1)*3 + (dz+1) with dx on coordinate column 1;
cross-correlation sign (the voxel at c + offset_k meets W[k], as in a dense
conv3d with padding 1); no neighbours across batches or off the grid;
duplicates and out-of-range coordinates are errors.

Two tiers
---------
Tier A is the definition written out with a dict and loops (small inputs).
Tier B restates it with numpy sorting, gathers and float64 BLAS products (any
size); tests cross-check the tiers and pin both to dense convolution,
hand-derived cases and invariants.  Floats are float64 on the exact values of
the (already rounded) inputs.
"""
from __future__ import annotations

import numpy as np

SENTINEL = np.uint32(0xFFFFFFFF)
V = 27

# k = (dx+1)*9 + (dy+1)*3 + (dz+1)
OFFSETS = np.array([(dx, dy, dz) for dx in (-1, 0, 1) for dy in (-1, 0, 1) for dz in (-1, 0, 1)],
                   dtype=np.int64)
CENTRE = 13


def _f64(a) -> np.ndarray:
    """float64 numpy copy of a numpy array or CPU torch tensor (any float dtype)."""
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def _take(a, idx) -> np.ndarray:
    """float64 rows a[idx] of a numpy array or CPU torch tensor."""
    idx = np.asarray(idx, dtype=np.int64)
    if hasattr(a, "detach"):
        import torch
        return a.index_select(0, torch.from_numpy(idx)).double().numpy()
    return np.asarray(a)[idx].astype(np.float64)


def _take_col(a, idx, col: int) -> np.ndarray:
    """float64 entries a[idx, col] of a numpy array or CPU torch tensor."""
    idx = np.asarray(idx, dtype=np.int64)
    if hasattr(a, "detach"):
        import torch
        return a[:, col].index_select(0, torch.from_numpy(idx)).double().numpy()
    return np.asarray(a)[idx, col].astype(np.float64)


def validate(coords: np.ndarray, shape) -> None:
    """Raise ValueError for coordinates outside [0, B) x [0, X) x [0, Y) x [0, Z)."""
    coords = np.asarray(coords)
    if coords.ndim != 2 or coords.shape[1] != 4:
        raise ValueError("coords must be [N, 4]")
    lim = np.asarray(shape, dtype=np.int64)
    c = coords.astype(np.int64)
    if c.size and ((c < 0).any() or (c >= lim[None, :]).any()):
        raise ValueError("coordinate out of range")


# ============================================================================
# Tier A: the definition, with a dict and loops
# ============================================================================

def neighbor_map_dict(coords: np.ndarray, shape) -> np.ndarray:
    """nmap[i][k] = row of the voxel at coords[i] + offset_k, or the sentinel.

    A dict from (b, x, y, z) to row index stands in for the pages' coordinate
    hashmap (page 1, kernels.cuda.hash: insert, then lookup).
    """
    validate(coords, shape)
    B, X, Y, Z = (int(s) for s in shape)
    table: dict[tuple, int] = {}
    for i, (b, x, y, z) in enumerate(np.asarray(coords).tolist()):
        if (b, x, y, z) in table:
            raise ValueError("duplicate coordinate")
        table[(b, x, y, z)] = i
    n = len(table)
    nmap = np.full((n, V), SENTINEL, dtype=np.uint32)
    for i, (b, x, y, z) in enumerate(np.asarray(coords).tolist()):
        for k, (dx, dy, dz) in enumerate(OFFSETS.tolist()):
            px, py, pz = x + dx, y + dy, z + dz
            if 0 <= px < X and 0 <= py < Y and 0 <= pz < Z:
                j = table.get((b, px, py, pz))
                if j is not None:
                    nmap[i, k] = j
    return nmap


def ceil_log2(v: int) -> int:
    """Smallest e >= 0 with 2^e >= v."""
    e = 0
    while (1 << e) < v:
        e += 1
    return e


def morton_bits(shape) -> int:
    """Bits per axis of the z-order code: ceil(log2(max(X, Y, Z)))."""
    return ceil_log2(max(int(s) for s in shape[1:]))


def morton_code(x: int, y: int, z: int, nbits: int) -> int:
    """z-order code, built bit by bit from the top: each triplet is (x, y, z), x most significant."""
    code = 0
    for bit in range(nbits - 1, -1, -1):
        code = (code << 3) | (((x >> bit) & 1) << 2) | (((y >> bit) & 1) << 1) | ((z >> bit) & 1)
    return code


def morton_decode(code: int, nbits: int) -> tuple:
    x = y = z = 0
    for bit in range(nbits):
        z |= ((code >> (3 * bit)) & 1) << bit
        y |= ((code >> (3 * bit + 1)) & 1) << bit
        x |= ((code >> (3 * bit + 2)) & 1) << bit
    return x, y, z


def zorder_key(b: int, x: int, y: int, z: int, shape) -> int:
    """Batch index above the z-order code of (x, y, z)."""
    nb = morton_bits(shape)
    return (b << (3 * nb)) | morton_code(x, y, z, nb)


def masks_loop(nmap: np.ndarray) -> list:
    """mask[i] = sum over k of 2^k for the offsets whose neighbour exists."""
    out = []
    for row in np.asarray(nmap).tolist():
        m = 0
        for k, j in enumerate(row):
            if j != int(SENTINEL):
                m |= 1 << k
        out.append(m)
    return out


def sort_perm_tuples(coords: np.ndarray, nmap: np.ndarray, shape) -> np.ndarray:
    """perm[r] = original row at sorted position r; ascending by (mask, z-order key).

    Coordinates are unique, so the z-order key alone is unique and the order is total.
    """
    masks = masks_loop(nmap)
    keys = [(masks[i], zorder_key(b, x, y, z, shape))
            for i, (b, x, y, z) in enumerate(np.asarray(coords).tolist())]
    return np.array(sorted(range(len(keys)), key=lambda i: keys[i]), dtype=np.int64)


def fwd_loops(feats, weight, bias, nmap) -> np.ndarray:
    """out[i] = bias + sum over k with nmap[i][k] = j valid of X[j] @ W[k]."""
    X, W = _f64(feats), _f64(weight)
    n, co = X.shape[0], W.shape[2]
    bvec = np.zeros(co) if bias is None else _f64(bias)
    out = np.zeros((n, co))
    for i in range(n):
        acc = bvec.copy()
        for k in range(V):
            j = int(nmap[i, k])
            if j != int(SENTINEL):
                acc += X[j] @ W[k]
        out[i] = acc
    return out


def dgrad_scatter(dout, weight, nmap) -> np.ndarray:
    """Input gradient in scatter form: every valid (i, k, j = nmap[i][k]) adds W[k] @ dY[i] to dX[j]."""
    dY, W = _f64(dout), _f64(weight)
    n, ci = dY.shape[0], W.shape[1]
    dX = np.zeros((n, ci))
    for i in range(n):
        for k in range(V):
            j = int(nmap[i, k])
            if j != int(SENTINEL):
                dX[j] += W[k] @ dY[i]
    return dX


def wgrad_loops(feats, dout, nmap) -> np.ndarray:
    """dW[k] = sum over rows i with nmap[i][k] = j valid of outer(X[j], dY[i])."""
    X, dY = _f64(feats), _f64(dout)
    ci, co = X.shape[1], dY.shape[1]
    dW = np.zeros((V, ci, co))
    for i in range(X.shape[0]):
        for k in range(V):
            j = int(nmap[i, k])
            if j != int(SENTINEL):
                dW[k] += np.outer(X[j], dY[i])
    return dW


def dbias_loops(dout) -> np.ndarray:
    """dbias = sum over rows of dY."""
    dY = _f64(dout)
    acc = np.zeros(dY.shape[1])
    for i in range(dY.shape[0]):
        acc += dY[i]
    return acc


# ============================================================================
# Tier B: the same definition, vectorised
# ============================================================================

def linear_keys(coords: np.ndarray, shape) -> np.ndarray:
    """((b X + x) Y + y) Z + z as int64."""
    _, X, Y, Z = (int(s) for s in shape)
    c = np.asarray(coords).astype(np.int64)
    return ((c[:, 0] * X + c[:, 1]) * Y + c[:, 2]) * Z + c[:, 3]


def neighbor_map(coords: np.ndarray, shape) -> np.ndarray:
    """Tier B neighbour map: sorted linear keys + binary search, with per-axis bounds first."""
    validate(coords, shape)
    _, X, Y, Z = (int(s) for s in shape)
    c = np.asarray(coords).astype(np.int64)
    n = c.shape[0]
    keys = linear_keys(c, shape)
    order = np.argsort(keys, kind="stable")
    skeys = keys[order]
    if n > 1 and (np.diff(skeys) == 0).any():
        raise ValueError("duplicate coordinate")
    nmap = np.full((n, V), SENTINEL, dtype=np.uint32)
    if n == 0:
        return nmap
    lim = np.array([X, Y, Z], dtype=np.int64)
    for k in range(V):
        p = c[:, 1:] + OFFSETS[k][None, :]
        inb = ((p >= 0) & (p < lim[None, :])).all(axis=1)
        q = ((c[:, 0] * X + p[:, 0]) * Y + p[:, 1]) * Z + p[:, 2]
        pos = np.searchsorted(skeys, q)
        pos = np.minimum(pos, n - 1)
        hit = inb & (skeys[pos] == q)
        nmap[hit, k] = order[pos[hit]].astype(np.uint32)
    return nmap


def masks(nmap: np.ndarray) -> np.ndarray:
    valid = np.asarray(nmap) != SENTINEL
    return (valid.astype(np.int64) << np.arange(V, dtype=np.int64)[None, :]).sum(axis=1)


def zorder_keys(coords: np.ndarray, shape) -> np.ndarray:
    nb = morton_bits(shape)
    c = np.asarray(coords).astype(np.int64)
    code = np.zeros(c.shape[0], dtype=np.int64)
    for bit in range(nb):
        code |= ((c[:, 1] >> bit) & 1) << (3 * bit + 2)
        code |= ((c[:, 2] >> bit) & 1) << (3 * bit + 1)
        code |= ((c[:, 3] >> bit) & 1) << (3 * bit)
    return (c[:, 0] << (3 * nb)) | code


def sort_perm(coords: np.ndarray, nmap: np.ndarray, shape) -> np.ndarray:
    """Tier B permutation: lexsort by (mask, z-order key)."""
    return np.lexsort((zorder_keys(coords, shape), masks(nmap))).astype(np.int64)


def pairs(nmap: np.ndarray, k: int):
    """Rows I_k with a valid offset-k neighbour and those neighbours J_k (J_k is injective)."""
    col = np.asarray(nmap)[:, k]
    I = np.nonzero(col != SENTINEL)[0]
    return I, col[I].astype(np.int64)


def fwd(feats, weight, bias, nmap) -> np.ndarray:
    X, W = _f64(feats), _f64(weight)
    n, co = X.shape[0], W.shape[2]
    out = np.zeros((n, co))
    if bias is not None:
        out += _f64(bias)[None, :]
    for k in range(V):
        I, J = pairs(nmap, k)
        if I.size:
            out[I] += X[J] @ W[k]
    return out


def dgrad(dout, weight, nmap) -> np.ndarray:
    dY, W = _f64(dout), _f64(weight)
    dX = np.zeros((dY.shape[0], W.shape[1]))
    for k in range(V):
        I, J = pairs(nmap, k)
        if I.size:
            dX[J] += dY[I] @ W[k].T
    return dX


def wgrad(feats, dout, nmap) -> np.ndarray:
    X, dY = _f64(feats), _f64(dout)
    dW = np.zeros((V, X.shape[1], dY.shape[1]))
    for k in range(V):
        I, J = pairs(nmap, k)
        if I.size:
            dW[k] = X[J].T @ dY[I]
    return dW


def dbias(dout) -> np.ndarray:
    return _f64(dout).sum(axis=0)


# ---- sampled outputs (for inputs too large to compute whole) ---------------

def fwd_rows(feats, weight, bias, nmap, rows) -> np.ndarray:
    """out[rows] only: per row, the sum over its valid offsets (the definition, row by row)."""
    W = _f64(weight)
    co = W.shape[2]
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, co))
    if bias is not None:
        out += _f64(bias)[None, :]
    sub = np.asarray(nmap)[rows]
    for k in range(V):
        r = np.nonzero(sub[:, k] != SENTINEL)[0]
        if r.size:
            out[r] += _take(feats, sub[r, k]) @ W[k]
    return out


def dgrad_rows(dout, weight, nmap, rows) -> np.ndarray:
    """dX[rows] only, in scatter form: contributions (i, k) whose target nmap[i][k] is a sampled row."""
    W = _f64(weight)
    rows = np.asarray(rows, dtype=np.int64)
    where = {int(j): t for t, j in enumerate(rows.tolist())}
    dX = np.zeros((rows.size, W.shape[1]))
    nm = np.asarray(nmap)
    for k in range(V):
        col = nm[:, k].astype(np.int64)
        hit = np.nonzero(np.isin(col, rows))[0]
        if hit.size:
            tgt = np.array([where[int(j)] for j in col[hit]], dtype=np.int64)
            np.add.at(dX, tgt, _take(dout, hit) @ W[k].T)
    return dX


def wgrad_entries(feats, dout, nmap, entries) -> np.ndarray:
    """dW[k, a, c] for each (k, a, c) in entries: sum over valid rows i of X[nmap[i][k], a] * dY[i, c]."""
    out = np.zeros(len(entries))
    cache: dict[int, tuple] = {}
    for t, (k, a, c) in enumerate(entries):
        if k not in cache:
            cache[k] = pairs(nmap, k)
        I, J = cache[k]
        if I.size:
            out[t] = float(np.dot(_take_col(feats, J, a), _take_col(dout, I, c)))
    return out
