"""CPU oracle for voxel serialisation: z-order and Hilbert codes (test infrastructure).

This module is test infrastructure.  Only the test suite, the package smoke
check and the benchmark's CPU-baseline leg may import it; the HIP library and
its Python binding never do, and it shares no code with them.

What the pages fix (contributor report, page 1: section two, the module table
rows ops.serialize and kernels.cuda.serialize, and the key-function table
rows z_order_encode / decode, hilbert_encode / decode and encode_seq /
decode_seq; section three "minimal runnable", the serialize snippet):

* ``encode_seq(coords, shape, mode)`` maps int32 rows ``[b, x, y, z]`` to one
  code per voxel, ``mode`` is ``z_order`` or ``hilbert``, and
  ``decode_seq(codes, shape, mode)`` inverts it exactly (the snippet asserts
  the round trip);
* the code width, int32 or int64, is chosen from the spatial size.

The pages give no bit layout and no curve variant.  Readings taken here:

* n = ceil(log2(max(X, Y, Z))) bits per axis; the curve covers the cube of
  side 2**n that holds the grid.
* code = (b << 3n) | index(x, y, z): the batch sits above the spatial index,
  so the codes of one sample are contiguous.
* z-order index: bits interleaved from the top, each triplet (x, y, z) with x
  most significant -- the same key the row sort uses.
* Hilbert index: J. Skilling's transform ("Programming the Hilbert curve",
  AIP Conf. Proc. 707, 381 (2004)) with axes (x, y, z) in that order; the
  transposed bits are interleaved like the z-order index.
* width: int32 when the code needs at most 31 bits (so every code is a
  non-negative int32), else int64.

Pinned by tests/test_oracle_serialize.py against properties the curves must
have (bijection, unit steps, aligned sub-cubes, endpoints, round trips) and
the consistency of the z-order code with the row sort's key.  Skilling's
orientation convention itself has no published value table to pin against
here: within the family of Hilbert curves, the orientation is a reading.
"""
from __future__ import annotations

import numpy as np

from .subm import ceil_log2, morton_code, morton_decode

MODES = ("z_order", "hilbert")


def axis_bits(shape) -> int:
    """n = ceil(log2(max(X, Y, Z))) for shape (B, X, Y, Z)."""
    return ceil_log2(max(int(s) for s in shape[1:]))


def code_bits(shape) -> int:
    """Bits of a code: 3n for the spatial index plus ceil(log2(B)) for the batch."""
    return 3 * axis_bits(shape) + ceil_log2(int(shape[0]))


def code_width(shape) -> int:
    """32 when every code fits a non-negative int32, else 64."""
    return 32 if code_bits(shape) <= 31 else 64


# ---------------------------------------------------------------------------
# Hilbert: Skilling's transform between axes and the "transposed" index
# ---------------------------------------------------------------------------

def hilbert_transpose(x: int, y: int, z: int, nbits: int) -> list:
    """Axes -> transposed Hilbert index (Skilling): bit j of t[i] is index bit 3j + (2 - i)."""
    t = [x, y, z]
    if nbits == 0:
        return t
    top = 1 << (nbits - 1)
    q = top
    while q > 1:  # undo the excess work, from the top bit down
        low = q - 1
        for i in range(3):
            if t[i] & q:
                t[0] ^= low
            else:
                swap = (t[0] ^ t[i]) & low
                t[0] ^= swap
                t[i] ^= swap
        q >>= 1
    for i in (1, 2):  # Gray encode
        t[i] ^= t[i - 1]
    flip = 0
    q = top
    while q > 1:
        if t[2] & q:
            flip ^= q - 1
        q >>= 1
    return [v ^ flip for v in t]


def hilbert_untranspose(t: list, nbits: int) -> list:
    """Transposed Hilbert index -> axes: the inverse of hilbert_transpose."""
    a = list(t)
    if nbits == 0:
        return a
    g = a[2] >> 1  # Gray decode
    for i in (2, 1):
        a[i] ^= a[i - 1]
    a[0] ^= g
    q = 2
    while q != (1 << nbits):  # redo the work, from the bottom bit up
        low = q - 1
        for i in (2, 1, 0):
            if a[i] & q:
                a[0] ^= low
            else:
                swap = (a[0] ^ a[i]) & low
                a[0] ^= swap
                a[i] ^= swap
        q <<= 1
    return a


def hilbert_index(x: int, y: int, z: int, nbits: int) -> int:
    t = hilbert_transpose(x, y, z, nbits)
    return morton_code(t[0], t[1], t[2], nbits)


def hilbert_point(h: int, nbits: int) -> tuple:
    t = morton_decode(h, nbits)
    return tuple(hilbert_untranspose(list(t), nbits))


# ---------------------------------------------------------------------------
# encode_seq / decode_seq
# ---------------------------------------------------------------------------

def _check_mode(mode: str) -> None:
    if mode not in MODES:
        raise ValueError(f"mode must be one of {MODES}, got {mode!r}")


def encode_seq(coords, shape, mode: str) -> np.ndarray:
    """code[i] = (b << 3n) | index(x, y, z); -1 for a row outside the grid.  int64 array."""
    _check_mode(mode)
    n = axis_bits(shape)
    B, X, Y, Z = (int(s) for s in shape)
    out = []
    for b, x, y, z in np.asarray(coords).reshape(-1, 4).tolist():
        if not (0 <= b < B and 0 <= x < X and 0 <= y < Y and 0 <= z < Z):
            out.append(-1)
            continue
        idx = morton_code(x, y, z, n) if mode == "z_order" else hilbert_index(x, y, z, n)
        out.append((b << (3 * n)) | idx)
    return np.array(out, dtype=np.int64)


def decode_seq(codes, shape, mode: str) -> np.ndarray:
    """Rows [b, x, y, z] of the codes; [-1, -1, -1, -1] for a code that names no grid cell."""
    _check_mode(mode)
    n = axis_bits(shape)
    B, X, Y, Z = (int(s) for s in shape)
    out = []
    for c in np.asarray(codes).reshape(-1).tolist():
        c = int(c)
        if c < 0:
            out.append([-1, -1, -1, -1])
            continue
        b = c >> (3 * n)
        idx = c & ((1 << (3 * n)) - 1)
        x, y, z = morton_decode(idx, n) if mode == "z_order" else hilbert_point(idx, n)
        if not (b < B and x < X and y < Y and z < Z):
            out.append([-1, -1, -1, -1])
        else:
            out.append([b, x, y, z])
    return np.array(out, dtype=np.int64).reshape(-1, 4)
