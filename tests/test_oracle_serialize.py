"""Pins for the serialisation oracle (CPU only).

The Hilbert index is checked against properties any Hilbert curve has, none of
which restates the transform: it is a bijection of the 2^n cube onto
[0, 8^n), consecutive indices are unit steps, every aligned block of 8^m
indices fills an aligned cube of side 2^m, the curve starts at the origin and
ends at a corner one edge away.  The z-order code is checked against the row
sort's key and against single-bit examples.  Round trips and the automatic
width follow the pages' encode_seq / decode_seq description.
"""
import json
import os

import numpy as np
import pytest

from oracle import serialize as S
from oracle import subm as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _all_cells(n):
    side = 1 << n
    g = np.stack(np.meshgrid(np.arange(side), np.arange(side), np.arange(side), indexing="ij"), -1)
    return g.reshape(-1, 3)


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_hilbert_bijection_and_unit_steps(n):
    side = 1 << n
    pts = [S.hilbert_point(h, n) for h in range(side ** 3)]
    assert len(set(pts)) == side ** 3
    assert all(0 <= v < side for p in pts for v in p)
    steps = np.abs(np.diff(np.array(pts), axis=0)).sum(axis=1)
    assert (steps == 1).all()
    for h, p in enumerate(pts):
        assert S.hilbert_index(*p, n) == h


@pytest.mark.parametrize("n", [2, 3, 4])
def test_hilbert_aligned_subcubes(n):
    pts = np.array([S.hilbert_point(h, n) for h in range(8 ** n)])
    for m in range(1, n):
        block = 8 ** m
        for k in range(8 ** (n - m)):
            p = pts[k * block:(k + 1) * block]
            lo, hi = p.min(axis=0), p.max(axis=0)
            assert ((lo % (1 << m)) == 0).all()
            assert ((hi - lo) == (1 << m) - 1).all()


@pytest.mark.parametrize("n", [1, 2, 3, 5])
def test_hilbert_endpoints(n):
    side = 1 << n
    assert S.hilbert_point(0, n) == (0, 0, 0)
    end = np.array(S.hilbert_point(side ** 3 - 1, n))
    assert sorted(end.tolist()) == [0, 0, side - 1]


def test_hilbert_planted_mistake_breaks_unit_steps():
    # drop the final Gray flip of the transpose: the curve must stop being continuous
    def broken(x, y, z, nbits):
        t = [x, y, z]
        top = 1 << (nbits - 1)
        q = top
        while q > 1:
            low = q - 1
            for i in range(3):
                if t[i] & q:
                    t[0] ^= low
                else:
                    sw = (t[0] ^ t[i]) & low
                    t[0] ^= sw
                    t[i] ^= sw
            q >>= 1
        for i in (1, 2):
            t[i] ^= t[i - 1]
        return t

    n = 3
    idx = {c: O.morton_code(*broken(*c, n), n) for c in map(tuple, _all_cells(n).tolist())}
    order = sorted(idx, key=idx.get)
    steps = np.abs(np.diff(np.array(order), axis=0)).sum(axis=1)
    assert not (steps == 1).all()


def test_zorder_matches_row_sort_key():
    rng = np.random.default_rng(3)
    shape = (3, 40, 17, 29)
    c = np.stack([rng.integers(0, s, 500) for s in shape], 1).astype(np.int32)
    codes = S.encode_seq(c, shape, "z_order")
    np.testing.assert_array_equal(codes, O.zorder_keys(c, shape))


def test_zorder_single_bits():
    # n = 3: x bit j lands at 3j + 2, y bit j at 3j + 1, z bit j at 3j
    shape = (1, 8, 8, 8)
    for j in range(3):
        assert S.encode_seq([[0, 1 << j, 0, 0]], shape, "z_order")[0] == 1 << (3 * j + 2)
        assert S.encode_seq([[0, 0, 1 << j, 0]], shape, "z_order")[0] == 1 << (3 * j + 1)
        assert S.encode_seq([[0, 0, 0, 1 << j]], shape, "z_order")[0] == 1 << (3 * j)
    assert S.encode_seq([[1, 0, 0, 0]], (2, 8, 8, 8), "z_order")[0] == 1 << 9


def test_pages_round_trip_example():
    # the pages' serialize snippet: two voxels in a 64^3 grid, round trip through z_order
    ex = json.load(open(os.path.join(GOLD, "serialize_example.json")))
    shape = tuple(ex["shape_bxyz"])
    c = np.array(ex["coords"], np.int64)
    for mode in S.MODES:
        codes = S.encode_seq(c, shape, mode)
        np.testing.assert_array_equal(S.decode_seq(codes, shape, mode), c)
    assert S.code_width(shape) == 32


@pytest.mark.parametrize("mode", S.MODES)
@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (2, 5, 9, 3), (3, 33, 20, 64), (1, 100, 7, 50)])
def test_round_trip_and_rejections(mode, shape):
    rng = np.random.default_rng(sum(shape))
    c = np.stack([rng.integers(0, s, 300) for s in shape], 1)
    codes = S.encode_seq(c, shape, mode)
    assert (codes >= 0).all() and (codes < (1 << S.code_bits(shape))).all()
    np.testing.assert_array_equal(S.decode_seq(codes, shape, mode), c)
    # distinct cells get distinct codes
    u = np.unique(c, axis=0)
    assert len(np.unique(S.encode_seq(u, shape, mode))) == len(u)
    # out of range in, -1 out; codes naming no grid cell decode to -1 rows
    bad = np.array([[-1, 0, 0, 0], [0, shape[1], 0, 0], [0, 0, 0, shape[3]], [shape[0], 0, 0, 0]])
    assert (S.encode_seq(bad, shape, mode) == -1).all()
    assert (S.decode_seq(np.array([-1, 1 << S.code_bits(shape)]), shape, mode) == -1).all()


def test_width_rule():
    assert S.code_bits((1, 64, 64, 64)) == 18 and S.code_width((1, 64, 64, 64)) == 32
    assert S.code_bits((2, 1024, 1024, 1024)) == 31 and S.code_width((2, 1024, 1024, 1024)) == 32
    assert S.code_bits((3, 1024, 1024, 1024)) == 32 and S.code_width((3, 1024, 1024, 1024)) == 64
    assert S.code_width((1, 2048, 1, 1)) == 64
    assert S.code_bits((1, 1, 1, 1)) == 0


def test_mode_is_checked():
    with pytest.raises(ValueError):
        S.encode_seq([[0, 0, 0, 0]], (1, 2, 2, 2), "morton")
