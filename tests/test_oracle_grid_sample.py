"""Pins for the sparse grid-sampling oracle (CPU only).

The oracle is checked against torch's dense ``grid_sample`` (trilinear,
align_corners=True, zero padding) on the zero-filled dense volume, a library
routine that shares nothing with it, and against that routine's autograd for
the backward pass; plus hand-derived cases, the adjoint identity between the
two passes and a planted mistake that the dense comparison must catch.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import grid_sample as G


def _sparse_set(rng, shape, p, C):
    B, X, Y, Z = shape
    act = rng.random((B, X, Y, Z)) < p
    coords = np.argwhere(act).astype(np.int32)
    feats = rng.standard_normal((len(coords), C))
    return coords, feats


def _points(rng, coords, shape, m):
    """Points near active voxels, anywhere in the box, and a few outside it or with bad batches."""
    B, X, Y, Z = shape
    k = m // 2
    pick = coords[rng.integers(0, len(coords), k)].astype(np.float64)
    near = pick + np.concatenate([np.zeros((k, 1)), rng.uniform(-1, 1, (k, 3))], 1)
    box = np.stack([rng.integers(0, B, m - k), rng.uniform(-1.5, X + 0.5, m - k),
                    rng.uniform(-1.5, Y + 0.5, m - k), rng.uniform(-1.5, Z + 0.5, m - k)], 1)
    return np.concatenate([near, box]).astype(np.float32).astype(np.float64)


def _dense_sample(coords, feats, shape, points, need_grad=False, dout=None):
    """torch grid_sample on the zero-filled dense volume, per sample; returns out (and dV at the sites)."""
    B, X, Y, Z = shape
    C = feats.shape[1]
    vol = torch.zeros((B, C, X, Y, Z), dtype=torch.float64)
    c = torch.from_numpy(coords.astype(np.int64))
    vol[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]] = torch.from_numpy(feats)
    vol.requires_grad_(need_grad)
    out = torch.zeros((len(points), C), dtype=torch.float64)
    for b in range(B):
        sel = np.nonzero(points[:, 0] == b)[0]
        if len(sel) == 0:
            continue
        p = torch.from_numpy(points[sel, 1:4])
        size = torch.tensor([X, Y, Z], dtype=torch.float64)
        g = 2.0 * p / (size - 1) - 1.0           # align_corners=True normalisation
        grid = g[:, [2, 1, 0]].reshape(1, len(sel), 1, 1, 3)  # (w, h, d) = (z, y, x)
        o = Fn.grid_sample(vol[b:b + 1], grid, mode="bilinear", padding_mode="zeros", align_corners=True)
        out = out.index_put((torch.from_numpy(sel),), o.reshape(C, len(sel)).T)
    if not need_grad:
        return out.detach().numpy()
    (out * torch.from_numpy(dout)).sum().backward()
    dV = vol.grad[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]]
    return out.detach().numpy(), dV.numpy()


SHAPE = (2, 7, 6, 9)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_forward_matches_dense_grid_sample(seed):
    rng = np.random.default_rng(seed)
    coords, feats = _sparse_set(rng, SHAPE, 0.4, 5)
    pts = _points(rng, coords, SHAPE, 400)
    ref = _dense_sample(coords, feats, SHAPE, pts)
    np.testing.assert_allclose(G.sample_fwd(coords, feats, SHAPE, pts), ref, atol=1e-12)
    np.testing.assert_allclose(G.sample_fwd_loops(coords, feats, SHAPE, pts), ref, atol=1e-12)


@pytest.mark.parametrize("seed", [3, 4])
def test_backward_matches_dense_autograd(seed):
    rng = np.random.default_rng(seed)
    coords, feats = _sparse_set(rng, SHAPE, 0.5, 4)
    pts = _points(rng, coords, SHAPE, 300)
    dout = rng.standard_normal((len(pts), 4))
    _, dV = _dense_sample(coords, feats, SHAPE, pts, need_grad=True, dout=dout)
    np.testing.assert_allclose(G.sample_bwd(coords, SHAPE, pts, dout), dV, atol=1e-12)
    np.testing.assert_allclose(G.sample_bwd_loops(coords, SHAPE, pts, dout), dV, atol=1e-12)


def test_adjoint_identity():
    rng = np.random.default_rng(5)
    coords, feats = _sparse_set(rng, SHAPE, 0.3, 3)
    pts = _points(rng, coords, SHAPE, 200)
    dout = rng.standard_normal((len(pts), 3))
    lhs = np.sum(G.sample_fwd(coords, feats, SHAPE, pts) * dout)
    rhs = np.sum(feats * G.sample_bwd(coords, SHAPE, pts, dout))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_hand_cases():
    shape = (2, 4, 4, 4)
    coords = np.array([[0, 1, 1, 1], [0, 2, 1, 1], [1, 0, 0, 0]], np.int32)
    a, b, c = np.array([1.0, 2.0]), np.array([10.0, -4.0]), np.array([7.0, 7.0])
    feats = np.stack([a, b, c])
    cases = [
        ([0, 1, 1, 1], a),                       # at a voxel: its features
        ([0, 1.5, 1, 1], 0.5 * a + 0.5 * b),     # midway along x
        ([0, 1.25, 1, 1], 0.75 * a + 0.25 * b),
        ([0, 1, 1.5, 1], 0.5 * a),               # the other corner along y is absent
        ([0, 1.5, 1.5, 1.5], (a + b) / 8),       # 2 of 8 corners present, 1/8 each
        ([1, 0, 0, 0], c),
        ([1, -0.5, 0, 0], 0.5 * c),              # half outside the grid: no renormalisation
        ([1, -1.5, 0, 0], 0 * c),                # wholly outside
        ([1, 1, 1, 1], 0 * c),                   # other sample's voxels are not seen
        ([2, 1, 1, 1], 0 * c),                   # batch out of range
        ([-1, 1, 1, 1], 0 * c),
        ([0.5, 1, 1, 1], 0 * c),                 # batch not an integer
        ([0, np.nan, 1, 1], 0 * c),
        ([0, np.inf, 1, 1], 0 * c),
    ]
    pts = np.array([p for p, _ in cases], np.float64)
    want = np.stack([v for _, v in cases])
    np.testing.assert_allclose(G.sample_fwd(coords, feats, shape, pts), want, atol=1e-15)
    np.testing.assert_allclose(G.sample_fwd_loops(coords, feats, shape, pts), want, atol=1e-15)
    # backward of one point midway along x: half of dout to each voxel
    d = G.sample_bwd(coords, shape, np.array([[0, 1.5, 1, 1]]), np.array([[2.0, 4.0]]))
    np.testing.assert_allclose(d, [[1.0, 2.0], [1.0, 2.0], [0.0, 0.0]], atol=1e-15)


def test_partition_of_unity():
    # constant features on a fully active box: any point with all corners inside samples the constant
    shape = (1, 5, 5, 5)
    coords = np.argwhere(np.ones(shape, bool)).astype(np.int32)
    feats = np.full((len(coords), 2), 3.5)
    rng = np.random.default_rng(6)
    pts = np.concatenate([np.zeros((100, 1)), rng.uniform(0, 4, (100, 3))], 1)
    np.testing.assert_allclose(G.sample_fwd(coords, feats, shape, pts), 3.5, atol=1e-13)


def test_planted_mistake_is_caught():
    # swapping t and 1 - t in the weights must disagree with the dense routine
    rng = np.random.default_rng(7)
    coords, feats = _sparse_set(rng, SHAPE, 0.5, 3)
    pts = _points(rng, coords, SHAPE, 200)
    ref = _dense_sample(coords, feats, SHAPE, pts)
    idx, w = G.corner_table(coords, SHAPE, pts)
    flipped = idx[:, ::-1]  # corner j read with the weight of corner 7 - j
    bad = np.zeros_like(ref)
    for j in range(8):
        hit = flipped[:, j] >= 0
        bad[hit] += w[hit, j:j + 1] * feats[flipped[hit, j]]
    assert np.abs(bad - ref).max() > 1e-3


def test_empty_inputs():
    shape = (1, 3, 3, 3)
    coords = np.zeros((0, 4), np.int32)
    assert G.sample_fwd(coords, np.zeros((0, 2)), shape, np.array([[0, 1.0, 1, 1]])).tolist() == [[0.0, 0.0]]
    assert G.sample_fwd(np.array([[0, 1, 1, 1]]), np.ones((1, 2)), shape, np.zeros((0, 4))).shape == (0, 2)
