"""Pins for the generalised (strided) sparse-convolution oracle (CPU only).

Expected values come from hand derivations (tests/golden/sparse_conv_hand.json),
an all-pairs search, torch's dense ``conv3d`` with stride and padding (float64)
on the zero-filled grid and its autograd, a dense all-ones convolution of the
occupancy for the output sites, and identities the operator must satisfy;
planted mistakes check that the dense comparison rejects plausible errors.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import sparse_conv as SC
from oracle import subm as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
S = int(SC.SENTINEL)
GEOMS = [(2, 2, 0), (3, 2, 1), (3, 1, 1), (3, 1, 0), (2, 1, 1), (1, 2, 0), (3, 3, 2), (2, 3, 1)]

with open(os.path.join(GOLD, "sparse_conv_hand.json")) as f:
    HAND = json.load(f)["cases"]


def _rows(n, dicts):
    out = np.full((n, 27), S, dtype=np.uint32)
    for i, d in enumerate(dicts):
        for k, j in d.items():
            out[i, int(k)] = j
    return out


def _grid(rng, shape, p):
    act = rng.random(shape) < p
    return np.argwhere(act).astype(np.int32)


@pytest.mark.parametrize("name", sorted(HAND))
@pytest.mark.parametrize("tier", ["A", "B"])
def test_hand_cases(name, tier):
    c = HAND[name]
    coords = np.array(c["coords"], dtype=np.int32)
    shape, ks, s, p = tuple(c["shape"]), c["ks"], c["stride"], c["pad"]
    oc = SC.out_coords_loops(coords, shape, ks, s, p) if tier == "A" else SC.out_coords(coords, shape, ks, s, p)
    assert oc.tolist() == c["out_coords"]
    nm = (SC.neighbor_map_dict if tier == "A" else SC.neighbor_map)(coords, shape, oc, ks, s, p)
    assert np.array_equal(nm, _rows(len(oc), c["nmap"]))
    assert SC.masks(nm).tolist() == c["mask"]
    assert SC.sort_perm(oc, nm, SC.out_shape(shape, ks, s, p)).tolist() == c["perm"]
    if "numeric" in c:
        v = c["numeric"]
        X = np.array(v["X"], dtype=np.float64)[:, None]
        W = np.array(v["W"], dtype=np.float64)[:, None, None]
        b = np.array([v["bias"]])
        dY = np.array(v["dY"], dtype=np.float64)[:, None]
        if tier == "A":
            out, dX = SC.fwd_loops(X, W, b, nm), SC.dgrad_scatter(dY, W, nm, len(X))
            dW = SC.wgrad_loops(X, dY, nm, ks ** 3)
        else:
            out, dX, dW = SC.fwd(X, W, b, nm), SC.dgrad(dY, W, nm, len(X)), SC.wgrad(X, dY, nm, ks ** 3)
        assert out[:, 0].tolist() == v["out"]
        assert dX[:, 0].tolist() == v["dX"]
        assert dW[:, 0, 0].tolist() == v["dW"]
        assert SC.dbias(dY)[0] == v["dbias"]


def _dense_sites(coords, shape, ks, s, p):
    """Output sites from torch: an all-ones conv3d of the occupancy, non-zero sites in C order."""
    B = shape[0]
    occ = torch.zeros((B, 1) + tuple(shape[1:]), dtype=torch.float64)
    c = torch.from_numpy(coords.astype(np.int64))
    occ[c[:, 0], 0, c[:, 1], c[:, 2], c[:, 3]] = 1.0
    cnt = Fn.conv3d(occ, torch.ones((1, 1, ks, ks, ks), dtype=torch.float64), stride=s, padding=p)
    return np.argwhere(cnt[:, 0].numpy() > 0).astype(np.int32), cnt[:, 0].numpy()


@pytest.mark.parametrize("ks,s,p", GEOMS)
@pytest.mark.parametrize("seed", [0, 1])
def test_out_sites_against_dense_occupancy(ks, s, p, seed):
    rng = np.random.default_rng(100 + seed)
    shape = (2, 9, 7, 8)
    coords = _grid(rng, shape, 0.08)
    ref, cnt = _dense_sites(coords, shape, ks, s, p)
    assert SC.out_coords(coords, shape, ks, s, p).tolist() == ref.tolist()
    assert SC.out_coords_loops(coords, shape, ks, s, p).tolist() == ref.tolist()
    # the map's popcount is the number of active inputs in each output's window
    nm = SC.neighbor_map(coords, shape, ref, ks, s, p)
    pc = (nm != S).sum(axis=1)
    assert pc.tolist() == [int(cnt[b, x, y, z]) for b, x, y, z in ref.tolist()]


def _brute(coords_in, coords_out, ks, s, p):
    """All-pairs search: input j sits in output o's window at position d = c_j - (o s - p) in [0, ks)^3."""
    ci = np.asarray(coords_in, dtype=np.int64)
    co = np.asarray(coords_out, dtype=np.int64)
    nm = np.full((len(co), 27), S, dtype=np.uint32)
    for o in range(len(co)):
        for j in range(len(ci)):
            if ci[j, 0] != co[o, 0]:
                continue
            d = ci[j, 1:] - (co[o, 1:] * s - p)
            if np.all((d >= 0) & (d < ks)):
                nm[o, int((d[0] * ks + d[1]) * ks + d[2])] = j
    return nm


@pytest.mark.parametrize("ks,s,p", GEOMS)
def test_map_bruteforce(ks, s, p):
    rng = np.random.default_rng(7)
    shape = (2, 7, 6, 5)
    coords = _grid(rng, shape, 0.15)
    rng.shuffle(coords)
    oc = SC.out_coords(coords, shape, ks, s, p)
    ref = _brute(coords, oc, ks, s, p)
    assert np.array_equal(SC.neighbor_map(coords, shape, oc, ks, s, p), ref)
    assert np.array_equal(SC.neighbor_map_dict(coords, shape, oc, ks, s, p), ref)
    # columns past the kernel volume are never used
    assert (ref[:, ks ** 3:] == S).all()


def test_submanifold_special_case():
    """ks=3, s=1, p=1 with the input sites as outputs is the submanifold map (pinned on its own)."""
    rng = np.random.default_rng(3)
    shape = (2, 8, 8, 8)
    coords = _grid(rng, shape, 0.2)
    rng.shuffle(coords)
    nm = SC.neighbor_map(coords, shape, coords, 3, 1, 1)
    assert np.array_equal(nm, O.neighbor_map(coords, shape))
    assert np.array_equal(SC.sort_perm(coords, nm, shape), O.sort_perm(coords, nm, shape))


def _dense_pin(coords, oc, shape, ks, s, p, X, W, b, dY):
    """fwd, dX and dW from torch conv3d (stride s, padding p, float64) and its autograd."""
    B = shape[0]
    ci = X.shape[1]
    vol = torch.zeros((B, ci) + tuple(shape[1:]), dtype=torch.float64)
    c = torch.from_numpy(coords.astype(np.int64))
    vol[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]] = torch.from_numpy(X)
    vol.requires_grad_(True)
    V = ks ** 3
    # dense weight [co][ci][a][b][c] = W[(a ks + b) ks + c][ci][co]
    Wd = torch.from_numpy(W).reshape(ks, ks, ks, ci, -1).permute(4, 3, 0, 1, 2).contiguous()
    Wd.requires_grad_(True)
    y = Fn.conv3d(vol, Wd, bias=torch.from_numpy(b), stride=s, padding=p)
    o = torch.from_numpy(oc.astype(np.int64))
    out = y[o[:, 0], :, o[:, 1], o[:, 2], o[:, 3]]
    (out * torch.from_numpy(dY)).sum().backward()
    dX = vol.grad[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]].numpy()
    dW = Wd.grad.permute(2, 3, 4, 1, 0).reshape(V, ci, -1).numpy()
    return out.detach().numpy(), dX, dW


@pytest.mark.parametrize("ks,s,p", GEOMS)
def test_against_dense_conv(ks, s, p):
    rng = np.random.default_rng(11 + ks * 10 + s)
    shape = (2, 8, 9, 7)
    coords = _grid(rng, shape, 0.12)
    rng.shuffle(coords)
    ci, co = 3, 4
    X = rng.standard_normal((len(coords), ci))
    W = rng.standard_normal((ks ** 3, ci, co))
    b = rng.standard_normal(co)
    oc = SC.out_coords(coords, shape, ks, s, p)
    dY = rng.standard_normal((len(oc), co))
    out_r, dX_r, dW_r = _dense_pin(coords, oc, shape, ks, s, p, X, W, b, dY)
    nm = SC.neighbor_map(coords, shape, oc, ks, s, p)
    np.testing.assert_allclose(SC.fwd(X, W, b, nm), out_r, rtol=0, atol=1e-12)
    np.testing.assert_allclose(SC.dgrad(dY, W, nm, len(X)), dX_r, rtol=0, atol=1e-12)
    np.testing.assert_allclose(SC.wgrad(X, dY, nm, ks ** 3), dW_r, rtol=0, atol=1e-12)
    np.testing.assert_allclose(SC.dbias(dY), dY.sum(0), rtol=0, atol=1e-12)
    # Tier A on the same case
    nmA = SC.neighbor_map_dict(coords, shape, oc, ks, s, p)
    np.testing.assert_allclose(SC.fwd_loops(X, W, b, nmA), out_r, rtol=0, atol=1e-12)
    np.testing.assert_allclose(SC.dgrad_scatter(dY, W, nmA, len(X)), dX_r, rtol=0, atol=1e-12)
    np.testing.assert_allclose(SC.wgrad_loops(X, dY, nmA, ks ** 3), dW_r, rtol=0, atol=1e-12)


def _planted_map(kind, coords, shape, oc, ks, s, p):
    """Maps with a plausible mistake: swapped window axes, or the padding added instead of subtracted."""
    ci = np.asarray(coords, dtype=np.int64)
    lut = {tuple(t): j for j, t in enumerate(ci.tolist())}
    nm = np.full((len(oc), 27), S, dtype=np.uint32)
    for o, (b, x, y, z) in enumerate(np.asarray(oc).tolist()):
        for k, (a, bb, c) in enumerate(SC.offsets(ks).tolist()):
            if kind == "axes":
                a, c = c, a
            sgn = 1 if kind == "pad_sign" else -1
            q = (b, x * s + sgn * p + a, y * s + sgn * p + bb, z * s + sgn * p + c)
            if q in lut:
                nm[o, k] = lut[q]
    return nm


@pytest.mark.parametrize("kind", ["axes", "pad_sign", "transposed_w"])
def test_dense_pin_rejects_planted_mistakes(kind):
    rng = np.random.default_rng(5)
    shape, ks, s, p = (1, 8, 8, 8), 3, 2, 1
    coords = _grid(rng, shape, 0.3)
    ci = co = 3
    X = rng.standard_normal((len(coords), ci))
    W = rng.standard_normal((ks ** 3, ci, co))
    b = np.zeros(co)
    oc = SC.out_coords(coords, shape, ks, s, p)
    dY = rng.standard_normal((len(oc), co))
    out_r, _, _ = _dense_pin(coords, oc, shape, ks, s, p, X, W, b, dY)
    if kind == "transposed_w":
        bad = SC.fwd(X, np.ascontiguousarray(W.transpose(0, 2, 1)), b, SC.neighbor_map(coords, shape, oc, ks, s, p))
    else:
        bad = SC.fwd(X, W, b, _planted_map(kind, coords, shape, oc, ks, s, p))
    assert np.abs(bad - out_r).max() > 1e-3


def test_adjoint_and_integer_counts():
    rng = np.random.default_rng(9)
    shape, ks, s, p = (2, 10, 10, 10), 3, 2, 1
    coords = _grid(rng, shape, 0.1)
    oc = SC.out_coords(coords, shape, ks, s, p)
    nm = SC.neighbor_map(coords, shape, oc, ks, s, p)
    X = rng.standard_normal((len(coords), 5))
    W = rng.standard_normal((27, 5, 6))
    dY = rng.standard_normal((len(oc), 6))
    # <fwd(X), dY> = <X, dX>
    lhs = float((SC.fwd(X, W, None, nm) * dY).sum())
    rhs = float((X * SC.dgrad(dY, W, nm, len(X))).sum())
    assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(lhs))
    # <dW, U> = <fwd_U(X), dY>
    U = rng.standard_normal(W.shape)
    assert abs(float((SC.wgrad(X, dY, nm, 27) * U).sum()) - float((SC.fwd(X, U, None, nm) * dY).sum())) <= 1e-9 * 1e3
    # ones: fwd counts the window's inputs, dX counts the outputs each input feeds, dW[k] counts pairs
    one_x, one_w, one_y = np.ones((len(coords), 1)), np.ones((27, 1, 1)), np.ones((len(oc), 1))
    assert SC.fwd(one_x, one_w, None, nm)[:, 0].tolist() == (nm != S).sum(1).tolist()
    fed = np.zeros(len(coords))
    for j in nm[nm != S].astype(np.int64):
        fed[j] += 1
    assert SC.dgrad(one_y, one_w, nm, len(coords))[:, 0].tolist() == fed.tolist()
    assert SC.wgrad(one_x, one_y, nm, 27)[:, 0, 0].tolist() == (nm != S).sum(0)[:27].tolist()


def test_errors_and_empty():
    shape = (1, 4, 4, 4)
    with pytest.raises(ValueError):
        SC.out_coords(np.array([[0, 4, 0, 0]], np.int32), shape, 2, 2, 0)
    with pytest.raises(ValueError):
        SC.neighbor_map(np.array([[0, 1, 1, 1], [0, 1, 1, 1]], np.int32), shape, np.zeros((0, 4), np.int32), 2, 2, 0)
    with pytest.raises(ValueError):
        SC.neighbor_map(np.array([[0, 1, 1, 1]], np.int32), shape, np.array([[0, 0, 0, 0]] * 2, np.int32), 2, 2, 0)
    with pytest.raises(ValueError):
        SC.out_coords(np.zeros((0, 4), np.int32), shape, 4, 1, 0)
    with pytest.raises(ValueError):
        SC.out_coords(np.zeros((0, 4), np.int32), shape, 2, 1, 2)
    assert SC.out_coords(np.zeros((0, 4), np.int32), shape, 2, 2, 0).shape == (0, 4)
    assert SC.out_coords_loops(np.zeros((0, 4), np.int32), shape, 2, 2, 0).shape == (0, 4)
    assert SC.out_shape((2, 64, 63, 1), 3, 2, 1) == (2, 32, 32, 1)
