"""GPU parity of ssc_grid_sample_fwd / ssc_grid_sample_bwd against the grid-sampling oracle.

Tolerance as for the convolution: max|err| / max|ref| <= 1e-5 for fp32 and
2e-2 for fp16 / bf16 inputs with fp32 accumulation (the backward pass sums
each voxel's bucket in the order integer atomics placed it, so its last bits
may differ between runs).
"""
import numpy as np
import pytest
import torch

from oracle import grid_sample as G
from sparse_submanifold_convolution_amd import workloads as WL

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}


@pytest.fixture(scope="module")
def ssc():
    import sparse_submanifold_convolution_amd as m
    m.lib()
    return m


def _rel(got, ref):
    got = got.detach().float().cpu().double().numpy()
    den = max(np.abs(ref).max(), 1e-30)
    return np.abs(got - ref).max() / den


def _case(seed, B, dims, p, C, dt, m):
    # co = 16: the workload's weight tensor is not used here
    w = WL.random_workload(seed, B, dims, p, C, 16, dt, random_bias=False, shuffle=True)
    pts = WL.sample_points(w.coords, w.shape, m, seed + 100)
    dout = WL.normal(np.random.default_rng(seed + 200), (m, C), dt)
    return w, pts, dout


CASES = [  # seed, B, dims, p, C, dtype, m, key_bits
    (1, 1, (10, 12, 9), 0.3, 16, "f32", 3000, 0),
    (2, 2, (17, 11, 20), 0.2, 64, "f16", 5000, 0),
    (3, 2, (17, 11, 20), 0.2, 64, "bf16", 5000, 64),
    (4, 1, (30, 30, 30), 0.05, 72, "f16", 4000, 0),     # 9 vectors per row: lanes of a group idle
    (5, 3, (9, 9, 9), 0.5, 256, "bf16", 2000, 32),
    (6, 1, (12, 12, 12), 0.3, 1024, "bf16", 700, 0),   # 2 vectors per lane
    (7, 1, (12, 12, 12), 0.3, 4096, "f32", 300, 64),   # widest row: 16 KiB, the zero row's size
    (8, 1, (40, 3, 5), 0.6, 8, "f16", 2345, 0),        # one vector per row
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}-{c[5]}-C{c[4]}" for c in CASES])
def test_forward_and_backward_parity(ssc, case):
    seed, B, dims, p, C, dt, m, kb = case
    w, pts, dout = _case(seed, B, dims, p, C, dt, m)
    print(f"[grid_sample] seed={seed} n={w.n} m={m} C={C} {dt} key_bits={kb}", flush=True)
    plan = ssc.build_neighbor_map(torch.from_numpy(w.coords).to(DEV), w.shape, key_bits=kb)
    X = w.feats.to(DEV)
    P = torch.from_numpy(pts).to(DEV)
    out = ssc.grid_sample_fwd(plan, X, P)
    dX = ssc.grid_sample_bwd(plan, P, dout.to(DEV))
    torch.cuda.synchronize()
    ref = G.sample_fwd(w.coords, w.feats, w.shape, pts)
    assert np.abs(ref).max() > 0
    assert _rel(out, ref) <= TOL[dt]
    dref = G.sample_bwd(w.coords, w.shape, pts, dout)
    assert np.abs(dref).max() > 0
    assert _rel(dX, dref) <= TOL[dt]


def test_invalid_points_sample_zero(ssc):
    w = WL.values_for(np.array([[0, 1, 1, 1], [0, 2, 1, 1], [1, 0, 0, 0]], np.int32), (2, 4, 4, 4), 0, 16, 16,
                      "f32")
    pts = np.array([[0, 1.5, 1, 1], [1, -0.5, 0, 0], [1, -1.5, 0, 0], [2, 1, 1, 1], [-1, 1, 1, 1],
                    [0.5, 1, 1, 1], [0, np.nan, 1, 1], [0, np.inf, 1, 1], [np.nan, 1, 1, 1], [0, 1, 1, 1]],
                   np.float32)
    plan = ssc.build_neighbor_map(torch.from_numpy(w.coords).to(DEV), w.shape)
    out = ssc.grid_sample_fwd(plan, w.feats.to(DEV), torch.from_numpy(pts).to(DEV)).cpu().double().numpy()
    ref = G.sample_fwd(w.coords, w.feats, w.shape, pts)
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-6)
    assert (out[2:9] == 0).all()


def test_empty_voxels_and_points(ssc):
    # no voxels: samples are zero; no points: the gradient is zero
    e = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    plan0 = ssc.build_neighbor_map(e, (1, 8, 8, 8))
    P = torch.tensor([[0, 1.5, 2, 3]], dtype=torch.float32, device=DEV)
    out = torch.full((1, 16), 7.0, dtype=torch.float16, device=DEV)
    ssc.grid_sample_fwd(plan0, torch.zeros((0, 16), dtype=torch.float16, device=DEV), P, out=out)
    assert (out == 0).all()
    w = WL.random_workload(9, 1, (6, 6, 6), 0.5, 16, 16, "bf16")
    plan = ssc.build_neighbor_map(torch.from_numpy(w.coords).to(DEV), w.shape)
    d = torch.full((w.n, 16), 3.0, dtype=torch.bfloat16, device=DEV)
    ssc.grid_sample_bwd(plan, torch.zeros((0, 4), dtype=torch.float32, device=DEV),
                        torch.zeros((0, 16), dtype=torch.bfloat16, device=DEV), dfeats=d)
    assert (d == 0).all()
    assert ssc.grid_sample_fwd(plan, w.feats.to(DEV), torch.zeros((0, 4), device=DEV)).shape == (0, 16)


def test_autograd_wrapper(ssc):
    w, pts, dout = _case(11, 1, (14, 14, 14), 0.3, 32, "f32", 1500)
    plan = ssc.build_neighbor_map(torch.from_numpy(w.coords).to(DEV), w.shape)
    X = w.feats.to(DEV).requires_grad_(True)
    y = ssc.grid_sample(X, plan, torch.from_numpy(pts).to(DEV))
    y.backward(dout.to(DEV))
    assert _rel(X.grad, G.sample_bwd(w.coords, w.shape, pts, dout)) <= 1e-5


def test_config2_voxels_full_check(ssc):
    """Config 2 voxel set (2 x 64^3 shells, C = 64, fp16), two points per voxel: every output checked."""
    w = WL.make_workload(2)
    m = 2 * w.n
    pts = WL.sample_points(w.coords, w.shape, m, 2)
    dout = WL.normal(np.random.default_rng(22), (m, w.ci), w.dtype)
    plan = ssc.build_neighbor_map(torch.from_numpy(w.coords).to(DEV), w.shape, key_bits=w.key_bits)
    P = torch.from_numpy(pts).to(DEV)
    out = ssc.grid_sample_fwd(plan, w.feats.to(DEV), P)
    dX = ssc.grid_sample_bwd(plan, P, dout.to(DEV))
    torch.cuda.synchronize()
    assert _rel(out, G.sample_fwd(w.coords, w.feats, w.shape, pts)) <= 2e-2
    assert _rel(dX, G.sample_bwd(w.coords, w.shape, pts, dout)) <= 2e-2


def test_config4_voxels_sampled(ssc):
    """Config 4 voxel set (1024^3 shells, 6,416,526 voxels, 64-bit keys, C = 64, fp16), one point per voxel,
    as the benchmark runs it: sampled forward rows against the oracle, and the adjoint identity
    <fwd(F), G> = <F, bwd(G)> over the whole run."""
    w = WL.make_workload(4)
    m = w.n
    pts = WL.sample_points(w.coords, w.shape, m, 4)
    plan = ssc.build_neighbor_map(torch.from_numpy(w.coords).to(DEV), w.shape, key_bits=w.key_bits)
    P = torch.from_numpy(pts).to(DEV)
    F = w.feats.to(DEV)
    out = ssc.grid_sample_fwd(plan, F, P)
    Gd = WL.normal(np.random.default_rng(44), (m, w.ci), w.dtype).to(DEV)
    dF = ssc.grid_sample_bwd(plan, P, Gd)
    torch.cuda.synchronize()
    idx = np.random.default_rng(0).choice(m, 20000, replace=False)
    ref = G.sample_fwd(w.coords, w.feats, w.shape, pts[idx])
    assert _rel(out[torch.from_numpy(idx).to(DEV)], ref) <= 2e-2
    a = out.double() * Gd.double()
    b = F.double() * dF.double()
    lhs, rhs = float(a.sum()), float(b.sum())
    # rounding of out and dF to fp16 moves each sum by about 2^-11 * sqrt(sum of squares); a dropped or
    # misweighted corner would move rhs by a fair fraction of |rhs| ~ that same root
    scale = float(torch.sqrt((a * a).sum() + (b * b).sum()))
    assert abs(lhs - rhs) <= 0.025 * scale
