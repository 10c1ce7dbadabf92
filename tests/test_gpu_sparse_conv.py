"""Strided sparse convolution: HIP path against the CPU oracle, through the C ABI (needs an MI355X).

Output sites, the map and the output rows' GEMM order must match the oracle
bit for bit; fwd, dX, dW and dbias must satisfy max|err| / max|ref| <= 1e-5
(fp32) or <= 2e-2 (fp16 / bf16 inputs with fp32 accumulation) per tensor.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import sparse_conv as SC
from sparse_submanifold_convolution_amd import workloads as WL

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
DEV = torch.device("cuda:0")
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def ssc():
    import sparse_submanifold_convolution_amd as m
    m.lib()
    return m


def _rel(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = np.abs(ref).max()
    err = np.abs(got - ref).max()
    return float(err / den) if den > 0 else float(err)


def _grid(seed, shape, p, shuffle=False):
    rng = np.random.default_rng(seed)
    coords = np.argwhere(rng.random(shape) < p).astype(np.int32)
    if shuffle and len(coords) > 1:
        coords = coords[rng.permutation(len(coords))]
    return np.ascontiguousarray(coords)


def _check(ssc, coords, shape, ks, s, p, ci, co, dtype, seed=1, out_coords=None, key_bits=0):
    print(f"[case] shape={shape} n_in={len(coords)} ks={ks} s={s} p={p} Ci={ci} Co={co} {dtype} "
          f"given_out={out_coords is not None} key_bits={key_bits}", flush=True)
    ci_t = torch.from_numpy(coords).to(DEV)
    oc_t = None if out_coords is None else torch.from_numpy(out_coords).to(DEV)
    plan = ssc.build_sparse_map(ci_t, shape, ks, s, p, out_coords=oc_t, key_bits=key_bits)
    oc_ref = SC.out_coords(coords, shape, ks, s, p) if out_coords is None else out_coords
    assert np.array_equal(plan.out_coords.cpu().numpy(), oc_ref), "output sites differ"
    nm = SC.neighbor_map(coords, shape, oc_ref, ks, s, p)
    assert np.array_equal(plan.nmap.cpu().numpy().view(np.uint32), nm), "map differs"
    oshape = SC.out_shape(shape, ks, s, p)
    assert np.array_equal(plan.perm.cpu().numpy().astype(np.int64), SC.sort_perm(oc_ref, nm, oshape)), \
        "GEMM order differs"
    X, W, b, dY = WL.strided_values(seed, len(coords), len(oc_ref), ks, ci, co, dtype)
    Xd, Wd, bd, dYd = (t.to(DEV) for t in (X, W, b, dY))
    out = ssc.sparse_conv3d_fwd(plan, Xd, Wd, bd)
    dX, dW, db = ssc.sparse_conv3d_bwd(plan, Xd, Wd, dYd)
    torch.cuda.synchronize()
    errs = {
        "out": _rel(out.double().cpu(), SC.fwd(X, W, b, nm)),
        "dX": _rel(dX.double().cpu(), SC.dgrad(dY, W, nm, len(coords))),
        "dW": _rel(dW.double().cpu(), SC.wgrad(X, dY, nm, ks ** 3)),
        "db": _rel(db.double().cpu(), SC.dbias(dY)),
    }
    print(f"[errs] {errs}", flush=True)
    for k, e in errs.items():
        assert e <= TOL[dtype], f"{k}: {e} > {TOL[dtype]}"
    return plan, (out, dX, dW, db)


HAND = json.load(open(os.path.join(GOLD, "sparse_conv_hand.json")))["cases"]


@pytest.mark.parametrize("name", sorted(HAND))
def test_hand_cases_gpu(ssc, name):
    c = HAND[name]
    coords = np.array(c["coords"], np.int32)
    plan, _ = _check(ssc, coords, tuple(c["shape"]), c["ks"], c["stride"], c["pad"], 16, 16, "f32")
    assert plan.out_coords.cpu().tolist() == c["out_coords"]
    assert plan.perm.cpu().tolist() == c["perm"]


GEOMS = [(2, 2, 0), (3, 2, 1), (3, 1, 1), (3, 1, 0), (2, 1, 1), (1, 2, 0), (3, 3, 2), (2, 3, 1)]


@pytest.mark.parametrize("ks,s,p", GEOMS)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_geometries(ssc, ks, s, p, dtype):
    coords = _grid(10 + ks * 7 + s, (2, 20, 18, 22), 0.15, shuffle=True)
    _check(ssc, coords, (2, 20, 18, 22), ks, s, p, 32, 48, dtype)


@pytest.mark.parametrize("ci,co", [(16, 16), (64, 128), (256, 64), (8, 24), (40, 8)])
def test_channels_several_tiles(ssc, ci, co):
    # a few thousand outputs: several GEMM tiles and a ragged tail
    coords = _grid(4, (2, 40, 40, 40), 0.2)
    _check(ssc, coords, (2, 40, 40, 40), 2, 2, 0, ci, co, "bf16")


def test_narrow_fp32_channels(ssc):
    # 16-byte fp32 rows (4 channels) and the pages' cached layer width (32 -> 8)
    coords = _grid(6, (1, 24, 24, 24), 0.2, shuffle=True)
    _check(ssc, coords, (1, 24, 24, 24), 3, 2, 1, 4, 12, "f32")
    _check(ssc, coords, (1, 24, 24, 24), 2, 2, 0, 32, 8, "f32")


def test_downsample_of_a_shell_workload(ssc):
    w = WL.make_workload(2, values=False)
    _check(ssc, w.coords, w.shape, 2, 2, 0, 64, 64, "f16")
    _check(ssc, w.coords, w.shape, 3, 2, 1, 64, 64, "f16", key_bits=64)


def test_given_output_sites_and_submanifold_case(ssc):
    """Outputs given by the caller; ks=3, s=1, p=1 on the input sites equals the submanifold path bit for bit."""
    shape = (2, 16, 16, 16)
    coords = _grid(21, shape, 0.25, shuffle=True)
    plan, (out, dX, dW, db) = _check(ssc, coords, shape, 3, 1, 1, 32, 32, "f16", out_coords=coords)
    X, W, b, dY = (t.to(DEV) for t in WL.strided_values(1, len(coords), len(coords), 3, 32, 32, "f16"))
    sp = ssc.build_neighbor_map(torch.from_numpy(coords).to(DEV), shape)
    assert torch.equal(sp.nmap, plan.nmap) and torch.equal(sp.perm, plan.perm)
    out2 = ssc.subm_conv3d_fwd(sp, X, W, b)
    dX2, dW2, db2 = ssc.subm_conv3d_bwd(sp, X, W, dY)
    torch.cuda.synchronize()
    for a, c in [(out, out2), (dX, dX2), (dW, dW2), (db, db2)]:
        assert torch.equal(a, c)
    # upsampling direction: the outputs of a stride-2 conv as sites of a caller-chosen output set
    down = SC.out_coords(coords, shape, 2, 2, 0)
    _check(ssc, coords, shape, 2, 2, 0, 16, 32, "f32", out_coords=np.ascontiguousarray(down[::-1]))


def test_empty_inputs_and_outputs(ssc):
    shape = (1, 8, 8, 8)
    none = np.zeros((0, 4), np.int32)
    plan, (out, dX, dW, db) = _check(ssc, none, shape, 2, 2, 0, 16, 32, "f16")
    assert out.shape == (0, 32) and dX.shape == (0, 16)
    assert float(dW.abs().max()) == 0.0 and float(db.abs().max()) == 0.0
    # inputs but no outputs: dX is zero
    coords = _grid(3, shape, 0.3)
    plan, (out, dX, dW, db) = _check(ssc, coords, shape, 2, 2, 0, 16, 16, "bf16", out_coords=none)
    assert float(dX.abs().max()) == 0.0
    # outputs with empty windows: bias only
    far = np.array([[0, 3, 3, 3]], np.int32)
    _check(ssc, np.array([[0, 0, 0, 0]], np.int32), shape, 2, 2, 0, 16, 16, "f32", out_coords=far)


def test_device_errors_are_reported(ssc):
    shape = (1, 8, 8, 8)
    bad = torch.tensor([[0, 1, 1, 1], [0, 8, 1, 1]], dtype=torch.int32, device=DEV)
    with pytest.raises(ssc.SSCError):
        ssc.sparse_out_coords(bad, shape, 2, 2, 0)
    good = torch.tensor([[0, 1, 1, 1], [0, 2, 2, 2]], dtype=torch.int32, device=DEV)
    dup = torch.tensor([[0, 0, 0, 0], [0, 0, 0, 0]], dtype=torch.int32, device=DEV)
    with pytest.raises(ssc.SSCError) as e:
        ssc.build_sparse_map(good, shape, 2, 2, 0, out_coords=dup)
    assert e.value.code == 6
    off = torch.tensor([[0, 4, 0, 0]], dtype=torch.int32, device=DEV)   # output grid is 4^3
    with pytest.raises(ssc.SSCError) as e:
        ssc.build_sparse_map(good, shape, 2, 2, 0, out_coords=off)
    assert e.value.code == 5


def test_autograd_and_determinism(ssc):
    shape = (1, 24, 24, 24)
    coords = _grid(8, shape, 0.2)
    plan = ssc.build_sparse_map(torch.from_numpy(coords).to(DEV), shape, 3, 2, 1)
    X, W, b, dY = (t.to(DEV) for t in WL.strided_values(2, plan.n_in, plan.n_out, 3, 32, 32, "bf16"))
    X.requires_grad_(True)
    W.requires_grad_(True)
    b.requires_grad_(True)
    y = ssc.sparse_conv3d(X, plan, W, b)
    y.backward(dY)
    ref = ssc.sparse_conv3d_bwd(plan, X.detach(), W.detach(), dY)
    assert torch.equal(X.grad, ref[0]) and torch.equal(W.grad, ref[1]) and torch.equal(b.grad, ref[2])
    again = ssc.sparse_conv3d_bwd(plan, X.detach(), W.detach(), dY)
    assert all(torch.equal(a, c) for a, c in zip(ref, again))


def test_row_range_weight_gradient_chunks(ssc):
    """More than 1024 blocks of 256 output rows at 64 channels: the weight gradient chunks by row ranges."""
    shape = (2, 128, 128, 128)
    coords = _grid(31, shape, 0.15)
    plan, _ = _check(ssc, coords, shape, 2, 2, 0, 64, 64, "f16")
    assert plan.n_out > 1024 * 256


@pytest.mark.parametrize("two_streams", [False, True], ids=["one_stream", "two_streams"])
def test_graph_replay_matches_eager(ssc, two_streams):
    """Map build + fwd + bwd captured once and replayed with eager work in between equals eager runs;
    two_streams runs the input gradient and the weight gradient concurrently on one workspace."""
    shape = (2, 30, 26, 28)
    coords = _grid(44, shape, 0.2, shuffle=True)
    ks, s, p = 3, 2, 1
    print(f"[case] strided graph replay n_in={len(coords)} two_streams={two_streams}", flush=True)
    ct = torch.from_numpy(coords).to(DEV)
    ref_plan = ssc.build_sparse_map(ct, shape, ks, s, p)
    X, W, b, dY = (t.to(DEV) for t in WL.strided_values(5, ref_plan.n_in, ref_plan.n_out, ks, 64, 32, "bf16"))
    ref = [ssc.sparse_conv3d_fwd(ref_plan, X, W, b), *ssc.sparse_conv3d_bwd(ref_plan, X, W, dY)]
    torch.cuda.synchronize()
    plan = ssc.build_sparse_map(ct, shape, ks, s, p, out_coords=ref_plan.out_coords)
    plan.nmap.zero_()
    plan.perm.zero_()
    plan.buf.zero_()
    ws = ssc.sparse_workspace(plan, 64, 32, X.dtype)
    out, dX, dW, db = (torch.empty_like(r) for r in ref)
    L = ssc.lib()
    P_ = ssc.binding._ptr
    B_, Xd, Yd, Zd = shape
    grad_side = torch.cuda.Stream(DEV)

    def step():
        r = L.ssc_build_sparse_map(P_(ct), plan.n_in, B_, Xd, Yd, Zd, P_(plan.out_coords), plan.n_out, ks, s, p, 0,
                                   P_(plan.nmap), P_(plan.perm), P_(plan.buf), plan.buf.numel(),
                                   ssc.binding._stream(DEV))
        assert r == 0
        ssc.sparse_conv3d_fwd(plan, X, W, b, out=out, ws=ws)
        if two_streams:
            cur = torch.cuda.current_stream(DEV)
            grad_side.wait_stream(cur)
            ssc.sparse_conv3d_bwd(plan, X, W, dY, ws=ws, outs=(dX, None, None))
            with torch.cuda.stream(grad_side):
                ssc.sparse_conv3d_bwd(plan, X, W, dY, ws=ws, outs=(None, dW, db))
            cur.wait_stream(grad_side)
        else:
            ssc.sparse_conv3d_bwd(plan, X, W, dY, ws=ws, outs=(dX, dW, db))

    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (out, dX, dW, db, plan.nmap, plan.perm):
            t.zero_()
        junk = (X.float() * 2).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.nmap, ref_plan.nmap) and torch.equal(plan.perm, ref_plan.perm)
        for got, r in zip((out, dX, dW, db), ref):
            assert torch.equal(got, r), f"replay {rep} differs"
        del junk


def test_benchmarked_size_config3_downsample(ssc):
    """The strided bench workload in full: config 3's 799,512 voxels, ks=2, stride 2, C=256, bf16."""
    w = WL.make_workload(3, values=False)
    plan, _ = _check(ssc, w.coords, w.shape, 2, 2, 0, 256, 256, "bf16", seed=1003)
    assert plan.n_out == 199175


def test_benchmarked_size_config4_downsample(ssc):
    """The largest strided bench workload in full: config 4's 6,416,526 voxels (64-bit keys), ks=2, stride 2,
    C=64, fp16 -- row-range weight-gradient chunks and 8-column maps at full size."""
    w = WL.make_workload(4, values=False)
    plan, _ = _check(ssc, w.coords, w.shape, 2, 2, 0, 64, 64, "f16", seed=1004, key_bits=w.key_bits)
    assert plan.n_out == 1649179
