"""The forward entry point that allocates nothing, against the one that takes a workspace (needs an MI355X).

ssc_subm_conv3d_fwd_noalloc runs the same kernels on the library's built-in
scratch array, so its output must equal ssc_subm_conv3d_fwd's bit for bit.
Two calls in a row, the second on a smaller input (the scratch keeps the first
call's contents), plus a layer whose Split-K partial sums live in the scratch.
Both are also held to the oracle's tolerance.
"""
import numpy as np
import pytest
import torch

from oracle import subm as O
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
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / den) if den > 0 else float(np.abs(got - ref).max())


def _case(ssc, w):
    print(f"[case] {w.desc} n={w.n} Ci={w.ci} Co={w.co} {w.dtype}", flush=True)
    plan = ssc.build_neighbor_map(torch.from_numpy(w.coords).to(DEV), w.shape)
    X, W, b = (t.to(DEV) for t in (w.feats, w.weight, w.bias))
    ref = ssc.subm_conv3d_fwd(plan, X, W, b)
    got = ssc.subm_conv3d_fwd_noalloc(plan, X, W, b)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), "no-allocation forward differs from the workspace forward"
    nm = plan.nmap.cpu().numpy().view(np.uint32)
    e = _rel(got.double().cpu(), O.fwd(w.feats, w.weight, w.bias, nm))
    print(f"[errs] out={e:.2e}", flush=True)
    assert e <= TOL[w.dtype]


def test_noalloc_forward_two_calls(ssc):
    # 8-wave tiles, then a smaller input on the same scratch
    _case(ssc, WL.random_workload(81, 2, (40, 40, 40), 0.35, 64, 96, "f16", random_bias=True, shuffle=True))
    _case(ssc, WL.random_workload(82, 1, (18, 17, 16), 0.3, 64, 96, "f16", random_bias=True))


def test_noalloc_forward_split_k_layer(ssc):
    # few rows: the offset set of each tile is split over workgroups whose fp32
    # partial sums live in the scratch; then a smaller fp32 layer
    _case(ssc, WL.random_workload(83, 1, (12, 12, 12), 0.3, 32, 32, "bf16", random_bias=True))
    _case(ssc, WL.random_workload(84, 1, (7, 7, 7), 0.3, 32, 8, "f32", random_bias=True))


def test_noalloc_forward_refuses_oversized_layer(ssc):
    w = WL.make_workload(5, values=False)
    plan = ssc.build_neighbor_map(torch.from_numpy(w.coords).to(DEV), w.shape)
    X = torch.zeros((w.n, 1024), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((27, 1024, 1024), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ssc.SSCError) as e:
        ssc.subm_conv3d_fwd_noalloc(plan, X, W)
    assert e.value.code == 8
