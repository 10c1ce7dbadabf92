"""The seeded generators produce workloads of the stated shapes, sizes and value statistics."""
import numpy as np
import pytest
import torch

from oracle import subm as O
from sparse_submanifold_convolution_amd import workloads as WL

# stated active-voxel ranges of the five workloads
RANGES = {1: (1872, 1872), 2: (20_000, 40_000), 3: (500_000, 1_000_000), 4: (5_000_000, 8_000_000),
          5: (600_000, 660_000)}


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_geometry_calibration(cfg):
    w = WL.make_workload(cfg, values=False)
    lo, hi = RANGES[cfg]
    assert lo <= w.n <= hi
    c = w.coords.astype(np.int64)
    assert c.dtype == np.int64 and w.coords.dtype == np.int32
    assert (c >= 0).all() and (c < np.array(w.shape)[None, :]).all()
    lin = O.linear_keys(c, w.shape)
    assert (np.diff(lin) > 0).all()          # unique and lexicographic
    assert set(np.unique(c[:, 0]).tolist()) == set(range(w.shape[0]))


def test_generator_is_deterministic_and_values_rounded():
    a = WL.make_workload(2)
    b = WL.make_workload(2)
    assert np.array_equal(a.coords, b.coords)
    assert torch.equal(a.feats, b.feats) and torch.equal(a.weight, b.weight) and torch.equal(a.dout, b.dout)
    assert a.feats.dtype == torch.float16 and a.weight.shape == (27, 64, 64)
    x = a.feats.double()
    assert abs(float(x.mean())) < 0.02 and abs(float(x.std()) - 1) < 0.02
    ws = float(a.weight.double().std()) * np.sqrt(27 * 64)
    assert abs(ws - 1) < 0.02
    assert float(a.bias.abs().max()) == 0.0


def test_config2_tiers_agree():
    w = WL.make_workload(2, values=False)
    assert np.array_equal(O.neighbor_map(w.coords, w.shape), O.neighbor_map_dict(w.coords, w.shape))


def test_random_workload_shapes():
    w = WL.random_workload(3, 2, (5, 6, 7), 0.2, 8, 16, "bf16", shuffle=True)
    assert w.feats.shape == (w.n, 8) and w.dout.shape == (w.n, 16) and w.weight.shape == (27, 8, 16)
    assert w.feats.dtype == torch.bfloat16
    e = WL.random_workload(3, 1, (3, 3, 3), 0.0, 8, 8, "f16")
    assert e.n == 0 and e.feats.shape == (0, 8)
