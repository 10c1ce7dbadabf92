"""GPU parity of ssc_encode_seq / ssc_decode_seq against the serialisation oracle (bit-exact)."""
import numpy as np
import pytest
import torch

from oracle import serialize as S
from sparse_submanifold_convolution_amd import workloads as WL

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def ssc():
    import sparse_submanifold_convolution_amd as m
    m.lib()
    return m


def _coords(seed, shape, n):
    rng = np.random.default_rng(seed)
    return np.stack([rng.integers(0, s, n) for s in shape], 1).astype(np.int32)


CASES = [
    (1, (1, 64, 64, 64), 5000),          # 18-bit codes
    (2, (2, 5, 9, 3), 300),              # tiny, non-power-of-two
    (3, (3, 33, 20, 64), 4000),
    (4, (1, 1, 1, 1), 10),               # zero spatial bits
    (5, (2, 1024, 1024, 1024), 20000),   # 31 bits: the widest int32 code
    (6, (3, 1024, 1024, 1024), 20000),   # 32 bits: int64
    (7, (5, 100000, 7, 3000), 3000),     # uneven axes, int64
]


@pytest.mark.parametrize("mode", S.MODES)
@pytest.mark.parametrize("case", CASES, ids=[f"c{c[0]}" for c in CASES])
def test_encode_decode_parity(ssc, mode, case):
    seed, shape, n = case
    c = _coords(seed, shape, n)
    print(f"[serialize] {mode} shape={shape} n={n}", flush=True)
    codes = ssc.encode_seq(torch.from_numpy(c).to(DEV), shape, mode)
    torch.cuda.synchronize()
    assert codes.dtype == (torch.int32 if S.code_width(shape) == 32 else torch.int64)
    ref = S.encode_seq(c, shape, mode)
    np.testing.assert_array_equal(codes.cpu().numpy().astype(np.int64), ref)
    back = ssc.decode_seq(codes, shape, mode)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(back.cpu().numpy(), c)


@pytest.mark.parametrize("mode", S.MODES)
def test_out_of_range_rows_and_codes(ssc, mode):
    shape = (2, 10, 12, 9)
    c = np.array([[0, 1, 2, 3], [-1, 0, 0, 0], [2, 0, 0, 0], [0, 10, 0, 0], [1, 9, 11, 8], [0, 0, 0, 9]],
                 np.int32)
    codes = ssc.encode_seq(torch.from_numpy(c).to(DEV), shape, mode).cpu().numpy().astype(np.int64)
    np.testing.assert_array_equal(codes, S.encode_seq(c, shape, mode))
    assert (codes[[1, 2, 3, 5]] == -1).all()
    # every code of the 16^3 cube that names no cell of the 10 x 12 x 9 grid decodes to -1 rows
    allc = np.arange(1 << S.code_bits(shape), dtype=np.int64)
    got = ssc.decode_seq(torch.from_numpy(allc).to(DEV).to(torch.int32), shape, mode).cpu().numpy()
    np.testing.assert_array_equal(got, S.decode_seq(allc, shape, mode))
    neg = ssc.decode_seq(torch.tensor([-1, -7], dtype=torch.int32, device=DEV), shape, mode).cpu().numpy()
    assert (neg == -1).all()


def test_hilbert_full_cube_on_gpu(ssc):
    n = 4
    shape = (1, 16, 16, 16)
    h = torch.arange(8 ** n, dtype=torch.int32, device=DEV)
    pts = ssc.decode_seq(h, shape, "hilbert").cpu().numpy()[:, 1:]
    assert len(np.unique(pts, axis=0)) == 8 ** n
    assert (np.abs(np.diff(pts, axis=0)).sum(axis=1) == 1).all()
    back = ssc.encode_seq(ssc.decode_seq(h, shape, "hilbert"), shape, "hilbert")
    torch.cuda.synchronize()
    assert torch.equal(back, h)


def test_five_dim_shape_and_empty(ssc):
    c = torch.tensor([[0, 10, 20, 30], [0, 15, 25, 35]], dtype=torch.int32, device=DEV)
    for mode in S.MODES:
        codes = ssc.encode_seq(c, (1, 1, 64, 64, 64), mode)
        assert torch.equal(ssc.decode_seq(codes, (1, 1, 64, 64, 64), mode), c)
    e = ssc.encode_seq(torch.empty((0, 4), dtype=torch.int32, device=DEV), (1, 8, 8, 8), "hilbert")
    assert e.numel() == 0


def test_config4_coordinates(ssc):
    """Full 1024^3 workload: GPU round trip for every row, oracle codes on a sample of rows."""
    w = WL.make_workload(4)
    shape = w.shape
    dc = torch.from_numpy(w.coords).to(DEV)
    rng = np.random.default_rng(0)
    idx = rng.choice(w.n, 20000, replace=False)
    for mode in S.MODES:
        codes = ssc.encode_seq(dc, shape, mode)
        back = ssc.decode_seq(codes, shape, mode)
        torch.cuda.synchronize()
        assert torch.equal(back, dc)
        got = codes.cpu().numpy().astype(np.int64)[idx]
        np.testing.assert_array_equal(got, S.encode_seq(w.coords[idx], shape, mode))
        assert len(np.unique(codes.cpu().numpy())) == w.n
