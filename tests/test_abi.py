"""libssc loads, exports every call include/ssc.h declares, and rejects bad arguments on the host.

No call here reaches the GPU: each one returns before any HIP runtime call.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssc.h")


@pytest.fixture(scope="module")
def L():
    import sparse_submanifold_convolution_amd as ssc
    return ssc.lib()


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssc_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared()
    for n in ["ssc_build_neighbor_map", "ssc_subm_conv3d_fwd", "ssc_subm_conv3d_bwd", "ssc_plan_bytes",
              "ssc_plan_status", "ssc_conv_workspace_bytes", "ssc_status_string"]:
        assert n in names


def test_every_declared_symbol_is_exported(L):
    from sparse_submanifold_convolution_amd.binding import SIGNATURES
    for name in declared():
        assert hasattr(L, name), name
        assert name in SIGNATURES, f"binding has no signature for {name}"


def test_status_strings(L):
    for code in range(9):
        assert L.ssc_status_string(code)
    assert L.ssc_status_string(99) == b"unknown status"


def test_plan_bytes_validation(L):
    assert L.ssc_plan_bytes(100, 1, 32, 32, 32, 0) > 0
    assert L.ssc_plan_bytes(-1, 1, 32, 32, 32, 0) == 0
    assert L.ssc_plan_bytes(100, 0, 32, 32, 32, 0) == 0
    assert L.ssc_plan_bytes(100, 1, 32, 32, 32, 17) == 0
    assert L.ssc_plan_bytes((1 << 26) + 1, 1, 32, 32, 32, 0) == 0
    # 32-bit keys cannot hold a 2 x 2048^3 volume; 64-bit can
    assert L.ssc_plan_bytes(100, 2, 2048, 2048, 2048, 32) == 0
    assert L.ssc_plan_bytes(100, 2, 2048, 2048, 2048, 0) > 0
    # table slots are 16 bytes for either key width
    assert L.ssc_plan_bytes(100, 1, 1024, 1024, 1024, 64) == L.ssc_plan_bytes(100, 1, 1024, 1024, 1024, 32) > 0
    assert L.ssc_plan_bytes(0, 1, 1, 1, 1, 0) > 0


def test_workspace_bytes_validation(L):
    assert L.ssc_conv_workspace_bytes(1000, 64, 64, 1) > 0
    # rows must be whole 16-byte vectors: multiples of 8 channels (16-bit), 4 (fp32)
    assert L.ssc_conv_workspace_bytes(1000, 24, 64, 1) > 0
    assert L.ssc_conv_workspace_bytes(1000, 8, 40, 2) > 0
    assert L.ssc_conv_workspace_bytes(1000, 32, 8, 0) > 0       # the pages' cached fp32 layer
    assert L.ssc_conv_workspace_bytes(1000, 4, 12, 0) > 0
    assert L.ssc_conv_workspace_bytes(1000, 12, 64, 1) == 0     # 24-byte fp16 rows
    assert L.ssc_conv_workspace_bytes(1000, 64, 4, 2) == 0      # 8-byte bf16 rows
    assert L.ssc_conv_workspace_bytes(1000, 64, 6, 0) == 0      # 24-byte fp32 rows
    assert L.ssc_conv_workspace_bytes(1000, 64, 64, 3) == 0     # unknown dtype
    assert L.ssc_conv_workspace_bytes(1000, 8192, 64, 2) == 0   # too wide


FAKE = ctypes.c_void_p(0x10000)   # aligned, never dereferenced: every call below fails its host checks first


def test_build_rejects_on_host(L):
    out = L.ssc_build_neighbor_map(None, 10, 1, 8, 8, 8, 0, FAKE, FAKE, FAKE, 1 << 30, None)
    assert out == 1
    out = L.ssc_build_neighbor_map(FAKE, 10, 1, 8, 8, 8, 0, FAKE, FAKE, FAKE, 16, None)
    assert out == 3                                   # plan buffer too small
    out = L.ssc_build_neighbor_map(FAKE, 10, 1, 8, 8, 8, 48, FAKE, FAKE, FAKE, 1 << 30, None)
    assert out == 1                                   # key_bits must be 0, 32 or 64
    out = L.ssc_build_neighbor_map(ctypes.c_void_p(0x10004), 10, 1, 8, 8, 8, 0, FAKE, FAKE, FAKE, 1 << 30, None)
    assert out == 1                                   # misaligned coords
    out = L.ssc_build_neighbor_map(FAKE, 10, 2, 2048, 2048, 2048, 32, FAKE, FAKE, FAKE, 1 << 30, None)
    assert out == 2                                   # volume does not fit 32-bit keys


def test_conv_rejects_on_host(L):
    f = L.ssc_subm_conv3d_fwd
    assert f(FAKE, FAKE, FAKE, 100, 32, 32, 5, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None) == 2   # dtype
    assert f(FAKE, FAKE, FAKE, 100, 18, 32, 0, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None) == 2   # fp32 Ci % 4
    assert f(FAKE, FAKE, FAKE, 100, 32, 20, 1, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None) == 2   # fp16 Co % 8
    assert f(FAKE, FAKE, FAKE, 100, 32, 32, 0, FAKE, FAKE, None, FAKE, FAKE, 64, None) == 3        # workspace
    assert f(FAKE, FAKE, FAKE, 100, 32, 32, 0, None, FAKE, None, FAKE, FAKE, 1 << 30, None) == 1   # feats NULL
    assert f(FAKE, FAKE, FAKE, -1, 32, 32, 0, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None) == 1
    b = L.ssc_subm_conv3d_bwd
    assert b(FAKE, FAKE, FAKE, 100, 32, 32, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, None) == 3
    assert b(FAKE, FAKE, FAKE, 100, 32, 32, 0, None, FAKE, FAKE, None, FAKE, None, FAKE, 1 << 30, None) == 1
    assert b(FAKE, FAKE, FAKE, 100, 32, 44, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 2
    assert b(FAKE, FAKE, FAKE, 100, 36, 32, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 2


def test_noalloc_forward_rejects_on_host(L):
    f = L.ssc_subm_conv3d_fwd_noalloc
    # arguments as ssc_subm_conv3d_fwd, checked before any HIP call
    assert f(FAKE, FAKE, FAKE, 100, 32, 32, 5, FAKE, FAKE, None, FAKE, None) == 2       # dtype
    assert f(FAKE, FAKE, FAKE, 100, 32, 20, 1, FAKE, FAKE, None, FAKE, None) == 2       # fp16 Co % 8
    assert f(FAKE, FAKE, FAKE, 100, 32, 32, 0, None, FAKE, None, FAKE, None) == 1       # feats NULL
    assert f(FAKE, FAKE, FAKE, -1, 32, 32, 0, FAKE, FAKE, None, FAKE, None) == 1
    assert f(FAKE, FAKE, FAKE, 0, 32, 32, 0, None, FAKE, None, None, None) == 0         # nothing to do
    # a layer whose workspace exceeds the built-in 64 MiB scratch (and every larger one) is refused
    assert L.ssc_conv_workspace_bytes(1 << 22, 1024, 1024, 2) > 64 << 20
    assert f(FAKE, FAKE, FAKE, 1 << 22, 1024, 1024, 2, FAKE, FAKE, None, FAKE, None) == 8
    assert L.ssc_status_string(8).startswith(b"larger than the built-in scratch")


def test_binding_raises_without_library(monkeypatch):
    from sparse_submanifold_convolution_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "_LIB_PATH", "/nonexistent/libssc.so")
    with pytest.raises(RuntimeError):
        binding.lib()


def test_seq_width_and_bits(L):
    assert L.ssc_seq_code_bits(1, 64, 64, 64) == 18 and L.ssc_seq_code_width(1, 64, 64, 64) == 32
    assert L.ssc_seq_code_bits(2, 1024, 1024, 1024) == 31 and L.ssc_seq_code_width(2, 1024, 1024, 1024) == 32
    assert L.ssc_seq_code_width(3, 1024, 1024, 1024) == 64
    assert L.ssc_seq_code_bits(1, 1, 1, 1) == 0
    assert L.ssc_seq_code_bits(0, 4, 4, 4) == -1 and L.ssc_seq_code_width(1, 0, 4, 4) == -1
    assert L.ssc_seq_code_width(1 << 20, 1 << 20, 1, 1) == -1  # 80-bit codes


def test_seq_rejections(L):
    ok, bad_arg, unsup = 0, 1, 2
    c = ctypes.c_void_p(FAKE.value)
    k = ctypes.c_void_p(FAKE.value + 256)
    enc, dec = L.ssc_encode_seq, L.ssc_decode_seq
    assert enc(c, -1, 1, 8, 8, 8, 0, k, 32, None) == bad_arg
    assert enc(c, 10, 0, 8, 8, 8, 0, k, 32, None) == bad_arg
    assert enc(c, 10, 1, 8, 8, 8, 2, k, 32, None) == unsup           # no such mode
    assert enc(c, 10, 1, 8, 8, 8, 0, k, 16, None) == unsup           # no such width
    assert enc(c, 10, 3, 1024, 1024, 1024, 0, k, 32, None) == unsup  # needs 64-bit codes
    assert enc(None, 10, 1, 8, 8, 8, 0, k, 32, None) == bad_arg
    assert enc(ctypes.c_void_p(FAKE.value + 4), 10, 1, 8, 8, 8, 0, k, 32, None) == bad_arg
    assert enc(c, 10, 1, 8, 8, 8, 0, ctypes.c_void_p(FAKE.value + 260), 64, None) == bad_arg
    assert enc(c, 0, 1, 8, 8, 8, 1, k, 64, None) == ok                # nothing to do
    assert dec(k, 10, 1, 8, 8, 8, 5, 32, c, None) == unsup
    assert dec(k, 10, 1, 8, 8, 8, 0, 32, None, None) == bad_arg
    assert dec(k, 10, 1, 8, 8, 8, 0, 32, ctypes.c_void_p(FAKE.value + 8), None) == bad_arg
    assert dec(k, 0, 1, 8, 8, 8, 0, 64, c, None) == ok


def test_grid_sample_workspace_and_rejections(L):
    ws = L.ssc_grid_sample_workspace_bytes
    assert ws(100, 1000) >= 8 * 100 + 64 * 1000 and ws(0, 0) > 0
    assert ws(-1, 10) == 0 and ws(10, -1) == 0 and ws(10, (1 << 28) + 1) == 0 and ws((1 << 26) + 1, 10) == 0
    f = L.ssc_grid_sample_fwd
    pts = ctypes.c_void_p(FAKE.value + 4096)
    assert f(None, 100, 1, 8, 8, 8, 0, 64, 1, FAKE, pts, 10, FAKE, None) == 1          # plan NULL
    assert f(FAKE, 100, 1, 8, 8, 8, 0, 64, 5, FAKE, pts, 10, FAKE, None) == 2          # dtype
    assert f(FAKE, 100, 1, 8, 8, 8, 0, 12, 1, FAKE, pts, 10, FAKE, None) == 2          # 24-byte rows
    assert f(FAKE, 100, 1, 8, 8, 8, 48, 64, 1, FAKE, pts, 10, FAKE, None) == 1         # key_bits
    assert f(FAKE, 100, 0, 8, 8, 8, 0, 64, 1, FAKE, pts, 10, FAKE, None) == 1          # B = 0
    assert f(FAKE, 100, 1, 8, 8, 8, 0, 64, 1, FAKE, pts, -1, FAKE, None) == 1          # m < 0
    assert f(FAKE, 100, 1, 8, 8, 8, 0, 64, 1, FAKE, ctypes.c_void_p(FAKE.value + 4), 10, FAKE, None) == 1
    assert f(FAKE, 100, 1, 8, 8, 8, 0, 64, 1, None, pts, 10, FAKE, None) == 1          # feats NULL
    assert f(FAKE, 100, 2, 2048, 2048, 2048, 32, 64, 1, FAKE, pts, 10, FAKE, None) == 2  # 32-bit keys too narrow
    b = L.ssc_grid_sample_bwd
    assert b(FAKE, 100, 1, 8, 8, 8, 0, 64, 1, pts, 10, FAKE, FAKE, FAKE, 64, None) == 3   # workspace small
    assert b(FAKE, 100, 1, 8, 8, 8, 0, 64, 5, pts, 10, FAKE, FAKE, FAKE, 1 << 30, None) == 2  # dtype
    assert b(FAKE, 100, 1, 8, 8, 8, 0, 64, 1, pts, 10, FAKE, FAKE, None, 1 << 30, None) == 1
    assert b(FAKE, 100, 1, 8, 8, 8, 0, 64, 1, pts, 10, None, FAKE, FAKE, 1 << 30, None) == 1  # dout NULL
    assert b(FAKE, 100, 1, 8, 8, 8, 0, 64, 1, pts, 10, FAKE, None, FAKE, 1 << 30, None) == 1  # dfeats NULL


def test_sparse_conv_sizes_and_rejections(L):
    dims = (ctypes.c_int32 * 4)()
    assert L.ssc_sparse_out_shape(2, 64, 63, 1, 3, 2, 1, dims) == 0 and list(dims) == [2, 32, 32, 1]
    assert L.ssc_sparse_out_shape(1, 8, 8, 8, 4, 1, 0, dims) == 1      # kernel side above 3
    assert L.ssc_sparse_out_shape(1, 8, 8, 8, 2, 1, 2, dims) == 1      # padding must stay below ks
    assert L.ssc_sparse_out_shape(1, 1, 8, 8, 3, 1, 0, dims) == 1      # empty output grid
    assert L.ssc_sparse_out_shape(1, 8, 8, 8, 2, 0, 0, dims) == 1      # stride 0
    # one bit per output site plus a count per 32 sites
    small = L.ssc_sparse_out_workspace_bytes(1, 64, 64, 64, 2, 2, 0)
    big = L.ssc_sparse_out_workspace_bytes(1, 64, 64, 64, 3, 1, 1)
    assert 0 < small < big and big >= 64 ** 3 // 4
    assert L.ssc_sparse_out_workspace_bytes(1, 8, 8, 8, 5, 1, 0) == 0
    assert L.ssc_sparse_plan_bytes(100, 50, 1, 32, 32, 32, 2, 2, 0, 0) > 0
    assert L.ssc_sparse_plan_bytes(100, 50, 1, 32, 32, 32, 2, 2, 0, 17) == 0
    assert L.ssc_sparse_plan_bytes(-1, 50, 1, 32, 32, 32, 2, 2, 0, 0) == 0
    assert L.ssc_sparse_plan_bytes(0, 0, 1, 32, 32, 32, 2, 2, 0, 0) > 0
    assert L.ssc_sparse_conv_workspace_bytes(1000, 200, 64, 128, 1) > 0
    assert L.ssc_sparse_conv_workspace_bytes(1000, 200, 64, 24, 1) > 0
    assert L.ssc_sparse_conv_workspace_bytes(1000, 200, 64, 20, 1) == 0
    cnt = ctypes.c_void_p(0x10008)
    assert L.ssc_sparse_out_count(None, 10, 1, 8, 8, 8, 2, 2, 0, FAKE, 1 << 30, cnt, None) == 1
    assert L.ssc_sparse_out_count(FAKE, 10, 1, 8, 8, 8, 2, 2, 0, FAKE, 16, cnt, None) == 3
    assert L.ssc_sparse_out_count(FAKE, 10, 1, 8, 8, 8, 2, 2, 3, FAKE, 1 << 30, cnt, None) == 1
    assert L.ssc_sparse_out_coords(FAKE, 16, 1, 8, 8, 8, 2, 2, 0, FAKE, 4, None) == 3
    assert L.ssc_sparse_out_coords(FAKE, 1 << 30, 1, 8, 8, 8, 2, 2, 0, None, 4, None) == 1
    b = L.ssc_build_sparse_map
    assert b(None, 10, 1, 8, 8, 8, FAKE, 4, 2, 2, 0, 0, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert b(FAKE, 10, 1, 8, 8, 8, FAKE, 4, 2, 2, 0, 0, FAKE, FAKE, FAKE, 16, None) == 3
    assert b(FAKE, 10, 1, 8, 8, 8, FAKE, 4, 2, 2, 0, 48, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert b(FAKE, 10, 1, 8, 8, 8, ctypes.c_void_p(0x10004), 4, 2, 2, 0, 0, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    f = L.ssc_sparse_conv3d_fwd
    assert f(FAKE, 100, 20, 2, FAKE, 32, 32, 5, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None) == 2
    assert f(FAKE, 100, 20, 2, FAKE, 32, 32, 0, FAKE, FAKE, None, FAKE, FAKE, 64, None) == 3
    assert f(FAKE, 100, 20, 4, FAKE, 32, 32, 0, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None) == 1
    assert f(FAKE, 100, 20, 2, None, 32, 32, 0, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None) == 1
    g = L.ssc_sparse_conv3d_bwd
    assert g(FAKE, 100, 20, 2, FAKE, 32, 32, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, None) == 3
    assert g(FAKE, 100, 20, 2, FAKE, 32, 32, 0, FAKE, None, FAKE, FAKE, None, None, FAKE, 1 << 30, None) == 1
