"""Thin ctypes binding of libssc (include/ssc.h): argument marshalling only.

Every step of the convolution runs in the HIP library.  torch supplies device
memory and the current stream; nothing here computes on the host or falls back
to another implementation.  If libssc.so is missing the calls raise.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssc.so")
_lib = None

SSC_OK = 0
STATUS_NAMES = {0: "SSC_OK", 1: "SSC_ERR_INVALID_ARG", 2: "SSC_ERR_UNSUPPORTED", 3: "SSC_ERR_WORKSPACE",
                4: "SSC_ERR_HIP", 5: "SSC_ERR_COORD_RANGE", 6: "SSC_ERR_DUPLICATE", 7: "SSC_ERR_HASH_FULL",
                8: "SSC_ERR_SCRATCH"}
DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

_VP, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
SIGNATURES = {
    "ssc_plan_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I32, _I32]),
    "ssc_build_neighbor_map": (ctypes.c_int, [_VP, _I64, _I32, _I32, _I32, _I32, _I32, _VP, _VP, _VP, _SZ, _VP]),
    "ssc_plan_status": (ctypes.c_int, [_VP, _VP, ctypes.POINTER(_I32)]),
    "ssc_plan_pair_counts": (ctypes.c_int, [_VP, _VP, ctypes.POINTER(_I64)]),
    "ssc_plan_row_orders": (ctypes.c_int, [_VP, _VP, ctypes.POINTER(_I64)]),
    "ssc_conv_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32]),
    "ssc_subm_conv3d_fwd": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "ssc_subm_conv3d_fwd_noalloc": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP]),
    "ssc_subm_conv3d_bwd": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                           _SZ, _VP]),
    "ssc_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ssc_seq_code_bits": (_I32, [_I32, _I32, _I32, _I32]),
    "ssc_seq_code_width": (_I32, [_I32, _I32, _I32, _I32]),
    "ssc_encode_seq": (ctypes.c_int, [_VP, _I64, _I32, _I32, _I32, _I32, _I32, _VP, _I32, _VP]),
    "ssc_decode_seq": (ctypes.c_int, [_VP, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _VP, _VP]),
    "ssc_grid_sample_workspace_bytes": (_SZ, [_I64, _I64]),
    "ssc_grid_sample_fwd": (ctypes.c_int, [_VP, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _VP, _VP, _I64,
                                           _VP, _VP]),
    "ssc_grid_sample_bwd": (ctypes.c_int, [_VP, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _VP, _I64, _VP,
                                           _VP, _VP, _SZ, _VP]),
    "ssc_sparse_out_shape": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(_I32)]),
    "ssc_sparse_out_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "ssc_sparse_out_count": (ctypes.c_int, [_VP, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _VP, _SZ, _VP,
                                            _VP]),
    "ssc_sparse_out_coords": (ctypes.c_int, [_VP, _SZ, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _VP, _I64, _VP]),
    "ssc_sparse_plan_bytes": (_SZ, [_I64, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "ssc_build_sparse_map": (ctypes.c_int, [_VP, _I64, _I32, _I32, _I32, _I32, _VP, _I64, _I32, _I32, _I32, _I32,
                                            _VP, _VP, _VP, _SZ, _VP]),
    "ssc_sparse_plan_status": (ctypes.c_int, [_VP, _I64, _VP, ctypes.POINTER(_I32)]),
    "ssc_sparse_conv_workspace_bytes": (_SZ, [_I64, _I64, _I32, _I32, _I32]),
    "ssc_sparse_conv3d_fwd": (ctypes.c_int, [_VP, _I64, _I64, _I32, _VP, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP,
                                             _SZ, _VP]),
    "ssc_sparse_conv3d_bwd": (ctypes.c_int, [_VP, _I64, _I64, _I32, _VP, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP,
                                             _VP, _VP, _SZ, _VP]),
}

SEQ_MODES = {"z_order": 0, "hilbert": 1}


class SSCError(RuntimeError):
    def __init__(self, func: str, code: int):
        self.code = code
        super().__init__(f"{func} failed: {STATUS_NAMES.get(code, code)} ({status_string(code)})")


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libssc; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"libssc.so not built at {_LIB_PATH}: run __graft_entry__.build()")
        l = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def status_string(code: int) -> str:
    return lib().ssc_status_string(int(code)).decode()


def _check(func: str, code: int) -> None:
    if code != SSC_OK:
        raise SSCError(func, code)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple, device: torch.device) -> None:
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


# ---------------------------------------------------------------------------
# plan
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Plan:
    """Neighbour map, permutation and neighbour cache of one coordinate set."""
    nmap: torch.Tensor      # [n, 27] uint32 (stored as int32 bits)
    perm: torch.Tensor      # [n] int32
    buf: torch.Tensor       # plan buffer (uint8)
    n: int
    shape: tuple
    key_bits: int

    @property
    def device(self) -> torch.device:
        return self.buf.device


def plan_bytes(n: int, shape, key_bits: int = 0) -> int:
    B, X, Y, Z = (int(s) for s in shape)
    return int(lib().ssc_plan_bytes(int(n), B, X, Y, Z, int(key_bits)))


def build_neighbor_map(coords: torch.Tensor, shape, key_bits: int = 0, check: bool = True) -> Plan:
    """ssc_build_neighbor_map on a device int32 [n, 4] coordinate tensor; raises on any error."""
    dev = coords.device
    n = int(coords.shape[0])
    _need(coords, "coords", torch.int32, (n, 4), dev)
    nbytes = plan_bytes(n, shape, key_bits)
    if nbytes == 0:
        raise SSCError("ssc_plan_bytes", 1)
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    nmap = torch.empty((n, 27), dtype=torch.int32, device=dev)
    perm = torch.empty((n,), dtype=torch.int32, device=dev)
    B, X, Y, Z = (int(s) for s in shape)
    _check("ssc_build_neighbor_map",
           lib().ssc_build_neighbor_map(_ptr(coords), n, B, X, Y, Z, int(key_bits), _ptr(nmap), _ptr(perm),
                                        _ptr(buf), nbytes, _stream(dev)))
    plan = Plan(nmap, perm, buf, n, tuple(int(s) for s in shape), int(key_bits))
    if check:
        st = plan_status(plan)
        if st != SSC_OK:
            raise SSCError("ssc_build_neighbor_map (device)", st)
    return plan


def plan_status(plan: Plan) -> int:
    out = ctypes.c_int32(-1)
    _check("ssc_plan_status", lib().ssc_plan_status(_ptr(plan.buf), _stream(plan.device), ctypes.byref(out)))
    return int(out.value)


def plan_pair_counts(plan: Plan) -> list[int]:
    arr = (ctypes.c_int64 * 27)()
    _check("ssc_plan_pair_counts", lib().ssc_plan_pair_counts(_ptr(plan.buf), _stream(plan.device), arr))
    return [int(v) for v in arr]


def plan_row_orders(plan: Plan) -> tuple[int, int, int]:
    """(row orders the GEMMs use: 1 or 3, the first order's 32-row group sum, the valid pairs)."""
    arr = (ctypes.c_int64 * 3)()
    _check("ssc_plan_row_orders", lib().ssc_plan_row_orders(_ptr(plan.buf), _stream(plan.device), arr))
    return int(arr[0]), int(arr[1]), int(arr[2])


# ---------------------------------------------------------------------------
# convolution
# ---------------------------------------------------------------------------

def conv_workspace_bytes(n: int, ci: int, co: int, dtype: torch.dtype) -> int:
    return int(lib().ssc_conv_workspace_bytes(int(n), int(ci), int(co), DTYPE_CODE[dtype]))


def workspace(plan: Plan, ci: int, co: int, dtype: torch.dtype) -> torch.Tensor:
    nbytes = conv_workspace_bytes(plan.n, ci, co, dtype)
    if nbytes == 0:
        raise SSCError("ssc_conv_workspace_bytes", 2)
    return torch.empty(nbytes, dtype=torch.uint8, device=plan.device)


def subm_conv3d_fwd(plan: Plan, feats: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor | None = None,
                    out: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    dev, dt, n = plan.device, feats.dtype, plan.n
    ci, co = int(weight.shape[1]), int(weight.shape[2])
    _need(feats, "feats", dt, (n, ci), dev)
    _need(weight, "weight", dt, (27, ci, co), dev)
    if bias is not None:
        _need(bias, "bias", dt, (co,), dev)
    if out is None:
        out = torch.empty((n, co), dtype=dt, device=dev)
    _need(out, "out", dt, (n, co), dev)
    if ws is None:
        ws = workspace(plan, ci, co, dt)
    if dt not in DTYPE_CODE:
        raise SSCError("ssc_subm_conv3d_fwd", 2)
    _check("ssc_subm_conv3d_fwd",
           lib().ssc_subm_conv3d_fwd(_ptr(plan.buf), _ptr(plan.nmap), _ptr(plan.perm), n, ci, co, DTYPE_CODE[dt],
                                     _ptr(feats), _ptr(weight), _ptr(bias), _ptr(out), _ptr(ws), ws.numel(),
                                     _stream(dev)))
    return out


def subm_conv3d_fwd_noalloc(plan: Plan, feats: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor | None = None,
                            out: torch.Tensor | None = None) -> torch.Tensor:
    """ssc_subm_conv3d_fwd_noalloc: the forward pass on the library's built-in scratch (no workspace)."""
    dev, dt, n = plan.device, feats.dtype, plan.n
    ci, co = int(weight.shape[1]), int(weight.shape[2])
    if dt not in DTYPE_CODE:
        raise SSCError("ssc_subm_conv3d_fwd_noalloc", 2)
    _need(feats, "feats", dt, (n, ci), dev)
    _need(weight, "weight", dt, (27, ci, co), dev)
    if bias is not None:
        _need(bias, "bias", dt, (co,), dev)
    if out is None:
        out = torch.empty((n, co), dtype=dt, device=dev)
    _need(out, "out", dt, (n, co), dev)
    _check("ssc_subm_conv3d_fwd_noalloc",
           lib().ssc_subm_conv3d_fwd_noalloc(_ptr(plan.buf), _ptr(plan.nmap), _ptr(plan.perm), n, ci, co,
                                             DTYPE_CODE[dt], _ptr(feats), _ptr(weight), _ptr(bias), _ptr(out),
                                             _stream(dev)))
    return out


def subm_conv3d_bwd(plan: Plan, feats: torch.Tensor, weight: torch.Tensor, dout: torch.Tensor,
                    need_dfeats: bool = True, need_dweight: bool = True, need_dbias: bool = True,
                    ws: torch.Tensor | None = None, outs: tuple | None = None):
    """Returns (dfeats, dweight, dbias); entries not asked for are None."""
    dev, dt, n = plan.device, dout.dtype, plan.n
    ci, co = int(weight.shape[1]), int(weight.shape[2])
    _need(feats, "feats", dt, (n, ci), dev)
    _need(weight, "weight", dt, (27, ci, co), dev)
    _need(dout, "dout", dt, (n, co), dev)
    if outs is not None:
        dX, dW, db = outs
    else:
        dX = torch.empty((n, ci), dtype=dt, device=dev) if need_dfeats else None
        dW = torch.empty((27, ci, co), dtype=dt, device=dev) if need_dweight else None
        db = torch.empty((co,), dtype=dt, device=dev) if need_dbias else None
    if ws is None:
        ws = workspace(plan, ci, co, dt)
    _check("ssc_subm_conv3d_bwd",
           lib().ssc_subm_conv3d_bwd(_ptr(plan.buf), _ptr(plan.nmap), _ptr(plan.perm), n, ci, co, DTYPE_CODE[dt],
                                     _ptr(feats), _ptr(weight), _ptr(dout), _ptr(dX), _ptr(dW), _ptr(db),
                                     _ptr(ws), ws.numel(), _stream(dev)))
    return dX, dW, db


class SubmConv3dFunction(torch.autograd.Function):
    """autograd wrapper: forward = ssc_subm_conv3d_fwd, backward = ssc_subm_conv3d_bwd."""

    @staticmethod
    def forward(ctx, feats, weight, bias, plan):
        ctx.plan = plan
        ctx.has_bias = bias is not None
        ctx.save_for_backward(feats, weight)
        return subm_conv3d_fwd(plan, feats.contiguous(), weight.contiguous(),
                               None if bias is None else bias.contiguous())

    @staticmethod
    def backward(ctx, dout):
        feats, weight = ctx.saved_tensors
        dX, dW, db = subm_conv3d_bwd(ctx.plan, feats, weight, dout.contiguous(),
                                     need_dfeats=ctx.needs_input_grad[0], need_dweight=ctx.needs_input_grad[1],
                                     need_dbias=ctx.has_bias and ctx.needs_input_grad[2])
        return dX, dW, db, None


def subm_conv3d(feats: torch.Tensor, plan: Plan, weight: torch.Tensor, bias: torch.Tensor | None = None):
    """Differentiable submanifold convolution over a built plan."""
    return SubmConv3dFunction.apply(feats, weight, bias, plan)


# ---------------------------------------------------------------------------
# strided (generalised) sparse convolution
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class SparsePlan:
    """Output sites, map and neighbour cache of a strided convolution over one input coordinate set."""
    out_coords: torch.Tensor  # [n_out, 4] int32
    nmap: torch.Tensor        # [n_out, 27] uint32 bits (int32)
    perm: torch.Tensor        # [n_out] int32: GEMM order of the output rows
    buf: torch.Tensor         # plan buffer (uint8)
    n_in: int
    n_out: int
    shape: tuple              # input grid (B, X, Y, Z)
    out_shape: tuple          # output grid (B, Xo, Yo, Zo)
    ks: int
    stride: int
    pad: int

    @property
    def device(self) -> torch.device:
        return self.buf.device


def sparse_out_shape(shape, ks: int, stride: int, pad: int) -> tuple:
    B, X, Y, Z = (int(s) for s in shape)
    dims = (ctypes.c_int32 * 4)()
    _check("ssc_sparse_out_shape", lib().ssc_sparse_out_shape(B, X, Y, Z, int(ks), int(stride), int(pad), dims))
    return tuple(int(d) for d in dims)


def sparse_out_coords(coords: torch.Tensor, shape, ks: int, stride: int, pad: int) -> torch.Tensor:
    """Active output sites (lexicographic order) of a strided convolution; reads the count on the host."""
    dev = coords.device
    n = int(coords.shape[0])
    _need(coords, "coords", torch.int32, (n, 4), dev)
    B, X, Y, Z = (int(s) for s in shape)
    geo = (int(ks), int(stride), int(pad))
    nbytes = int(lib().ssc_sparse_out_workspace_bytes(B, X, Y, Z, *geo))
    if nbytes == 0:
        raise SSCError("ssc_sparse_out_workspace_bytes", 1)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    count = torch.empty(1, dtype=torch.int64, device=dev)
    _check("ssc_sparse_out_count", lib().ssc_sparse_out_count(_ptr(coords), n, B, X, Y, Z, *geo, _ptr(ws), nbytes,
                                                              _ptr(count), _stream(dev)))
    n_out = int(count.item())
    if n_out < 0:
        raise SSCError("ssc_sparse_out_count (device)", 5)
    out = torch.empty((n_out, 4), dtype=torch.int32, device=dev)
    _check("ssc_sparse_out_coords", lib().ssc_sparse_out_coords(_ptr(ws), nbytes, B, X, Y, Z, *geo, _ptr(out),
                                                                n_out, _stream(dev)))
    return out


def build_sparse_map(coords: torch.Tensor, shape, ks: int, stride: int, pad: int,
                     out_coords: torch.Tensor | None = None, key_bits: int = 0, check: bool = True) -> SparsePlan:
    """sparse_neighbor_map: output sites (generated unless given), the map and the plan; raises on any error."""
    dev = coords.device
    n_in = int(coords.shape[0])
    _need(coords, "coords", torch.int32, (n_in, 4), dev)
    oshape = sparse_out_shape(shape, ks, stride, pad)
    if out_coords is None:
        out_coords = sparse_out_coords(coords, shape, ks, stride, pad)
    n_out = int(out_coords.shape[0])
    _need(out_coords, "out_coords", torch.int32, (n_out, 4), dev)
    B, X, Y, Z = (int(s) for s in shape)
    geo = (int(ks), int(stride), int(pad))
    nbytes = int(lib().ssc_sparse_plan_bytes(n_in, n_out, B, X, Y, Z, *geo, int(key_bits)))
    if nbytes == 0:
        raise SSCError("ssc_sparse_plan_bytes", 1)
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    nmap = torch.empty((n_out, 27), dtype=torch.int32, device=dev)
    perm = torch.empty((n_out,), dtype=torch.int32, device=dev)
    _check("ssc_build_sparse_map",
           lib().ssc_build_sparse_map(_ptr(coords), n_in, B, X, Y, Z, _ptr(out_coords), n_out, *geo, int(key_bits),
                                      _ptr(nmap), _ptr(perm), _ptr(buf), nbytes, _stream(dev)))
    plan = SparsePlan(out_coords, nmap, perm, buf, n_in, n_out, (B, X, Y, Z), oshape, *geo)
    if check:
        st = sparse_plan_status(plan)
        if st != SSC_OK:
            raise SSCError("ssc_build_sparse_map (device)", st)
    return plan


def sparse_plan_status(plan: SparsePlan) -> int:
    out = ctypes.c_int32(-1)
    _check("ssc_sparse_plan_status", lib().ssc_sparse_plan_status(_ptr(plan.buf), plan.n_out, _stream(plan.device),
                                                                  ctypes.byref(out)))
    return int(out.value)


def sparse_workspace(plan: SparsePlan, ci: int, co: int, dtype: torch.dtype) -> torch.Tensor:
    nbytes = int(lib().ssc_sparse_conv_workspace_bytes(plan.n_in, plan.n_out, int(ci), int(co), DTYPE_CODE[dtype]))
    if nbytes == 0:
        raise SSCError("ssc_sparse_conv_workspace_bytes", 2)
    return torch.empty(nbytes, dtype=torch.uint8, device=plan.device)


def sparse_conv3d_fwd(plan: SparsePlan, feats: torch.Tensor, weight: torch.Tensor,
                      bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
                      ws: torch.Tensor | None = None) -> torch.Tensor:
    dev, dt = plan.device, feats.dtype
    ci, co = int(weight.shape[1]), int(weight.shape[2])
    if dt not in DTYPE_CODE:
        raise SSCError("ssc_sparse_conv3d_fwd", 2)
    _need(feats, "feats", dt, (plan.n_in, ci), dev)
    _need(weight, "weight", dt, (plan.ks ** 3, ci, co), dev)
    if bias is not None:
        _need(bias, "bias", dt, (co,), dev)
    if out is None:
        out = torch.empty((plan.n_out, co), dtype=dt, device=dev)
    _need(out, "out", dt, (plan.n_out, co), dev)
    if ws is None:
        ws = sparse_workspace(plan, ci, co, dt)
    _check("ssc_sparse_conv3d_fwd",
           lib().ssc_sparse_conv3d_fwd(_ptr(plan.buf), plan.n_in, plan.n_out, plan.ks, _ptr(plan.perm), ci, co,
                                       DTYPE_CODE[dt], _ptr(feats), _ptr(weight), _ptr(bias), _ptr(out), _ptr(ws),
                                       ws.numel(), _stream(dev)))
    return out


def sparse_conv3d_bwd(plan: SparsePlan, feats: torch.Tensor, weight: torch.Tensor, dout: torch.Tensor,
                      need_dfeats: bool = True, need_dweight: bool = True, need_dbias: bool = True,
                      ws: torch.Tensor | None = None, outs: tuple | None = None):
    """Returns (dfeats, dweight, dbias); entries not asked for are None."""
    dev, dt = plan.device, dout.dtype
    ci, co = int(weight.shape[1]), int(weight.shape[2])
    V = plan.ks ** 3
    _need(feats, "feats", dt, (plan.n_in, ci), dev)
    _need(weight, "weight", dt, (V, ci, co), dev)
    _need(dout, "dout", dt, (plan.n_out, co), dev)
    if outs is not None:
        dX, dW, db = outs
    else:
        dX = torch.empty((plan.n_in, ci), dtype=dt, device=dev) if need_dfeats else None
        dW = torch.empty((V, ci, co), dtype=dt, device=dev) if need_dweight else None
        db = torch.empty((co,), dtype=dt, device=dev) if need_dbias else None
    if ws is None:
        ws = sparse_workspace(plan, ci, co, dt)
    _check("ssc_sparse_conv3d_bwd",
           lib().ssc_sparse_conv3d_bwd(_ptr(plan.buf), plan.n_in, plan.n_out, plan.ks, _ptr(plan.perm), ci, co,
                                       DTYPE_CODE[dt], _ptr(feats), _ptr(weight), _ptr(dout), _ptr(dX), _ptr(dW),
                                       _ptr(db), _ptr(ws), ws.numel(), _stream(dev)))
    return dX, dW, db


class SparseConv3dFunction(torch.autograd.Function):
    """autograd wrapper: forward = ssc_sparse_conv3d_fwd, backward = ssc_sparse_conv3d_bwd."""

    @staticmethod
    def forward(ctx, feats, weight, bias, plan):
        ctx.plan = plan
        ctx.has_bias = bias is not None
        ctx.save_for_backward(feats, weight)
        return sparse_conv3d_fwd(plan, feats.contiguous(), weight.contiguous(),
                                 None if bias is None else bias.contiguous())

    @staticmethod
    def backward(ctx, dout):
        feats, weight = ctx.saved_tensors
        dX, dW, db = sparse_conv3d_bwd(ctx.plan, feats, weight, dout.contiguous(),
                                       need_dfeats=ctx.needs_input_grad[0], need_dweight=ctx.needs_input_grad[1],
                                       need_dbias=ctx.has_bias and ctx.needs_input_grad[2])
        return dX, dW, db, None


def sparse_conv3d(feats: torch.Tensor, plan: SparsePlan, weight: torch.Tensor, bias: torch.Tensor | None = None):
    """Differentiable strided sparse convolution over a built plan (outputs at plan.out_coords)."""
    return SparseConv3dFunction.apply(feats, weight, bias, plan)


# ---------------------------------------------------------------------------
# serialisation
# ---------------------------------------------------------------------------

def _grid(shape) -> tuple:
    """(B, X, Y, Z) from a (B, X, Y, Z) or (B, C, X, Y, Z) shape; C is ignored."""
    s = tuple(int(v) for v in shape)
    if len(s) == 5:
        s = (s[0],) + s[2:]
    if len(s) != 4:
        raise ValueError(f"shape must be (B, X, Y, Z) or (B, C, X, Y, Z), got {shape}")
    return s


def _mode(mode: str) -> int:
    if mode not in SEQ_MODES:
        raise ValueError(f"mode must be one of {tuple(SEQ_MODES)}, got {mode!r}")
    return SEQ_MODES[mode]


def seq_code_width(shape) -> int:
    """32 or 64: the code width ssc_encode_seq picks for this grid."""
    w = int(lib().ssc_seq_code_width(*_grid(shape)))
    if w < 0:
        raise SSCError("ssc_seq_code_width", 2)
    return w


def encode_seq(coords: torch.Tensor, shape, mode: str = "z_order") -> torch.Tensor:
    """ssc_encode_seq: int32 [n, 4] rows (b, x, y, z) -> [n] codes (int32 or int64 by grid size)."""
    dev = coords.device
    n = int(coords.shape[0])
    _need(coords, "coords", torch.int32, (n, 4), dev)
    grid = _grid(shape)
    width = seq_code_width(grid)
    codes = torch.empty((n,), dtype=torch.int32 if width == 32 else torch.int64, device=dev)
    _check("ssc_encode_seq", lib().ssc_encode_seq(_ptr(coords), n, *grid, _mode(mode), _ptr(codes), width,
                                                  _stream(dev)))
    return codes


def decode_seq(codes: torch.Tensor, shape, mode: str = "z_order") -> torch.Tensor:
    """ssc_decode_seq: [n] int32 or int64 codes -> int32 [n, 4] rows; (-1, -1, -1, -1) where none."""
    dev = codes.device
    n = int(codes.shape[0])
    if codes.dtype not in (torch.int32, torch.int64) or codes.dim() != 1 or not codes.is_contiguous():
        raise ValueError(f"codes: expected a contiguous 1-d int32 or int64 tensor, got {codes.dtype} "
                         f"{tuple(codes.shape)}")
    grid = _grid(shape)
    width = 32 if codes.dtype == torch.int32 else 64
    coords = torch.empty((n, 4), dtype=torch.int32, device=dev)
    _check("ssc_decode_seq", lib().ssc_decode_seq(_ptr(codes), n, *grid, _mode(mode), width, _ptr(coords),
                                                  _stream(dev)))
    return coords


# ---------------------------------------------------------------------------
# sparse grid sampling
# ---------------------------------------------------------------------------

def grid_sample_workspace_bytes(n: int, m: int) -> int:
    """Workspace bytes of grid_sample_bwd for n voxels and m points."""
    return int(lib().ssc_grid_sample_workspace_bytes(int(n), int(m)))


def grid_sample_fwd(plan: Plan, feats: torch.Tensor, points: torch.Tensor,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """ssc_grid_sample_fwd: trilinear samples [m, C] of the plan's voxel features at float32 [m, 4] points."""
    dev, dt, n = plan.device, feats.dtype, plan.n
    c, m = int(feats.shape[1]), int(points.shape[0])
    _need(feats, "feats", dt, (n, c), dev)
    _need(points, "points", torch.float32, (m, 4), dev)
    if dt not in DTYPE_CODE:
        raise SSCError("ssc_grid_sample_fwd", 2)
    if out is None:
        out = torch.empty((m, c), dtype=dt, device=dev)
    _need(out, "out", dt, (m, c), dev)
    B, X, Y, Z = plan.shape
    _check("ssc_grid_sample_fwd",
           lib().ssc_grid_sample_fwd(_ptr(plan.buf), n, B, X, Y, Z, plan.key_bits, c, DTYPE_CODE[dt], _ptr(feats),
                                     _ptr(points), m, _ptr(out), _stream(dev)))
    return out


def grid_sample_bwd(plan: Plan, points: torch.Tensor, dout: torch.Tensor, dfeats: torch.Tensor | None = None,
                    ws: torch.Tensor | None = None) -> torch.Tensor:
    """ssc_grid_sample_bwd: the feature gradient [n, C] of grid_sample_fwd for output gradient dout [m, C]."""
    dev, dt, n = plan.device, dout.dtype, plan.n
    c, m = int(dout.shape[1]), int(points.shape[0])
    _need(points, "points", torch.float32, (m, 4), dev)
    _need(dout, "dout", dt, (m, c), dev)
    if dt not in DTYPE_CODE:
        raise SSCError("ssc_grid_sample_bwd", 2)
    if dfeats is None:
        dfeats = torch.empty((n, c), dtype=dt, device=dev)
    _need(dfeats, "dfeats", dt, (n, c), dev)
    if ws is None:
        nbytes = grid_sample_workspace_bytes(n, m)
        if nbytes == 0:
            raise SSCError("ssc_grid_sample_workspace_bytes", 2)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    B, X, Y, Z = plan.shape
    _check("ssc_grid_sample_bwd",
           lib().ssc_grid_sample_bwd(_ptr(plan.buf), n, B, X, Y, Z, plan.key_bits, c, DTYPE_CODE[dt], _ptr(points),
                                     m, _ptr(dout), _ptr(dfeats), _ptr(ws), ws.numel(), _stream(dev)))
    return dfeats


class GridSampleFunction(torch.autograd.Function):
    """autograd wrapper: gradient with respect to the voxel features only."""

    @staticmethod
    def forward(ctx, feats, points, plan):
        ctx.plan = plan
        ctx.save_for_backward(points)
        return grid_sample_fwd(plan, feats.contiguous(), points.contiguous())

    @staticmethod
    def backward(ctx, dout):
        (points,) = ctx.saved_tensors
        d = grid_sample_bwd(ctx.plan, points, dout.contiguous()) if ctx.needs_input_grad[0] else None
        return d, None, None


def grid_sample(feats: torch.Tensor, plan: Plan, points: torch.Tensor) -> torch.Tensor:
    """Differentiable trilinear sampling of the voxel features at [m, 4] float32 points (b, x, y, z)."""
    return GridSampleFunction.apply(feats, points, plan)
