"""Python binding of the MI355X K-FAC hot-path library (libkfac.so).

The functions here carry the names of the C entry points in include/kfac.h
and do argument marshalling only: they check tensor shapes, dtypes and
devices, gather data pointers, take a workspace from PyTorch's allocator and
pass the current HIP stream.  Every step of the computation runs in the HIP
kernels of libkfac.so; there is no fallback.  If the library is missing the
import of this package succeeds but every call raises ``KfacLibraryError``.

PyTorch provides device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkfac.so")

KFAC_OK, KFAC_ERR_INVALID_VALUE, KFAC_ERR_WORKSPACE, KFAC_ERR_UNSUPPORTED, KFAC_ERR_HIP = range(5)
KFAC_F32, KFAC_BF16 = 0, 1
KFAC_PACK, KFAC_UNPACK = 0, 1

EXPORTS = (
    "kfac_abi_version", "kfac_status_string",
    "kfac_factors_workspace_size", "kfac_factors",
    "kfac_packed_size", "kfac_pack_workspace_size", "kfac_pack_sym",
    "kfac_inverse_workspace_size", "kfac_damped_inverse",
    "kfac_precondition_workspace_size", "kfac_precondition",
)


class KfacLibraryError(RuntimeError):
    pass


class KfacError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {status_string(status)} ({status})")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libkfac.so and declare its C signatures (no GPU needed)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise KfacLibraryError(f"{path} is missing: build it with `python -m linear_algebra_amd.build`")
    lib = ctypes.CDLL(path)
    i32, i64, sz, vp, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    sig = {
        "kfac_abi_version": (i32, []),
        "kfac_status_string": (ctypes.c_char_p, [i32]),
        "kfac_factors_workspace_size": (sz, [i32, vp, vp, i32]),
        "kfac_factors": (i32, [i32, vp, vp, vp, i32, vp, f32, i32, vp, sz, vp]),
        "kfac_packed_size": (i64, [i32, vp]),
        "kfac_pack_workspace_size": (sz, [i32, vp]),
        "kfac_pack_sym": (i32, [i32, vp, vp, vp, i32, vp, sz, vp]),
        "kfac_inverse_workspace_size": (sz, [i32, vp]),
        "kfac_damped_inverse": (i32, [i32, vp, vp, f32, vp, vp, vp, sz, vp]),
        "kfac_precondition_workspace_size": (sz, [i32, vp, vp]),
        "kfac_precondition": (i32, [i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load_library().kfac_status_string(int(status)).decode()
    except KfacLibraryError:
        return str(status)


# ------------------------------------------------------------ marshalling --

def _i64(values) -> ctypes.Array:
    values = [int(v) for v in values]
    return (ctypes.c_int64 * len(values))(*values)


def _ptrs(tensors) -> ctypes.Array:
    return (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])


def _stream(device, stream):
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(tensors, dtype, name):
    import torch
    dev = None
    for t in tensors:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name}: expected torch tensors")
        if t.device.type != "cuda":
            raise ValueError(f"{name}: tensors must live on the GPU")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name}: all tensors must be on one device")
    return dev


def _workspace(nbytes: int, device):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _call(status: int, where: str):
    if status != KFAC_OK:
        raise KfacError(status, where)


# ------------------------------------------------------------ entry points --

def kfac_factors(xs: Sequence, ms: Sequence, eps: float, first_step: bool, stream=None) -> None:
    """M_i <- F_i (first step) or eps*M_i + (1-eps)*F_i, F_i = x_i^T x_i / rows_i,
    upper triangle of each float32 M_i; x_i float32 or bfloat16 [rows_i, d_i]."""
    import torch
    lib = load_library()
    if len(xs) != len(ms) or len(xs) == 0:
        raise ValueError("kfac_factors: need equally many inputs and factors")
    dt = xs[0].dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise ValueError("kfac_factors: inputs must be float32 or bfloat16")
    dev = _check(list(xs), dt, "kfac_factors(x)")
    _check(list(ms), torch.float32, "kfac_factors(m)")
    rows, d = [], []
    for x, m in zip(xs, ms):
        if x.dim() != 2 or m.shape != (x.shape[1], x.shape[1]):
            raise ValueError("kfac_factors: x must be [rows, d] and m [d, d]")
        rows.append(x.shape[0])
        d.append(x.shape[1])
    n = len(xs)
    r64, d64 = _i64(rows), _i64(d)
    dtype = KFAC_BF16 if dt == torch.bfloat16 else KFAC_F32
    ws_bytes = lib.kfac_factors_workspace_size(n, r64, d64, dtype)
    if ws_bytes == 0:
        raise KfacError(KFAC_ERR_INVALID_VALUE, "kfac_factors_workspace_size")
    ws = _workspace(ws_bytes, dev)
    _call(lib.kfac_factors(n, _ptrs(xs), r64, d64, dtype, _ptrs(ms), ctypes.c_float(eps), int(bool(first_step)),
                           ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(dev, stream)), "kfac_factors")


def kfac_packed_size(dims: Sequence[int]) -> int:
    lib = load_library()
    v = lib.kfac_packed_size(len(dims), _i64(dims))
    if v < 0:
        raise KfacError(KFAC_ERR_INVALID_VALUE, "kfac_packed_size")
    return int(v)


def kfac_pack_sym(ms: Sequence, packed, direction: int, stream=None) -> None:
    """KFAC_PACK: upper triangles of ms -> packed.  KFAC_UNPACK: packed -> ms (both triangles)."""
    import torch
    lib = load_library()
    dev = _check(list(ms) + [packed], torch.float32, "kfac_pack_sym")
    d = []
    for m in ms:
        if m.dim() != 2 or m.shape[0] != m.shape[1]:
            raise ValueError("kfac_pack_sym: factors must be square")
        d.append(m.shape[0])
    n = len(ms)
    d64 = _i64(d)
    if packed.numel() != kfac_packed_size(d):
        raise ValueError("kfac_pack_sym: packed buffer has the wrong length")
    ws_bytes = lib.kfac_pack_workspace_size(n, d64)
    ws = _workspace(ws_bytes, dev)
    _call(lib.kfac_pack_sym(n, _ptrs(ms), d64, ctypes.c_void_p(packed.data_ptr()), int(direction),
                            ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(dev, stream)), "kfac_pack_sym")


def kfac_damped_inverse(xs: Sequence, gamma: float, xinvs: Sequence, info, stream=None) -> None:
    """xinv_i <- (X_i + gamma I)^-1 (X_i read from the upper triangle), info int32 [n]."""
    import torch
    lib = load_library()
    if len(xs) != len(xinvs) or len(xs) == 0:
        raise ValueError("kfac_damped_inverse: need equally many inputs and outputs")
    dev = _check(list(xs) + list(xinvs), torch.float32, "kfac_damped_inverse")
    _check([info], torch.int32, "kfac_damped_inverse(info)")
    if info.numel() != len(xs):
        raise ValueError("kfac_damped_inverse: info needs one entry per matrix")
    d = []
    for x, z in zip(xs, xinvs):
        if x.dim() != 2 or x.shape[0] != x.shape[1] or z.shape != x.shape:
            raise ValueError("kfac_damped_inverse: square inputs and outputs of equal shape")
        d.append(x.shape[0])
    n = len(xs)
    d64 = _i64(d)
    ws = _workspace(lib.kfac_inverse_workspace_size(n, d64), dev)
    _call(lib.kfac_damped_inverse(n, _ptrs(xs), d64, ctypes.c_float(gamma), _ptrs(xinvs),
                                  ctypes.c_void_p(info.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                  _stream(dev, stream)), "kfac_damped_inverse")


def kfac_precondition(ginvs: Sequence, grads: Sequence, ainvs: Sequence, outs: Sequence, stream=None) -> None:
    """out_l <- ginv_l . grad_l . ainv_l (ginv, ainv symmetric)."""
    import torch
    lib = load_library()
    n = len(grads)
    if not (len(ginvs) == len(ainvs) == len(outs) == n) or n == 0:
        raise ValueError("kfac_precondition: need equally many of every argument")
    dev = _check(list(ginvs) + list(grads) + list(ainvs) + list(outs), torch.float32, "kfac_precondition")
    dg, da = [], []
    for zg, g, za, o in zip(ginvs, grads, ainvs, outs):
        if g.dim() != 2 or zg.shape != (g.shape[0], g.shape[0]) or za.shape != (g.shape[1], g.shape[1]) \
                or o.shape != g.shape:
            raise ValueError("kfac_precondition: shapes must be ginv [dg,dg], grad [dg,da], ainv [da,da], out [dg,da]")
        dg.append(g.shape[0])
        da.append(g.shape[1])
    g64, a64 = _i64(dg), _i64(da)
    ws = _workspace(lib.kfac_precondition_workspace_size(n, g64, a64), dev)
    _call(lib.kfac_precondition(n, _ptrs(ginvs), _ptrs(grads), _ptrs(ainvs), g64, a64, _ptrs(outs),
                                ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(dev, stream)),
          "kfac_precondition")


__all__ = [
    "load_library", "status_string", "KfacError", "KfacLibraryError",
    "kfac_factors", "kfac_packed_size", "kfac_pack_sym", "kfac_damped_inverse", "kfac_precondition",
    "KFAC_F32", "KFAC_BF16", "KFAC_PACK", "KFAC_UNPACK", "EXPORTS",
]
