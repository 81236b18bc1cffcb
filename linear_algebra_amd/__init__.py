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
    "kfac_packed_size", "kfac_pack_workspace_size", "kfac_pack_sym", "kfac_pack_sym_static", "kfac_stream_copy",
    "kfac_matrix_rate",
    "kfac_inverse_workspace_size", "kfac_damped_inverse",
    "kfac_precondition_workspace_size", "kfac_precondition",
    "kfac_im2col_workspace_size", "kfac_im2col",
    "kfac_grad_rows_workspace_size", "kfac_grad_rows",
    "kfac_grad_matrix_workspace_size", "kfac_grad_matrix",
)


class KfacConv(ctypes.Structure):
    """kfac_conv_t: shape of a layer input and its convolution (1 x 1 for a
    fully connected layer)."""
    _fields_ = [("n", ctypes.c_int64), ("c", ctypes.c_int64), ("h", ctypes.c_int64), ("w", ctypes.c_int64),
                ("kh", ctypes.c_int32), ("kw", ctypes.c_int32), ("sh", ctypes.c_int32), ("sw", ctypes.c_int32),
                ("ph", ctypes.c_int32), ("pw", ctypes.c_int32), ("dh", ctypes.c_int32), ("dw", ctypes.c_int32),
                ("ones", ctypes.c_int32), ("reserved", ctypes.c_int32)]


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
        "kfac_pack_sym_static": (i32, [i32, vp, vp, vp, i32, vp]),
        "kfac_stream_copy": (i32, [vp, vp, sz, vp]),
        "kfac_matrix_rate": (i32, [i32, i64, i32, vp, vp, vp]),
        "kfac_inverse_workspace_size": (sz, [i32, vp]),
        "kfac_damped_inverse": (i32, [i32, vp, vp, f32, vp, vp, vp, sz, vp]),
        "kfac_precondition_workspace_size": (sz, [i32, vp, vp]),
        "kfac_precondition": (i32, [i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "kfac_im2col_workspace_size": (sz, [i32]),
        "kfac_im2col": (i32, [i32, vp, vp, i32, vp, vp, sz, vp]),
        "kfac_grad_rows_workspace_size": (sz, [i32]),
        "kfac_grad_rows": (i32, [i32, vp, vp, vp, vp, i32, f32, vp, vp, sz, vp]),
        "kfac_grad_matrix_workspace_size": (sz, [i32]),
        "kfac_grad_matrix": (i32, [i32, vp, vp, vp, vp, vp, i32, vp, sz, vp]),
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


def _keep_for(ws, stream) -> None:
    """The workspace comes from torch's allocator on the current stream; when
    the kernels run on another stream, the block must not be handed out
    again before that stream has passed them."""
    if stream is not None:
        ws.record_stream(stream)


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
    _keep_for(ws, stream)


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
    _keep_for(ws, stream)


def kfac_pack_sym_static(ms: Sequence, packed, direction: int, stream=None) -> None:
    """kfac_pack_sym without a workspace: the library's own device array holds
    the layer table, and nothing is allocated (at most 1024 factors; calls
    that may overlap on one GPU race)."""
    import torch
    lib = load_library()
    dev = _check(list(ms) + [packed], torch.float32, "kfac_pack_sym_static")
    d = []
    for m in ms:
        if m.dim() != 2 or m.shape[0] != m.shape[1]:
            raise ValueError("kfac_pack_sym_static: factors must be square")
        d.append(m.shape[0])
    if packed.numel() != kfac_packed_size(d):
        raise ValueError("kfac_pack_sym_static: packed buffer has the wrong length")
    _call(lib.kfac_pack_sym_static(len(ms), _ptrs(ms), _i64(d), ctypes.c_void_p(packed.data_ptr()), int(direction),
                                   _stream(dev, stream)), "kfac_pack_sym_static")


def kfac_stream_copy(src, dst, stream=None) -> None:
    """dst <- src, a plain device copy (the streaming reference of pack)."""
    lib = load_library()
    dev = _check([src, dst], None, "kfac_stream_copy")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("kfac_stream_copy: source and destination sizes differ")
    _call(lib.kfac_stream_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes,
                               _stream(dev, stream)), "kfac_stream_copy")


KFAC_RATE_BF16, KFAC_RATE_F64, KFAC_RATE_F32 = 0, 1, 2


def kfac_matrix_rate(kind: int, iters: int, sink, stream=None) -> float:
    """Register-only matrix-core product loops (the measured reference of the
    matrix-core-bound stages); sink float32 with 4 entries per workgroup.
    Returns the flops the call runs."""
    import torch
    lib = load_library()
    dev = _check([sink], torch.float32, "kfac_matrix_rate")
    if sink.numel() % 4 != 0 or sink.numel() == 0:
        raise ValueError("kfac_matrix_rate: sink needs 4 floats per workgroup")
    flops = ctypes.c_double(0.0)
    _call(lib.kfac_matrix_rate(int(kind), int(iters), sink.numel() // 4, ctypes.c_void_p(sink.data_ptr()),
                               ctypes.byref(flops), _stream(dev, stream)), "kfac_matrix_rate")
    return flops.value


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
    _keep_for(ws, stream)


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
    _keep_for(ws, stream)


__all__ = [
    "load_library", "status_string", "KfacError", "KfacLibraryError",
    "kfac_factors", "kfac_packed_size", "kfac_pack_sym", "kfac_pack_sym_static", "kfac_stream_copy",
    "kfac_matrix_rate", "KFAC_RATE_BF16", "KFAC_RATE_F64", "KFAC_RATE_F32",
    "kfac_damped_inverse",
    "kfac_precondition",
    "KFAC_F32", "KFAC_BF16", "KFAC_PACK", "KFAC_UNPACK", "EXPORTS",
]


def conv_out_hw(h: int, w: int, kh: int, kw: int, stride=(1, 1), padding=(0, 0), dilation=(1, 1)):
    """Output height and width of a convolution (the formula of kfac_im2col)."""
    oh = (h + 2 * padding[0] - dilation[0] * (kh - 1) - 1) // stride[0] + 1
    ow = (w + 2 * padding[1] - dilation[1] * (kw - 1) - 1) // stride[1] + 1
    return oh, ow


def kfac_im2col(xs: Sequence, shapes: Sequence[dict], outs: Sequence, stream=None) -> None:
    """a = patches of x as rows (kfac_im2col).  xs[i]: [n, c, h, w] float32 or
    bfloat16; shapes[i]: dict with kh, kw, stride, padding, dilation, ones;
    outs[i]: [n*oh*ow, c*kh*kw + ones] of the same dtype."""
    import torch
    lib = load_library()
    if len(xs) != len(shapes) or len(xs) != len(outs) or len(xs) == 0:
        raise ValueError("kfac_im2col: need equally many inputs, shapes and outputs")
    dt = xs[0].dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise ValueError("kfac_im2col: inputs must be float32 or bfloat16")
    dev = _check(list(xs) + list(outs), dt, "kfac_im2col")
    n = len(xs)
    arr = (KfacConv * n)()
    for i, (x, sh, o) in enumerate(zip(xs, shapes, outs)):
        if x.dim() != 4:
            raise ValueError("kfac_im2col: inputs must be [n, c, h, w]")
        kh, kw = sh.get("kernel", (1, 1))
        st, pd, dl = sh.get("stride", (1, 1)), sh.get("padding", (0, 0)), sh.get("dilation", (1, 1))
        ones = int(bool(sh.get("ones", False)))
        oh, ow = conv_out_hw(x.shape[2], x.shape[3], kh, kw, st, pd, dl)
        if o.dim() != 2 or o.shape != (x.shape[0] * oh * ow, x.shape[1] * kh * kw + ones):
            raise ValueError("kfac_im2col: output has the wrong shape")
        arr[i] = KfacConv(x.shape[0], x.shape[1], x.shape[2], x.shape[3], kh, kw, st[0], st[1], pd[0], pd[1],
                          dl[0], dl[1], ones, 0)
    ws = _workspace(lib.kfac_im2col_workspace_size(n), dev)
    dtype = KFAC_BF16 if dt == torch.bfloat16 else KFAC_F32
    _call(lib.kfac_im2col(n, _ptrs(xs), ctypes.cast(arr, ctypes.c_void_p), dtype, _ptrs(outs),
                          ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(dev, stream)), "kfac_im2col")
    _keep_for(ws, stream)


def kfac_grad_rows(gys: Sequence, scale: float, outs: Sequence, stream=None) -> None:
    """g[b*hw + p][c] = scale * gy[b][c][p] (kfac_grad_rows).  gys[i]:
    [b, c] or [b, c, H, W], float32 or bfloat16; outs[i]: [b*H*W, c]."""
    import torch
    lib = load_library()
    if len(gys) != len(outs) or len(gys) == 0:
        raise ValueError("kfac_grad_rows: need equally many gradients and outputs")
    dt = gys[0].dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise ValueError("kfac_grad_rows: gradients must be float32 or bfloat16")
    dev = _check(list(gys) + list(outs), dt, "kfac_grad_rows")
    b, c, hw = [], [], []
    for gy, o in zip(gys, outs):
        if gy.dim() < 2:
            raise ValueError("kfac_grad_rows: gradients must be [b, c, ...]")
        p = 1
        for s_ in gy.shape[2:]:
            p *= s_
        if o.shape != (gy.shape[0] * p, gy.shape[1]):
            raise ValueError("kfac_grad_rows: output has the wrong shape")
        b.append(gy.shape[0]); c.append(gy.shape[1]); hw.append(p)
    n = len(gys)
    ws = _workspace(lib.kfac_grad_rows_workspace_size(n), dev)
    dtype = KFAC_BF16 if dt == torch.bfloat16 else KFAC_F32
    _call(lib.kfac_grad_rows(n, _ptrs(gys), _i64(b), _i64(c), _i64(hw), dtype, ctypes.c_float(scale), _ptrs(outs),
                             ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(dev, stream)), "kfac_grad_rows")
    _keep_for(ws, stream)


def kfac_grad_matrix(wgrads: Sequence, bgrads: Sequence, mats: Sequence, direction: int, stream=None) -> None:
    """KFAC_PACK: mats[i] = [wgrad | bgrad]; KFAC_UNPACK: the reverse.
    wgrads[i]: float32 with d_out = shape[0] and d_in = the rest flattened;
    bgrads[i]: [d_out] or None; mats[i]: [d_out, d_in + has_bias]."""
    import torch
    lib = load_library()
    if len(wgrads) != len(bgrads) or len(wgrads) != len(mats) or len(wgrads) == 0:
        raise ValueError("kfac_grad_matrix: need equally many weights, biases and matrices")
    dev = _check(list(wgrads) + [b for b in bgrads if b is not None] + list(mats), torch.float32, "kfac_grad_matrix")
    d_out, d_in = [], []
    for w, b, m in zip(wgrads, bgrads, mats):
        do = w.shape[0]
        di = w.numel() // do
        if b is not None and b.numel() != do:
            raise ValueError("kfac_grad_matrix: bias gradient has the wrong length")
        if m.shape != (do, di + (b is not None)):
            raise ValueError("kfac_grad_matrix: matrix has the wrong shape")
        d_out.append(do); d_in.append(di)
    n = len(wgrads)
    bptr = (ctypes.c_void_p * n)(*[b.data_ptr() if b is not None else None for b in bgrads])
    ws = _workspace(lib.kfac_grad_matrix_workspace_size(n), dev)
    _call(lib.kfac_grad_matrix(n, _ptrs(wgrads), ctypes.cast(bptr, ctypes.c_void_p), _i64(d_out), _i64(d_in),
                               _ptrs(mats), int(direction), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                               _stream(dev, stream)), "kfac_grad_matrix")
    _keep_for(ws, stream)
