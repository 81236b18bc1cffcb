"""fp64 CPU oracle for the per-GPU K-FAC hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The GPU library never calls it
and shares no code with it.

Every function states the passage of "Accelerating Distributed K-FAC with
Smart Parallelism of Computing and Communication Tasks" it follows.  The page's
equation bodies did not survive extraction; where a formula is missing the
plain reading is used and listed in the design notes:

* factor      F = (1/rows) a^T a (Kronecker factors A and G; paragraph that
              introduces the Kronecker factors as symmetric matrices, Eqs.
              (7)-(8) as referenced in the pipelining paragraph);  computed as
              one fp64 matrix product.
* running avg M = F on the first step, else eps*M + (1-eps)*F (not on the
              page; the plainest average whose weights sum to one).
* pack        upper triangle incl. diagonal, d(d+1)/2 elements per factor,
              concatenated into one buffer (tensor-fusion paragraph; paragraph
              on broadcasting only upper triangles).  Written in C as index
              loops (kfac_oracle.c).
* inverse     (X + gamma I)^-1 through a Cholesky factorisation (paragraph on
              Tikhonov damping; paragraph on the Cholesky-based inverse).
              Written in C: textbook outer-product Cholesky, then forward and
              back substitution against columns of the identity.
* precondition P = (G+gamma I)^-1 grad (A+gamma I)^-1 (the damped update rule
              after the Kronecker inverse property, Eq. (4) onwards); computed
              as two fp64 matrix products of the given inverses.
* layers      the factor inputs of real layers, taken in the forward
              pre-hook (layer input) and the backward hook (gradient of the
              layer output) of the pipelining paragraph: the patches of a
              convolution input as rows (one per sample and output position,
              a column of ones for a bias), the output gradient as rows
              [b*H*W, c] times a scale, and a layer's weight and bias
              gradients as one matrix.  Written as index loops over the
              kernel taps.

Inputs are the exact values given to the GPU (float32 and bf16 upcast to
float64 exactly).  gamma and eps are float32 in the GPU library; callers pass
the same float32 value here.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.build()
        lib = ctypes.CDLL(path)
        i64, vp, dbl = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        lib.oracle_packed_size.restype = i64
        lib.oracle_packed_size.argtypes = [ctypes.c_int, vp]
        lib.oracle_pack.restype = None
        lib.oracle_pack.argtypes = [ctypes.c_int, vp, vp, vp]
        lib.oracle_unpack.restype = None
        lib.oracle_unpack.argtypes = [ctypes.c_int, vp, vp, vp]
        lib.oracle_cholesky_upper.restype = i64
        lib.oracle_cholesky_upper.argtypes = [vp, i64]
        lib.oracle_damped_inverse.restype = i64
        lib.oracle_damped_inverse.argtypes = [vp, i64, dbl, vp]
        lib.oracle_damped_inverse_columns.restype = i64
        lib.oracle_damped_inverse_columns.argtypes = [vp, i64, dbl, vp, i64, vp]
        _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def upcast(x, in_dtype: str = "f32") -> np.ndarray:
    """Exact fp64 copy of a GPU input (float32 array or uint16 bf16 bits)."""
    if in_dtype == "bf16":
        bits = np.ascontiguousarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ------------------------------------------------------------------ factor --

def factor(x) -> np.ndarray:
    """F = (1/rows) x^T x for x of shape [rows, d]; full symmetric fp64 d x d.
    Kronecker factor A (x = layer input a) or G (x = output gradient g)."""
    x = _f64(x)
    return (x.T @ x) / x.shape[0]


def factor_entries(x, ii, jj) -> np.ndarray:
    """Selected entries F[ii[q], jj[q]] = (1/rows) sum_r x[r, ii[q]] x[r, jj[q]]."""
    x = np.asarray(x)
    ii = np.asarray(ii, dtype=np.int64)
    jj = np.asarray(jj, dtype=np.int64)
    out = np.empty(ii.shape[0], dtype=np.float64)
    for q in range(ii.shape[0]):
        out[q] = np.dot(x[:, ii[q]].astype(np.float64), x[:, jj[q]].astype(np.float64))
    return out / x.shape[0]


def factor_diagonal(x) -> np.ndarray:
    """Diagonal of the factor: F[i][i] = (1/rows) sum_r x[r, i]^2."""
    x = _f64(x)
    return np.einsum("ri,ri->i", x, x) / x.shape[0]


def running_average(m_prev, f, eps: float, first: bool) -> np.ndarray:
    """M = F on the first step, else eps * M_prev + (1 - eps) * F."""
    f = _f64(f)
    if first:
        return f.copy()
    eps = float(eps)
    return eps * _f64(m_prev) + (1.0 - eps) * f


# -------------------------------------------------------------------- pack --

def packed_size(dims) -> int:
    d = np.ascontiguousarray(dims, dtype=np.int64)
    return int(_load().oracle_packed_size(len(d), _ptr(d)))


def pack(mats, dims=None) -> np.ndarray:
    """Concatenate the row-major upper triangles (incl. diagonal) of float32
    d x d matrices; returns float32 with the inputs' exact bit patterns."""
    mats = [np.ascontiguousarray(m, dtype=np.float32) for m in mats]
    d = np.ascontiguousarray([m.shape[0] for m in mats] if dims is None else dims, dtype=np.int64)
    for m, dl in zip(mats, d):
        assert m.shape == (dl, dl)
    out = np.empty(packed_size(d), dtype=np.float32)
    ptrs = (ctypes.c_void_p * len(mats))(*[m.ctypes.data for m in mats])
    _load().oracle_pack(len(mats), ctypes.cast(ptrs, ctypes.c_void_p), _ptr(d), _ptr(out))
    return out


def unpack(packed, dims):
    """Inverse of :func:`pack`: list of full symmetric float32 matrices."""
    packed = np.ascontiguousarray(packed, dtype=np.float32)
    d = np.ascontiguousarray(dims, dtype=np.int64)
    assert packed.shape[0] == packed_size(d)
    mats = [np.zeros((int(dl), int(dl)), dtype=np.float32) for dl in d]
    ptrs = (ctypes.c_void_p * len(mats))(*[m.ctypes.data for m in mats])
    _load().oracle_unpack(len(mats), _ptr(packed), _ptr(d), ctypes.cast(ptrs, ctypes.c_void_p))
    return mats


# ----------------------------------------------------------------- inverse --

def cholesky_upper(y):
    """U with Y = U^T U from the upper triangle of y; returns (U, info)."""
    y = _f64(y).copy()
    info = int(_load().oracle_cholesky_upper(_ptr(y), y.shape[0]))
    return np.triu(y), info


def damped_inverse(x, gamma: float):
    """(X + gamma I)^-1 with X read from the upper triangle of x.
    Returns (Z, info); Z is meaningful only when info == 0."""
    x = _f64(x)
    d = x.shape[0]
    z = np.zeros((d, d), dtype=np.float64)
    info = int(_load().oracle_damped_inverse(_ptr(x), d, float(gamma), _ptr(z)))
    return z, info


def damped_inverse_columns(x, gamma: float, cols):
    """Columns ``cols`` of (X + gamma I)^-1; returns (array [len(cols), d], info)."""
    x = _f64(x)
    d = x.shape[0]
    c = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.zeros((c.shape[0], d), dtype=np.float64)
    info = int(_load().oracle_damped_inverse_columns(_ptr(x), d, float(gamma), _ptr(c), c.shape[0], _ptr(out)))
    return out, info


# ------------------------------------------------------------ precondition --

def precondition(zg, grad, za) -> np.ndarray:
    """P = Z_G grad Z_A, with Z_G = (G+gamma I)^-1 [d_g, d_g],
    grad [d_g, d_a], Z_A = (A+gamma I)^-1 [d_a, d_a]."""
    return (_f64(zg) @ _f64(grad)) @ _f64(za)


def precondition_entries(zg, grad, za, ii, jj) -> np.ndarray:
    """Selected entries P[ii[q], jj[q]] = Z_G[ii[q], :] grad Z_A[:, jj[q]]."""
    zg, grad, za = np.asarray(zg), np.asarray(grad), np.asarray(za)
    ii = np.asarray(ii, dtype=np.int64)
    jj = np.asarray(jj, dtype=np.int64)
    rows = zg[ii, :].astype(np.float64) @ grad.astype(np.float64)       # [q, d_a]
    cols = za[:, jj].astype(np.float64)                                  # [d_a, q]
    return np.einsum("qk,kq->q", rows, cols)


# ---------------------------------------------------------------- compare --

def rel_fro(x, ref) -> float:
    """||x - ref||_F / ||ref||_F in fp64."""
    x = _f64(x)
    ref = _f64(ref)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x - ref))


def rel_fro_upper(x, ref) -> float:
    """rel_fro over the upper triangle including the diagonal."""
    iu = np.triu_indices(np.asarray(ref).shape[0])
    return rel_fro(np.asarray(x)[iu], np.asarray(ref)[iu])


__all__ = [
    "upcast", "factor", "factor_entries", "factor_diagonal", "running_average", "packed_size", "pack", "unpack",
    "cholesky_upper", "damped_inverse", "damped_inverse_columns", "precondition",
    "precondition_entries", "rel_fro", "rel_fro_upper",
]


# ----------------------------------------------------------------- layers --

def conv_out_hw(h, w, kh, kw, stride=(1, 1), padding=(0, 0), dilation=(1, 1)):
    """Output size of a convolution: (h + 2p - d (k - 1) - 1) // s + 1."""
    oh = (h + 2 * padding[0] - dilation[0] * (kh - 1) - 1) // stride[0] + 1
    ow = (w + 2 * padding[1] - dilation[1] * (kw - 1) - 1) // stride[1] + 1
    return oh, ow


def im2col(x, kernel=(1, 1), stride=(1, 1), padding=(0, 0), dilation=(1, 1), ones=False) -> np.ndarray:
    """Patches of x [n, c, h, w] as rows: row (ni*oh + y)*ow + xo, column
    (ci*kh + i)*kw + j holds x[ni, ci, y*sh - ph + i*dh, xo*sw - pw + j*dw]
    (zero outside the input), then a column of ones if `ones`.  Same dtype
    as x (values are copied)."""
    x = np.asarray(x)
    n, c, h, w = x.shape
    kh, kw = kernel
    oh, ow = conv_out_hw(h, w, kh, kw, stride, padding, dilation)
    out = np.zeros((n, oh, ow, c, kh, kw), dtype=x.dtype)
    for i in range(kh):
        for j in range(kw):
            for y in range(oh):
                yy = y * stride[0] - padding[0] + i * dilation[0]
                if yy < 0 or yy >= h:
                    continue
                for xo in range(ow):
                    xx = xo * stride[1] - padding[1] + j * dilation[1]
                    if 0 <= xx < w:
                        out[:, y, xo, :, i, j] = x[:, :, yy, xx]
    a = out.reshape(n * oh * ow, c * kh * kw)
    if ones:
        a = np.concatenate([a, np.ones((a.shape[0], 1), dtype=x.dtype)], axis=1)
    return a


def bf16_round(x32) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to
    even; NaN stays NaN."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def grad_rows(gy, scale: float, bf16: bool = False) -> np.ndarray:
    """g[b*hw + p][ci] = scale * gy[b][ci][p] for gy [b, c, ...] (positions
    flattened), the product in float32; bfloat16 inputs are given as their
    uint16 bit patterns and the result is rounded back to bfloat16."""
    gy = np.asarray(gy)
    b, c = gy.shape[0], gy.shape[1]
    v = gy.reshape(b, c, -1)
    if bf16:
        v = (v.astype(np.uint32) << 16).view(np.float32)
    g = np.empty((b * v.shape[2], c), dtype=np.float32)
    s = np.float32(scale)
    for bi in range(b):
        for p in range(v.shape[2]):
            g[bi * v.shape[2] + p, :] = s * v[bi, :, p]
    return bf16_round(g) if bf16 else g


def grad_matrix(wgrad, bgrad=None) -> np.ndarray:
    """[wgrad | bgrad]: wgrad [d_out, ...] read as [d_out, d_in], the bias
    gradient as the last column."""
    w = np.asarray(wgrad)
    w = w.reshape(w.shape[0], -1)
    if bgrad is None:
        return w.copy()
    return np.concatenate([w, np.asarray(bgrad).reshape(-1, 1)], axis=1)

