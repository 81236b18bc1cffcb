"""Host-side checks of the C ABI: the library loads without a GPU, exports
every entry point include/kfac.h declares, and rejects bad arguments before
enqueuing anything (these calls never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

import linear_algebra_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from linear_algebra_amd import build
    build.build()
    return la.load_library()


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(kfac_[a-z0-9_]+)\s*\(", text))
    return names


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("kfac_factors", "kfac_pack_sym", "kfac_damped_inverse", "kfac_precondition"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names == set(la.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.kfac_abi_version() == 1
    assert la.status_string(0) == "KFAC_OK"
    assert la.status_string(2) == "KFAC_ERR_WORKSPACE"
    assert la.status_string(99) == "KFAC_ERR_UNKNOWN"


def i64(v):
    return (ctypes.c_int64 * len(v))(*v)


def vps(v):
    return (ctypes.c_void_p * len(v))(*v)


def test_packed_size(lib):
    d = [1, 2, 65, 4608]
    assert lib.kfac_packed_size(len(d), i64(d)) == sum(x * (x + 1) // 2 for x in d)
    assert lib.kfac_packed_size(0, i64([1])) == -1
    assert lib.kfac_packed_size(1, i64([0])) == -1
    assert lib.kfac_packed_size(1, i64([16385])) == -1


def test_workspace_sizes(lib):
    d, rows = [65, 2049], [32, 128]
    assert lib.kfac_factors_workspace_size(2, i64(rows), i64(d), 0) > 0
    assert lib.kfac_factors_workspace_size(2, i64(rows), i64(d), 7) == 0
    assert lib.kfac_factors_workspace_size(1, i64([0]), i64([4]), 0) == 0
    # the inverse keeps one float64 copy of every padded matrix
    ws = lib.kfac_inverse_workspace_size(2, i64(d))
    assert ws >= 8 * (128 * 128 + 2112 * 2112)
    assert lib.kfac_inverse_workspace_size(0, i64(d)) == 0
    assert lib.kfac_precondition_workspace_size(1, i64([32]), i64([65])) >= 4 * 32 * 65
    assert lib.kfac_pack_workspace_size(2, i64(d)) > 0


def test_split_k_partials_for_tall_inputs(lib):
    # a 401408 x 147 input needs split-K partial tiles beyond the descriptor table
    small = lib.kfac_factors_workspace_size(1, i64([128]), i64([147]), 0)
    tall = lib.kfac_factors_workspace_size(1, i64([401408]), i64([147]), 0)
    assert tall > small + 3 * 128 * 128 * 4


FAKE = 0x10000   # never dereferenced: every call below fails validation first


def test_factors_rejects_bad_arguments(lib):
    x, m = vps([FAKE]), vps([FAKE])
    ws = ctypes.c_void_p(FAKE)
    call = lambda n=1, x=x, rows=i64([8]), d=i64([4]), dt=0, m=m, eps=0.5, wsb=1 << 30, w=ws: \
        lib.kfac_factors(n, x, rows, d, dt, m, ctypes.c_float(eps), 0, w, wsb, None)
    assert call(n=0) == la.KFAC_ERR_INVALID_VALUE
    assert call(d=i64([0])) == la.KFAC_ERR_INVALID_VALUE
    assert call(d=i64([16385])) == la.KFAC_ERR_INVALID_VALUE           # past the largest order
    assert call(rows=i64([0])) == la.KFAC_ERR_INVALID_VALUE
    assert call(rows=i64([1 << 31])) == la.KFAC_ERR_INVALID_VALUE       # rows past 2^31 - 1
    assert call(eps=1.5) == la.KFAC_ERR_INVALID_VALUE
    assert call(eps=float("nan")) == la.KFAC_ERR_INVALID_VALUE
    assert call(dt=3) == la.KFAC_ERR_INVALID_VALUE
    assert call(x=vps([0])) == la.KFAC_ERR_INVALID_VALUE
    assert call(x=vps([FAKE + 2])) == la.KFAC_ERR_INVALID_VALUE       # misaligned float32
    assert call(wsb=16) == la.KFAC_ERR_WORKSPACE
    assert call(w=ctypes.c_void_p(FAKE + 8)) == la.KFAC_ERR_WORKSPACE  # misaligned workspace
    assert call(w=ctypes.c_void_p(0)) == la.KFAC_ERR_WORKSPACE


def test_inverse_rejects_bad_arguments(lib):
    x, z = vps([FAKE]), vps([FAKE])
    info = ctypes.c_void_p(FAKE)
    ws = ctypes.c_void_p(FAKE)
    call = lambda n=1, d=i64([4]), g=1e-3, info=info, wsb=1 << 30: \
        lib.kfac_damped_inverse(n, x, d, ctypes.c_float(g), z, info, ws, wsb, None)
    assert call(g=-1.0) == la.KFAC_ERR_INVALID_VALUE
    assert call(g=float("inf")) == la.KFAC_ERR_INVALID_VALUE
    assert call(info=ctypes.c_void_p(0)) == la.KFAC_ERR_INVALID_VALUE
    assert call(n=4097, d=i64([4] * 4097)) == la.KFAC_ERR_INVALID_VALUE
    assert call(n=0) == la.KFAC_ERR_INVALID_VALUE
    assert call(d=i64([0])) == la.KFAC_ERR_INVALID_VALUE
    assert call(d=i64([16385])) == la.KFAC_ERR_INVALID_VALUE
    assert call(wsb=100) == la.KFAC_ERR_WORKSPACE


def test_pack_and_precondition_reject_bad_arguments(lib):
    m = vps([FAKE])
    ws = ctypes.c_void_p(FAKE)
    assert lib.kfac_pack_sym(1, m, i64([4]), ctypes.c_void_p(FAKE), 2, ws, 1 << 20, None) == la.KFAC_ERR_INVALID_VALUE
    assert lib.kfac_pack_sym(1, m, i64([4]), ctypes.c_void_p(0), 0, ws, 1 << 20, None) == la.KFAC_ERR_INVALID_VALUE
    assert lib.kfac_pack_sym(1, m, i64([4]), ctypes.c_void_p(FAKE), 0, ws, 0, None) == la.KFAC_ERR_WORKSPACE
    p = vps([FAKE])
    assert lib.kfac_precondition(1, p, p, p, i64([0]), i64([4]), p, ws, 1 << 20, None) == la.KFAC_ERR_INVALID_VALUE
    assert lib.kfac_precondition(1, p, vps([0]), p, i64([4]), i64([4]), p, ws, 1 << 20, None) == la.KFAC_ERR_INVALID_VALUE
    assert lib.kfac_precondition(1, p, p, p, i64([4]), i64([4]), p, ws, 8, None) == la.KFAC_ERR_WORKSPACE


def test_static_pack_rejects_bad_arguments(lib):
    """The allocation-free pack validates like kfac_pack_sym and refuses more
    factors than its array holds, all before any device call."""
    n = 1025
    m = vps([FAKE] * n)
    packed = ctypes.c_void_p(FAKE)
    assert lib.kfac_pack_sym_static(n, m, i64([4] * n), packed, 0, None) == la.KFAC_ERR_UNSUPPORTED
    assert lib.kfac_pack_sym_static(1, m, i64([4]), packed, 2, None) == la.KFAC_ERR_INVALID_VALUE
    assert lib.kfac_pack_sym_static(1, m, i64([0]), packed, 0, None) == la.KFAC_ERR_INVALID_VALUE
    assert lib.kfac_pack_sym_static(1, m, i64([4]), ctypes.c_void_p(0), 0, None) == la.KFAC_ERR_INVALID_VALUE
    assert lib.kfac_pack_sym_static(1, vps([FAKE + 2]), i64([4]), packed, 1, None) == la.KFAC_ERR_INVALID_VALUE


def test_stream_copy_rejects_bad_arguments(lib):
    src, dst = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + (1 << 20))
    assert lib.kfac_stream_copy(src, dst, 0, None) == la.KFAC_OK                          # nothing to do
    assert lib.kfac_stream_copy(src, dst, 24, None) == la.KFAC_ERR_INVALID_VALUE          # not a multiple of 16
    assert lib.kfac_stream_copy(ctypes.c_void_p(FAKE + 4), dst, 16, None) == la.KFAC_ERR_INVALID_VALUE
    assert lib.kfac_stream_copy(src, ctypes.c_void_p(FAKE + 8), 4096, None) == la.KFAC_ERR_INVALID_VALUE
    assert lib.kfac_stream_copy(src, ctypes.c_void_p(FAKE + 16), 4096, None) == la.KFAC_ERR_INVALID_VALUE  # overlap
    assert lib.kfac_stream_copy(ctypes.c_void_p(0), dst, 16, None) == la.KFAC_ERR_INVALID_VALUE


def test_matrix_rate_rejects_bad_arguments(lib):
    sink = ctypes.c_void_p(FAKE)
    flops = ctypes.c_double(-1.0)
    rate = lib.kfac_matrix_rate
    assert rate(3, 10, 1, sink, ctypes.byref(flops), None) == la.KFAC_ERR_INVALID_VALUE          # unknown kind
    assert rate(0, 0, 1, sink, None, None) == la.KFAC_ERR_INVALID_VALUE                           # no rounds
    assert rate(0, (1 << 24) + 1, 1, sink, None, None) == la.KFAC_ERR_INVALID_VALUE               # too many rounds
    assert rate(1, 10, 0, sink, None, None) == la.KFAC_ERR_INVALID_VALUE                          # no workgroups
    assert rate(1, 10, 65537, sink, None, None) == la.KFAC_ERR_INVALID_VALUE
    assert rate(2, 10, 1, ctypes.c_void_p(0), None, None) == la.KFAC_ERR_INVALID_VALUE            # no sink
    assert rate(2, 10, 1, ctypes.c_void_p(FAKE + 2), None, None) == la.KFAC_ERR_INVALID_VALUE     # misaligned sink
    assert flops.value == -1.0                                                                     # untouched on error


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 3)
    m = torch.zeros(3, 3)
    with pytest.raises((ValueError, la.KfacLibraryError)):
        la.kfac_factors([x], [m], 0.95, True)


def conv_shape(**kw):
    """A valid kfac_conv_t (2 x 3 x 8 x 8 input, 3 x 3 kernel, padding 1)
    with the given fields changed."""
    c = la.KfacConv(2, 3, 8, 8, 3, 3, 1, 1, 1, 1, 1, 1, 0, 0)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_layer_entry_points_reject_bad_arguments(lib):
    ws = ctypes.c_void_p(FAKE)
    out = vps([FAKE])

    def im2col(shape, n=1, dtype=0, wsb=1 << 20, x=None):
        arr = (la.KfacConv * 1)(shape)
        return lib.kfac_im2col(n, x if x is not None else vps([FAKE]), ctypes.cast(arr, ctypes.c_void_p), dtype,
                               out, ws, wsb, None)

    bad = la.KFAC_ERR_INVALID_VALUE
    assert im2col(conv_shape(), n=0) == bad
    assert im2col(conv_shape(), dtype=7) == bad
    assert im2col(conv_shape(), x=vps([0])) == bad
    assert im2col(conv_shape(), x=vps([FAKE + 2])) == bad           # not 4-byte aligned for float32
    for field, value in [("n", 0), ("c", 0), ("kh", 0), ("sw", 0), ("ph", -1), ("dw", 0), ("ones", 2),
                         ("reserved", 1)]:
        assert im2col(conv_shape(**{field: value})) == bad, field
    assert im2col(conv_shape(kh=11)) == bad                         # kernel wider than the padded input
    assert im2col(conv_shape(c=1 << 20, h=1 << 11, w=1 << 11, kh=1, kw=1, ph=0, pw=0)) == bad   # c h w >= 2^31
    assert im2col(conv_shape(n=1 << 20, c=64, h=64, w=64)) == bad   # more than 2^31 - 1 patch elements
    assert im2col(conv_shape(), wsb=0) == la.KFAC_ERR_WORKSPACE

    def grad_rows(batch=4, c=8, hw=9, dtype=0, scale=1.0, gy=None, wsb=1 << 20):
        return lib.kfac_grad_rows(1, gy if gy is not None else vps([FAKE]), i64([batch]), i64([c]), i64([hw]),
                                  dtype, ctypes.c_float(scale), out, ws, wsb, None)

    assert grad_rows(batch=0) == bad
    assert grad_rows(c=0) == bad
    assert grad_rows(hw=0) == bad
    assert grad_rows(dtype=3) == bad
    assert grad_rows(scale=float("nan")) == bad
    assert grad_rows(gy=vps([0])) == bad
    assert grad_rows(wsb=0) == la.KFAC_ERR_WORKSPACE

    def grad_matrix(d_out=4, d_in=6, direction=0, mat=None, wsb=1 << 20):
        return lib.kfac_grad_matrix(1, vps([FAKE]), None, i64([d_out]), i64([d_in]),
                                    mat if mat is not None else vps([FAKE]), direction, ws, wsb, None)

    assert grad_matrix(d_out=0) == bad
    assert grad_matrix(d_in=0) == bad
    assert grad_matrix(direction=2) == bad
    assert grad_matrix(mat=vps([0])) == bad
    assert grad_matrix(mat=vps([FAKE + 1])) == bad
    assert grad_matrix(wsb=0) == la.KFAC_ERR_WORKSPACE
    assert lib.kfac_im2col_workspace_size(0) == 0
    assert lib.kfac_grad_rows_workspace_size(1) > 0
