"""Pins for the fp64 oracle: closed forms, brute force on tiny inputs,
invariants, a textbook library cross-check and the page's printed counts.

Page: "Accelerating Distributed K-FAC with Smart Parallelism of Computing and
Communication Tasks".  Each test names the passage or mathematical fact it
holds the oracle to.  None of these tests touches the GPU library.
"""
from fractions import Fraction
import json
import os

import numpy as np
import pytest

import oracle
from workloads import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def spd(rng, d, rows=None, scale=1.0):
    rows = 2 * d if rows is None else rows
    x = rng.standard_normal((rows, d)) * scale
    return x.T @ x / rows


# ------------------------------------------------------------------ factor --

@pytest.mark.parametrize("rows,d", [(1, 1), (3, 2), (5, 8), (8, 3)])
def test_factor_brute_force_exact(rows, d):
    """Factor definition (Kronecker factors built from a layer's input or
    output gradient, symmetric): F[i][j] = (1/rows) sum_r x_ri x_rj,
    summed exactly with rationals from small integers."""
    rng = np.random.default_rng(rows * 31 + d)
    x = rng.integers(-7, 8, size=(rows, d))
    f = oracle.factor(x.astype(np.float64))
    for i in range(d):
        for j in range(d):
            s = Fraction(0)
            for r in range(rows):
                s += Fraction(int(x[r, i])) * Fraction(int(x[r, j]))
            # the integer sum is exact in fp64 and the division is correctly rounded
            assert f[i, j] == float(s / rows)


def test_factor_trace_closed_form():
    """trace(F) = ||x||_F^2 / rows."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((37, 19))
    f = oracle.factor(x)
    assert abs(np.trace(f) - (x * x).sum() / 37) <= 1e-12 * np.trace(f)


def test_factor_bias_column_closed_form():
    """With a trailing ones column: F[d-1][d-1] = 1 and F[i][d-1] = mean of column i."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((41, 9))
    x[:, -1] = 1.0
    f = oracle.factor(x)
    assert f[-1, -1] == 1.0
    np.testing.assert_allclose(f[:-1, -1], x[:, :-1].mean(axis=0), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(f[-1, :-1], x[:, :-1].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_factor_all_ones():
    f = oracle.factor(np.ones((13, 6)))
    np.testing.assert_array_equal(f, np.ones((6, 6)))


def test_factor_symmetric_psd():
    """The page states the Kronecker factors are symmetric; as Gram matrices
    they are also positive semi-definite."""
    rng = np.random.default_rng(3)
    x = np.maximum(rng.standard_normal((20, 50)), 0)       # rank-deficient: rows < d
    f = oracle.factor(x)
    np.testing.assert_array_equal(f, f.T)
    w = np.linalg.eigvalsh(f)
    assert w.min() >= -1e-12 * np.linalg.norm(f)


def test_factor_diagonal_is_trace_split():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((29, 11))
    np.testing.assert_allclose(oracle.factor_diagonal(x), (x * x).sum(axis=0) / 29, rtol=1e-14)
    np.testing.assert_allclose(oracle.factor_diagonal(x), np.diag(oracle.factor(x)), rtol=1e-13)


def test_factor_entries_agree_with_full():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((300, 40)).astype(np.float32)
    f = oracle.factor(oracle.upcast(x))
    ii = rng.integers(0, 40, 50)
    jj = rng.integers(0, 40, 50)
    np.testing.assert_allclose(oracle.factor_entries(x, ii, jj), f[ii, jj], rtol=1e-13, atol=1e-15)


# --------------------------------------------------------- running average --

def test_running_average_limits():
    rng = np.random.default_rng(5)
    m, f = spd(rng, 7), spd(rng, 7)
    np.testing.assert_array_equal(oracle.running_average(m, f, 0.0, False), f)
    np.testing.assert_array_equal(oracle.running_average(m, f, 1.0, False), m)
    np.testing.assert_array_equal(oracle.running_average(m, f, 0.95, True), f)


def test_running_average_constant_input():
    rng = np.random.default_rng(6)
    f = spd(rng, 5)
    m = oracle.running_average(None, f, 0.95, True)
    for _ in range(4):
        m = oracle.running_average(m, f, 0.95, False)
        np.testing.assert_allclose(m, f, rtol=1e-14, atol=1e-15)


def test_running_average_three_steps_closed_form():
    """eps = 0.95 over three steps: M = 0.9025 F0 + 0.0475 F1 + 0.05 F2."""
    rng = np.random.default_rng(7)
    fs = [spd(rng, 6) for _ in range(3)]
    m = oracle.running_average(None, fs[0], 0.95, True)
    m = oracle.running_average(m, fs[1], 0.95, False)
    m = oracle.running_average(m, fs[2], 0.95, False)
    np.testing.assert_allclose(m, 0.9025 * fs[0] + 0.0475 * fs[1] + 0.05 * fs[2], rtol=1e-13, atol=1e-15)


# -------------------------------------------------------------------- pack --

def _read_literal(golden_dir):
    dims, packed = None, None
    with open(os.path.join(golden_dir, "pack_literal.txt")) as fh:
        for line in fh:
            if line.startswith("dims"):
                dims = [int(t) for t in line.split()[1:]]
            elif line.startswith("packed"):
                packed = [float(t) for t in line.split()[1:]]
    return dims, packed


def test_pack_literal(golden_dir):
    dims, expect = _read_literal(golden_dir)
    mats = [np.array([[100 * l + 10 * i + j for j in range(d)] for i in range(d)], dtype=np.float32)
            for l, d in enumerate(dims)]
    np.testing.assert_array_equal(oracle.pack(mats), np.array(expect, dtype=np.float32))
    back = oracle.unpack(np.array(expect, dtype=np.float32), dims)
    for l, (m, d) in enumerate(zip(back, dims)):
        up = np.triu(mats[l])
        np.testing.assert_array_equal(m, up + np.triu(up, 1).T)


def test_pack_size_closed_form():
    """d(d+1)/2 per factor (tensor-fusion paragraph), summed over factors."""
    dims = [1, 2, 3, 64, 65, 147, 2049]
    assert oracle.packed_size(dims) == sum(d * (d + 1) // 2 for d in dims)
    assert oracle.packed_size(CONFIGS[3].factor_dims()) == 76967027


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_pack_matches_library_index_map(seed):
    """Row-major upper order equals numpy's triu_indices order."""
    rng = np.random.default_rng(seed)
    dims = [int(v) for v in rng.integers(1, 70, size=6)] + [1, 2]
    mats = [rng.standard_normal((d, d)).astype(np.float32) for d in dims]
    ref = np.concatenate([m[np.triu_indices(m.shape[0])] for m in mats])
    got = oracle.pack(mats)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_pack_unpack_round_trip_bits():
    """Pack and unpack are pure copies: arbitrary 32-bit patterns (NaN payloads,
    -0.0, denormals) survive both round trips bit for bit."""
    rng = np.random.default_rng(9)
    dims = [5, 1, 17, 2]
    mats = [rng.integers(0, 2**32, size=(d, d), dtype=np.uint64).astype(np.uint32).view(np.float32) for d in dims]
    p = oracle.pack(mats)
    back = oracle.unpack(p, dims)
    for m, b in zip(mats, back):
        iu = np.triu_indices(m.shape[0])
        np.testing.assert_array_equal(b.view(np.uint32)[iu], m.view(np.uint32)[iu])
        np.testing.assert_array_equal(b.view(np.uint32), b.view(np.uint32).T)
    np.testing.assert_array_equal(oracle.pack(back).view(np.uint32), p.view(np.uint32))


def test_pack_adjoint():
    """Adjoint test for linear data movement ("A Linear Algebraic Approach to
    Model Parallelism in Deep Learning", paragraph on verifying data-movement
    operators): <pack(M), p> = <M, pack^T(p)>, where pack^T scatters p into the
    upper triangle (= upper triangle of unpack(p)).  Small integers make both
    sides exact in float64."""
    rng = np.random.default_rng(10)
    dims = [4, 9, 1, 30]
    mats = [rng.integers(-20, 21, size=(d, d)).astype(np.float32) for d in dims]
    p = rng.integers(-20, 21, size=oracle.packed_size(dims)).astype(np.float32)
    lhs = float(np.dot(oracle.pack(mats).astype(np.float64), p.astype(np.float64)))
    rhs = sum(float(np.sum(np.triu(m).astype(np.float64) * np.triu(u).astype(np.float64)))
              for m, u in zip(mats, oracle.unpack(p, dims)))
    assert lhs == rhs


# ----------------------------------------------------------------- inverse --

@pytest.mark.parametrize("d,gamma", [(1, 0.5), (7, 1e-3), (64, 1e-3), (150, 1e-2)])
def test_inverse_residual(d, gamma):
    """(X + gamma I) Z = I to fp64 accuracy."""
    rng = np.random.default_rng(d)
    x = spd(rng, d, rows=max(1, d // 2))            # rank-deficient, as real factors often are
    z, info = oracle.damped_inverse(x, gamma)
    assert info == 0
    r = (x + gamma * np.eye(d)) @ z - np.eye(d)
    assert np.linalg.norm(r) / np.sqrt(d) <= 1e-10


def test_inverse_diagonal_closed_form():
    x = np.diag(np.linspace(0.0, 5.0, 11))
    z, info = oracle.damped_inverse(x, 0.25)
    assert info == 0
    np.testing.assert_allclose(z, np.diag(1.0 / (np.diag(x) + 0.25)), rtol=1e-15, atol=1e-300)


def test_inverse_zero_matrix():
    z, info = oracle.damped_inverse(np.zeros((9, 9)), 1e-3)
    assert info == 0
    np.testing.assert_allclose(z, np.eye(9) / 1e-3, rtol=1e-14, atol=0)


@pytest.mark.parametrize("c,d,gamma", [(1.0, 10, 1e-3), (0.3, 33, 0.01)])
def test_inverse_sherman_morrison(c, d, gamma):
    """X = c 11^T: (X + gamma I)^-1 = (1/gamma)(I - c/(gamma + c d) 11^T)."""
    x = c * np.ones((d, d))
    z, info = oracle.damped_inverse(x, gamma)
    assert info == 0
    ref = (np.eye(d) - c / (gamma + c * d) * np.ones((d, d))) / gamma
    np.testing.assert_allclose(z, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())


def test_inverse_two_by_two():
    a, b, c, g = 2.0, 0.7, 1.5, 0.1
    z, info = oracle.damped_inverse(np.array([[a, b], [b, c]]), g)
    det = (a + g) * (c + g) - b * b
    np.testing.assert_allclose(z, np.array([[c + g, -b], [-b, a + g]]) / det, rtol=1e-15)


def test_inverse_reads_upper_triangle_only():
    rng = np.random.default_rng(11)
    x = spd(rng, 12)
    z0, _ = oracle.damped_inverse(x, 1e-2)
    xg = x.copy()
    xg[np.tril_indices(12, -1)] = rng.standard_normal(66) * 1e6
    z1, _ = oracle.damped_inverse(xg, 1e-2)
    np.testing.assert_array_equal(z0, z1)


@pytest.mark.parametrize("d", [3, 40, 200, 512])
def test_inverse_against_lapack(d):
    """Textbook special case: the Cholesky-based inverse equals LAPACK
    dpotrf + dpotri (the page inverts through a Cholesky decomposition)."""
    from scipy.linalg import lapack
    rng = np.random.default_rng(100 + d)
    x = spd(rng, d, rows=d + 3)
    gamma = 1e-3
    z, info = oracle.damped_inverse(x, gamma)
    y = x + gamma * np.eye(d)
    u, i1 = lapack.dpotrf(y, lower=0)
    zi, i2 = lapack.dpotri(u, lower=0)
    assert i1 == 0 and i2 == 0 and info == 0
    zi = np.triu(zi) + np.triu(zi, 1).T
    assert oracle.rel_fro(z, zi) <= 1e-10


def test_cholesky_recovers_known_factor():
    """Y = U^T U for an integer upper-triangular U with positive diagonal is
    factored back to U."""
    u = np.array([[2.0, 1.0, -1.0, 3.0], [0, 3.0, 2.0, 0.0], [0, 0, 1.0, 4.0], [0, 0, 0, 5.0]])
    y = u.T @ u
    got, info = oracle.cholesky_upper(y)
    assert info == 0
    np.testing.assert_allclose(got, u, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("k", [1, 2, 5, 8])
def test_inverse_info_first_failing_pivot(k):
    """A non-positive leading minor of order k gives info = k (LAPACK xPOTRF)."""
    d = 8
    gamma = 1e-3
    x = np.eye(d)
    x[k - 1, k - 1] = -1.0 - gamma           # pivot k is -1
    _, info = oracle.damped_inverse(x, gamma)
    assert info == k
    _, info = oracle.damped_inverse(-2 * gamma * np.eye(d), gamma)
    assert info == 1
    xn = np.eye(d)
    xn[k - 1, k - 1] = np.nan
    _, info = oracle.damped_inverse(xn, gamma)
    assert info == k


def test_inverse_columns_agree_with_full():
    rng = np.random.default_rng(12)
    x = spd(rng, 45, rows=20)
    z, info = oracle.damped_inverse(x, 1e-3)
    cols = [0, 7, 44, 13]
    zc, info2 = oracle.damped_inverse_columns(x, 1e-3, cols)
    assert info == info2 == 0
    np.testing.assert_allclose(zc, z[:, cols].T, rtol=1e-12, atol=1e-12 * np.abs(z).max())


# ------------------------------------------------------------ precondition --

def _kron_brute(a, g, gamma, grad):
    """(A + gamma I) (x) (G + gamma I), built index by index, then vec(P)
    solved from K vec(P) = vec(grad) with column-major vec: the Kronecker
    inverse property turns the preconditioned update into G^-1 grad A^-1."""
    da, dg = a.shape[0], g.shape[0]
    ad = a + gamma * np.eye(da)
    gd = g + gamma * np.eye(dg)
    K = np.empty((da * dg, da * dg))
    for p in range(da):
        for q in range(da):
            K[p * dg:(p + 1) * dg, q * dg:(q + 1) * dg] = ad[p, q] * gd
    vec = grad.T.reshape(-1)                               # column-major vec of [dg, da]
    x = np.linalg.solve(K, vec)
    return x.reshape(da, dg).T


@pytest.mark.parametrize("da,dg", [(1, 1), (3, 5), (16, 16), (9, 2)])
def test_precondition_kronecker_brute_force(da, dg):
    rng = np.random.default_rng(da * 100 + dg)
    a, g = spd(rng, da, rows=da + 2), spd(rng, dg, rows=dg + 1)
    grad = rng.standard_normal((dg, da))
    gamma = 1e-2
    za, ia = oracle.damped_inverse(a, gamma)
    zg, ig = oracle.damped_inverse(g, gamma)
    assert ia == ig == 0
    p = oracle.precondition(zg, grad, za)
    ref = _kron_brute(a, g, gamma, grad)
    assert oracle.rel_fro(p, ref) <= 1e-9


def test_precondition_kronecker_fc1_shape():
    """Whole single-FC workload shape (d_a = 65, d_g = 32): K is 2080 x 2080."""
    from workloads import gen_a, gen_g, gen_grad
    cfg = CONFIGS[1]
    a = oracle.factor(oracle.upcast(gen_a(cfg, 0, 0)))
    g = oracle.factor(oracle.upcast(gen_g(cfg, 0, 0)))
    grad = oracle.upcast(gen_grad(cfg, 0, 0))
    gamma = float(np.float32(0.01))
    za, _ = oracle.damped_inverse(a, gamma)
    zg, _ = oracle.damped_inverse(g, gamma)
    assert oracle.rel_fro(oracle.precondition(zg, grad, za), _kron_brute(a, g, gamma, grad)) <= 1e-8


def test_precondition_closed_forms():
    rng = np.random.default_rng(13)
    grad = rng.standard_normal((6, 4))
    gamma = 0.05
    z4, _ = oracle.damped_inverse(np.zeros((4, 4)), gamma)
    z6, _ = oracle.damped_inverse(np.zeros((6, 6)), gamma)
    np.testing.assert_allclose(oracle.precondition(z6, grad, z4), grad / gamma**2, rtol=1e-13)
    z4, _ = oracle.damped_inverse(np.eye(4), gamma)
    z6, _ = oracle.damped_inverse(np.eye(6), gamma)
    np.testing.assert_allclose(oracle.precondition(z6, grad, z4), grad / (1 + gamma) ** 2, rtol=1e-13)


def test_precondition_entries_agree_with_full():
    rng = np.random.default_rng(14)
    zg, za = spd(rng, 11), spd(rng, 23)
    grad = rng.standard_normal((11, 23))
    p = oracle.precondition(zg, grad, za)
    ii, jj = rng.integers(0, 11, 30), rng.integers(0, 23, 30)
    np.testing.assert_allclose(oracle.precondition_entries(zg, grad, za, ii, jj), p[ii, jj], rtol=1e-12)


# --------------------------------------------------------------- workloads --

def test_resnet50_counts_reproduce_page(golden_dir):
    """The ResNet-50 layer list reproduces the page's printed counts."""
    with open(os.path.join(golden_dir, "resnet50_factor_counts.json")) as fh:
        gold = json.load(fh)
    L = CONFIGS[3].layers
    a = sum(l.d_a * (l.d_a + 1) // 2 for l in L)
    g = sum(l.d_g * (l.d_g + 1) // 2 for l in L)
    params = sum(l.d_a * l.d_g for l in L)
    per = [d * (d + 1) // 2 for l in L for d in (l.d_a, l.d_g)]
    assert round(a / 1e6, 1) == gold["a_upper_millions"]
    assert round(g / 1e6, 1) == gold["g_upper_millions"]
    assert round(params / 1e6, 1) == gold["params_millions"]
    assert min(per) == gold["min_factor_elements"]
    assert max(per) == gold["max_factor_elements"]


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(15)
    x = (rng.standard_normal(100000) * 0.02).astype(np.float32)
    # exact ties: low 16 bits 0x8000, with even and odd kept parts
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40008000], dtype=np.uint32).view(np.float32)
    x = np.concatenate([x, ties, np.array([1.0, -0.0, 0.0], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(x), ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


# ----------------------------------------------------------------- layers --

CONV_CASES = [
    dict(shape=(2, 3, 7, 6), kernel=(3, 3), stride=(1, 1), padding=(1, 1), dilation=(1, 1)),
    dict(shape=(1, 4, 9, 8), kernel=(3, 2), stride=(2, 1), padding=(1, 0), dilation=(1, 2)),
    dict(shape=(3, 2, 5, 5), kernel=(1, 1), stride=(2, 2), padding=(0, 0), dilation=(1, 1)),
    dict(shape=(2, 3, 8, 8), kernel=(7, 7), stride=(2, 2), padding=(3, 3), dilation=(1, 1)),
]


def test_im2col_matches_torch_unfold():
    """Patch matrix against torch's CPU unfold (a different implementation):
    unfold gives [n, c*kh*kw, oh*ow] with the same column order."""
    import torch
    rng = np.random.default_rng(41)
    for case in CONV_CASES:
        x = rng.standard_normal(case["shape"])
        a = oracle.im2col(x, case["kernel"], case["stride"], case["padding"], case["dilation"], ones=True)
        u = torch.nn.functional.unfold(torch.from_numpy(x), case["kernel"], dilation=case["dilation"],
                                       padding=case["padding"], stride=case["stride"])
        ref = u.permute(0, 2, 1).reshape(-1, u.shape[1]).numpy()
        np.testing.assert_array_equal(a[:, :-1], ref)
        assert np.all(a[:, -1] == 1.0)


def test_im2col_hand_example():
    """3 x 3 image 1..9, 2 x 2 kernel: the four patches written out."""
    x = np.arange(1.0, 10.0).reshape(1, 1, 3, 3)
    a = oracle.im2col(x, (2, 2))
    np.testing.assert_array_equal(a, [[1, 2, 4, 5], [2, 3, 5, 6], [4, 5, 7, 8], [5, 6, 8, 9]])
    # padding 1 puts zeros around: the first patch is [0, 0, 0, 1]
    b = oracle.im2col(x, (2, 2), padding=(1, 1))
    assert b.shape == (16, 4)
    np.testing.assert_array_equal(b[0], [0, 0, 0, 1])
    np.testing.assert_array_equal(b[-1], [9, 0, 0, 0])


def test_conv_weight_gradient_is_g_rows_times_patches():
    """For a convolution, autograd's weight gradient equals g^T a with
    g = grad_rows(dL/dy, 1) and a = im2col(x): this ties the row order of
    both factor inputs and the column order of the patches to the weight
    layout [c_out, c, kh, kw].  The bias gradient is g^T 1."""
    import torch
    rng = np.random.default_rng(42)
    for case in CONV_CASES:
        n, c, h, w = case["shape"]
        x = torch.from_numpy(rng.standard_normal(case["shape"]))
        conv = torch.nn.Conv2d(c, 5, case["kernel"], stride=case["stride"], padding=case["padding"],
                               dilation=case["dilation"], bias=True).double()
        y = conv(x)
        gy = torch.from_numpy(rng.standard_normal(tuple(y.shape)))
        y.backward(gy)
        a = oracle.im2col(x.numpy(), case["kernel"], case["stride"], case["padding"], case["dilation"], ones=True)
        g = oracle.grad_rows(gy.numpy().astype(np.float32), 1.0).astype(np.float64)
        gw = g.T @ a
        np.testing.assert_allclose(gw[:, :-1], conv.weight.grad.reshape(5, -1).numpy(), rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(gw[:, -1], conv.bias.grad.numpy(), rtol=1e-6, atol=1e-6)


def test_grad_rows_layout_and_scale():
    gy = np.arange(2 * 3 * 4, dtype=np.float32).reshape(2, 3, 2, 2)
    g = oracle.grad_rows(gy, 0.5)
    assert g.shape == (8, 3)
    for b in range(2):
        for ci in range(3):
            for p in range(4):
                assert g[b * 4 + p, ci] == np.float32(0.5) * gy[b, ci, p // 2, p % 2]
    # a fully connected layer: [b, c] scaled, no reordering
    np.testing.assert_array_equal(oracle.grad_rows(gy[:, :, 0, 0], 4.0), 4.0 * gy[:, :, 0, 0])


def test_grad_rows_bf16_rounding():
    """bfloat16 gradients: the scaled float32 value rounded to nearest even,
    checked against torch's conversion, including exact ties."""
    import torch
    rng = np.random.default_rng(43)
    x32 = (rng.standard_normal((4, 5, 3)) * 0.02).astype(np.float32)
    bits = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.grad_rows(bits, 3.0, bf16=True)
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float() * 3.0
    ref = vals.permute(0, 2, 1).reshape(12, 5).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000], dtype=np.uint32).view(np.float32)
    np.testing.assert_array_equal(oracle.bf16_round(ties), [0x3F80, 0x3F82, 0xBF80])


def test_grad_matrix_concatenates_bias():
    w = np.arange(12, dtype=np.float32).reshape(2, 3, 2)
    b = np.array([100.0, 200.0], dtype=np.float32)
    m = oracle.grad_matrix(w, b)
    np.testing.assert_array_equal(m, [[0, 1, 2, 3, 4, 5, 100], [6, 7, 8, 9, 10, 11, 200]])
    np.testing.assert_array_equal(oracle.grad_matrix(w), w.reshape(2, 6))
