"""GPU: every stage at the largest order the library accepts (16384).

- factors: a float32 input of 64 rows; sampled entries and every diagonal
  entry against the oracle's entry-wise sums;
- pack and unpack of a 16384 x 16384 matrix, bit for bit against the
  oracle's index loops;
- damped inverse of X = c 11^T (every block of the factorisation and of the
  triangular inverse is dense) against its closed form (Sherman-Morrison):
  (X + gamma I)^-1 = (I - c / (gamma + c d) 11^T) / gamma, in full;
- preconditioning with d_A = 16384 (d_G = 64) against the oracle's fp64
  products, in full."""
import numpy as np
import pytest

import linear_algebra_amd as la
import oracle
from tests.gpu_helpers import nan_f32, rel_fro, say, to_dev, to_host

pytestmark = pytest.mark.gpu

DMAX = 16384


@pytest.mark.timeout(600)
def test_largest_order_every_stage():
    import torch
    rng = np.random.default_rng(DMAX)
    d = DMAX

    say(f"max order {d}: factors")
    x = rng.standard_normal((64, d)).astype(np.float32)
    m = nan_f32(d, d)
    la.kfac_factors([to_dev(x)], [m], 0.95, True)
    got = to_host(m)
    ii = np.concatenate([rng.integers(0, d, 200), [0, d - 1]])
    jj = np.concatenate([rng.integers(0, d, 200), [d - 1, d - 1]])
    ii, jj = np.minimum(ii, jj), np.maximum(ii, jj)
    diag = oracle.factor_diagonal(x)
    err = np.abs(got[ii, jj] - oracle.factor_entries(x, ii, jj)) / np.sqrt(diag[ii] * diag[jj])
    derr = np.abs(np.diag(got) - diag) / diag
    say(f"  factor: worst sampled rel err {err.max():.3e}, diagonal {derr.max():.3e}")
    assert err.max() <= 1e-5 and derr.max() <= 1e-5
    del m, got

    say(f"max order {d}: pack and unpack")
    y = rng.standard_normal((d, d)).astype(np.float32)
    dy = to_dev(y)
    packed = torch.full((la.kfac_packed_size([d]),), float("nan"), device="cuda:0")
    la.kfac_pack_sym([dy], packed, la.KFAC_PACK)
    ref = oracle.pack([y])
    np.testing.assert_array_equal(to_host(packed).view(np.uint32), ref.view(np.uint32))
    back = nan_f32(d, d)
    la.kfac_pack_sym([back], packed, la.KFAC_UNPACK)
    np.testing.assert_array_equal(to_host(back).view(np.uint32), oracle.unpack(ref, [d])[0].view(np.uint32))
    del dy, packed, back, y, ref

    say(f"max order {d}: damped inverse of c 11^T")
    c, gamma = 1.0 / d, np.float32(1e-3)
    xd = to_dev(np.full((d, d), c, dtype=np.float32))
    z = nan_f32(d, d)
    info = torch.full((1,), -7, dtype=torch.int32, device="cuda:0")
    la.kfac_damped_inverse([xd], float(gamma), [z], info)
    assert int(to_host(info)[0]) == 0
    zh = to_host(z)
    del xd, z
    g = float(gamma)
    closed = np.full((d, d), -c / (g + c * d) / g)
    closed[np.diag_indices(d)] += 1.0 / g
    err = rel_fro(zh, closed)
    say(f"  inverse: rel err against the closed form {err:.3e}")
    assert err <= 1e-3
    np.testing.assert_array_equal(zh, zh.T)
    del zh, closed

    say(f"max order {d}: preconditioning, d_G = 64, d_A = {d}")
    dg = 64
    za = rng.standard_normal((d, d)).astype(np.float32)
    za = ((za + za.T) * np.float32(0.5)).astype(np.float32)
    zg = rng.standard_normal((dg, dg)).astype(np.float32)
    zg = ((zg + zg.T) * np.float32(0.5)).astype(np.float32)
    grad = (1e-3 * rng.standard_normal((dg, d))).astype(np.float32)
    out = nan_f32(dg, d)
    la.kfac_precondition([to_dev(zg)], [to_dev(grad)], [to_dev(za)], [out])
    err = rel_fro(to_host(out), oracle.precondition(zg, grad, za))
    say(f"  precondition: rel err {err:.3e}")
    assert err <= 1e-3
