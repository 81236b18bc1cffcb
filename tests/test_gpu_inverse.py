"""GPU parity: damped SPD inverse against the fp64 oracle.

Gate: relative Frobenius error <= 1e-3 (for gamma >= 1e-3; the large-factor
workload's gamma = 1e-4 is held to the same bound).  Both sides invert the
same float32 matrix; the inputs are float32 roundings of oracle factors of
the workloads' seeded activations and gradients (rank-deficient whenever a
layer has fewer rows than its dimension), so the condition numbers are the
workloads' own.  Outputs must also be exactly symmetric."""
import numpy as np
import pytest

import linear_algebra_amd as la
import oracle
from tests.gpu_helpers import nan_f32, rel_fro, say, to_dev, to_host
from workloads import CONFIGS, gen_a, gen_g

pytestmark = pytest.mark.gpu

TOL = 1e-3


def gpu_inverse(xs, gamma):
    import torch
    dx = [to_dev(x) for x in xs]
    zs = [nan_f32(*x.shape) for x in xs]
    info = torch.full((len(xs),), -7, dtype=torch.int32, device="cuda:0")
    la.kfac_damped_inverse(dx, gamma, zs, info)
    return [to_host(z) for z in zs], to_host(info)


def factor_input(x, in_dtype="f32"):
    return oracle.factor(oracle.upcast(x, in_dtype)).astype(np.float32)


def spd_f32(rng, d, rows):
    x = np.maximum(rng.standard_normal((rows, d)), 0).astype(np.float32)
    return factor_input(x)


@pytest.mark.parametrize("dims", [[1], [2, 3], [63, 64, 65], [100, 128, 129, 1], [200, 257, 64, 64, 31]])
def test_inverse_small_batch(dims):
    say("inverse small", dims)
    rng = np.random.default_rng(sum(dims))
    gamma = np.float32(1e-3)
    xs = [spd_f32(rng, d, max(1, d // 2)) for d in dims]   # rank-deficient
    zs, info = gpu_inverse(xs, gamma)
    assert np.all(info == 0), info
    for x, z in zip(xs, zs):
        ref, rinfo = oracle.damped_inverse(x, gamma)
        assert rinfo == 0
        err = rel_fro(z, ref)
        say("  d", x.shape[0], "err", err)
        assert err <= TOL
        np.testing.assert_array_equal(z, z.T)


def test_inverse_reads_upper_only():
    rng = np.random.default_rng(8)
    x = spd_f32(rng, 150, 300)
    xg = x.copy()
    xg[np.tril_indices(150, -1)] = 1e30
    z1, _ = gpu_inverse([x], 1e-2)
    z2, _ = gpu_inverse([xg], 1e-2)
    np.testing.assert_array_equal(z1[0], z2[0])


def test_inverse_closed_forms():
    gamma = np.float32(0.25)
    d = 130
    diag = np.linspace(0.0, 5.0, d).astype(np.float32)
    zs, info = gpu_inverse([np.diag(diag), np.zeros((70, 70), np.float32)], gamma)
    assert np.all(info == 0)
    np.testing.assert_allclose(zs[0], np.diag(1.0 / (diag.astype(np.float64) + float(gamma))), rtol=1e-6, atol=1e-30)
    np.testing.assert_allclose(zs[1], np.eye(70) / float(gamma), rtol=1e-6, atol=0)


@pytest.mark.parametrize("k", [1, 5, 64, 65, 100])
def test_inverse_info_reports_first_failing_pivot(k):
    """A matrix whose leading minor of order k is negative reports info = k,
    like the oracle; its neighbours in the batch are unaffected."""
    d = 130
    gamma = np.float32(1e-3)
    bad = np.eye(d, dtype=np.float32)
    bad[k - 1, k - 1] = np.float32(-1.0) - gamma
    good = spd_f32(np.random.default_rng(k), 90, 200)
    zs, info = gpu_inverse([good, bad, good], gamma)
    _, rinfo = oracle.damped_inverse(bad, gamma)
    assert rinfo == k
    assert list(info) == [0, k, 0]
    ref, _ = oracle.damped_inverse(good, gamma)
    assert rel_fro(zs[0], ref) <= TOL and rel_fro(zs[2], ref) <= TOL


def test_inverse_nan_reports_info():
    d = 70
    x = np.eye(d, dtype=np.float32)
    x[10, 10] = np.nan
    _, info = gpu_inverse([x], 1e-3)
    _, rinfo = oracle.damped_inverse(x, np.float32(1e-3))
    assert info[0] == rinfo == 11


# Orders one above a multiple of 64 (the factor A of a layer with a bias)
# factor the leading part in blocks and attach the last row and column
# afterwards as a border; these cases aim at that path.
@pytest.mark.parametrize("k", [1, 64, 65, 100, 129])
def test_inverse_bordered_info_reports_first_failing_pivot(k):
    d = 129
    say("inverse bordered info", k)
    gamma = np.float32(1e-3)
    bad = np.eye(d, dtype=np.float32)
    bad[k - 1, k - 1] = np.float32(-1.0) - gamma
    good = spd_f32(np.random.default_rng(k), d, 300)
    zs, info = gpu_inverse([good, bad, good], gamma)
    _, rinfo = oracle.damped_inverse(bad, gamma)
    assert rinfo == k
    assert list(info) == [0, k, 0]
    ref, _ = oracle.damped_inverse(good, gamma)
    assert rel_fro(zs[0], ref) <= TOL and rel_fro(zs[2], ref) <= TOL


@pytest.mark.parametrize("where", [(5, 128), (128, 128)])
def test_inverse_bordered_nan_in_border_reports_info(where):
    d = 129
    x = np.eye(d, dtype=np.float32)
    x[where] = np.nan
    _, info = gpu_inverse([x], 1e-3)
    _, rinfo = oracle.damped_inverse(x, np.float32(1e-3))
    assert info[0] == rinfo == d


def test_inverse_bordered_closed_form_and_upper_only():
    gamma = np.float32(0.25)
    d = 193
    diag = np.linspace(0.0, 5.0, d).astype(np.float32)
    zs, info = gpu_inverse([np.diag(diag)], gamma)
    assert info[0] == 0
    np.testing.assert_allclose(zs[0], np.diag(1.0 / (diag.astype(np.float64) + float(gamma))), rtol=1e-6, atol=1e-30)
    x = spd_f32(np.random.default_rng(3), d, 400)
    xg = x.copy()
    xg[np.tril_indices(d, -1)] = 1e30
    z1, _ = gpu_inverse([x], 1e-2)
    z2, _ = gpu_inverse([xg], 1e-2)
    np.testing.assert_array_equal(z1[0], z2[0])
    ref, _ = oracle.damped_inverse(x, np.float32(1e-2))
    assert rel_fro(z1[0], ref) <= TOL


def test_inverse_bordered_nearly_dependent_last_row():
    """The last row is nearly a combination of the others, so its pivot
    xi - w^T w is small (cancellation) and the inverse is large along one
    direction."""
    rng = np.random.default_rng(12)
    n = 128
    x11 = spd_f32(rng, n, 3 * n).astype(np.float64)
    a = rng.standard_normal(n) / np.sqrt(n)
    col = x11 @ a
    x = np.zeros((n + 1, n + 1))
    x[:n, :n] = x11
    x[:n, n] = x[n, :n] = col
    x[n, n] = a @ x11 @ a + 1e-2
    x = x.astype(np.float32)
    gamma = np.float32(1e-3)
    zs, info = gpu_inverse([x], gamma)
    ref, rinfo = oracle.damped_inverse(x, gamma)
    assert info[0] == rinfo == 0
    err = rel_fro(zs[0], ref)
    say("  bordered, small last pivot: err", err, "z_nn", zs[0][n, n])
    assert err <= TOL
    np.testing.assert_array_equal(zs[0], zs[0].T)


_FACTOR_CACHE = {}


def config_factor_inputs(cid, rows_cap=None):
    """float32 factors (A's then G's) of a workload's first step, from the
    oracle; rows_cap limits the rows drawn per layer (same recipe).  Layers
    are drawn and reduced in parallel threads (numpy releases the GIL), and
    the result is kept for the other tests of this module."""
    from concurrent.futures import ThreadPoolExecutor
    key = (cid, rows_cap)
    if key in _FACTOR_CACHE:
        return _FACTOR_CACHE[key]
    cfg = CONFIGS[cid]

    def rows(l):
        return l.rows if rows_cap is None else min(l.rows, rows_cap)

    jobs = [(gen_a, li) for li in range(cfg.n_layers)] + [(gen_g, li) for li in reversed(range(cfg.n_layers))]

    def one(j):
        f = factor_input(j[0](cfg, 0, j[1], rows=rows(cfg.layers[j[1]])), cfg.in_dtype)
        if f.shape[0] >= 1024:
            say(f"  oracle factor: config {cid} layer {j[1]} {'A' if j[0] is gen_a else 'G'} ({f.shape[0]})")
        return f

    with ThreadPoolExecutor(max_workers=4) as ex:
        xs = list(ex.map(one, jobs))
    _FACTOR_CACHE.clear()
    _FACTOR_CACHE[key] = xs
    return xs


def check_sampled(xs, zs, gamma, pick, ncols=6, seed=0):
    """Oracle columns of the picked matrices (one Cholesky each)."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for k in pick:
        d = xs[k].shape[0]
        cols = np.unique(np.concatenate([[0, d - 1], rng.integers(0, d, ncols)]))
        ref, info = oracle.damped_inverse_columns(xs[k], gamma, cols)
        assert info == 0
        err = rel_fro(zs[k][:, cols].T, ref)
        worst = max(worst, err)
        if d >= 1024:
            say(f"  matrix {k} (order {d}): {len(cols)} oracle columns, rel err {err:.3e}")
        assert err <= TOL, (k, d, err)
    return worst


def check_full_per_order(xs, zs, gamma):
    """The whole inverse of the first matrix of every order against the
    oracle's (Cholesky, then every column by substitution)."""
    worst, seen = 0.0, set()
    for k, x in enumerate(xs):
        d = x.shape[0]
        if d in seen:
            continue
        seen.add(d)
        ref, info = oracle.damped_inverse(x, gamma)
        assert info == 0
        err = rel_fro(zs[k], ref)
        worst = max(worst, err)
        say(f"  matrix {k} (order {d}): whole inverse, rel err {err:.3e}")
        assert err <= TOL, (k, d, err)
    return worst


def test_inverse_config1_full():
    xs = config_factor_inputs(1)
    gamma = np.float32(0.01)
    zs, info = gpu_inverse(xs, gamma)
    assert np.all(info == 0)
    for x, z in zip(xs, zs):
        ref, _ = oracle.damped_inverse(x, gamma)
        assert rel_fro(z, ref) <= TOL


def test_inverse_config2_full():
    xs = config_factor_inputs(2)
    gamma = np.float32(1e-3)
    say("config 2 inverse", [x.shape[0] for x in xs])
    zs, info = gpu_inverse(xs, gamma)
    assert np.all(info == 0)
    for z in zs:
        np.testing.assert_array_equal(z, z.T)
    worst = check_sampled(xs, zs, gamma, range(len(xs)), ncols=8)
    # the two 1025-wide and the 10-wide factors in full
    for k, x in enumerate(xs):
        if x.shape[0] <= 1025:
            ref, _ = oracle.damped_inverse(x, gamma)
            err = rel_fro(zs[k], ref)
            worst = max(worst, err)
            assert err <= TOL
    say(f"config 2 inverse: worst rel err {worst:.3e}")


def bucket_representatives(xs):
    seen, pick = set(), []
    for k, x in enumerate(xs):
        b = (x.shape[0] + 63) // 64
        if b not in seen:
            seen.add(b)
            pick.append(k)
    return pick


def test_inverse_config3_full_batch():
    """All 108 ResNet-50 factors, at the workload's full row counts, in one
    call; one matrix of every size bucket checked against oracle columns,
    the first matrix of every order in whole, every output checked for
    symmetry."""
    xs = config_factor_inputs(3)
    gamma = np.float32(1e-3)
    say("config 3 inverse: 108 matrices")
    zs, info = gpu_inverse(xs, gamma)
    assert np.all(info == 0), info
    for z in zs:
        np.testing.assert_array_equal(z, z.T)
    worst = check_sampled(xs, zs, gamma, bucket_representatives(xs))
    worst = max(worst, check_full_per_order(xs, zs, gamma))
    say(f"config 3 inverse: worst rel err (sampled and whole) {worst:.3e}")


def size_representatives(xs):
    """The first and the last matrix of every distinct order."""
    first, last = {}, {}
    for k, x in enumerate(xs):
        first.setdefault(x.shape[0], k)
        last[x.shape[0]] = k
    return sorted(set(first.values()) | set(last.values()))


@pytest.mark.timeout(600)
def test_inverse_config4_full_batch():
    """The encoder's 96 factors (orders 1024, 1025, 3072, 4096, 4097; the
    bf16 inputs upcast exactly) in one call, the configuration the benchmark
    runs: the first and last matrix of every order against oracle columns,
    the first matrix of every order in whole, every output checked for
    symmetry."""
    xs = config_factor_inputs(4)
    gamma = np.float32(1e-3)
    say("config 4 inverse:", len(xs), "matrices, orders", sorted({x.shape[0] for x in xs}))
    zs, info = gpu_inverse(xs, gamma)
    assert np.all(info == 0), info
    for z in zs:
        np.testing.assert_array_equal(z, z.T)
    worst = check_sampled(xs, zs, gamma, size_representatives(xs), ncols=6, seed=4)
    worst = max(worst, check_full_per_order(xs, zs, gamma))
    say(f"config 4 inverse: worst rel err (sampled and whole) {worst:.3e}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("gamma", [1e-2, 1e-4])
def test_inverse_config5_full_batch(gamma):
    """The large-factor workload's 32 factors at its full 25,088 rows, in one
    call as the benchmark makes it (the bordered 2305 and 4609 with the
    plain 512, 2048 and 4096 in one launch sequence): every matrix against
    oracle columns, the first matrix of every order in whole, every output
    checked for symmetry.  gamma = 1e-4 is held to the same bound."""
    xs = config_factor_inputs(5)
    gamma = np.float32(gamma)
    say("config 5 inverse, full batch, gamma", float(gamma), [x.shape[0] for x in xs])
    zs, info = gpu_inverse(xs, gamma)
    assert np.all(info == 0), info
    for z in zs:
        np.testing.assert_array_equal(z, z.T)
    worst = check_sampled(xs, zs, gamma, range(len(xs)), ncols=3, seed=int(1 / gamma))
    worst = max(worst, check_full_per_order(xs, zs, gamma))
    say(f"config 5 inverse gamma={float(gamma)}: worst rel err (sampled and whole) {worst:.3e}")


@pytest.mark.parametrize("gamma", [1e-2, 1e-4])
def test_inverse_config5_ill_conditioned(gamma):
    """Large factors with 10% of the input columns scaled x100: the largest
    condition numbers of the five workloads."""
    cfg = CONFIGS[5]
    xs = [factor_input(gen_a(cfg, 0, li, rows=6000)) for li in (0, 1)] + \
         [factor_input(gen_g(cfg, 0, li, rows=6000)) for li in (0, 1, 2)]
    gamma = np.float32(gamma)
    say("config 5 inverse, gamma", float(gamma), [x.shape[0] for x in xs])
    zs, info = gpu_inverse(xs, gamma)
    assert np.all(info == 0), info
    worst = check_sampled(xs, zs, gamma, range(len(xs)), ncols=4)
    say(f"config 5 inverse gamma={float(gamma)}: worst sampled rel err {worst:.3e}")


def test_inverse_well_conditioned_to_float32_rounding():
    """With a condition number near 10 the only error left is the float32
    rounding of the output: every matrix within 1e-6 of the oracle."""
    rng = np.random.default_rng(21)
    gamma = np.float32(0.5)
    xs = [spd_f32(rng, d, 4 * d) for d in (64, 100, 257, 700)]
    zs, info = gpu_inverse(xs, gamma)
    assert np.all(info == 0)
    for x, z in zip(xs, zs):
        ref, _ = oracle.damped_inverse(x, gamma)
        err = rel_fro(z, ref)
        say("  well-conditioned d", x.shape[0], "err", err)
        assert err <= 1e-6


@pytest.mark.timeout(400)
def test_inverse_max_dimension_8192():
    """The largest dimension of the inverse-time sweep, d = 8192, against
    oracle columns, and the residual (X + gamma I) z_j - e_j of those
    columns in fp64."""
    d, gamma = 8192, np.float32(1e-3)
    rng = np.random.default_rng(8192)
    a = np.maximum(rng.standard_normal((d, d), dtype=np.float32), 0)
    x = ((a.T @ a) / np.float32(d)).astype(np.float32)
    x = np.triu(x) + np.triu(x, 1).T
    say("inverse d=8192")
    zs, info = gpu_inverse([x], gamma)
    assert info[0] == 0
    z = zs[0]
    cols = np.array([0, 1234, 5000, d - 1])
    ref, rinfo = oracle.damped_inverse_columns(x, gamma, cols)
    assert rinfo == 0
    err = rel_fro(z[:, cols].T, ref)
    xd = x.astype(np.float64) + float(gamma) * np.eye(d)
    res = xd @ z[:, cols].astype(np.float64) - np.eye(d)[:, cols]
    say(f"inverse d=8192: rel err {err:.3e}, max residual {np.abs(res).max():.3e}")
    assert err <= TOL
    # backward error of a float32-stored inverse: a few units of float32
    # rounding times ||X + gamma I|| ||z_j||
    for q in range(len(cols)):
        bound = 64 * 2.0 ** -24 * np.linalg.norm(xd, 1) * np.abs(z[:, cols[q]]).sum()
        assert np.abs(res[:, q]).max() <= bound


def test_inverse_many_ragged_matrices():
    """Seventy factors of ragged sizes (odd and even block counts, sizes one
    off a multiple of 64) in one call: enough 2 x 2 groups of blocks
    (sum over matrices of n2 (n2 + 1) / 2 with n2 = ceil(ceil(d / 64) / 2),
    at least 1024) for the product V V^T to run on 128 x 128 tiles.  Every
    matrix against the oracle in full."""
    rng = np.random.default_rng(70)
    edge = [1, 2, 63, 64, 65, 127, 128, 129, 191, 192, 193, 1023, 1025]
    dims = edge + [int(x) for x in rng.integers(100, 1400, 70 - len(edge))]
    groups = sum(((d + 127) // 128) * ((d + 127) // 128 + 1) // 2 for d in dims)
    assert groups >= 1024, groups
    gamma = np.float32(1e-3)
    xs = [spd_f32(rng, d, max(1, d // 2)) for d in dims]
    say("inverse 70 ragged matrices, groups", groups)
    zs, info = gpu_inverse(xs, gamma)
    assert np.all(info == 0), info
    worst = 0.0
    for x, z in zip(xs, zs):
        ref, rinfo = oracle.damped_inverse(x, gamma)
        assert rinfo == 0
        err = rel_fro(z, ref)
        worst = max(worst, err)
        assert err <= TOL, (x.shape[0], err)
        np.testing.assert_array_equal(z, z.T)
    say(f"70 ragged matrices: worst rel err {worst:.3e}")
