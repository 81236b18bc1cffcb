"""GPU parity: two-sided preconditioning against the fp64 oracle.

Gate: relative Frobenius error <= 1e-3 per layer.  Inputs: seeded weight
gradients of the workloads and exactly symmetric float32 matrices standing in
for the damped inverses (the kernel is a product of the three; symmetry is
its documented precondition)."""
import numpy as np
import pytest

import linear_algebra_amd as la
import oracle
from tests.gpu_helpers import empty_f32, rel_fro, say, to_dev, to_host
from workloads import CONFIGS, gen_grad

pytestmark = pytest.mark.gpu

TOL = 1e-3


def sym_f32(rng, d):
    """Symmetric positive definite stand-in with a spread spectrum."""
    q = rng.standard_normal((d, d)).astype(np.float32) / np.float32(np.sqrt(d))
    s = (q + q.T) * np.float32(0.5) + np.eye(d, dtype=np.float32) * np.float32(2.0)
    return np.ascontiguousarray(s)


def run(zgs, grads, zas):
    zg_d = [to_dev(z) for z in zgs]
    za_d = [to_dev(z) for z in zas]
    g_d = [to_dev(g) for g in grads]
    outs = [empty_f32(*g.shape) for g in grads]
    la.kfac_precondition(zg_d, g_d, za_d, outs)
    return [to_host(o) for o in outs]


@pytest.mark.parametrize("shapes", [[(1, 1)], [(32, 65)], [(10, 1025), (2048, 129), (7, 3)], [(300, 257), (128, 128)]])
def test_precondition_small(shapes):
    say("precondition small", shapes)
    rng = np.random.default_rng(sum(a * b for a, b in shapes))
    zgs = [sym_f32(rng, dg) for dg, _ in shapes]
    zas = [sym_f32(rng, da) for _, da in shapes]
    grads = [rng.standard_normal((dg, da)).astype(np.float32) for dg, da in shapes]
    outs = run(zgs, grads, zas)
    for zg, g, za, o in zip(zgs, grads, zas, outs):
        err = rel_fro(o, oracle.precondition(zg, g, za))
        assert err <= TOL, err


def test_precondition_identity_closed_form():
    """Z_G = Z_A = I / (1 + gamma): out = grad / (1 + gamma)^2 (equal up to float32 rounding)."""
    rng = np.random.default_rng(2)
    g = rng.standard_normal((200, 300)).astype(np.float32)
    c = np.float32(1.0 / 1.01)
    out = run([np.eye(200, dtype=np.float32) * c], [g], [np.eye(300, dtype=np.float32) * c])[0]
    np.testing.assert_allclose(out, g.astype(np.float64) * float(c) ** 2, rtol=1e-6, atol=1e-30)


def test_precondition_float32_rounding():
    """The products run on the bf16 matrix cores as six products of exact
    three-way splits: the result stays within float32 rounding (2e-6; a
    two-way split leaves about 1e-5)."""
    rng = np.random.default_rng(13)
    zg, za = sym_f32(rng, 640), sym_f32(rng, 1153)
    g = rng.standard_normal((640, 1153)).astype(np.float32)
    out = run([zg], [g], [za])[0]
    err = rel_fro(out, oracle.precondition(zg, g, za))
    say("precondition f32 rounding err", err)
    assert err <= 2e-6, err


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_precondition_config_full(cid):
    """Every layer of a workload in one call, compared in full."""
    cfg = CONFIGS[cid]
    rng = np.random.default_rng(100 + cid)
    L = cfg.layers
    # one stand-in inverse per distinct dimension keeps the host work small
    cache = {}
    def z(d):
        if d not in cache:
            cache[d] = sym_f32(rng, d)
        return cache[d]
    zgs = [z(l.d_g) for l in L]
    zas = [z(l.d_a) for l in L]
    grads = [gen_grad(cfg, 0, li) for li in range(len(L))]
    say(f"precondition config {cid}: {len(L)} layers")
    outs = run(zgs, grads, zas)
    worst = 0.0
    for k in range(len(L)):
        err = rel_fro(outs[k], oracle.precondition(zgs[k], grads[k], zas[k]))
        worst = max(worst, err)
        assert err <= TOL, (L[k].name, err)
    say(f"config {cid} precondition: worst rel err {worst:.3e}")
