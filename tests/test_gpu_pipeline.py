"""End to end: the whole per-GPU K-FAC step on the GPU (factors with running
average, pack and unpack through the fused buffer, damped inverses,
preconditioning) against the oracle pipeline run from the same raw inputs.

The stage tests gate each kernel; here the oracle's factors are fp64 while the
GPU's are float32, so the inverse amplifies the factor rounding by the
condition number.  The single-FC workload (gamma = 0.01) is gated at 1e-3;
the MLP workload's end-to-end error is checked against a bound of 1e-2."""
import numpy as np
import pytest

import linear_algebra_amd as la
import oracle
from tests.gpu_helpers import empty_f32, nan_f32, rel_fro, say, to_dev, to_host
from workloads import CONFIGS, gen_layer_step

pytestmark = pytest.mark.gpu


def run_pipeline(cid, steps, inverse_at):
    import torch
    cfg = CONFIGS[cid]
    L = cfg.layers
    eps = np.float32(cfg.eps)
    gamma = np.float32(cfg.gammas[0])
    ma = [nan_f32(l.d_a, l.d_a) for l in L]
    mg = [nan_f32(l.d_g, l.d_g) for l in L]
    za = [nan_f32(l.d_a, l.d_a) for l in L]
    zg = [nan_f32(l.d_g, l.d_g) for l in L]
    info = torch.full((2 * len(L),), -1, dtype=torch.int32, device="cuda:0")
    dims = [l.d_a for l in L] + [l.d_g for l in L]
    packed = empty_f32(la.kfac_packed_size(dims))
    ra, rg = [None] * len(L), [None] * len(L)
    rza, rzg = [None] * len(L), [None] * len(L)
    errs = []
    for t in range(steps):
        data = gen_layer_step(cfg, t, threads=8)
        la.kfac_factors([to_dev(d[0]) for d in data], ma, float(eps), t == 0)
        la.kfac_factors([to_dev(d[1]) for d in data], mg, float(eps), t == 0)
        la.kfac_pack_sym(ma + mg, packed, la.KFAC_PACK)
        la.kfac_pack_sym(ma + mg, packed, la.KFAC_UNPACK)
        for k, d in enumerate(data):
            ra[k] = oracle.running_average(ra[k], oracle.factor(oracle.upcast(d[0])), eps, t == 0)
            rg[k] = oracle.running_average(rg[k], oracle.factor(oracle.upcast(d[1])), eps, t == 0)
        if t in inverse_at:
            la.kfac_damped_inverse(ma + mg, float(gamma), za + zg, info)
            assert np.all(to_host(info) == 0)
            for k in range(len(L)):
                rza[k] = oracle.damped_inverse(ra[k], gamma)[0]
                rzg[k] = oracle.damped_inverse(rg[k], gamma)[0]
        if rza[0] is None:
            continue
        grads = [d[2] for d in data]
        outs = [empty_f32(*g.shape) for g in grads]
        la.kfac_precondition(zg, [to_dev(g) for g in grads], za, outs)
        for k in range(len(L)):
            errs.append(rel_fro(to_host(outs[k]), oracle.precondition(rzg[k], grads[k], rza[k])))
    return max(errs)


def test_pipeline_config1():
    err = run_pipeline(1, 3, inverse_at={2})
    say(f"config 1 end-to-end rel err {err:.3e}")
    assert err <= 1e-3


def test_pipeline_config2_first_steps():
    err = run_pipeline(2, 2, inverse_at={0})
    say(f"config 2 end-to-end rel err {err:.3e}")
    assert err <= 1e-2


@pytest.mark.timeout(600)
def test_pipeline_config2_full_schedule():
    """The MLP workload's whole schedule: 20 steps of factors with their
    running average, pack and unpack, inverses at steps 0 and 10 (of the
    running averages at those steps), every step preconditioned with the
    latest inverses, against the oracle pipeline from the same raw inputs."""
    cfg = CONFIGS[2]
    err = run_pipeline(2, cfg.steps, inverse_at=set(cfg.inverse_steps))
    say(f"config 2 full schedule ({cfg.steps} steps, inverses at {cfg.inverse_steps}): end-to-end rel err {err:.3e}")
    assert err <= 1e-2
