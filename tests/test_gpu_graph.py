"""GPU: one whole K-FAC step captured in a HIP graph and replayed.

Every entry point only enqueues work on the caller's stream (descriptor
tables go up by a kernel launch, no memset or copy), so a step can be
captured.  The test captures factors with their running average, pack and
unpack (the workspace form and the allocation-free form), the damped
inverses and the preconditioning, replays the graph several times with eager
work and synchronisations between the replays, and after every replay
compares every output bit for bit with the same step run eagerly on a second
set of buffers (the kernels are deterministic).  The first replay is also
checked against the oracle."""
import numpy as np
import pytest

import linear_algebra_amd as la
import oracle
from tests.gpu_helpers import DEV, rel_fro, say, to_dev, to_host

pytestmark = pytest.mark.gpu

# (d_a, d_g, rows): a bordered order (257 = 4 * 64 + 1), ragged orders, split-K rows
LAYERS = [(130, 64, 300), (257, 100, 700), (65, 200, 2500)]
EPS, GAMMA = 0.95, 1e-2


def make_state(torch):
    s = {}
    s["ma"] = [torch.zeros(da, da, device=DEV) for da, _, _ in LAYERS]
    s["mg"] = [torch.zeros(dg, dg, device=DEV) for _, dg, _ in LAYERS]
    s["za"] = [torch.zeros(da, da, device=DEV) for da, _, _ in LAYERS]
    s["zg"] = [torch.zeros(dg, dg, device=DEV) for _, dg, _ in LAYERS]
    s["out"] = [torch.zeros(dg, da, device=DEV) for da, dg, _ in LAYERS]
    dims = [da for da, _, _ in LAYERS] + [dg for _, dg, _ in LAYERS]
    s["packed"] = torch.zeros(la.kfac_packed_size(dims), device=DEV)
    s["packed2"] = torch.zeros(la.kfac_packed_size(dims), device=DEV)
    s["info"] = torch.zeros(len(dims), dtype=torch.int32, device=DEV)
    return s


def step(s, a, g, w, first):
    facs = s["ma"] + s["mg"]
    la.kfac_factors(a, s["ma"], EPS, first)
    la.kfac_factors(g, s["mg"], EPS, first)
    la.kfac_pack_sym(facs, s["packed"], la.KFAC_PACK)
    la.kfac_pack_sym_static(facs, s["packed2"], la.KFAC_PACK)
    la.kfac_pack_sym(facs, s["packed"], la.KFAC_UNPACK)
    la.kfac_damped_inverse(facs, GAMMA, s["za"] + s["zg"], s["info"])
    la.kfac_precondition(s["zg"], w, s["za"], s["out"])


def outputs(s):
    keys = ["ma", "mg", "za", "zg", "out"]
    res = {k: [to_host(t) for t in s[k]] for k in keys}
    res["packed"] = to_host(s["packed"])
    res["packed2"] = to_host(s["packed2"])
    res["info"] = to_host(s["info"])
    return res


def test_step_captured_in_a_graph():
    import torch
    rng = np.random.default_rng(31)
    a = [to_dev(np.concatenate([np.maximum(rng.standard_normal((r, da - 1)), 0), np.ones((r, 1))], 1)
                .astype(np.float32)) for da, _, r in LAYERS]
    g = [to_dev((1e-2 * rng.standard_normal((r, dg))).astype(np.float32)) for _, dg, r in LAYERS]
    w = [to_dev((1e-3 * rng.standard_normal((dg, da))).astype(np.float32)) for da, dg, _ in LAYERS]
    cap, ref = make_state(torch), make_state(torch)

    # first step (M <- F) eagerly on both sets, and warm-up on a side stream
    # before capture, as torch asks
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(cap, a, g, w, True)
    torch.cuda.current_stream().wait_stream(side)
    step(ref, a, g, w, True)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(cap, a, g, w, False)     # the running-average form: M is read and updated
    torch.cuda.synchronize()

    for replay in range(4):
        say(f"graph replay {replay}")
        graph.replay()
        # eager work between replays, with its own synchronisation
        junk = torch.randn(1 << 20, device=DEV)
        float(junk.sum())
        step(ref, a, g, w, False)
        got, want = outputs(cap), outputs(ref)
        assert np.all(got["info"] == 0) and np.all(want["info"] == 0)
        for k in want:
            for x, y in zip(got[k] if isinstance(got[k], list) else [got[k]],
                            want[k] if isinstance(want[k], list) else [want[k]]):
                assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                                      y.view(np.uint32) if y.dtype == np.float32 else y), (replay, k)
        np.testing.assert_array_equal(got["packed"], got["packed2"])
        if replay == 0:
            # the state after the first replay: two running-average steps of the same data
            errs = []
            for k, (da, dg, _) in enumerate(LAYERS):
                fa = oracle.factor(oracle.upcast(to_host(a[k])))
                fg = oracle.factor(oracle.upcast(to_host(g[k])))
                za = oracle.damped_inverse(got["ma"][k], np.float32(GAMMA))[0]
                zg = oracle.damped_inverse(got["mg"][k], np.float32(GAMMA))[0]
                errs.append(rel_fro(np.triu(got["ma"][k]), np.triu(fa)))
                errs.append(rel_fro(np.triu(got["mg"][k]), np.triu(fg)))
                errs.append(rel_fro(got["out"][k], oracle.precondition(zg, to_host(w[k]), za)))
            say(f"  first replay against the oracle: worst rel err {max(errs):.3e}")
            assert max(errs) <= 1e-3
