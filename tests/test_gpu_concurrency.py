"""GPU: entry points called concurrently.

The library keeps no state between calls (beyond the table of the
allocation-free pack), so calls on different streams with different
workspaces may overlap on the GPU, and calls from different host threads may
overlap on the host.  Two host threads each run a factor -> pack -> unpack ->
inverse -> preconditioning sequence on a stream of their own, several times,
while the other does the same on different data; every result must equal,
bit for bit, the same sequence run alone on the default stream (the kernels
are deterministic)."""
import threading

import numpy as np
import pytest

import linear_algebra_amd as la
from tests.gpu_helpers import DEV, say, to_dev, to_host

pytestmark = pytest.mark.gpu

LAYERS = [(257, 96, 900), (130, 200, 400)]


def inputs(seed):
    rng = np.random.default_rng(seed)
    a = [np.maximum(rng.standard_normal((r, da)), 0).astype(np.float32) for da, _, r in LAYERS]
    g = [(1e-2 * rng.standard_normal((r, dg))).astype(np.float32) for _, dg, r in LAYERS]
    w = [(1e-3 * rng.standard_normal((dg, da))).astype(np.float32) for da, dg, _ in LAYERS]
    return [to_dev(x) for x in a], [to_dev(x) for x in g], [to_dev(x) for x in w]


def sequence(a, g, w, stream=None):
    import torch
    ma = [torch.zeros(x.shape[1], x.shape[1], device=DEV) for x in a]
    mg = [torch.zeros(x.shape[1], x.shape[1], device=DEV) for x in g]
    za = [torch.zeros_like(m) for m in ma]
    zg = [torch.zeros_like(m) for m in mg]
    out = [torch.zeros_like(x) for x in w]
    info = torch.zeros(len(ma) + len(mg), dtype=torch.int32, device=DEV)
    facs = ma + mg
    packed = torch.zeros(la.kfac_packed_size([m.shape[0] for m in facs]), device=DEV)
    la.kfac_factors(a, ma, 0.95, True, stream=stream)
    la.kfac_factors(g, mg, 0.95, True, stream=stream)
    la.kfac_pack_sym(facs, packed, la.KFAC_PACK, stream=stream)
    la.kfac_pack_sym(facs, packed, la.KFAC_UNPACK, stream=stream)
    la.kfac_damped_inverse(facs, 1e-2, za + zg, info, stream=stream)
    la.kfac_precondition(zg, w, za, out, stream=stream)
    return [packed, info] + za + zg + out


def test_two_host_threads_two_streams():
    import torch
    data = [inputs(1), inputs(2)]
    # buffers are made on the default stream; the side streams wait for them
    torch.cuda.synchronize()
    alone = [[to_host(t) for t in sequence(*d)] for d in data]
    results = [[], []]
    errors = []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            for _ in range(3):
                with torch.cuda.stream(s):
                    outs = sequence(*data[k], stream=s)
                s.synchronize()
                results[k].append([to_host(t) for t in outs])
        except Exception as e:   # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for k in range(2):
        say(f"thread {k}: {len(results[k])} runs")
        assert len(results[k]) == 3
        for run in results[k]:
            for x, y in zip(run, alone[k]):
                assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                                      y.view(np.uint32) if y.dtype == np.float32 else y)
        assert np.all(alone[k][1] == 0)
