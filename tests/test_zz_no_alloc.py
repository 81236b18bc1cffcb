"""GPU: the allocation-free pack (kfac_pack_sym_static) against kfac_pack_sym.

Both directions, bit for bit, on two calls in a row (the second with fewer
and smaller factors, so the library's array still holds the first call's
larger table), and at the largest factor count the array holds.  The static
calls must not allocate through torch either."""
import numpy as np
import pytest

import linear_algebra_amd as la
import oracle
from tests.gpu_helpers import nan_f32, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def bits(rng, d):
    return rng.integers(0, 2**32, size=(d, d), dtype=np.uint64).astype(np.uint32).view(np.float32)


def allocations():
    import torch
    return torch.cuda.memory_stats().get("allocation.all.allocated", 0)


def check_both_directions(dims, rng):
    import torch
    mats = [bits(rng, d) for d in dims]
    dm = [to_dev(m) for m in mats]
    size = la.kfac_packed_size(dims)
    p_ws, p_st = nan_f32(size), nan_f32(size)
    la.kfac_pack_sym(dm, p_ws, la.KFAC_PACK)
    torch.cuda.synchronize()
    before = allocations()
    la.kfac_pack_sym_static(dm, p_st, la.KFAC_PACK)
    torch.cuda.synchronize()
    assert allocations() == before
    got_ws, got_st = to_host(p_ws).view(np.uint32), to_host(p_st).view(np.uint32)
    np.testing.assert_array_equal(got_st, got_ws)
    np.testing.assert_array_equal(got_st, oracle.pack(mats).view(np.uint32))
    u_ws = [nan_f32(d, d) for d in dims]
    u_st = [nan_f32(d, d) for d in dims]
    la.kfac_pack_sym(u_ws, p_ws, la.KFAC_UNPACK)
    torch.cuda.synchronize()
    before = allocations()
    la.kfac_pack_sym_static(u_st, p_ws, la.KFAC_UNPACK)
    torch.cuda.synchronize()
    assert allocations() == before
    for a, b in zip(u_ws, u_st):
        np.testing.assert_array_equal(to_host(b).view(np.uint32), to_host(a).view(np.uint32))


def test_static_pack_two_calls_second_smaller():
    rng = np.random.default_rng(91)
    for dims in ([300, 257, 17, 1025, 64, 2, 129, 700], [65, 3, 129]):
        say("static pack", dims)
        check_both_directions(dims, rng)


def test_static_pack_most_factors():
    """KFAC_STATIC_MAX_FACTORS factors of orders 1..4 (many layer boundaries
    inside one 16-byte unit), then a single factor."""
    rng = np.random.default_rng(92)
    dims = [1 + (k % 4) for k in range(1024)]
    say("static pack, 1024 factors")
    check_both_directions(dims, rng)
    check_both_directions([33], rng)
