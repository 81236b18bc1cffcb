"""GPU: the matrix-core rate reference (kfac_matrix_rate) runs each kind of
product loop, writes one finite, non-zero float per wave, and reports the
flops of the call (rounds x 4 products x 4 waves x workgroups x flops per
product).  It is a measuring aid, not a stage of the path."""
import pytest

import linear_algebra_amd as la
from tests.gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu

PER_PRODUCT = {la.KFAC_RATE_BF16: 32 * 32 * 16 * 2, la.KFAC_RATE_F64: 16 * 16 * 4 * 2, la.KFAC_RATE_F32: 32 * 32 * 2 * 2}


@pytest.mark.parametrize("kind", sorted(PER_PRODUCT))
def test_matrix_rate_runs(kind):
    import torch
    blocks, iters = 8, 2000
    say(f"matrix rate kind {kind}, {blocks} workgroups, {iters} rounds")
    sink = torch.zeros(4 * blocks, device=DEV)
    flops = la.kfac_matrix_rate(kind, iters, sink)
    torch.cuda.synchronize()
    assert flops == iters * 4 * 4 * blocks * PER_PRODUCT[kind]
    assert bool(torch.isfinite(sink).all())
    assert bool((sink != 0).all())
