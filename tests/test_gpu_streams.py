"""GPU: entry points called on a side stream.

The binding takes each call's workspace from torch's caching allocator on the
current stream.  When the kernels run on another stream, the block must stay
reserved until that stream has passed them, or the allocator may hand it to
new work on the current stream while the kernels still use it.  The test
holds the side stream behind a timed spin on the current stream, so the
kernels have not started when the call returns, and checks that an
allocation of the same size made right away gets other memory, then that the
result matches the oracle."""
import numpy as np
import pytest

import linear_algebra_amd as la
import oracle
from tests.gpu_helpers import DEV, rel_fro, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_workspace_kept_for_side_stream(monkeypatch):
    import torch
    rng = np.random.default_rng(17)
    dg, da = 300, 520
    zg = rng.standard_normal((dg, dg)).astype(np.float32)
    zg = (zg + zg.T).astype(np.float32)
    za = rng.standard_normal((da, da)).astype(np.float32)
    za = (za + za.T).astype(np.float32)
    grad = rng.standard_normal((dg, da)).astype(np.float32)
    d_zg, d_za, d_grad = to_dev(zg), to_dev(za), to_dev(grad)
    out = torch.full((dg, da), float("nan"), device=DEV)

    seen = []
    real = la._workspace

    def spy(nbytes, device):
        ws = real(nbytes, device)
        seen.append((ws.data_ptr(), ws.numel()))
        return ws

    monkeypatch.setattr(la, "_workspace", spy)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    torch.cuda._sleep(200_000_000)            # a bounded spin on the current stream
    ready = torch.cuda.Event()
    ready.record()
    side.wait_event(ready)
    la.kfac_precondition([d_zg], [d_grad], [d_za], [out], stream=side)
    ptr, nbytes = seen[-1]
    other = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    say("workspace", hex(ptr), nbytes, "next allocation", hex(other.data_ptr()))
    assert other.data_ptr() != ptr
    other.fill_(0xFF)
    torch.cuda.synchronize()
    err = rel_fro(to_host(out), oracle.precondition(zg, grad, za))
    say("side-stream precondition rel err", err)
    assert err <= 1e-5
