"""GPU parity: triangular pack / unpack against the oracle, bit for bit."""
import numpy as np
import pytest

import linear_algebra_amd as la
import oracle
from tests.gpu_helpers import empty_f32, nan_f32, say, to_dev, to_host
from workloads import CONFIGS

pytestmark = pytest.mark.gpu


def random_bits(rng, d):
    """float32 matrices with arbitrary bit patterns, including NaN payloads,
    infinities, signed zeros and denormals: the copy must not touch them."""
    b = rng.integers(0, 2**32, size=(d, d), dtype=np.uint64).astype(np.uint32)
    return b.view(np.float32)


def run_pack_case(dims, rng, values="bits"):
    import torch
    mats = [random_bits(rng, d) if values == "bits" else rng.standard_normal((d, d)).astype(np.float32) for d in dims]
    ref = oracle.pack(mats)
    dm = [to_dev(m) for m in mats]
    packed = nan_f32(la.kfac_packed_size(dims))
    la.kfac_pack_sym(dm, packed, la.KFAC_PACK)
    got = to_host(packed)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    # unpack into fresh buffers and compare both triangles with the oracle
    out = [nan_f32(d, d) for d in dims]
    la.kfac_pack_sym(out, to_dev(ref), la.KFAC_UNPACK)
    ref_mats = oracle.unpack(ref, dims)
    for o, r in zip(out, ref_mats):
        np.testing.assert_array_equal(to_host(o).view(np.uint32), r.view(np.uint32))
    torch.cuda.synchronize()


@pytest.mark.parametrize("dims", [[1], [2], [3, 1, 2], [63, 64, 65], [5, 129, 1, 200, 4], [300, 257, 17]])
def test_pack_unpack_small(dims):
    say("pack/unpack", dims)
    run_pack_case(dims, np.random.default_rng(sum(dims)))


def test_pack_misaligned_buffer():
    """A packed buffer that is not 16-byte aligned takes the scalar store path."""
    import torch
    rng = np.random.default_rng(5)
    dims = [7, 33]
    mats = [rng.standard_normal((d, d)).astype(np.float32) for d in dims]
    ref = oracle.pack(mats)
    base = torch.full((ref.size + 1,), float("nan"), dtype=torch.float32, device="cuda:0")
    view = base[1:]
    la.kfac_pack_sym([to_dev(m) for m in mats], view, la.KFAC_PACK)
    np.testing.assert_array_equal(to_host(view).view(np.uint32), ref.view(np.uint32))


def test_pack_layer_boundaries_inside_vector():
    """Many tiny layers: a 4-element store group spans several layers."""
    dims = [1, 1, 2, 1, 3, 1, 1, 2, 5, 1]
    say("pack tiny layers", dims)
    run_pack_case(dims, np.random.default_rng(11))


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_pack_unpack_full_config(cid):
    """All factors of a workload, at its real dimensions, in one call each way."""
    dims = CONFIGS[cid].factor_dims()
    say(f"pack/unpack config {cid}: {len(dims)} factors, {sum(d * (d + 1) // 2 for d in dims)} packed elements")
    run_pack_case(dims, np.random.default_rng(cid), values="normal")
