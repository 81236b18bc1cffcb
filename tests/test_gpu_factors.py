"""GPU parity: Kronecker factors with running average against the fp64 oracle.

Gate (relative Frobenius error on the upper triangle incl. the diagonal):
1e-5 for float32 inputs, 2e-3 for bfloat16 inputs.  The oracle consumes the
exact values given to the GPU (bf16 upcast exactly)."""
import numpy as np
import pytest

import linear_algebra_amd as la
import oracle
from tests.gpu_helpers import nan_f32, say, to_dev, to_host, upper_rel_fro
from workloads import CONFIGS, gen_a, gen_g, gen_layer_step

pytestmark = pytest.mark.gpu

TOL_F32, TOL_BF16 = 1e-5, 2e-3
EPS = 0.95


def gpu_factors(xs, ms, eps, first):
    la.kfac_factors([to_dev(x) if isinstance(x, np.ndarray) else x for x in xs], ms, eps, first)


@pytest.mark.parametrize("shapes", [
    [(1, 1)],
    [(32, 65), (32, 32)],
    [(100, 129), (7, 300), (1000, 64), (3, 2)],
    [(5000, 257), (2000, 130), (600, 1)],
])
def test_factors_small_running_average(shapes):
    """First step, then two running-average steps, several layers per call
    (ragged tails in rows and in both tile directions)."""
    say("factors small", shapes)
    rng = np.random.default_rng(len(shapes) * 7 + shapes[0][1])
    ms = [nan_f32(d, d) for _, d in shapes]
    ref = [None] * len(shapes)
    for step in range(3):
        xs = [np.maximum(rng.standard_normal((r, d)), 0).astype(np.float32) for r, d in shapes]
        gpu_factors(xs, ms, EPS, step == 0)
        for k, x in enumerate(xs):
            ref[k] = oracle.running_average(ref[k], oracle.factor(oracle.upcast(x)), np.float32(EPS), step == 0)
        for k, m in enumerate(ms):
            got = to_host(m)
            err = upper_rel_fro(got, ref[k])
            assert err <= TOL_F32, (shapes[k], step, err)
            # strict lower triangle is left as it was (NaN sentinel)
            assert np.all(np.isnan(got[np.tril_indices(shapes[k][1], -1)]))


def test_factors_tall_split_k():
    """Very tall inputs use split-K partial tiles and the fixed-order reduce."""
    say("factors tall split-K")
    rng = np.random.default_rng(3)
    xs = [np.maximum(rng.standard_normal((200000, 147)), 0).astype(np.float32),
          rng.standard_normal((150000, 64)).astype(np.float32)]
    ms = [nan_f32(147, 147), nan_f32(64, 64)]
    gpu_factors(xs, ms, EPS, True)
    for x, m in zip(xs, ms):
        err = upper_rel_fro(to_host(m), oracle.factor(oracle.upcast(x)))
        say("  tall err", x.shape, err)
        assert err <= TOL_F32


def test_factors_deterministic():
    rng = np.random.default_rng(4)
    x = to_dev(rng.standard_normal((70000, 300)).astype(np.float32))
    m1, m2 = nan_f32(300, 300), nan_f32(300, 300)
    la.kfac_factors([x], [m1], EPS, True)
    la.kfac_factors([x], [m2], EPS, True)
    np.testing.assert_array_equal(to_host(m1).view(np.uint32)[np.triu_indices(300)],
                                  to_host(m2).view(np.uint32)[np.triu_indices(300)])


def test_factors_f32_float32_rounding():
    """float32 inputs run on the bf16 matrix cores as six products of exact
    three-way splits.  With values that use all 24 significand bits (and a
    2^40 spread of magnitudes) the factor stays within float32 rounding:
    1e-6, a tenth of the gate (a two-way split leaves about 1e-5)."""
    say("factors f32 rounding")
    rng = np.random.default_rng(12)
    x = rng.standard_normal((6000, 300)).astype(np.float32)
    y = (rng.standard_normal((3000, 257)) * np.exp2(rng.integers(-20, 20, size=(1, 257)))).astype(np.float32)
    ms = [nan_f32(300, 300), nan_f32(257, 257)]
    gpu_factors([x, y], ms, EPS, True)
    for h, m in zip((x, y), ms):
        err = upper_rel_fro(to_host(m), oracle.factor(oracle.upcast(h)))
        say("  f32 rounding err", h.shape, err)
        assert err <= 1e-6, (h.shape, err)


def test_factors_bf16_small():
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(5)
    shapes = [(4096, 1025), (300, 70)]
    xs = [f32_to_bf16_bits(0.02 * rng.standard_normal((r, d)).astype(np.float32)) for r, d in shapes]
    ms = [nan_f32(d, d) for _, d in shapes]
    gpu_factors(xs, ms, EPS, True)
    for x, m in zip(xs, ms):
        err = upper_rel_fro(to_host(m), oracle.factor(oracle.upcast(x, "bf16")))
        say("  bf16 err", x.shape, err)
        assert err <= TOL_BF16


def test_factors_bf16_row_alignment():
    """bfloat16 rows that start 4-byte aligned (even width, aligned base) are
    copied into LDS whole; rows of odd width, or an input whose base sits one
    element past an aligned address, are read element by element.  One call
    mixes both kinds (widths that are even but not a multiple of 8, an odd
    one, a tall split-K one), two running-average steps, and the same data
    at both alignments gives results within rounding of each other."""
    import torch
    from workloads import f32_to_bf16_bits
    say("factors bf16 row alignment")
    rng = np.random.default_rng(6)
    shapes = [(300, 70), (257, 33), (1000, 1026), (90000, 130), (513, 128)]
    ms = [nan_f32(d, d) for _, d in shapes]
    ref = [None] * len(shapes)
    for step in range(2):
        hs = [f32_to_bf16_bits(0.05 * rng.standard_normal((r, d)).astype(np.float32)) for r, d in shapes]
        xs = [to_dev(h) for h in hs]
        # the last input: same values, base one element past an aligned address
        r, d = shapes[-1]
        flat = torch.empty(r * d + 8, dtype=torch.bfloat16, device=xs[-1].device)
        shifted = flat[1:1 + r * d].view(r, d)
        shifted.copy_(xs[-1])
        assert shifted.data_ptr() % 4 == 2
        m_shift = nan_f32(d, d)
        gpu_factors(xs, ms, EPS, step == 0)
        gpu_factors([shifted], [m_shift], EPS, True)
        for k, h in enumerate(hs):
            ref[k] = oracle.running_average(ref[k], oracle.factor(oracle.upcast(h, "bf16")), np.float32(EPS), step == 0)
            err = upper_rel_fro(to_host(ms[k]), ref[k])
            say("  bf16 err", shapes[k], step, err)
            assert err <= TOL_BF16, (shapes[k], step, err)
        one = oracle.factor(oracle.upcast(hs[-1], "bf16"))
        assert upper_rel_fro(to_host(m_shift), one) <= TOL_BF16
        if step == 0:
            assert upper_rel_fro(to_host(m_shift), to_host(ms[-1]).astype(np.float64)) <= 1e-6


@pytest.mark.parametrize("dtype,rows,d", [
    ("bf16", 97, 1025), ("bf16", 33, 65), ("bf16", 1000, 33), ("bf16", 65, 4097),
    ("bf16", 97, 130), ("f32", 97, 1025), ("f32", 1000, 33),
])
def test_factors_slab_and_matrix_ends(dtype, rows, d):
    """Only the last two columns are nonzero, in the last row of every 32-row
    slab and in the matrix's last row: the elements read at the end of each
    slab's address range and at the very end of the input.  The factor is a
    handful of exact sums, so any element lost at a range end shows."""
    from workloads import f32_to_bf16_bits
    say("factors slab ends", dtype, rows, d)
    x = np.zeros((rows, d), dtype=np.float32)
    ends = sorted(set(list(range(31, rows, 32)) + [rows - 1]))
    x[ends, d - 1] = 1.0
    if d > 1:
        x[ends, d - 2] = 2.0
    h = f32_to_bf16_bits(x) if dtype == "bf16" else x
    m = nan_f32(d, d)
    gpu_factors([h], [m], EPS, True)
    ref = oracle.factor(oracle.upcast(h, "bf16") if dtype == "bf16" else oracle.upcast(h))
    got = to_host(m).astype(np.float64)
    assert got[d - 1, d - 1] == pytest.approx(len(ends) / rows, rel=1e-6)
    assert upper_rel_fro(got, ref) <= 1e-6


def test_factors_bf16_wide_tiles():
    """bf16 launches with enough tiles, no split of K and at most 16384 rows
    take 256 x 128 tiles.  One call over orders with every kind of edge
    (multiples of 256, of 128 only, 64m + 1, others; 1223 wide tiles in
    all), rows not a multiple of the 32-row slab, two running-average steps.
    The last layer carries the slab-end pattern: only its last two columns
    are nonzero, in the last row of every slab and in the last row."""
    from workloads import f32_to_bf16_bits
    say("factors bf16 wide tiles")
    rng = np.random.default_rng(8)
    rows = 1000
    dims = [4097, 4096, 3000, 2049, 2000, 1025, 1000, 513, 384, 257, 130, 4097]
    ms = [nan_f32(d, d) for d in dims]
    ref = [None] * len(dims)
    ends = sorted(set(list(range(31, rows, 32)) + [rows - 1]))
    for step in range(2):
        fs = [0.05 * rng.standard_normal((rows, d)).astype(np.float32) for d in dims]
        last = np.zeros((rows, dims[-1]), dtype=np.float32)
        last[ends, -1] = 1.0
        last[ends, -2] = 2.0
        fs[-1] = last
        hs = [f32_to_bf16_bits(f) for f in fs]
        gpu_factors(hs, ms, EPS, step == 0)
        for k, h in enumerate(hs):
            ref[k] = oracle.running_average(ref[k], oracle.factor(oracle.upcast(h, "bf16")), np.float32(EPS), step == 0)
            got = to_host(ms[k])
            err = upper_rel_fro(got, ref[k])
            say("  wide err", dims[k], step, err)
            assert err <= TOL_BF16, (dims[k], step, err)
            assert np.all(np.isnan(got[np.tril_indices(dims[k], -1)]))
        got = to_host(ms[-1]).astype(np.float64)
        assert upper_rel_fro(got, ref[-1]) <= 1e-6
        assert got[-1, -1] == pytest.approx(ref[-1][-1, -1], rel=1e-6)


def run_config_factors(cid, steps=None):
    """A factors then G factors of every layer, as one call each, for the
    given steps of the workload's schedule; full comparison with the oracle."""
    cfg = CONFIGS[cid]
    steps = cfg.steps if steps is None else steps
    L = cfg.layers
    ma = [nan_f32(l.d_a, l.d_a) for l in L]
    mg = [nan_f32(l.d_g, l.d_g) for l in L]
    ref_a, ref_g = [None] * len(L), [None] * len(L)
    worst = 0.0
    for step in range(steps):
        data = gen_layer_step(cfg, step, threads=16)
        a = [t[0] for t in data]
        g = [t[1] for t in data]
        gpu_factors(a, ma, EPS, step == 0)
        gpu_factors(g, mg, EPS, step == 0)
        tol = TOL_BF16 if cfg.in_dtype == "bf16" else TOL_F32
        for k in range(len(L)):
            fa = oracle.factor(oracle.upcast(a[k], cfg.in_dtype))
            fg = oracle.factor(oracle.upcast(g[k], cfg.in_dtype))
            ref_a[k] = oracle.running_average(ref_a[k], fa, np.float32(EPS), step == 0)
            ref_g[k] = oracle.running_average(ref_g[k], fg, np.float32(EPS), step == 0)
            ea = upper_rel_fro(to_host(ma[k]), ref_a[k])
            eg = upper_rel_fro(to_host(mg[k]), ref_g[k])
            worst = max(worst, ea, eg)
            assert ea <= tol and eg <= tol, (cid, step, L[k].name, ea, eg)
        del data, a, g
    say(f"config {cid}: worst factor rel err {worst:.3e} over {steps} step(s)")


def test_factors_config1():
    run_config_factors(1)


def test_factors_config2_two_steps():
    run_config_factors(2, steps=2)


def test_factors_config3_full():
    say("config 3 factors (ResNet-50 shapes, 108 factors)")
    run_config_factors(3)


def test_factors_config4_bf16_full():
    say("config 4 factors (encoder, bf16 inputs)")
    run_config_factors(4)


def test_factors_config5_sampled():
    """Large-factor workload: the A factors and the G factors of every layer,
    one call per side as the benchmark makes it, checked on sampled entries
    and on every diagonal entry against the oracle's entry-wise sums, and in
    full (relative Frobenius error of the upper triangle, the gate) on the
    first layer of every distinct order on each side (A 2305 and 4609; G 512,
    2048 and 4096) at the full 25,088 rows."""
    cfg = CONFIGS[5]
    say("config 5 factors (16 large layers, A and G), sampled")
    data = gen_layer_step(cfg, 0, threads=16)
    L = cfg.layers
    rng = np.random.default_rng(55)
    worst = 0.0
    for side in (0, 1):
        dims = [l.d_a if side == 0 else l.d_g for l in L]
        ms = [nan_f32(d, d) for d in dims]
        la.kfac_factors([to_dev(t[side]) for t in data], ms, EPS, True)
        for k in range(len(L)):
            x = data[k][side]
            d = x.shape[1]
            got = to_host(ms[k])
            ii = rng.integers(0, d, 24)
            jj = rng.integers(0, d, 24)
            ii, jj = np.minimum(ii, jj), np.maximum(ii, jj)
            # the last row and column (a bias column of ones on the A side)
            ii = np.concatenate([ii, [0, d - 1]])
            jj = np.concatenate([jj, [d - 1, d - 1]])
            diag = oracle.factor_diagonal(x)
            ref = oracle.factor_entries(x, ii, jj)
            scale = np.sqrt(diag[ii] * diag[jj])
            err = np.abs(got[ii, jj] - ref) / scale
            derr = np.abs(np.diag(got) - diag) / diag
            worst = max(worst, err.max(), derr.max())
            assert err.max() <= TOL_F32 and derr.max() <= TOL_F32, ("AG"[side], L[k].name, err.max(), derr.max())
        seen = set()
        for k in range(len(L)):
            d = dims[k]
            if d in seen:
                continue
            seen.add(d)
            full = upper_rel_fro(to_host(ms[k]), oracle.factor(oracle.upcast(data[k][side])))
            say(f"  {'AG'[side]} factor of order {d}, layer {L[k].name}: full rel err {full:.3e}")
            worst = max(worst, full)
            assert full <= TOL_F32, ("AG"[side], L[k].name, full)
        del ms
    say(f"config 5: worst relative error (sampled and full) {worst:.3e}")
