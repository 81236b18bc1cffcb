"""GPU parity: factor inputs of real layers (kfac_im2col, kfac_grad_rows) and
the weight/bias gradient matrix (kfac_grad_matrix) against the oracle.

All three move data (grad_rows also scales in float32), so the gate is
bit-exact, in float32 and bfloat16, single and batched, over shapes that
span many 64 x 64 tiles with ragged edges."""
import numpy as np
import pytest

import linear_algebra_amd as la
import oracle
from tests.gpu_helpers import DEV, say, to_dev

pytestmark = pytest.mark.gpu

CASES = [  # (n, c, h, w), kernel, stride, padding, dilation, ones
    ((2, 3, 7, 6), (3, 3), (1, 1), (1, 1), (1, 1), True),
    ((1, 4, 9, 8), (3, 2), (2, 1), (1, 0), (1, 2), False),
    ((3, 2, 5, 5), (1, 1), (2, 2), (0, 0), (1, 1), True),
    ((4, 64, 28, 28), (3, 3), (1, 1), (1, 1), (1, 1), False),
    ((2, 3, 56, 56), (7, 7), (2, 2), (3, 3), (1, 1), False),
    ((5, 130, 9, 11), (3, 3), (2, 2), (1, 1), (1, 1), True),
    ((37, 1025, 1, 1), (1, 1), (1, 1), (0, 0), (1, 1), True),   # a fully connected layer with bias
    # four-element gathers (1 x 1, stride 1, h w % 4 == 0) and writes (columns % 4 == 0)
    ((3, 64, 14, 14), (1, 1), (1, 1), (0, 0), (1, 1), False),   # both; 588 rows, a ragged row tile
    ((2, 130, 6, 6), (1, 1), (1, 1), (0, 0), (1, 1), True),     # gather only: 131 columns
    ((2, 68, 5, 5), (3, 3), (1, 1), (1, 1), (1, 1), False),     # write only: 612 columns
    ((3, 72, 7, 7), (1, 1), (1, 1), (0, 0), (1, 1), False),     # write only: h w = 49
    ((32, 1024, 1, 1), (1, 1), (1, 1), (0, 0), (1, 1), False),  # fully connected, no bias: both
    # degenerate shapes: a 1 x 1 output, a stride wider than the kernel, one channel with dilation 2
    ((2, 3, 5, 5), (7, 7), (1, 1), (1, 1), (1, 1), True),
    ((1, 2, 9, 9), (2, 2), (3, 3), (0, 0), (1, 1), False),
    ((3, 1, 6, 6), (3, 3), (1, 1), (0, 0), (2, 2), False),
]


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def shape_dict(kernel, stride, padding, dilation, ones):
    return dict(kernel=kernel, stride=stride, padding=padding, dilation=dilation, ones=ones)


def inputs(rng, shp, bf16):
    x = rng.standard_normal(shp).astype(np.float32)
    return oracle.bf16_round(x) if bf16 else x


def gpu_im2col(xs, shapes):
    import torch
    outs = []
    for x, s in zip(xs, shapes):
        oh, ow = la.conv_out_hw(x.shape[2], x.shape[3], *s["kernel"], s["stride"], s["padding"], s["dilation"])
        outs.append(torch.full((x.shape[0] * oh * ow, x.shape[1] * s["kernel"][0] * s["kernel"][1] + int(s["ones"])),
                               float("nan"), dtype=x.dtype, device=DEV))
    la.kfac_im2col(xs, shapes, outs)
    return [host(o) for o in outs]


@pytest.mark.parametrize("bf16", [False, True])
def test_im2col_each_case(bf16):
    rng = np.random.default_rng(51)
    for shp, k, s, p, d, ones in CASES:
        say("im2col", shp, k, s, p, d, ones, "bf16" if bf16 else "f32")
        x = inputs(rng, shp, bf16)
        (got,) = gpu_im2col([to_dev(x)], [shape_dict(k, s, p, d, ones)])
        ref = oracle.im2col(x, k, s, p, d, ones)
        if bf16:
            ref[:, -1] = 0x3F80 if ones else ref[:, -1]   # a bf16 one, as bits
        np.testing.assert_array_equal(got, ref)


def test_im2col_batched_mixed_layers():
    rng = np.random.default_rng(52)
    xs = [inputs(rng, c[0], False) for c in CASES]
    shapes = [shape_dict(*c[1:]) for c in CASES]
    got = gpu_im2col([to_dev(x) for x in xs], shapes)
    for x, c, g in zip(xs, CASES, got):
        np.testing.assert_array_equal(g, oracle.im2col(x, *c[1:]))


def test_im2col_resnet50_conv1_full_size():
    """The first ResNet-50 convolution at batch 32 (224 x 224, 7 x 7, stride 2,
    padding 3): 401,408 patch rows; the rows of three samples against the
    oracle run on those samples alone."""
    rng = np.random.default_rng(53)
    x = rng.standard_normal((32, 3, 224, 224)).astype(np.float32)
    s = shape_dict((7, 7), (2, 2), (3, 3), (1, 1), False)
    (got,) = gpu_im2col([to_dev(x)], [s])
    assert got.shape == (401408, 147)
    per = 112 * 112
    for ni in (0, 17, 31):
        np.testing.assert_array_equal(got[ni * per:(ni + 1) * per], oracle.im2col(x[ni:ni + 1], *s.values()))


@pytest.mark.parametrize("shp,k,st,pd", [((32, 64, 56, 56), (1, 1), (1, 1), (0, 0)),
                                         ((32, 128, 28, 28), (3, 3), (1, 1), (1, 1)),
                                         ((32, 256, 56, 56), (1, 1), (2, 2), (0, 0))])
def test_im2col_resnet50_layers_full_size(shp, k, st, pd):
    """ResNet-50 bottleneck convolutions at batch 32 (a 1 x 1, a 3 x 3 and a
    stride-2 shortcut): the rows of three samples against the oracle."""
    rng = np.random.default_rng(55)
    say("im2col full size", shp, k, st, pd)
    x = rng.standard_normal(shp).astype(np.float32)
    s = shape_dict(k, st, pd, (1, 1), False)
    (got,) = gpu_im2col([to_dev(x)], [s])
    oh, ow = la.conv_out_hw(shp[2], shp[3], *k, st, pd)
    per = oh * ow
    assert got.shape == (shp[0] * per, shp[1] * k[0] * k[1])
    for ni in (0, 13, 31):
        np.testing.assert_array_equal(got[ni * per:(ni + 1) * per], oracle.im2col(x[ni:ni + 1], *s.values()))


@pytest.mark.parametrize("bf16", [False, True])
def test_grad_rows(bf16):
    import torch
    rng = np.random.default_rng(54)
    shapes = [(4, 64, 28, 28), (8, 10), (3, 130, 7, 9), (130, 70), (2, 5, 1, 1), (1, 3, 65, 3),
              (2, 132, 10, 10), (3, 66, 8, 8), (2, 12, 7, 7)]
    gys = [inputs(rng, s, bf16) for s in shapes]
    scale = 37.0
    outs = []
    for g in gys:
        p = int(np.prod(g.shape[2:])) if g.ndim > 2 else 1
        outs.append(torch.full((g.shape[0] * p, g.shape[1]), float("nan"),
                               dtype=torch.bfloat16 if bf16 else torch.float32, device=DEV))
    la.kfac_grad_rows([to_dev(g) for g in gys], scale, outs)
    for g, o in zip(gys, outs):
        np.testing.assert_array_equal(host(o), oracle.grad_rows(g, scale, bf16))


def test_grad_matrix_round_trip():
    import torch
    rng = np.random.default_rng(55)
    specs = [((1000, 2048), True), ((64, 3, 7, 7), False), ((10, 1025), True), ((1, 1), True), ((130, 65), False)]
    ws = [rng.standard_normal(s).astype(np.float32) for s, _ in specs]
    bs = [rng.standard_normal(s[0]).astype(np.float32) if has else None for s, has in specs]
    dw = [to_dev(w) for w in ws]
    db = [to_dev(b) if b is not None else None for b in bs]
    mats = [torch.full((w.shape[0], w[0].size + (b is not None)), float("nan"), device=DEV) for w, b in zip(ws, bs)]
    la.kfac_grad_matrix(dw, db, mats, la.KFAC_PACK)
    for w, b, m in zip(ws, bs, mats):
        np.testing.assert_array_equal(host(m), oracle.grad_matrix(w, b))
    # scatter back into fresh gradients
    w2 = [torch.full_like(w, float("nan")) for w in dw]
    b2 = [torch.full_like(b, float("nan")) if b is not None else None for b in db]
    la.kfac_grad_matrix(w2, b2, mats, la.KFAC_UNPACK)
    for w, b, w_, b_ in zip(ws, bs, w2, b2):
        np.testing.assert_array_equal(host(w_), w)
        if b is not None:
            np.testing.assert_array_equal(host(b_), b)
