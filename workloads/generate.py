"""Seeded generators for the workloads in :mod:`workloads.configs`.

Every tensor is drawn from its own ``numpy.random.Generator`` seeded with
``SeedSequence([config_id, step, layer, tensor_id])`` where tensor_id is
0 for the activations a, 1 for the output gradients g, 2 for the weight
gradient and 3 for the choice of scaled columns.  Draws are float32.

bf16 workloads are returned as uint16 bit patterns, rounded from the float32
draw to nearest, ties to even; a ones column is exactly 1.0 (0x3F80).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Config

TENSOR_A, TENSOR_G, TENSOR_GRAD, TENSOR_COLS = 0, 1, 2, 3


def seed_rng(cid: int, step: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(cid), int(step), int(layer), int(tensor_id)]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.
    Inputs must be finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng, shape, scale):
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def gen_a(cfg: Config, step: int, li: int, rows: int | None = None) -> np.ndarray:
    """Activation matrix of layer ``li`` at ``step``: [rows, d_a] float32, or
    uint16 bf16 bits for bf16 workloads.  ``rows`` overrides the layer's row
    count (smaller test cases use the same recipe)."""
    layer = cfg.layers[li]
    rows = layer.rows if rows is None else int(rows)
    d_feat = layer.d_a - (1 if layer.bias else 0)
    rng = seed_rng(cfg.cid, step, li, TENSOR_A)
    x = np.empty((rows, layer.d_a), dtype=np.float32)
    x[:, :d_feat] = _normal(rng, (rows, d_feat), cfg.a_scale)
    if cfg.a_kind in ("relu_normal", "relu_normal_scaled_cols"):
        np.maximum(x[:, :d_feat], np.float32(0.0), out=x[:, :d_feat])
    if cfg.a_kind == "relu_normal_scaled_cols":
        nscale = int(np.floor(cfg.col_scale_frac * d_feat))
        cols = np.sort(seed_rng(cfg.cid, 0, li, TENSOR_COLS).choice(d_feat, size=nscale, replace=False))
        x[:, cols] *= np.float32(cfg.col_scale)
    if layer.bias:
        x[:, d_feat] = np.float32(1.0)
    if cfg.in_dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def gen_g(cfg: Config, step: int, li: int, rows: int | None = None) -> np.ndarray:
    """Output-gradient matrix of layer ``li`` at ``step``: [rows, d_g]."""
    layer = cfg.layers[li]
    rows = layer.rows if rows is None else int(rows)
    rng = seed_rng(cfg.cid, step, li, TENSOR_G)
    x = _normal(rng, (rows, layer.d_g), cfg.g_std)
    if cfg.in_dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def gen_grad(cfg: Config, step: int, li: int) -> np.ndarray:
    """Weight gradient of layer ``li`` at ``step``: [d_g, d_a] float32."""
    layer = cfg.layers[li]
    rng = seed_rng(cfg.cid, step, li, TENSOR_GRAD)
    return _normal(rng, (layer.d_g, layer.d_a), cfg.grad_std)


def gen_layer_step(cfg: Config, step: int, threads: int = 8, layers=None):
    """All three inputs of every layer at ``step``: list of (a, g, grad).
    Layers are drawn in parallel threads (numpy releases the GIL while
    drawing); the result does not depend on ``threads``."""
    idx = list(range(cfg.n_layers)) if layers is None else list(layers)

    def one(li):
        return gen_a(cfg, step, li), gen_g(cfg, step, li), gen_grad(cfg, step, li)

    if threads <= 1 or len(idx) == 1:
        return [one(li) for li in idx]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(one, idx))
