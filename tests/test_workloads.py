"""Seeded input generators: determinism, shapes and the stated recipes."""
import numpy as np

from workloads import CONFIGS, bf16_bits_to_f32, gen_a, gen_g, gen_grad, gen_layer_step


def test_generators_deterministic_and_step_dependent():
    cfg = CONFIGS[2]
    a0 = gen_a(cfg, 0, 1, rows=16)
    np.testing.assert_array_equal(a0, gen_a(cfg, 0, 1, rows=16))
    assert not np.array_equal(a0, gen_a(cfg, 1, 1, rows=16))
    assert not np.array_equal(gen_g(cfg, 0, 0), gen_g(cfg, 0, 1)[:, :2048])


def test_shapes_and_bias_column():
    for cid in (1, 2):
        cfg = CONFIGS[cid]
        for li, layer in enumerate(cfg.layers):
            a, g, w = gen_a(cfg, 0, li), gen_g(cfg, 0, li), gen_grad(cfg, 0, li)
            assert a.shape == (layer.rows, layer.d_a) and a.dtype == np.float32
            assert g.shape == (layer.rows, layer.d_g)
            assert w.shape == (layer.d_g, layer.d_a)
            assert np.all(a[:, -1] == 1.0)


def test_relu_and_scaled_columns():
    cfg = CONFIGS[5]
    a = gen_a(cfg, 0, 0, rows=64)
    assert a.min() >= 0.0
    d_feat = cfg.layers[0].d_a - 1
    big = np.sum(a[:, :d_feat].max(axis=0) > 20.0)
    assert big == int(0.1 * d_feat)            # 10% of the non-bias columns scaled x100


def test_bf16_workload_has_exact_ones_column():
    cfg = CONFIGS[4]
    a = gen_a(cfg, 0, 3, rows=8)
    assert a.dtype == np.uint16 and a.shape == (8, 4097)
    assert np.all(a[:, -1] == 0x3F80)
    v = bf16_bits_to_f32(a[:, :-1])
    assert 0.005 < float(np.std(v)) < 0.05


def test_parallel_generation_matches_serial():
    cfg = CONFIGS[2]
    s = gen_layer_step(cfg, 3, threads=1)
    p = gen_layer_step(cfg, 3, threads=4)
    for x, y in zip(s, p):
        for u, v in zip(x, y):
            np.testing.assert_array_equal(u, v)
