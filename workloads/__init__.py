"""Seeded synthetic inputs for the per-GPU K-FAC hot path.

This package holds the five workload definitions (layer shapes, value
distributions, damping, running-average weight, schedule) and the seeded
generators that turn them into arrays.  It is shared by the oracle side and
the GPU side of every test and of the benchmark, and by nothing else.  It
contains none of the method's arithmetic: no factor, no pack index map, no
inverse, no product.  Inputs are drawn once on the host and handed to both
sides unchanged.

Shapes follow "Accelerating Distributed K-FAC with Smart Parallelism of
Computing and Communication Tasks": the ResNet-50 layer list reproduces the
factor element counts that page gives in the paragraph on the MPD-KFAC bar of
Fig. 2 and in the paragraph on the dimension distributions of Fig. 3.
"""
from .configs import CONFIGS, Config, Layer, get_config, resnet50_layers  # noqa: F401
from .generate import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    gen_a,
    gen_g,
    gen_grad,
    gen_layer_step,
    seed_rng,
)
