"""The five synthetic workloads of the K-FAC hot path.

Each workload is a list of layers.  A layer is described by the dimensions of
its two Kronecker factors and by the number of rows of the matrices they are
built from:

* ``d_a``  -- dimension of the input-side factor A (layer input width, plus one
  trailing ones column when the layer has a bias);
* ``d_g``  -- dimension of the output-side factor G (layer output width);
* ``rows`` -- rows of the activation and gradient matrices (batch size for a
  fully connected layer, batch x output height x output width for an
  im2col'd convolution).

The weight gradient of a layer is ``[d_g, d_a]`` (output-major, bias gradient
in the last column when the layer has a bias).

Value distributions are written as (mean, standard deviation).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Layer:
    name: str
    d_a: int
    d_g: int
    rows: int
    bias: bool


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    layers: Tuple[Layer, ...]
    in_dtype: str            # "f32" or "bf16" for the activation / output-gradient matrices
    a_kind: str              # "normal", "relu_normal", "relu_normal_scaled_cols"
    a_scale: float           # multiplier applied to the N(0,1) draw of a
    g_std: float             # g ~ N(0, g_std)
    grad_std: float          # weight gradient ~ N(0, grad_std)
    gammas: Tuple[float, ...]
    eps: float
    steps: int
    inverse_steps: Tuple[int, ...]
    note: str = ""
    col_scale: float = 1.0            # factor applied to the scaled columns of a
    col_scale_frac: float = 0.0       # fraction of non-bias columns that are scaled

    @property
    def n_layers(self) -> int:
        return len(self.layers)

    def factor_dims(self):
        """Dimensions of all factors in call order: every A (forward order),
        then every G (backward order, last layer first)."""
        return [l.d_a for l in self.layers] + [l.d_g for l in reversed(self.layers)]


def _conv(name, c_in, k, c_out, rows):
    return Layer(name, c_in * k * k, c_out, rows, False)


def resnet50_layers(batch: int = 32) -> Tuple[Layer, ...]:
    """ResNet-50 at 224x224 input, stride on the 3x3 convolution of each
    down-sampling bottleneck, no bias on convolutions, bias on the final
    fully connected layer.  rows = batch x H_out x W_out."""
    L = []
    r112, r56, r28, r14, r7 = (batch * s * s for s in (112, 56, 28, 14, 7))
    L.append(_conv("conv1", 3, 7, 64, r112))
    stages = [  # (name, blocks, width, out, in_channels, rows_in, rows_out)
        ("layer1", 3, 64, 256, 64, r56, r56),
        ("layer2", 4, 128, 512, 256, r56, r28),
        ("layer3", 6, 256, 1024, 512, r28, r14),
        ("layer4", 3, 512, 2048, 1024, r14, r7),
    ]
    for sname, nblocks, width, out, c_in0, rows_in, rows_out in stages:
        for b in range(nblocks):
            c_in = c_in0 if b == 0 else out
            rows_c1 = rows_in if b == 0 else rows_out
            L.append(_conv(f"{sname}.{b}.conv1", c_in, 1, width, rows_c1))
            L.append(_conv(f"{sname}.{b}.conv2", width, 3, width, rows_out))
            L.append(_conv(f"{sname}.{b}.conv3", width, 1, out, rows_out))
            if b == 0:
                L.append(_conv(f"{sname}.{b}.downsample", c_in, 1, out, rows_out))
    L.append(Layer("fc", 2048 + 1, 1000, batch, True))
    return tuple(L)


def _c4_layers():
    L = []
    for blk in range(12):
        L.append(Layer(f"enc{blk}.qkv", 1025, 3072, 4096, True))
        L.append(Layer(f"enc{blk}.out", 1025, 1024, 4096, True))
        L.append(Layer(f"enc{blk}.ffn1", 1025, 4096, 4096, True))
        L.append(Layer(f"enc{blk}.ffn2", 4097, 1024, 4096, True))
    return tuple(L)


def _c5_layers():
    return tuple(
        Layer(f"stress{i}", (2305, 4609)[i % 2], (512, 2048, 4096)[i % 3], 25088, True)
        for i in range(16)
    )


CONFIGS = {
    1: Config(
        cid=1, name="fc1",
        layers=(Layer("fc", 64 + 1, 32, 32, True),),
        in_dtype="f32", a_kind="normal", a_scale=1.0, g_std=1.0, grad_std=1.0,
        gammas=(0.01,), eps=0.95, steps=3, inverse_steps=(2,),
        note="single fully connected layer, batch 32, 64 inputs + ones column, 32 outputs",
    ),
    2: Config(
        cid=2, name="mlp4",
        layers=(
            Layer("fc1", 1024 + 1, 2048, 128, True),
            Layer("fc2", 2048 + 1, 2048, 128, True),
            Layer("fc3", 2048 + 1, 1024, 128, True),
            Layer("fc4", 1024 + 1, 10, 128, True),
        ),
        in_dtype="f32", a_kind="relu_normal", a_scale=1.0, g_std=1e-2, grad_std=1e-3,
        gammas=(1e-3,), eps=0.95, steps=20, inverse_steps=(0, 10),
        note="MLP 1024-2048-2048-1024-10, batch 128",
    ),
    3: Config(
        cid=3, name="resnet50",
        layers=resnet50_layers(32),
        in_dtype="f32", a_kind="relu_normal", a_scale=1.0, g_std=1e-3, grad_std=1e-3,
        gammas=(1e-3,), eps=0.95, steps=1, inverse_steps=(0,),
        note="ResNet-50 factor shapes (53 conv + fc), batch 32, 224x224",
    ),
    4: Config(
        cid=4, name="encoder12",
        layers=_c4_layers(),
        in_dtype="bf16", a_kind="normal", a_scale=0.02, g_std=0.02, grad_std=0.02,
        gammas=(1e-3,), eps=0.95, steps=1, inverse_steps=(0,),
        note="12-layer encoder, hidden 1024, FFN 4096, 4096 tokens; bf16 a and g",
    ),
    5: Config(
        cid=5, name="stress16",
        layers=_c5_layers(),
        in_dtype="f32", a_kind="relu_normal_scaled_cols", a_scale=1.0, g_std=1e-3, grad_std=1e-3,
        gammas=(1e-2, 1e-4), eps=0.95, steps=3, inverse_steps=(0, 1, 2),
        col_scale=100.0, col_scale_frac=0.1,
        note="16 large-factor layers, rows 25088, 10% of a's columns scaled x100",
    ),
}


def get_config(cid: int) -> Config:
    return CONFIGS[int(cid)]
