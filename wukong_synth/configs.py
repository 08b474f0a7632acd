"""Shapes of the synthetic Wukong interaction-stack workloads.

A Wukong layer (Wukong paper, section 2.2 "Wukong", as summarised on the
xdnf.cn repost of the Zhihu article) maps a per-example feature matrix
X in R^{n x d} to a new n x d matrix: a Factorization Machine Block (FMB)
compresses the n embeddings to k, interacts them with X, and an MLP turns the
flattened interaction into n_F embeddings; a Linear Compress Block (LCB) maps
the n embeddings to n_L; both are concatenated, the residual is added and a
LayerNorm is applied.  The scaling knobs l, n_F, n_L, k and the MLP widths are
listed in section 2.3 of the same page; the embedding width 160 comes from its
section 3.2.1 (training setup), the 720 features from its dataset description
and the 8-dim "units" from section 2.1.

This module holds shapes only.  It performs none of the layer's arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class LayerShape:
    """One Wukong layer: n embeddings of width d in, n_F + n_L = n out.

    mlp is the full list of FMB-MLP widths m_0 = n*k, m_1, ..., m_T = n_F*d.
    """

    n: int
    d: int
    k: int
    n_f: int
    n_l: int
    mlp: Tuple[int, ...]

    def __post_init__(self):
        if self.n_f + self.n_l != self.n:
            raise ValueError("the residual needs n_F + n_L == n")
        if len(self.mlp) < 2:
            raise ValueError("the FMB MLP needs at least one Linear layer")
        if self.mlp[0] != self.n * self.k:
            raise ValueError("first MLP width must be n*k (the flattened interaction)")
        if self.mlp[-1] != self.n_f * self.d:
            raise ValueError("last MLP width must be n_F*d (reshaped to n_F x d)")

    @property
    def num_linear(self) -> int:
        return len(self.mlp) - 1

    def flops_per_example(self) -> int:
        """Algorithmic FLOPs of one layer for one example.

        compress Z = Phi.X (2knd) + interaction X.Z^T (2ndk) + LCB W_L.X
        (2 n_L n d) + every MLP Linear (2 m_{t-1} m_t).  LayerNorm, residual
        and ReLU are not counted.
        """
        n, d, k = self.n, self.d, self.k
        f = 2 * k * n * d + 2 * n * d * k + 2 * self.n_l * n * d
        for a, b in zip(self.mlp[:-1], self.mlp[1:]):
            f += 2 * a * b
        return f


@dataclass(frozen=True)
class WukongConfig:
    name: str
    dtype: str  # "f32" or "bf16": storage type of inputs, weights and outputs
    batch: int
    layers: Tuple[LayerShape, ...]
    x_dist: str = "normal"  # "normal" or "feature_scaled_units"
    unit_width: int = 0  # width of the embedding units a feature row is built from
    description: str = ""
    units_per_feature: int = 1  # rows of X that belong to one feature (unit-level layers)

    @property
    def num_layers(self) -> int:
        return len(self.layers)

    def flops_per_example(self) -> int:
        return sum(s.flops_per_example() for s in self.layers)

    def head_dims(self, hidden: Tuple[int, ...] = (1024, 256), outputs: int = 1) -> Tuple[int, ...]:
        """Widths of the prediction head on this stack's output: the page names
        an MLP after the Wukong layers but gives no sizes, so the hidden widths
        default to 1024 and 256 and one output (a click probability)."""
        s = self.layers[-1]
        return (s.n * s.d,) + tuple(hidden) + (outputs,)

    def with_batch(self, batch: int) -> "WukongConfig":
        return replace(self, batch=batch)

    def with_layers(self, num_layers: int) -> "WukongConfig":
        return replace(self, layers=self.layers[:num_layers])


def _stack(shape: LayerShape, l: int) -> Tuple[LayerShape, ...]:
    return tuple([shape] * l)


# Tiny fp32 single layer: n=16, d=16, k=4, n_F = n_L = 8, MLP 64 -> 64 -> 128.
TINY_F32 = WukongConfig(
    "tiny_f32", "f32", 64,
    _stack(LayerShape(16, 16, 4, 8, 8, (64, 64, 128)), 1),
    description="tiny single layer, fp32, B=64, n=16, d=16, k=4, n_F=n_L=8",
)

# Single bf16 layer at the pages' embedding width d=160.
LAYER_D160 = WukongConfig(
    "layer_d160", "bf16", 4096,
    _stack(LayerShape(128, 160, 32, 64, 64, (4096, 2048, 10240)), 1),
    description="single layer, bf16, B=4096, n=128, d=160, k=32, n_F=n_L=64, MLP 4096-2048-10240",
)

# 8-layer stack, n stays 256.
STACK8_N256 = WukongConfig(
    "stack8_n256", "bf16", 16384,
    _stack(LayerShape(256, 160, 48, 128, 128, (12288, 4096, 4096, 20480)), 8),
    description="8-layer stack, bf16, B=16384, n=256, d=160, k=48, n_F=n_L=128, MLP 12288-4096-4096-20480",
)

# Large-compute 8-layer stack (~13.5 GFLOP/example).
STACK8_N512 = WukongConfig(
    "stack8_n512", "bf16", 2048,
    _stack(LayerShape(512, 160, 96, 256, 256, (49152, 8192, 8192, 40960)), 8),
    description="8-layer stack, bf16, B=2048, n=512, d=160, k=96, n_F=n_L=256, MLP 49152-8192-8192-40960",
)

# Small-d irregular layer: 720 features of d=32 built from four 8-dim units.
SMALLD_N720 = WukongConfig(
    "smalld_n720", "bf16", 8192,
    _stack(LayerShape(720, 32, 24, 360, 360, (17280, 1024, 11520)), 1),
    x_dist="feature_scaled_units", unit_width=8,
    description="single layer, bf16, B=8192, n=720, d=32 (4 units of 8), k=24, n_F=n_L=360, MLP 17280-1024-11520",
)

# Unit-level interaction (section 2.1 of the same page: each 8-wide unit takes
# part in the interaction as a feature of its own): the n = 720 workload's
# features split into their 4 units, so n = 2880 rows of width 8.  k, n_F,
# n_L and the MLP keep the n = 720 layer's proportions (the page gives none).
UNITS_N2880 = WukongConfig(
    "units_n2880", "bf16", 8192,
    _stack(LayerShape(2880, 8, 24, 1440, 1440, (69120, 1024, 11520)), 1),
    x_dist="feature_scaled_unit_rows", unit_width=8, units_per_feature=4,
    description="unit-level single layer, bf16, B=8192, n=2880 units of d=8 (4 per feature), k=24, "
                "n_F=n_L=1440, MLP 69120-1024-11520",
)

CONFIGS = (TINY_F32, LAYER_D160, STACK8_N256, STACK8_N512, SMALLD_N720)
BY_NAME = {c.name: c for c in CONFIGS + (UNITS_N2880,)}


def get(name_or_index) -> WukongConfig:
    if isinstance(name_or_index, int):
        return CONFIGS[name_or_index]
    return BY_NAME[name_or_index]
