"""Seeded synthetic inputs and weights for the Wukong interaction stack.

Both the CPU oracle's tests and the GPU path's tests and benchmark draw their
host arrays from here, so the two sides see bit-identical inputs.  Nothing in
this module computes any part of the layer: it only draws random numbers,
scales them and rounds them to the storage type.

Random streams
--------------
Every tensor has a tag such as ``"stack8_n256/L3/mlp_w1"``.  The tag and the
seed are hashed (BLAKE2b) to a 128-bit Philox-4x64 key; the tensor is filled
in fixed-size chunks, each with its own key (tag + chunk index), so the values
do not depend on how many threads fill them.  Philox is a counter-based
generator (Salmon et al., "Parallel random numbers: as easy as 1, 2, 3",
SC 2011) and numpy's implementation of its raw stream is platform-stable.

Distributions
-------------
* inputs X: N(0, 1); for the small-d workload each 32-wide feature row is four
  8-wide units side by side, all scaled by one per-feature factor
  s_i = 10**U(-1, 1) (log-uniform on [0.1, 10]) shared by every example;
* weights: Xavier-uniform, bound sqrt(6 / (fan_in + fan_out)) with PyTorch's
  fan convention for an [out, in] matrix (fan_in = in, fan_out = out);
* LayerNorm gamma = 1, beta = 0 and biases = 0 for the measured runs, or
  gamma = 1 + U(-0.5, 0.5), beta and biases U(-0.5, 0.5) for parity runs.

Storage
-------
fp32 configurations return float32 arrays.  bf16 configurations return the
bf16 bit patterns as uint16 arrays, rounded once from float32 with
round-to-nearest-even.
"""
from __future__ import annotations

import hashlib
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from .configs import LayerShape, WukongConfig

CHUNK = 1 << 22  # elements per independently keyed chunk


def stream_key(seed: int, tag: str) -> int:
    h = hashlib.blake2b(f"{seed}|{tag}".encode(), digest_size=16).digest()
    return int.from_bytes(h, "little")


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _run_chunks(nchunks: int, work) -> None:
    if nchunks <= 1:
        for i in range(nchunks):
            work(i)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(work, range(nchunks)))


def _bf16_round_bits(x32: np.ndarray) -> np.ndarray:
    b = x32.view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def _draw(seed: int, tag: str, size: int, kind: str, scale: float = 1.0, offset: float = 0.0,
          dtype: str = "f32") -> np.ndarray:
    """`size` draws, each chunk keyed independently, transformed to scale*v + offset.

    kind 'uniform_pm' draws v = 2u - 1 with u ~ U[0,1) (so v ~ U[-1,1)); kind
    'normal' draws v ~ N(0,1).  The result is stored as float32 or bf16 bits.
    """
    out = np.empty(size, dtype=np.float32 if dtype == "f32" else np.uint16)
    nchunks = (size + CHUNK - 1) // CHUNK
    sc, of = np.float32(scale), np.float32(offset)

    def work(i):
        lo, hi = i * CHUNK, min(size, (i + 1) * CHUNK)
        g = np.random.Generator(np.random.Philox(key=stream_key(seed, f"{tag}#{i}")))
        v = np.empty(hi - lo, dtype=np.float32)
        if kind == "uniform_pm":
            g.random(dtype=np.float32, out=v)
            v *= np.float32(2.0)
            v -= np.float32(1.0)
        elif kind == "normal":
            g.standard_normal(dtype=np.float32, out=v)
        else:  # pragma: no cover
            raise ValueError(kind)
        if scale != 1.0:
            v *= sc
        if offset != 0.0:
            v += of
        out[lo:hi] = v if dtype == "f32" else _bf16_round_bits(v)

    _run_chunks(nchunks, work)
    return out


def _fill(seed: int, tag: str, size: int, kind: str) -> np.ndarray:
    """float32 U[0,1) draws (kind 'uniform'), keyed per chunk like _draw."""
    assert kind == "uniform"
    out = np.empty(size, dtype=np.float32)

    def work(i):
        lo, hi = i * CHUNK, min(size, (i + 1) * CHUNK)
        g = np.random.Generator(np.random.Philox(key=stream_key(seed, f"{tag}#{i}")))
        g.random(dtype=np.float32, out=out[lo:hi])

    _run_chunks((size + CHUNK - 1) // CHUNK, work)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1)
    flat_out = out.reshape(-1)
    n = flat_in.size

    def work(i):
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        flat_out[lo:hi] = _bf16_round_bits(flat_in[lo:hi])

    _run_chunks((n + CHUNK - 1) // CHUNK, work)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


def xavier_uniform(seed: int, tag: str, out_features: int, in_features: int, dtype: str) -> np.ndarray:
    a = math.sqrt(6.0 / (in_features + out_features))
    w = _draw(seed, tag, out_features * in_features, "uniform_pm", scale=a, dtype=dtype)
    return w.reshape(out_features, in_features)


def _uniform_pm(seed: int, tag: str, size: int, half_width: float, center: float = 0.0) -> np.ndarray:
    return _draw(seed, tag, size, "uniform_pm", scale=half_width, offset=center)


@dataclass
class HostLayerWeights:
    """Host copies of one layer's parameters (float32, or uint16 bf16 bits)."""

    phi: np.ndarray            # [k, n]
    w_l: np.ndarray            # [n_L, n]
    fm_gamma: np.ndarray       # [n*k]
    fm_beta: np.ndarray        # [n*k]
    mlp_w: List[np.ndarray]    # W_t: [m_t, m_{t-1}]
    mlp_b: List[np.ndarray]    # b_t: [m_t]
    out_gamma: np.ndarray      # [d]
    out_beta: np.ndarray       # [d]
    dtype: str = "f32"

    def nbytes(self) -> int:
        arrs = [self.phi, self.w_l, self.fm_gamma, self.fm_beta, self.out_gamma, self.out_beta]
        arrs += self.mlp_w + self.mlp_b
        return int(sum(a.nbytes for a in arrs))


def make_layer_weights(cfg_name: str, layer: int, shape: LayerShape, dtype: str, seed: int,
                       affine: str = "identity") -> HostLayerWeights:
    """Xavier-uniform weights of one layer.  affine: 'identity' or 'random'."""
    return _module_weights(f"{cfg_name}/L{layer}", shape.n, shape.d, shape.k, shape.n_l, shape.mlp, dtype, seed,
                           affine)


def make_expert_weights(tag: str, expert: int, n: int, d: int, k: int, n_l: int, mlp, dtype: str, seed: int,
                        affine: str = "identity") -> HostLayerWeights:
    """Xavier-uniform weights of one expert of a mixture-of-experts layer (a
    Wukong module with its own k, LCB rows n_l and MLP widths mlp, ending in
    n_F * d).  Its out_gamma / out_beta are drawn but the layer's own are used."""
    return _module_weights(f"{tag}/E{expert}", n, d, k, n_l, tuple(mlp), dtype, seed, affine)


def _module_weights(t: str, n: int, d: int, k: int, n_l: int, mlp, dtype: str, seed: int,
                    affine: str) -> HostLayerWeights:
    phi = xavier_uniform(seed, f"{t}/phi", k, n, dtype)
    w_l = xavier_uniform(seed, f"{t}/w_l", n_l, n, dtype)
    mlp_w, mlp_b = [], []
    for i, (a, b) in enumerate(zip(mlp[:-1], mlp[1:])):
        mlp_w.append(xavier_uniform(seed, f"{t}/mlp_w{i}", b, a, dtype))
        if affine == "random":
            mlp_b.append(_store(_uniform_pm(seed, f"{t}/mlp_b{i}", b, 0.5), dtype))
        else:
            mlp_b.append(_store(np.zeros(b, np.float32), dtype))
    if affine == "random":
        fm_g = _uniform_pm(seed, f"{t}/fm_gamma", n * k, 0.5, 1.0)
        fm_b = _uniform_pm(seed, f"{t}/fm_beta", n * k, 0.5)
        o_g = _uniform_pm(seed, f"{t}/out_gamma", d, 0.5, 1.0)
        o_b = _uniform_pm(seed, f"{t}/out_beta", d, 0.5)
    elif affine == "identity":
        fm_g, fm_b = np.ones(n * k, np.float32), np.zeros(n * k, np.float32)
        o_g, o_b = np.ones(d, np.float32), np.zeros(d, np.float32)
    else:
        raise ValueError(affine)
    return HostLayerWeights(phi, w_l, _store(fm_g, dtype), _store(fm_b, dtype), mlp_w, mlp_b,
                            _store(o_g, dtype), _store(o_b, dtype), dtype)


def make_stack_weights(cfg: WukongConfig, seed: int, affine: str = "identity",
                       num_layers: Optional[int] = None) -> List[HostLayerWeights]:
    l = cfg.num_layers if num_layers is None else num_layers
    return [make_layer_weights(cfg.name, i, cfg.layers[i], cfg.dtype, seed, affine) for i in range(l)]


def make_head_weights(cfg_name: str, dims, dtype: str, seed: int, affine: str = "identity"):
    """Xavier-uniform weights [m_t, m_{t-1}] and biases [m_t] of the prediction
    head's Linears (biases 0 for 'identity', U(-0.5, 0.5) for 'random')."""
    dims = tuple(dims)
    w, b = [], []
    for i, (a, o) in enumerate(zip(dims[:-1], dims[1:])):
        w.append(xavier_uniform(seed, f"{cfg_name}/head/w{i}", o, a, dtype))
        if affine == "random":
            b.append(_store(_uniform_pm(seed, f"{cfg_name}/head/b{i}", o, 0.5), dtype))
        elif affine == "identity":
            b.append(_store(np.zeros(o, np.float32), dtype))
        else:
            raise ValueError(affine)
    return w, b


@dataclass
class HostFusionWeights:
    """Host copies of WHALE fusion-step parameters (float32, or uint16 bf16 bits)."""

    w_f: np.ndarray               # [d, 2d]
    b_f: Optional[np.ndarray]     # [d]
    gamma: Optional[np.ndarray]   # [d]
    beta: Optional[np.ndarray]    # [d]
    w_up: np.ndarray              # [d_ff, d]
    b_up: Optional[np.ndarray]    # [d_ff]
    w_down: np.ndarray            # [d, d_ff]
    b_down: Optional[np.ndarray]  # [d]


def make_fusion_weights(tag: str, d: int, d_ff: int, dtype: str, seed: int,
                        affine: str = "identity") -> HostFusionWeights:
    """Xavier-uniform Linear weights; biases 0 / LN gamma 1, beta 0 ('identity') or U(+-0.5) ('random')."""
    w_f = xavier_uniform(seed, f"{tag}/fusion/w_f", d, 2 * d, dtype)
    w_up = xavier_uniform(seed, f"{tag}/fusion/w_up", d_ff, d, dtype)
    w_down = xavier_uniform(seed, f"{tag}/fusion/w_down", d, d_ff, dtype)
    if affine == "random":
        vec = lambda name, k, c=0.0: _store(_uniform_pm(seed, f"{tag}/fusion/{name}", k, 0.5, c), dtype)  # noqa: E731
        return HostFusionWeights(w_f, vec("b_f", d), vec("gamma", d, 1.0), vec("beta", d), w_up, vec("b_up", d_ff),
                                 w_down, vec("b_down", d))
    if affine != "identity":
        raise ValueError(affine)
    z = lambda k: _store(np.zeros(k, np.float32), dtype)  # noqa: E731
    return HostFusionWeights(w_f, z(d), _store(np.ones(d, np.float32), dtype), z(d), w_up, z(d_ff), w_down, z(d))


def make_sequence(tag: str, batch: int, L: int, d: int, dtype: str, seed: int) -> np.ndarray:
    """A stand-in for the sequence branch's output H_s [batch, L, d]: N(0, 1) entries."""
    return _draw(seed, f"{tag}/h_s", batch * L * d, "normal", dtype=dtype).reshape(batch, L, d)


def feature_scales(cfg: WukongConfig, seed: int, count: Optional[int] = None) -> np.ndarray:
    """Per-feature scale s_i = 10**U(-1,1), shared by all examples (float32 [count], default n)."""
    n = cfg.layers[0].n if count is None else count
    u = _fill(seed, f"{cfg.name}/x_feature_scale", n, "uniform")
    return np.power(np.float32(10.0), u * np.float32(2.0) - np.float32(1.0)).astype(np.float32)


def make_input(cfg: WukongConfig, seed: int, batch: Optional[int] = None,
               first_example: int = 0) -> np.ndarray:
    """X of shape [batch, n, d] in the config's storage type.

    Examples are drawn independently per index, so make_input(..., batch=b,
    first_example=s) equals rows s..s+b of the full batch: a subset can be
    regenerated without drawing the whole batch.
    """
    s0 = cfg.layers[0]
    n, d = s0.n, s0.d
    b = cfg.batch if batch is None else batch
    per = n * d
    x = np.empty((b, n, d), dtype=np.float32)
    # examples are keyed in blocks of EX_BLOCK so any sub-range can be regenerated
    ex_block = max(1, CHUNK // per)
    blk0 = first_example // ex_block
    blk1 = (first_example + b + ex_block - 1) // ex_block

    def work(blk):
        lo_ex = blk * ex_block
        vals = np.empty(ex_block * per, dtype=np.float32)
        g = np.random.Generator(np.random.Philox(key=stream_key(seed, f"{cfg.name}/x#{blk}")))
        g.standard_normal(dtype=np.float32, out=vals)
        vals = vals.reshape(ex_block, n, d)
        a = max(lo_ex, first_example)
        z = min(lo_ex + ex_block, first_example + b)
        if a < z:
            x[a - first_example:z - first_example] = vals[a - lo_ex:z - lo_ex]

    blocks = list(range(blk0, blk1))
    if len(blocks) <= 1:
        for blk in blocks:
            work(blk)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(work, blocks))
    if cfg.x_dist == "feature_scaled_units":
        # each row is unit_width-wide units side by side; one scale per feature row
        assert cfg.unit_width > 0 and d % cfg.unit_width == 0
        x *= feature_scales(cfg, seed)[None, :, None]
    elif cfg.x_dist == "feature_scaled_unit_rows":
        # each row is one unit; units_per_feature consecutive rows share their feature's scale
        upf = cfg.units_per_feature
        assert d == cfg.unit_width and n % upf == 0
        s = feature_scales(cfg, seed, n // upf)
        x *= np.repeat(s, upf)[None, :, None]
    elif cfg.x_dist != "normal":
        raise ValueError(cfg.x_dist)
    return _store(x, cfg.dtype)


def make_upstream_grad(cfg: WukongConfig, seed: int, batch: Optional[int] = None) -> np.ndarray:
    """A stand-in for dLoss/dY of a layer output [batch, n, d]: N(0, 1) entries."""
    s0 = cfg.layers[0]
    b = cfg.batch if batch is None else batch
    return _draw(seed, f"{cfg.name}/dy", b * s0.n * s0.d, "normal", dtype=cfg.dtype).reshape(b, s0.n, s0.d)


def make_out_layernorm(tag: str, d: int, dtype: str, seed: int, affine: str = "identity"):
    """(gamma, beta) [d] of a layer's output LayerNorm: 1 and 0, or 1 + U(-0.5, 0.5) and U(-0.5, 0.5)."""
    if affine == "identity":
        return _store(np.ones(d, np.float32), dtype), _store(np.zeros(d, np.float32), dtype)
    if affine != "random":
        raise ValueError(affine)
    return (_store(_uniform_pm(seed, f"{tag}/out_gamma", d, 0.5, 1.0), dtype),
            _store(_uniform_pm(seed, f"{tag}/out_beta", d, 0.5), dtype))
