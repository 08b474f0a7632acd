"""Shared plumbing of the GPU parity tests: seeded host inputs -> device,
HIP path through the C ABI, oracle on the same host arrays, error metric."""
from __future__ import annotations

import sys
import time
from typing import List, Optional, Sequence

import numpy as np
import torch

import oracle
import recommender_feature_interaction_amd as wk
import wukong_synth as ws
from _metrics import TOL_BF16, TOL_BF16_RMS, TOL_F32, normwise_err, rel_err, rms_err

# Tensors the bf16 HIP path stores in bf16 (include/wukong.h): Z as a product
# operand, Fn, each h_t, M and Y.  The LCB output is not rounded.
BF16_STORAGE = ("Z", "Fn", "h", "M", "Y")


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def spec_of(shape: ws.LayerShape, dtype: str, eps: float = 1e-5) -> wk.LayerSpec:
    return wk.LayerSpec(shape.n, shape.d, shape.k, shape.n_f, shape.n_l, tuple(shape.mlp), eps, dtype)


def device_layers(cfg: ws.WukongConfig, host: Sequence[ws.HostLayerWeights]) -> List[wk.DeviceLayer]:
    return [wk.DeviceLayer.from_host(spec_of(cfg.layers[i], cfg.dtype), h) for i, h in enumerate(host)]


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def host_f64(a: np.ndarray) -> np.ndarray:
    """GPU output on the host -> float64 (bf16 bits widened exactly)."""
    if a.dtype == np.uint16:
        return ws.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def storage_for(cfg: ws.WukongConfig):
    return BF16_STORAGE if cfg.dtype == "bf16" else ()


def sample_indices(batch: int, count: int, seed: int) -> np.ndarray:
    """First, last and seeded random distinct example indices."""
    if count >= batch:
        return np.arange(batch)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, batch - 1), size=count - 2, replace=False)
    return np.unique(np.concatenate([[0, batch - 1], mid]))


class Run:
    """Generate a workload, run it through the C ABI, keep host copies."""

    def __init__(self, cfg: ws.WukongConfig, seed: int, affine: str = "random",
                 num_layers: Optional[int] = None, batch: Optional[int] = None):
        t0 = time.time()
        if batch is not None:
            cfg = cfg.with_batch(batch)
        if num_layers is not None:
            cfg = cfg.with_layers(num_layers)
        self.cfg = cfg
        self.host_w = ws.make_stack_weights(cfg, seed, affine)
        self.x = ws.make_input(cfg, seed)
        log(f"[{cfg.name} B={cfg.batch} l={cfg.num_layers}] generated in {time.time() - t0:.1f}s")
        self.layers = device_layers(cfg, self.host_w)
        self.xd = wk.to_device(self.x, cfg.dtype, "cuda")

    def forward(self, workspace=None, trace=None) -> torch.Tensor:
        y = wk.stack_forward(self.xd, self.layers, workspace=workspace, trace=trace)
        torch.cuda.synchronize()
        return y

    def oracle(self, idx=None, storage=None):
        x = self.x if idx is None else self.x[idx]
        st = storage_for(self.cfg) if storage is None else storage
        return oracle.wukong_stack(x, self.host_w, storage=st)


def check(name: str, got: np.ndarray, ref: np.ndarray, dtype: str, elementwise: bool = True) -> dict:
    """The parity gate (tests/_metrics.py): fp32 elementwise <= 1e-4; bf16
    normwise <= 2e-2 and rms <= 1e-2, plus elementwise <= 2e-2 when asked."""
    e = {"elementwise": rel_err(got, ref), "normwise": normwise_err(got, ref), "rms": rms_err(got, ref)}
    log(f"  {name}: elementwise={e['elementwise']:.3e} normwise={e['normwise']:.3e} rms={e['rms']:.3e}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    if dtype == "f32":
        assert e["elementwise"] <= TOL_F32, f"{name}: elementwise {e['elementwise']:.3e} > {TOL_F32:.0e}"
    else:
        assert e["normwise"] <= TOL_BF16, f"{name}: normwise {e['normwise']:.3e} > {TOL_BF16:.0e}"
        assert e["rms"] <= TOL_BF16_RMS, f"{name}: rms {e['rms']:.3e} > {TOL_BF16_RMS:.0e}"
        if elementwise:
            assert e["elementwise"] <= TOL_BF16, f"{name}: elementwise {e['elementwise']:.3e} > {TOL_BF16:.0e}"
    return e
