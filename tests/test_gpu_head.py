"""Parity of the prediction head (top MLP + logistic function) with the oracle.

The head reads a layer output Y [batch, n, d]; here Y is a seeded synthetic
stand-in with a LayerNorm output's statistics (N(0, 1) entries), so the head
is checked on its own, and once end to end after a real layer on the GPU
against the oracle's layer followed by its head.  fp32 heads are gated
elementwise at 1e-4 against the pure fp64 oracle; bf16 heads against the
oracle with the hidden activations rounded to bf16 where produced (the
library stores them in bf16), at the bf16 gate.
"""
import numpy as np
import pytest
import torch

import oracle
import recommender_feature_interaction_amd as wk
import wukong_synth as ws
from _gpu_helpers import Run, check, host_f64, log, sample_indices, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    wk.load_library()


def _y_standin(batch, n, d, dtype, seed):
    cfg = ws.WukongConfig(f"head_y_n{n}_d{d}", dtype, batch,
                          (ws.LayerShape(n, d, 1, n, 0, (n, n * d)),))
    return ws.make_input(cfg, seed)


class HeadRun:
    def __init__(self, dims, batch, dtype, seed, affine="random", y_host=None, n=None):
        dims = tuple(dims)
        if y_host is None:
            n = n or 8
            assert dims[0] % n == 0
            y_host = _y_standin(batch, n, dims[0] // n, dtype, seed)
        self.y = y_host
        self.dims, self.dtype = dims, dtype
        self.w, self.b = ws.make_head_weights(f"head{len(dims)}", dims, dtype, seed, affine)
        self.head = wk.DeviceHead(wk.HeadSpec(dims, dtype), self.w, self.b)
        self.yd = wk.to_device(y_host, dtype, "cuda")

    def forward(self, y=None, trace=None):
        p = wk.head_forward(self.yd if y is None else y, self.head, trace=trace)
        torch.cuda.synchronize()
        return p

    def oracle(self, idx=None, y=None):
        yy = self.y if y is None else y
        if idx is not None:
            yy = yy[idx]
        st = ("h",) if self.dtype == "bf16" else ()
        return oracle.prediction_head(yy, self.w, self.b, storage=st)


def test_f32_head_elementwise():
    for dims, batch in [((64, 40, 24, 3), 37), ((60, 12, 5), 9), ((96, 1), 130)]:
        r = HeadRun(dims, batch, "f32", seed=2, n=4)
        log(f"f32 head dims={dims} B={batch}")
        p = r.forward()
        assert p.shape == (batch, dims[-1]) and p.dtype == torch.float32
        check("prob", host_f64(to_host(p)), r.oracle(), "f32")


HEADS_BF16 = [
    ((20480, 1024, 256, 1), 48),       # the default head on the d=160, n=128 layer output
    ((256, 136, 40, 3), 37),           # ragged widths: K % 64 != 0 on the second Linear
    ((128, 2), 5),                     # no hidden layer
    ((512, 64, 1), 1),
    ((4096, 72, 1), 37),               # the hidden Linear split in two along K (ragged rows and columns)
    ((81920, 1024, 256, 1), 40),       # the n = 512 stack's head: 8 K splits
]


@pytest.mark.parametrize("dims,batch", HEADS_BF16, ids=lambda v: str(v))
def test_bf16_head(dims, batch):
    r = HeadRun(dims, batch, "bf16", seed=3, n=8 if dims[0] % 8 == 0 else 1)
    log(f"bf16 head dims={dims} B={batch}")
    p = host_f64(to_host(r.forward()))
    check("prob", p, r.oracle(), "bf16")
    _, z = oracle.prediction_head(r.y, r.w, r.b, storage=("h",), logits=True)
    log(f"  logits span [{z.min():.2f}, {z.max():.2f}] (probabilities not saturated)")


def test_head_without_biases():
    """NULL biases mean zero bias (both the GEMM and the output kernel)."""
    r = HeadRun((4096, 72, 1), 37, "bf16", seed=5)
    head = wk.DeviceHead(wk.HeadSpec(r.dims, "bf16"), r.w)
    p = host_f64(to_host(wk.head_forward(r.yd, head)))
    torch.cuda.synchronize()
    check("prob (no biases)", p, oracle.prediction_head(r.y, r.w, None, storage=("h",)), "bf16")


def test_head_after_layer_end_to_end():
    """X -> Wukong layer -> head on the GPU against the oracle's layer and head."""
    cfg = ws.LAYER_D160
    r = Run(cfg, seed=6, affine="random", batch=24)
    y = r.forward()
    dims = cfg.head_dims()
    w, b = ws.make_head_weights("e2e", dims, "bf16", 6, "random")
    head = wk.DeviceHead(wk.HeadSpec(dims, "bf16"), w, b)
    p = host_f64(to_host(wk.head_forward(y, head)))
    torch.cuda.synchronize()
    y_ref = oracle.wukong_stack(r.x, r.host_w, storage=("Z", "Fn", "h", "M", "Y"))
    p_ref = oracle.prediction_head(y_ref, w, b, storage=("h",))
    check("prob after the layer", p, p_ref, "bf16")


def test_head_determinism_batch_invariance_and_trace():
    r = HeadRun((20480, 1024, 256, 1), 64, "bf16", seed=4, n=128)
    tr = wk.Trace(capacity=16)
    p1 = to_host(r.forward(trace=tr))
    recs = tr.records()
    tr.close()
    kinds = [(x["kernel"], x["index"]) for x in recs]
    assert kinds == [("head_linear", 0), ("head_linear", 1), ("head_out", 0)], kinds
    assert all(x["ms"] > 0 for x in recs)
    p2 = to_host(r.forward())
    assert np.array_equal(p1, p2), "two runs differ"
    sub = wk.head_forward(r.yd[7:30].contiguous(), r.head)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(sub), p1[7:30]), "a subset's rows differ from the full batch's"
    empty = wk.head_forward(r.yd[:0], r.head)
    torch.cuda.synchronize()
    assert empty.shape == (0, 1)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_head_full_batch_sampled():
    """The default head at the d=160 workload's full batch; the oracle recomputes sampled rows."""
    cfg = ws.LAYER_D160
    dims = cfg.head_dims()
    r = HeadRun(dims, cfg.batch, "bf16", seed=9, affine="identity", n=cfg.layers[0].n)
    p = r.forward()
    assert torch.isfinite(p).all().item()
    idx = sample_indices(cfg.batch, 16, seed=2)
    check(f"prob at examples {idx.tolist()}", host_f64(to_host(p))[idx], r.oracle(idx), "bf16")
