"""Parity of the Wukong mixture-of-experts layer on the GPU with the CPU oracle.

Each expert is a Wukong module with its own k, FMB rows n_F,e, LCB rows
n_L,e and MLP; the experts' rows add up to n.  The HIP path (experts as
grouped launches of the layer kernels, each writing its share of the output
rows) runs through the C ABI; the oracle (oracle/wukong_moe_oracle.py, pinned
in test_moe_oracle_pins.py) runs on the same seeded host arrays at the bf16
storage points Z, Fn, h_t, M and Y (fp32: none), with the gate of the
single-layer tests (bf16: elementwise and normwise 2e-2, rms 1e-2; fp32:
elementwise 1e-4).
"""
import numpy as np
import pytest
import torch

import oracle
import recommender_feature_interaction_amd as wk
import wukong_synth as ws
from _gpu_helpers import BF16_STORAGE, check, host_f64, log, sample_indices, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    wk.load_library()


class MoeRun:
    """experts: list of (k, n_f, n_l, hidden widths)."""

    def __init__(self, tag, n, d, experts, batch, dtype="bf16", seed=3, affine="random"):
        self.dtype = dtype
        self.specs, self.host = [], []
        for e, (k, n_f, n_l, hidden) in enumerate(experts):
            mlp = (n * k,) + tuple(hidden) + (n_f * d,)
            self.specs.append(wk.LayerSpec(n, d, k, n_f, n_l, mlp, 1e-5, dtype))
            self.host.append(ws.make_expert_weights(tag, e, n, d, k, n_l, mlp, dtype, seed, affine))
        self.out_gamma, self.out_beta = ws.make_out_layernorm(tag, d, dtype, seed, affine)
        cfg = ws.WukongConfig(tag, dtype, batch, (ws.LayerShape(n, d, 1, n - 1, 1, (n, (n - 1) * d)),))
        self.x = ws.make_input(cfg, seed)
        self.spec = wk.MoeSpec(self.specs)
        self.moe = wk.DeviceMoe(self.spec, [wk.DeviceLayer.from_host(s, h) for s, h in zip(self.specs, self.host)],
                                self.out_gamma, self.out_beta)
        self.xd = wk.to_device(self.x, dtype, "cuda")

    def forward(self, trace=None):
        y = wk.moe_forward(self.xd, self.moe, trace=trace)
        torch.cuda.synchronize()
        return y

    def oracle(self, idx=None):
        x = self.x if idx is None else self.x[idx]
        st = BF16_STORAGE if self.dtype == "bf16" else ()
        return oracle.wukong_moe_layer(x, self.host, self.out_gamma, self.out_beta, storage=st)


CASES = [
    # (tag, n, d, experts, batch)
    ("moe_mixed", 40, 32, [(12, 8, 4, (72,)), (8, 6, 10, (96, 64)), (4, 2, 10, (40,))], 37),
    ("moe4_d160", 128, 160, [(32, 16, 16, (2048,))] * 4, 24),  # four experts of the d = 160 layer's width
    ("moe2_d16", 16, 16, [(4, 4, 4, (32,)), (8, 4, 4, (64,))], 130),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_moe_parity(case):
    tag, n, d, experts, B = case
    r = MoeRun(tag, n, d, experts, B)
    log(f"moe {tag}: n={n} d={d} experts={experts} B={B}")
    check("Y", host_f64(to_host(r.forward())), r.oracle(), "bf16")


def test_moe_fp32():
    r = MoeRun("moe_f32", 16, 16, [(4, 4, 4, (32,)), (4, 4, 4, (64, 16))], 64, dtype="f32")
    check("Y (fp32)", host_f64(to_host(r.forward())), r.oracle(), "f32")


def test_one_expert_is_the_layer():
    """One expert covering every row launches exactly the single layer's kernels."""
    r = MoeRun("moe_one", 40, 32, [(12, 16, 24, (72,))], 37)
    y_moe = to_host(r.forward())
    layer = wk.DeviceLayer(r.specs[0], r.host[0].phi, r.host[0].w_l, r.host[0].mlp_w, r.host[0].mlp_b,
                           r.host[0].fm_gamma, r.host[0].fm_beta, r.out_gamma, r.out_beta)
    y_layer = wk.layer_forward(r.xd, layer)
    torch.cuda.synchronize()
    assert np.array_equal(y_moe, to_host(y_layer))


def test_moe_trace_and_determinism():
    r = MoeRun("moe_mixed", 40, 32, CASES[0][3], 37)
    tr = wk.Trace(capacity=64)
    y1 = to_host(r.forward(trace=tr))
    recs = tr.records()
    tr.close()
    experts = sorted({x["layer"] for x in recs})
    assert experts == [0, 1, 2], experts
    assert [x["kernel"] for x in recs if x["layer"] == 1].count("mlp_linear") == 3
    assert np.array_equal(y1, to_host(r.forward())), "two runs differ"


def test_moe_grouped_last_linears():
    """Experts whose last Linears carry the output LayerNorm run those as one grouped launch
    (recorded as layer = number of experts); each expert launches its FMB+LCB and first Linear."""
    tag, n, d, experts, B = CASES[1]
    r = MoeRun(tag, n, d, experts, B)
    tr = wk.Trace(capacity=64)
    y = r.forward(trace=tr)
    recs = [(x["kernel"], x["layer"], x["index"]) for x in tr.records()]
    tr.close()
    assert recs.count(("mlp_linear", len(experts), 0)) == 1, recs
    for e in range(len(experts)):
        assert [k for k in recs if k[1] == e] == [("fmb_lcb", e, 0), ("mlp_linear", e, 0)], recs
    check("Y (grouped last Linears)", host_f64(to_host(y)), r.oracle(), "bf16")
    assert np.array_equal(to_host(y), to_host(r.forward())), "two runs differ"


def test_moe_grouped_launches_of_four():
    """Six experts with fused last Linears: those run as two grouped launches (four, then two)."""
    experts = [(16, 8, 8, (128,))] * 2 + [(24, 12, 12, (192,))] * 4  # rows 2 * 16 + 4 * 24 = 128
    r = MoeRun("moe6_d160", 128, 160, experts, 20)
    tr = wk.Trace(capacity=64)
    y = r.forward(trace=tr)
    recs = [(x["kernel"], x["layer"], x["index"]) for x in tr.records()]
    tr.close()
    assert [k for k in recs if k[1] == len(experts)] == [("mlp_linear", 6, 0), ("mlp_linear", 6, 1)], recs
    check("Y (six experts)", host_f64(to_host(y)), r.oracle(), "bf16")


def test_moe_empty_and_single_example():
    r = MoeRun("moe_mixed", 40, 32, CASES[0][3], 1)
    check("Y (one example)", host_f64(to_host(r.forward())), r.oracle(), "bf16")
    empty = wk.moe_forward(r.xd[:0], r.moe)
    torch.cuda.synchronize()
    assert empty.shape == (0, 40, 32)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_moe_full_batch_sampled():
    """Four experts of the d = 160 layer's width at the full batch of 4096; sampled examples checked."""
    tag, n, d, experts, _ = CASES[1]
    r = MoeRun(tag, n, d, experts, 4096)
    y = host_f64(to_host(r.forward()))
    idx = sample_indices(4096, 8, seed=5)
    check(f"Y at examples {idx.tolist()}", y[idx], r.oracle(idx), "bf16")
