"""Parity of WHALE's fusion step (shared K = V cross-attention, Fusion Linear,
pre-norm shared-gate SwiGLU FFN) on the GPU with the CPU oracle.

Inputs are seeded stand-ins: H_w with a LayerNorm output's statistics and the
sequence output H_s, both N(0, 1).  The oracle runs at the library's bf16
storage points (the softmax weights where they multiply H_s, A, Q, LN(Q),
silu(U) * U and H_f) and is gated like the layer (bf16: elementwise 2e-2
with an rms floor, normwise 2e-2, rms 1e-2); intermediates read back from the
workspace are gated the same way.
"""
import numpy as np
import pytest
import torch

import oracle
import recommender_feature_interaction_amd as wk
import wukong_synth as ws
from _gpu_helpers import check, host_f64, log, sample_indices, to_host

pytestmark = pytest.mark.gpu

STORAGE = ("P", "A", "Q", "Qn", "G", "Hf")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    wk.load_library()


class FusionRun:
    def __init__(self, B, n, d, L, dff, seed, affine="random", hw_scale=1.0):
        self.spec = wk.FusionSpec(n, d, L, dff)
        tag = f"fusion_n{n}_d{d}_L{L}"
        hw = ws.bf16_bits_to_f32(ws.make_sequence(tag + "/hw", B, n, d, "bf16", seed)) * np.float32(hw_scale)
        self.hw = ws.to_bf16_bits(hw)
        self.hs = ws.make_sequence(tag, B, L, d, "bf16", seed)
        self.w = ws.make_fusion_weights(tag, d, dff, "bf16", seed, affine)
        w = self.w
        self.dev = wk.DeviceFusion(self.spec, w.w_f, w.w_up, w.w_down, w.b_f, w.gamma, w.beta, w.b_up, w.b_down)
        self.hwd = wk.to_device(self.hw, "bf16", "cuda")
        self.hsd = wk.to_device(self.hs, "bf16", "cuda")
        self.B = B

    def forward(self, workspace=None, trace=None):
        out = wk.fusion_forward(self.hwd, self.hsd, self.dev, workspace=workspace, trace=trace)
        torch.cuda.synchronize()
        return out

    def oracle(self, idx=None, intermediates=False):
        hw, hs = (self.hw, self.hs) if idx is None else (self.hw[idx], self.hs[idx])
        return oracle.whale_fusion(hw, hs, self.w, storage=STORAGE, intermediates=intermediates)


# Key tiles hold 32 positions at d >= 96, 64 at d = 64 and 128 at d = 32; the ring has 4
# slots, so the number of tiles T modulo 4 selects the slot the Fusion Linear's W_f
# stream starts from.
CASES = [
    (5, 32, 64, 50, 256),      # d = 64: one ragged key tile
    (3, 48, 64, 130, 256),     # d = 64: three key tiles, the last ragged (T % 4 = 3)
    (2, 48, 64, 300, 256),     # d = 64: five key tiles, the last ragged (T % 4 = 1)
    (3, 48, 32, 300, 128),     # d = 32: three 128-position tiles, the last ragged (T % 4 = 3)
    (2, 32, 32, 600, 128),     # d = 32: five tiles, the last ragged (T % 4 = 1)
    (2, 16, 32, 520, 128),     # d = 32: five tiles, a last tile of 8 positions
    (4, 128, 160, 1024, 640),  # the measured shape
    (3, 16, 32, 1, 128),       # one position: A equals it for every query
    (2, 48, 96, 33, 384),      # a partly filled query chunk
    (2, 144, 128, 100, 512),   # two query chunks
    (3, 48, 160, 70, 200),     # d_ff % 32 != 0: the FFN as separate kernels
    (7, 80, 160, 20, 32),      # one d_ff chunk; 560 rows, a ragged last FFN tile
    (1, 128, 160, 1024, 640),  # one example of the measured shape: 128 rows, half an FFN tile
]


@pytest.mark.parametrize("B,n,d,L,dff", CASES, ids=lambda v: str(v))
def test_fusion_parity_and_intermediates(B, n, d, L, dff):
    r = FusionRun(B, n, d, L, dff, seed=3)
    wst = wk.alloc_workspace(wk.fusion_workspace_size(r.spec, B))
    hf = host_f64(to_host(r.forward(workspace=wst)))
    ref, it = r.oracle(intermediates=True)
    log(f"fusion B={B} n={n} d={d} L={L} d_ff={dff}")
    check("H_f", hf, ref, "bf16")
    rows = B * n
    # Q = [H_w, A] W_f^T + b_f, written by the attention kernel at the start of the workspace
    q = host_f64(to_host(wst[:rows * d * 2].view(torch.bfloat16))).reshape(B, n, d)
    check("Q", q, it["Q"], "bf16")


def test_fusion_sharp_softmax_and_identity_affine():
    """Logits scaled up 8x (near one-hot attention) with identity LayerNorm / zero biases."""
    r = FusionRun(3, 64, 128, 300, 512, seed=4, affine="identity", hw_scale=8.0)
    check("H_f (sharp attention)", host_f64(to_host(r.forward())), r.oracle(), "bf16")


FUSED_KINDS = [("fusion_attention", 0), ("fusion_ffn", 0)]
UNFUSED_KINDS = [("fusion_attention", 0), ("fusion_ln", 0), ("fusion_linear", 1), ("fusion_linear", 2)]


@pytest.mark.parametrize("dff,kinds", [(640, FUSED_KINDS), (200, UNFUSED_KINDS)], ids=["fused_ffn", "unfused_ffn"])
def test_fusion_trace_determinism_and_batch_invariance(dff, kinds):
    r = FusionRun(6, 128, 160, 257, dff, seed=5)
    tr = wk.Trace(capacity=16)
    y1 = to_host(r.forward(trace=tr))
    got = [(x["kernel"], x["index"]) for x in tr.records()]
    tr.close()
    assert got == kinds, got
    assert np.array_equal(y1, to_host(r.forward())), "two runs differ"
    sub = wk.fusion_forward(r.hwd[2:5].contiguous(), r.hsd[2:5].contiguous(), r.dev)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(sub), y1[2:5]), "a subset's rows differ from the full batch's"
    empty = wk.fusion_forward(r.hwd[:0], r.hsd[:0], r.dev)
    torch.cuda.synchronize()
    assert empty.shape == (0, 128, 160)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_fusion_full_batch_sampled():
    """The measured shape at its full batch (4096 examples, L = 1024); sampled examples checked."""
    r = FusionRun(4096, 128, 160, 1024, 640, seed=9, affine="identity")
    hf = r.forward()
    assert torch.isfinite(hf.float()).all().item()
    idx = sample_indices(r.B, 6, seed=3)
    check(f"H_f at examples {idx.tolist()}", host_f64(to_host(hf))[idx], r.oracle(idx), "bf16")
