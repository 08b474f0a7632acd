"""Parity of one Wukong layer's backward pass (bf16) on the GPU with the CPU oracle.

The HIP path runs the training forward (which keeps Fn, h_t and M) and the
backward through the C ABI; the oracle (oracle/wukong_backward.py, pinned by
finite differences in test_backward_oracle_pins.py) runs on the same seeded
host arrays at the library's bf16 storage points: the forward's Z, Fn, h_t, M
and the backward's dR, g_t, d_Fn, dF, dZ and dX.  Inputs: X as the layer
workloads draw it, dY ~ N(0, 1) as a stand-in for the loss gradient, weights
Xavier-uniform with random LayerNorm affines and biases.  Every output (dX
and every weight gradient) passes the bf16 gate: elementwise 2e-2 with an rms
floor, normwise 2e-2, rms 1e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import recommender_feature_interaction_amd as wk
import wukong_synth as ws
from _gpu_helpers import check, host_f64, log, spec_of, to_host
from _metrics import TOL_BF16, TOL_BF16_RMS, normwise_err, rel_err, rms_err

pytestmark = pytest.mark.gpu

FWD_STORAGE = ("Z", "Fn", "h", "M")
BWD_STORAGE = ("dR", "dh", "dFn", "dF", "dZ", "dX")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    wk.load_library()


def _custom(name, n, d, k, n_f, mlp, batch):
    return ws.WukongConfig(name, "bf16", batch, (ws.LayerShape(n, d, k, n_f, n - n_f, tuple(mlp)),))


CASES = [
    _custom("bwd_tiny", 16, 16, 4, 8, (64, 64, 128), 37),                 # the tiny layer's shape in bf16
    _custom("bwd_layer_d160_b40", 128, 160, 32, 64, (4096, 2048, 10240), 40),  # the d = 160 layer, ragged batch
    _custom("bwd_padded", 40, 32, 20, 16, (800, 96, 72, 512), 70),        # k, n_l, n padded; three Linears
    _custom("bwd_d48", 24, 48, 12, 16, (288, 64, 768), 65),               # d % 32 == 16
    _custom("bwd_tiny_b600", 16, 16, 4, 8, (64, 64, 128), 600),           # 2-3 examples per workgroup
]


# Wide layers (n of 256 .. 720): the backward of wukong_backward_wide.hip (output rows, FM part per
# example, the [Phi; W_L] products as GEMMs over the batch-major gradient matrix)
# The oracle's own elementwise floor (test_tolerance_floor.py::test_wide_backward_floor) reaches
# the 2e-2 line for dX and d_Phi at the n = 256 layer's shape (and is taken to at the larger n = 512
# one), and for the MLP weight gradients of
# these small batches (2e-2 .. 3.5e-2): those are gated normwise and by rms at the fixed
# tolerances, everything else elementwise as well.
WIDE_ELEMENTWISE = {"bwd_wide_n256": False, "bwd_wide_n512": False}
WIDE_CASES = [
    _custom("bwd_wide_n256", 256, 160, 48, 128, (12288, 4096, 4096, 20480), 6),  # the n = 256 stack's layer
    _custom("bwd_wide_n720", 720, 32, 24, 360, (17280, 1024, 11520), 8),         # the n = 720 layer
    _custom("bwd_wide_n512", 512, 160, 96, 256, (49152, 8192, 8192, 40960), 3),  # the n = 512 stack's layer
    _custom("bwd_wide_n192_k40", 192, 160, 40, 96, (7680, 264, 15360), 5),       # k % 16 = 8
    _custom("bwd_wide_n360_k20", 360, 32, 20, 176, (7200, 136, 5632), 7),        # n % 32 = 8, k % 16 = 4
]


class BackwardRun:
    def __init__(self, cfg, seed, affine="random", batch=None):
        if batch is not None:
            cfg = cfg.with_batch(batch)
        self.cfg = cfg
        self.host_w = ws.make_stack_weights(cfg, seed, affine)[0]
        self.x = ws.make_input(cfg, seed)
        self.dy = ws.make_upstream_grad(cfg, seed)
        self.spec = spec_of(cfg.layers[0], "bf16")
        self.layer = wk.DeviceLayer.from_host(self.spec, self.host_w)
        self.xd = wk.to_device(self.x, "bf16", "cuda")
        self.dyd = wk.to_device(self.dy, "bf16", "cuda")

    def run(self, trace=None, grads=None):
        y, saved = wk.layer_forward_train(self.xd, self.layer)
        dx, grads = wk.layer_backward(self.xd, saved, self.dyd, self.layer, grads=grads, trace=trace)
        torch.cuda.synchronize()
        return y, saved, dx, grads

    def oracle(self, x=None, dy=None):
        x = self.x if x is None else x
        dy = self.dy if dy is None else dy
        return oracle.layer_backward(x, self.host_w, dy, storage=FWD_STORAGE + BWD_STORAGE)


def _grad_host(t):
    return t.detach().cpu().double().numpy()


def check_grads(got: wk.LayerGrads, ref: dict, T: int, elementwise: bool = True, mlp_elementwise=None):
    mlp_elementwise = elementwise if mlp_elementwise is None else mlp_elementwise
    check("d_phi", _grad_host(got.phi), ref["phi"], "bf16", elementwise)
    check("d_w_l", _grad_host(got.w_l), ref["w_l"], "bf16", elementwise)
    for name in ("fm_gamma", "fm_beta", "out_gamma", "out_beta"):
        check(f"d_{name}", _grad_host(getattr(got, name)), ref[name], "bf16", elementwise)
    for t in range(T):
        check(f"d_W{t}", _grad_host(got.mlp_w[t]), ref["mlp_w"][t], "bf16", mlp_elementwise)
        check(f"d_b{t}", _grad_host(got.mlp_b[t]), ref["mlp_b"][t], "bf16", mlp_elementwise)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_backward_parity(cfg):
    r = BackwardRun(cfg, seed=5)
    log(f"backward {cfg.name} B={cfg.batch} shape={cfg.layers[0]}")
    y, saved, dx, grads = r.run()
    ref = r.oracle()
    y_ref = oracle.wukong_layer(r.x, r.host_w, storage=FWD_STORAGE + ("Y",))
    check("Y (training forward)", host_f64(to_host(y)), y_ref, "bf16")
    check("dX", host_f64(to_host(dx)), ref["dX"], "bf16")
    check_grads(grads, ref, len(cfg.layers[0].mlp) - 1)


def subset_run(r, keep):
    """The same layer and weights on the examples `keep` of r's batch."""
    s = BackwardRun.__new__(BackwardRun)
    s.cfg = r.cfg.with_batch(int(np.count_nonzero(keep)))
    s.host_w, s.spec, s.layer = r.host_w, r.spec, r.layer
    s.x, s.dy = np.ascontiguousarray(r.x[keep]), np.ascontiguousarray(r.dy[keep])
    s.xd, s.dyd = wk.to_device(s.x, "bf16", "cuda"), wk.to_device(s.dy, "bf16", "cuda")
    return s


@pytest.mark.parametrize("cfg", WIDE_CASES, ids=lambda c: c.name)
def test_backward_parity_wide(cfg):
    """The wide layers' backward against the oracle, every output elementwise.  An
    example holding a ReLU near-tie decided the other way (relu_flip_examples) is
    compared normwise only, and the weight gradients, which sum over the batch,
    elementwise on the batch without it (examples are independent)."""
    r = BackwardRun(cfg, seed=15)
    log(f"backward {cfg.name} B={cfg.batch} shape={cfg.layers[0]}")
    tr = wk.Trace(capacity=128)
    y, saved, dx, grads = r.run(trace=tr)
    T = len(cfg.layers[0].mlp) - 1
    recs = [(x["kernel"], x["index"]) for x in tr.records()]
    tr.close()
    assert ("bwd_transpose", 3 * T) in recs and ("bwd_wgrad", T + 1) in recs, "not the wide-layer backward"
    ref = r.oracle()
    y_ref = oracle.wukong_layer(r.x, r.host_w, storage=FWD_STORAGE + ("Y",))
    check("Y (training forward)", host_f64(to_host(y)), y_ref, "bf16")
    got = host_f64(to_host(dx))
    elem = WIDE_ELEMENTWISE.get(cfg.name, True)
    flip, _ = relu_flip_examples(r, saved)
    if not flip.any():
        check("dX", got, ref["dX"], "bf16", elem)
        check_grads(grads, ref, T, elem, mlp_elementwise=False)
        return
    log(f"  examples {np.flatnonzero(flip).tolist()} hold a ReLU near-tie decided the other way")
    e_nw = normwise_err(got[flip], ref["dX"][flip])
    log(f"  dX (those examples): normwise={e_nw:.3e}")
    assert e_nw <= TOL_BF16, f"dX of the near-tie examples: normwise {e_nw:.3e}"
    check("dX (the others)", got[~flip], ref["dX"][~flip], "bf16", elem)
    s = subset_run(r, ~flip)
    _, saved2, dx2, grads2 = s.run()
    assert not relu_flip_examples(s, saved2)[0].any()
    ref2 = s.oracle()
    check("dX (batch without them)", host_f64(to_host(dx2)), ref2["dX"], "bf16", elem)
    check_grads(grads2, ref2, T, elem, mlp_elementwise=False)


def test_saved_activations_match_the_forward():
    cfg = CASES[2]
    r = BackwardRun(cfg, seed=6)
    _, saved, _, _ = r.run()
    _, it = oracle.wukong_layer(r.x, r.host_w, storage=FWD_STORAGE, intermediates=True)
    lay = wk.saved_layout(r.spec, cfg.batch)
    B, n, k, d = cfg.batch, r.spec.n, r.spec.k, r.spec.d

    def view(off, cols):
        raw = saved[off:off + B * cols * 2].view(torch.bfloat16)
        return host_f64(to_host(raw)).reshape(B, cols)

    check("Fn (saved)", view(lay["fn"], n * k), it["Fn"], "bf16")
    for t, off in enumerate(lay["hidden"]):
        check(f"h_{t + 1} (saved)", view(off, r.spec.mlp[t + 1]), it["h"][t], "bf16")
    check("M (saved)", view(lay["m"], r.spec.n_f * d), it["M"].reshape(B, -1), "bf16")


def test_backward_empty_and_single_example():
    """An empty batch: empty dX, zero gradients, and gradients passed in are left as they were.
    One example: every batch sum has a single term (the weight gradients are outer products)."""
    r = BackwardRun(CASES[2], seed=10, batch=1)
    _, _, dx, grads = r.run()
    ref = r.oracle()
    check("dX (one example)", host_f64(to_host(dx)), ref["dX"], "bf16")
    check_grads(grads, ref, len(CASES[2].layers[0].mlp) - 1)
    x0, dy0 = r.xd[:0], r.dyd[:0]
    y0, saved0 = wk.layer_forward_train(x0, r.layer)
    dx0, g0 = wk.layer_backward(x0, saved0, dy0, r.layer)
    torch.cuda.synchronize()
    assert y0.shape == dx0.shape == (0, r.spec.n, r.spec.d)
    for name, t in g0.as_dict().items():
        for u in t if isinstance(t, list) else [t]:
            assert u is not None and torch.count_nonzero(u).item() == 0, name
    before = [t.clone() for t in grads.mlp_w]
    wk.layer_backward(x0, saved0, dy0, r.layer, grads=grads)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(before, grads.mlp_w))


def test_backward_identity_affine_no_bias_effects():
    """Identity LayerNorm affines and zero biases (their gradients are still computed)."""
    r = BackwardRun(CASES[0], seed=7, affine="identity")
    _, _, dx, grads = r.run()
    ref = r.oracle()
    check("dX", host_f64(to_host(dx)), ref["dX"], "bf16")
    check_grads(grads, ref, 2)


def test_backward_determinism_trace_and_batch_rows():
    cfg = CASES[1]
    r = BackwardRun(cfg, seed=8)
    tr = wk.Trace(capacity=64)
    _, _, dx1, g1 = r.run(trace=tr)
    kinds = [x["kernel"] for x in tr.records()]
    tr.close()
    log(f"  launches: {kinds}")
    assert kinds[0] == "bwd_out" and "bwd_fmb" in kinds and kinds.count("bwd_wgrad") == 2
    assert kinds.count("bwd_dgrad") == 2
    dx1 = to_host(dx1)
    g1 = {k: (v if not isinstance(v, list) else [t.clone() for t in v]) for k, v in g1.as_dict().items()}
    g1 = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in g1.items()}
    _, _, dx2, g2 = r.run()
    assert np.array_equal(dx1, to_host(dx2)), "dX differs between two runs"
    for k, v in g2.as_dict().items():
        if isinstance(v, list):
            for a, b in zip(g1[k], v):
                assert torch.equal(a, b), k
        elif v is not None:
            assert torch.equal(g1[k], v), k
    # dX of an example depends on that example only
    sub = slice(3, 17)
    y, saved = wk.layer_forward_train(r.xd[sub].contiguous(), r.layer)
    dxs, _ = wk.layer_backward(r.xd[sub].contiguous(), saved, r.dyd[sub].contiguous(), r.layer)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(dxs), dx1[sub]), "a subset's dX rows differ from the full batch's"


def relu_flip_examples(r, saved, band=1e-2):
    """Examples where the kernels' ReLU mask differs from the oracle's.

    The mask is a decision taken from a rounded sum: the kernels take it from
    fp32 sums of the bf16 values they stored, the oracle from fp64 sums of its
    own, so a unit whose pre-activation is within rounding of zero can go
    either way, and both are correct results of the method.  Everything in such
    an example downstream of the mask (d_Fn, dF, dZ, dX) then differs by the
    flipped unit's contribution, and so do the weight-gradient entries that
    sum over the flipped unit: row j of d_W_t and entry j of d_b_t for unit j
    of h_{t+1}, column j of d_W_{t+1}.  This returns the examples holding a
    flip and the flipped units of each h_{t+1}, and checks that every flip is
    such a near-tie: the oracle's pre-activation (fp64, from its bf16-stored
    input) lies within `band` x rms of zero."""
    _, it = oracle.wukong_layer(r.x, r.host_w, storage=FWD_STORAGE, intermediates=True)
    lay = wk.saved_layout(r.spec, r.cfg.batch)
    acts = [it["Fn"]] + list(it["h"][:-1])
    B = r.cfg.batch
    flip = np.zeros(B, dtype=bool)
    units = {}
    for t, off in enumerate(lay["hidden"]):
        m = r.spec.mlp[t + 1]
        h_gpu = host_f64(to_host(saved[off:off + B * m * 2].view(torch.bfloat16))).reshape(B, m)
        W = oracle.to_f64(r.host_w.mlp_w[t])
        pre = acts[t] @ W.T + oracle.to_f64(r.host_w.mlp_b[t])
        differ = (h_gpu > 0) != (pre > 0)
        if differ.any():
            worst = float(np.abs(pre[differ]).max() / np.sqrt(np.mean(pre * pre)))
            log(f"  h_{t + 1}: {int(differ.sum())} mask flips, largest |pre-activation| {worst:.2e} x rms")
            assert worst < band, "a ReLU decision differs away from zero"
        flip |= differ.any(axis=1)
        units[t] = np.flatnonzero(differ.any(axis=0))
    return flip, units


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["layer_d160", "smalld_n720"])
def test_backward_full_batch(name):
    """The d = 160 layer at its full batch of 4096 (the fused per-example backward)
    and the n = 720 layer at its full batch of 8192 (the wide-layer backward): every
    gradient against the oracle over all examples (normwise and rms), and dX
    elementwise on every example whose ReLU masks agree with the oracle's
    (relu_flip_examples)."""
    r = BackwardRun(ws.BY_NAME[name], seed=9)
    _, saved, dx, grads = r.run()
    ref = r.oracle()
    got = host_f64(to_host(dx))
    check("dX (all examples)", got, ref["dX"], "bf16", elementwise=False)
    flip, units = relu_flip_examples(r, saved)
    log(f"  {int(flip.sum())} of {r.cfg.batch} examples hold a ReLU near-tie decided the other way")
    assert flip.sum() <= 0.05 * r.cfg.batch
    # elementwise per example: over thousands of examples the bf16 floor's largest values reach the
    # 2e-2 line (about 1.4e-2 is typical for one example of the n = 720 layer), so at most 0.1 % of
    # the examples may exceed it; all are within it normwise and by rms
    check("dX (examples whose masks agree)", got[~flip], ref["dX"][~flip], "bf16", elementwise=False)
    per = np.array([rel_err(got[b], ref["dX"][b]) for b in np.flatnonzero(~flip)])
    log(f"  dX elementwise per example: median {np.median(per):.2e}, 99.9th percentile "
        f"{np.percentile(per, 99.9):.2e}, above 2e-2: {int((per > TOL_BF16).sum())}")
    assert (per > TOL_BF16).mean() <= 1e-3
    # The weight gradients sum over the batch, near-tie examples included, whose contributions
    # differ legitimately (reading of the pages: both ReLU decisions are results of the method):
    # normwise and rms over the whole batch, and elementwise on the batch without those examples
    # (GPU and oracle run again on it; examples are independent).  The n = 720 layer's MLP
    # weight gradients stay normwise and rms there too: their floor lies above 2e-2
    # elementwise (test_tolerance_floor.py).
    T = len(r.cfg.layers[0].mlp) - 1
    mlp_elem = name != "smalld_n720"
    check_grads(grads, ref, T, elementwise=False)
    if flip.any():
        s = subset_run(r, ~flip)
        _, saved2, _, grads2 = s.run()
        assert not relu_flip_examples(s, saved2)[0].any()
        check_grads(grads2, s.oracle(), T, mlp_elementwise=mlp_elem)
    else:
        check_grads(grads, ref, T, mlp_elementwise=mlp_elem)


# Oracle parity of stacks runs on shapes with narrow hidden layers.  With the
# d = 160 layer's 2048-unit hidden layer, the upper layer's input (the lower
# layer's bf16 output, whose rounding differs from the oracle's by flips) also
# moves a few of its ReLU decisions, each of which changes one example's
# gradient as a whole, a random event no tolerance derived from the arithmetic
# bounds; that stack is checked bit for bit against the layer backward chained
# by hand (test_stack_backward_chains_the_layer_backward), the layer backward
# itself against the oracle above.
STACK_CASES = [
    # (name, n, d, k, n_f, mlp, layers, batch)
    ("bwd_stack2_padded", 40, 32, 20, 16, (800, 96, 512), 2, 37),
    ("bwd_stack3_tiny", 16, 16, 4, 8, (64, 64, 128), 3, 300),   # several examples per workgroup
    ("bwd_stack2_wide_d32", 360, 32, 20, 176, (7200, 136, 5632), 2, 6),  # wide layers
]
STACK_D160 = ("bwd_stack2_d160", 128, 160, 32, 64, (4096, 2048, 10240), 2, 24)


def _stack_run(case):
    name, n, d, k, n_f, mlp, layers, B = case
    shape = ws.LayerShape(n, d, k, n_f, n - n_f, tuple(mlp))
    cfg = ws.WukongConfig(name, "bf16", B, tuple([shape] * layers))
    host = ws.make_stack_weights(cfg, 5, "random")
    x = ws.make_input(cfg, 5)
    dy = ws.make_upstream_grad(cfg, 5)
    spec = spec_of(shape, "bf16")
    dev_layers = [wk.DeviceLayer.from_host(spec, h) for h in host]
    return cfg, host, x, dy, spec, dev_layers


@pytest.mark.parametrize("case", STACK_CASES, ids=lambda c: c[0])
def test_stack_backward_parity(case):
    """Stacks against the bf16-storage oracle, normwise and by rms at the fixed
    bf16 gate (2e-2 normwise, 1e-2 rms) for dX and every layer's weight
    gradients.  A layer's input is the previous layer's bf16 output, whose
    rounding flips against the oracle's carry into every later gradient, so the
    elementwise view is left to the per-layer test below.  The oracle's own
    floor (the same stack with the inter-layer activations kept in fp64
    instead of bf16) is logged beside each error as a diagnostic only."""
    name, n, d, k, n_f, mlp, layers, B = case
    cfg, host, x, dy, spec, dev_layers = _stack_run(case)
    xd = wk.to_device(x, "bf16", "cuda")
    y, saved = wk.stack_forward_train(xd, dev_layers)
    tr = wk.Trace(capacity=256)
    dx, grads = wk.stack_backward(xd, saved, wk.to_device(dy, "bf16", "cuda"), dev_layers, trace=tr)
    torch.cuda.synchronize()
    assert sorted({r["layer"] for r in tr.records()}) == list(range(layers))
    tr.close()
    log(f"stack backward {name}: {layers} layers, B={B}")
    st = FWD_STORAGE + ("Y",)
    check("Y (stack training forward)", host_f64(to_host(y)), oracle.wukong_stack(x, host, storage=st), "bf16",
          elementwise=False)
    ref_dx, ref = oracle.stack_backward(x, host, dy, storage=st + BWD_STORAGE)
    alt_dx, alt = oracle.stack_backward(x, host, dy, storage=FWD_STORAGE + BWD_STORAGE)  # fp64 between layers

    def items(dx_, g_):
        out = [("dX", dx_)]
        for i in range(layers):
            gi = g_[i] if isinstance(g_[i], dict) else {k_: (v.cpu().double().numpy() if isinstance(v, torch.Tensor)
                                                             else [t.cpu().double().numpy() for t in v])
                                                        for k_, v in g_[i].as_dict().items() if v is not None}
            for key in ("phi", "w_l", "fm_gamma", "fm_beta", "out_gamma", "out_beta"):
                out.append((f"layer {i} d_{key}", gi[key]))
            for t in range(len(mlp) - 1):
                out.append((f"layer {i} d_W{t}", gi["mlp_w"][t]))
                out.append((f"layer {i} d_b{t}", gi["mlp_b"][t]))
        return out

    for (label, g_), (_, r_), (_, a_) in zip(items(host_f64(to_host(dx)), grads), items(ref_dx, ref),
                                             items(alt_dx, alt)):
        nw_floor, rms_floor = normwise_err(a_, r_), rms_err(a_, r_)
        e_nw, e_rms = normwise_err(g_, r_), rms_err(g_, r_)
        log(f"  {label}: normwise={e_nw:.3e} rms={e_rms:.3e} (oracle floor: normwise {nw_floor:.2e}, "
            f"rms {rms_floor:.2e})")
        assert np.all(np.isfinite(g_)), label
        assert e_nw <= TOL_BF16 and e_rms <= TOL_BF16_RMS, f"{label}: normwise {e_nw:.3e}, rms {e_rms:.3e}"


def test_stack_backward_chains_the_layer_backward():
    """The stack backward equals the layer backward called layer by layer, last
    to first, on the inputs and activations the stack's training forward kept
    (bit for bit: the same kernels on the same data)."""
    cfg, host, x, dy, spec, dev_layers = _stack_run(STACK_D160)
    layers = len(dev_layers)
    xd = wk.to_device(x, "bf16", "cuda")
    dyd = wk.to_device(dy, "bf16", "cuda")
    y, saved = wk.stack_forward_train(xd, dev_layers)
    dx, grads = wk.stack_backward(xd, saved, dyd, dev_layers)
    # by hand: the training forward layer by layer, then the backward in reverse
    xs, sv = [xd], []
    for i, l in enumerate(dev_layers):
        yi, si = wk.layer_forward_train(xs[-1], l)
        sv.append(si)
        xs.append(yi)
    g = dyd
    hand = [None] * layers
    for i in range(layers - 1, -1, -1):
        g, hand[i] = wk.layer_backward(xs[i], sv[i], g.contiguous(), dev_layers[i])
    torch.cuda.synchronize()
    assert torch.equal(xs[-1], y)
    assert torch.equal(g, dx)
    for i in range(layers):
        for key, v in grads[i].as_dict().items():
            w = hand[i].as_dict()[key]
            if isinstance(v, list):
                assert all(torch.equal(a, b) for a, b in zip(v, w)), (i, key)
            elif v is not None:
                assert torch.equal(v, w), (i, key)


def test_stack_backward_empty_batch():
    """An empty batch through a stack: empty outputs and zero gradients for every layer."""
    _, _, x, dy, spec, dev_layers = _stack_run(STACK_CASES[0])
    xd = wk.to_device(x, "bf16", "cuda")[:0]
    dyd = wk.to_device(dy, "bf16", "cuda")[:0]
    y, saved = wk.stack_forward_train(xd, dev_layers)
    dx, grads = wk.stack_backward(xd, saved, dyd, dev_layers)
    torch.cuda.synchronize()
    assert y.shape == dx.shape == (0, spec.n, spec.d) and len(grads) == len(dev_layers)
    for g in grads:
        for name, t in g.as_dict().items():
            for u in t if isinstance(t, list) else [t]:
                assert u is not None and torch.count_nonzero(u).item() == 0, name


@pytest.mark.parametrize("case", STACK_CASES, ids=lambda c: c[0])
def test_stack_backward_teacher_forced_per_layer(case):
    """Each layer of a stack's backward, elementwise at the bf16 gate: layer i on
    the GPU takes the oracle's bf16 input of that layer (the oracle's forward
    output of the layer below) and the oracle's bf16 gradient arriving from the
    layer above, so no rounding flip of another layer reaches the comparison."""
    name, n, d, k, n_f, mlp, layers, B = case
    cfg, host, x, dy, spec, dev_layers = _stack_run(case)
    st_f = FWD_STORAGE + ("Y",)
    xs = [x]
    for i in range(layers - 1):  # the oracle's bf16 input of every layer
        yi = oracle.wukong_layer(xs[-1], host[i], storage=st_f)
        xs.append(ws.to_bf16_bits(yi.astype(np.float32)))
    g = dy
    log(f"stack backward per layer {name}: {layers} layers, B={B}")
    for i in range(layers - 1, -1, -1):
        r = BackwardRun.__new__(BackwardRun)
        r.cfg, r.host_w, r.x, r.dy, r.spec, r.layer = cfg.with_layers(1), host[i], xs[i], g, spec, dev_layers[i]
        r.xd, r.dyd = wk.to_device(xs[i], "bf16", "cuda"), wk.to_device(g, "bf16", "cuda")
        _, _, dx, grads = r.run()
        ref = r.oracle()
        log(f" layer {i}")
        check("  dX", host_f64(to_host(dx)), ref["dX"], "bf16")
        check_grads(grads, ref, len(mlp) - 1)
        g = ws.to_bf16_bits(ref["dX"].astype(np.float32))  # dX is stored in bf16: exact
