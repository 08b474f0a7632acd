"""Pins of the Wukong layer's backward oracle against facts that do not come from it.

  * central finite differences of the forward oracle (itself pinned by
    test_oracle_pins) along random directions of X and of every weight, at
    fp64 on tiny layers with one and two hidden Linears;
  * the output LayerNorm's input gradient is orthogonal to the ones vector
    and to the normalised row (eps = 0, unit gamma);
  * the output scale's gradient equals sum dY * (Y - beta) / gamma read off
    the forward's own output;
  * a zero upstream gradient gives zero gradients everywhere;
  * two stacked layers: the chained backward against central differences of
    the stack's loss.
Each planted mistake in MUTANTS must fail at least one pin.
"""
import math
import types

import numpy as np
import pytest

import oracle.wukong_backward as WB
from oracle.wukong_oracle import wukong_layer


def _weights(n, d, k, n_l, hidden, seed, affine=True, bias=True):
    g = np.random.default_rng(seed)
    dims = [n * k] + list(hidden) + [(n - n_l) * d]
    return types.SimpleNamespace(
        phi=g.normal(size=(k, n)) / math.sqrt(n), w_l=g.normal(size=(n_l, n)) / math.sqrt(n),
        fm_gamma=1 + 0.2 * g.normal(size=n * k) if affine else None,
        fm_beta=0.2 * g.normal(size=n * k) if affine else None,
        mlp_w=[g.normal(size=(dims[t + 1], dims[t])) / math.sqrt(dims[t]) for t in range(len(dims) - 1)],
        mlp_b=[0.3 * g.normal(size=dims[t + 1]) for t in range(len(dims) - 1)] if bias else None,
        out_gamma=1 + 0.2 * g.normal(size=d) if affine else None,
        out_beta=0.2 * g.normal(size=d) if affine else None)


def _case(hidden=(8,), seed=0, S=3, n=6, d=4, k=3, n_l=2, **kw):
    g = np.random.default_rng(seed + 100)
    w = _weights(n, d, k, n_l, hidden, seed, **kw)
    return w, g.normal(size=(S, n, d)), g.normal(size=(S, n, d))


def _params(w):
    """(name, index, array) of every differentiable weight present in w."""
    out = [("phi", None, w.phi), ("w_l", None, w.w_l)]
    for name in ("fm_gamma", "fm_beta", "out_gamma", "out_beta"):
        if getattr(w, name) is not None:
            out.append((name, None, getattr(w, name)))
    for t, W in enumerate(w.mlp_w):
        out.append(("mlp_w", t, W))
    if w.mlp_b is not None:
        for t, b in enumerate(w.mlp_b):
            out.append(("mlp_b", t, b))
    return out


def _fd_check(mod, w, X, dY, h=1e-6, tol=2e-6):
    grads = mod.layer_backward(X, w, dY)
    rng = np.random.default_rng(11)
    # the input
    V = rng.normal(size=X.shape)
    fd = (WB.layer_loss(X + h * V, w, dY) - WB.layer_loss(X - h * V, w, dY)) / (2 * h)
    an = float((grads["dX"] * V).sum())
    assert abs(fd - an) <= tol * max(1.0, abs(fd)), ("dX", fd, an)
    # every weight
    for name, t, P in _params(w):
        V = rng.normal(size=P.shape)
        P0 = P.copy()
        P[...] = P0 + h * V
        lp = WB.layer_loss(X, w, dY)
        P[...] = P0 - h * V
        lm = WB.layer_loss(X, w, dY)
        P[...] = P0
        fd = (lp - lm) / (2 * h)
        g = grads[name] if t is None else grads[name][t]
        an = float((g * V).sum())
        assert abs(fd - an) <= tol * max(1.0, abs(fd)), (name, t, fd, an)


def pin_finite_differences_one_hidden(mod):
    _fd_check(mod, *_case(hidden=(8,), seed=1))


def pin_finite_differences_two_hidden(mod):
    _fd_check(mod, *_case(hidden=(7, 5), seed=2, S=2, n=8, d=3, k=2, n_l=3))


def pin_finite_differences_no_affine_no_bias(mod):
    w, X, dY = _case(hidden=(6,), seed=3, affine=False, bias=False)
    _fd_check(mod, w, X, dY)


def pin_layernorm_projection(mod):
    w, X, dY = _case(hidden=(8,), seed=4, affine=False)
    out = mod.layer_backward(X, w, dY, eps=0.0, intermediates=True)
    _, it = wukong_layer(X, w, eps=0.0, intermediates=True)
    R = it["R"]
    R_hat = (R - R.mean(-1, keepdims=True)) / R.std(-1, keepdims=True)
    dR = out["inter"]["dR"]
    assert np.abs(dR.sum(-1)).max() < 1e-10
    assert np.abs((dR * R_hat).sum(-1)).max() < 1e-10
    assert np.abs(dR).max() > 1e-3


def pin_out_gamma_from_forward(mod):
    w, X, dY = _case(hidden=(8,), seed=5)
    out = mod.layer_backward(X, w, dY)
    Y = wukong_layer(X, w)
    want = (dY * (Y - w.out_beta) / w.out_gamma).sum(axis=(0, 1))
    assert np.allclose(out["out_gamma"], want, atol=1e-10)
    assert np.allclose(out["out_beta"], dY.sum(axis=(0, 1)), atol=1e-12)


def pin_zero_upstream(mod):
    w, X, _ = _case(hidden=(8,), seed=6)
    out = mod.layer_backward(X, w, np.zeros_like(X))
    for key in ("dX", "phi", "w_l", "fm_gamma", "fm_beta", "out_gamma", "out_beta"):
        assert not np.any(out[key]), key
    for t in range(len(w.mlp_w)):
        assert not np.any(out["mlp_w"][t]) and not np.any(out["mlp_b"][t])


def pin_stack_finite_differences(mod):
    """Two stacked layers: the chained backward against central differences of the stack's loss."""
    w1, X, dY = _case(hidden=(8,), seed=8)
    w2, _, _ = _case(hidden=(5,), seed=9)
    ws_ = [w1, w2]
    dX, grads = mod.stack_backward(X, ws_, dY)
    h, rng = 1e-6, np.random.default_rng(12)
    V = rng.normal(size=X.shape)
    fd = (WB.stack_loss(X + h * V, ws_, dY) - WB.stack_loss(X - h * V, ws_, dY)) / (2 * h)
    assert abs(fd - float((dX * V).sum())) <= 2e-6 * max(1.0, abs(fd))
    for li, name in ((0, "phi"), (0, "w_l"), (1, "phi"), (1, "out_gamma")):
        P = getattr(ws_[li], name)
        V = rng.normal(size=P.shape)
        P0 = P.copy()
        P[...] = P0 + h * V
        lp = WB.stack_loss(X, ws_, dY)
        P[...] = P0 - h * V
        lm = WB.stack_loss(X, ws_, dY)
        P[...] = P0
        fd = (lp - lm) / (2 * h)
        assert abs(fd - float((grads[li][name] * V).sum())) <= 2e-6 * max(1.0, abs(fd)), (li, name)


PINS = {f.__name__: f for f in (pin_finite_differences_one_hidden, pin_finite_differences_two_hidden,
                                 pin_finite_differences_no_affine_no_bias, pin_layernorm_projection,
                                 pin_out_gamma_from_forward, pin_zero_upstream, pin_stack_finite_differences)}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    PINS[name](WB)


def test_storage_names_and_rounding():
    w, X, dY = _case(hidden=(8,), seed=7)
    with pytest.raises(ValueError):
        WB.layer_backward(X, w, dY, storage=("dQ",))
    full = ("Z", "Fn", "h", "M", "dR", "dh", "dFn", "dF", "dZ", "dX")
    out = WB.layer_backward(X, w, dY, storage=full, intermediates=True)
    assert np.array_equal(out["dX"], WB.round_bf16(out["dX"]))
    assert np.array_equal(out["inter"]["dF"], WB.round_bf16(out["inter"]["dF"]))
    ref = WB.layer_backward(X, w, dY)
    rel = np.linalg.norm(out["dX"] - ref["dX"]) / np.linalg.norm(ref["dX"])
    assert 0 < rel < 2e-2, rel


MUTANTS = {
    "residual_dropped": ("dX = dR.copy()", "dX = np.zeros_like(dR)"),
    "lcb_input_term_dropped": ("dX = dX + np.matmul(w_l.T, dLc)", "dX = dX"),
    "ln_mean_term_dropped": ("return rstd * (g_hat - m1 - v_hat * m2)", "return rstd * (g_hat - v_hat * m2)"),
    "ln_projection_term_dropped": ("return rstd * (g_hat - m1 - v_hat * m2)", "return rstd * (g_hat - m1)"),
    "relu_mask_dropped": ("g = _r(g * (acts[t] > 0), \"dh\", storage)", "g = _r(g, \"dh\", storage)"),
    "phi_input_term_dropped": ("+ np.matmul(phi.T, dZ)", ""),
    "interaction_term_dropped": ("np.matmul(dF, Z) + ", ""),
    "fm_gamma_not_applied": ("layer_norm_backward(d_fn * g_fm,", "layer_norm_backward(d_fn,"),
    "dphi_from_z": ("np.einsum(\"bje,bme->jm\", dZ, X)", "np.einsum(\"bje,bme->jm\", Z, X)"),
    "bias_grad_mean": ("d_mlp_b[t] = g.sum(axis=0)", "d_mlp_b[t] = g.mean(axis=0)"),
    "out_gamma_unnormalised": ("(dY * R_hat).sum(axis=(0, 1))", "(dY * R).sum(axis=(0, 1))"),
    "dW_transposed_input": ("d_mlp_w[t] = g.T @ acts[t]", "d_mlp_w[t] = g.T @ (acts[t] * (acts[t] > 0))"),
    "dz_transposed": ("np.matmul(np.swapaxes(dF, 1, 2), X)", "np.matmul(np.swapaxes(dF, 1, 2), X) * 0.5"),
    "out_gamma_not_applied": ("layer_norm_backward(dY * g_out,", "layer_norm_backward(dY,"),
    "stack_first_input_everywhere": ("out = layer_backward(xs[i], weights[i], g, eps, storage)",
                                     "out = layer_backward(xs[0], weights[i], g, eps, storage)"),
    "stack_upstream_not_chained": ("        g = out[\"dX\"]\n", "        g = g\n"),
}


def make_mutant(old, new):
    src = open(WB.__file__).read()
    assert src.count(old) == 1, old
    src = src.replace(old, new).replace("from .wukong_oracle import", "from oracle.wukong_oracle import")
    mod = types.ModuleType("wukong_backward_mutant")
    mod.__file__ = WB.__file__
    exec(compile(src, "wukong_backward_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(mutant):
    mod = make_mutant(*MUTANTS[mutant])
    caught = []
    for name, pin in PINS.items():
        try:
            pin(mod)
        except Exception:
            caught.append(name)
    assert caught, f"no pin catches the planted mistake {mutant!r}"
