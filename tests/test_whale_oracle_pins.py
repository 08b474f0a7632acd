"""Pins of the WHALE fusion oracle against facts that do not come from it.

  * attention: explicit loops on tiny inputs (brute force); identical key
    rows give that row for every query; all-equal logits give the mean of
    the sequence (the mean pooling the WHALE ablation replaces attention
    with); one key with a much larger logit selects its row; a two-key case
    in closed form pins the 1/sqrt(d) scale;
  * silu and the shared gate: closed forms at u = 0, ln 3, -ln 3;
  * concatenation order: one-hot Fusion weights that read only H_w or only
    the attention output;
  * the pre-norm block: W_down = 0 leaves Q (the residual), the down
    projection's bias adds exactly, and scaling Q leaves the FFN branch
    unchanged (it sees LN(Q));
Each planted mistake in MUTANTS must fail at least one pin.
"""
import math
import types

import numpy as np
import pytest

import oracle.whale_oracle as WH

rng = np.random.default_rng(7)


def _w(d, dff, seed=0, bias=True):
    g = np.random.default_rng(seed)
    return types.SimpleNamespace(
        w_f=g.normal(size=(d, 2 * d)) / math.sqrt(2 * d), b_f=g.normal(size=d) * 0.1 if bias else None,
        gamma=1 + 0.1 * g.normal(size=d), beta=0.1 * g.normal(size=d),
        w_up=g.normal(size=(dff, d)) / math.sqrt(d), b_up=g.normal(size=dff) * 0.1 if bias else None,
        w_down=g.normal(size=(d, dff)) / math.sqrt(dff), b_down=g.normal(size=d) * 0.1 if bias else None)


def pin_brute_force(mod):
    Hw = rng.normal(size=(2, 3, 4))
    Hs = rng.normal(size=(2, 5, 4))
    A = mod.cross_attention(Hw, Hs)
    for b in range(2):
        ref = np.array(WH.brute_force_attention(Hw[b], Hs[b]))
        assert np.max(np.abs(A[b] - ref)) <= 1e-12


def pin_identical_keys(mod):
    v = rng.normal(size=6)
    Hs = np.tile(v, (1, 7, 1))
    Hw = rng.normal(size=(1, 4, 6))
    A = mod.cross_attention(Hw, Hs)
    assert np.allclose(A, np.tile(v, (1, 4, 1)), atol=1e-12)


def pin_mean_pooling(mod):
    Hs = rng.normal(size=(1, 9, 5))
    A = mod.cross_attention(np.zeros((1, 3, 5)), Hs)  # all logits 0: uniform weights
    assert np.allclose(A, np.tile(Hs.mean(axis=1), (1, 3, 1)), atol=1e-12)


def pin_dominant_key(mod):
    Hs = np.zeros((1, 4, 4))
    Hs[0, 2, 0] = 40.0  # the only key aligned with the query
    Hs[0, 0, 1] = Hs[0, 1, 2] = Hs[0, 3, 3] = 1.0
    Hw = np.zeros((1, 1, 4))
    Hw[0, 0, 0] = 1.0
    A = mod.cross_attention(Hw, Hs)  # logit 20 vs 0: weight 1 - 3e^-20
    assert np.allclose(A[0, 0], Hs[0, 2], atol=1e-6)


def pin_two_key_closed_form(mod):
    # d = 4, query (1, 0, 0, 0), keys k1 = (2, 1, 0, 0), k2 = (0, 0, 1, 0): logits 2/2 = 1 and 0
    Hw = np.array([[[1.0, 0, 0, 0]]])
    Hs = np.array([[[2.0, 1, 0, 0], [0, 0, 1.0, 0]]])
    p1 = math.e / (math.e + 1.0)
    want = p1 * Hs[0, 0] + (1 - p1) * Hs[0, 1]
    assert np.allclose(mod.cross_attention(Hw, Hs)[0, 0], want, atol=1e-14)


def pin_silu(mod):
    ln3 = math.log(3.0)
    assert mod.silu(np.array(0.0)) == 0.0
    assert abs(mod.silu(np.array(ln3)) - 0.75 * ln3) < 1e-15
    assert abs(mod.silu(np.array(-ln3)) + 0.25 * ln3) < 1e-15
    assert np.isfinite(mod.silu(np.array([-1000.0, 1000.0]))).all()


def _one_layer_case(mod, w, d=4, n=2, L=3, seed=1, eps=WH.LN_EPS):
    g = np.random.default_rng(seed)
    Hw = g.normal(size=(2, n, d))
    Hs = g.normal(size=(2, L, d))
    return Hw, Hs, mod.whale_fusion(Hw, Hs, w, eps=eps, intermediates=True)


def pin_concat_order(mod):
    d = 4
    w = _w(d, 16, bias=False)
    w.w_f = np.concatenate([np.eye(d), np.zeros((d, d))], axis=1)  # reads H_w only
    Hw, Hs, (_, it) = _one_layer_case(mod, w, d)
    assert np.allclose(it["Q"], Hw, atol=1e-14)
    w.w_f = np.concatenate([np.zeros((d, d)), np.eye(d)], axis=1)  # reads the attention output only
    Hw, Hs, (_, it) = _one_layer_case(mod, w, d)
    assert np.allclose(it["Q"], WH.cross_attention(Hw, Hs), atol=1e-14)


def pin_shared_gate(mod):
    d, dff = 4, 8
    w = _w(d, dff)
    Hw, Hs, (Hf, it) = _one_layer_case(mod, w, d)
    U = WH.layer_norm(it["Q"], w.gamma, w.beta) @ w.w_up.T + w.b_up
    assert np.allclose(it["G"], U * U / (1 + np.exp(-U)), atol=1e-13)


def pin_residual_and_down_bias(mod):
    d, dff = 4, 8
    w = _w(d, dff)
    w.w_down = np.zeros((d, dff))
    Hw, Hs, (Hf, it) = _one_layer_case(mod, w, d)
    assert np.allclose(Hf, it["Q"] + w.b_down, atol=1e-14)


def pin_prenorm(mod):
    d, dff = 4, 8
    w = _w(d, dff, bias=False)
    Hw, Hs, (Hf1, it1) = _one_layer_case(mod, w, d, eps=0.0)
    w2 = types.SimpleNamespace(**vars(w))
    w2.w_f = 3.0 * w.w_f  # Q -> 3Q; with eps = 0 the FFN branch sees LN(3Q) = LN(Q)
    Hw, Hs, (Hf2, it2) = _one_layer_case(mod, w2, d, eps=0.0)
    assert np.allclose(Hf2 - it2["Q"], Hf1 - it1["Q"], atol=1e-12)
    assert np.allclose(it2["Q"], 3.0 * it1["Q"], atol=1e-13)


PINS = {f.__name__: f for f in (pin_brute_force, pin_identical_keys, pin_mean_pooling, pin_dominant_key,
                                 pin_two_key_closed_form, pin_silu, pin_concat_order, pin_shared_gate,
                                 pin_residual_and_down_bias, pin_prenorm)}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    PINS[name](WH)


def test_storage_rounding_names():
    with pytest.raises(ValueError):
        WH.whale_fusion(np.zeros((1, 1, 2)), np.zeros((1, 1, 2)), _w(2, 4), storage=("X",))
    Hw = rng.normal(size=(1, 2, 4))
    Hs = rng.normal(size=(1, 3, 4))
    out = WH.whale_fusion(Hw, Hs, _w(4, 8), storage=("Hf",))
    assert np.array_equal(out, WH.round_bf16(out))


MUTANTS = {
    "scale_missing": ("/ math.sqrt(d)\n    m = S", "\n    m = S"),
    "softmax_wrong_axis": ("den = E.sum(axis=-1, keepdims=True)", "den = E.sum(axis=-2, keepdims=True)"),
    "concat_swapped": ("C = np.concatenate([Hw, A], axis=-1)", "C = np.concatenate([A, Hw], axis=-1)"),
    "residual_dropped": ("Hf = _r(Q + D, \"Hf\", storage)", "Hf = _r(D, \"Hf\", storage)"),
    "layernorm_missing": ("Qn = _r(layer_norm(Q, w.gamma, w.beta, eps), \"Qn\", storage)", "Qn = Q"),
    "gate_not_shared": ("G = _r(silu(U) * U, \"G\", storage)", "G = _r(silu(U), \"G\", storage)"),
    "silu_sign": ("np.where(u >= 0, 1.0 / (1.0 + e), e / (1.0 + e))", "np.where(u >= 0, e / (1.0 + e), 1.0 / (1.0 + e))"),
    "down_bias_dropped": ("D = D + to_f64(w.b_down)", "D = D"),
    "values_unnormalised": ("return _r(num / den, \"A\", storage)", "return _r(num, \"A\", storage)"),
    "max_not_subtracted_wrongly": ("E = np.exp(S - m)", "E = np.exp(S - m) * (1 + 0.01 * (m - S))"),
}


def make_mutant(old, new):
    src = open(WH.__file__).read()
    assert src.count(old) == 1, old
    src = src.replace(old, new).replace("from .wukong_oracle import", "from oracle.wukong_oracle import")
    mod = types.ModuleType("whale_oracle_mutant")
    mod.__file__ = WH.__file__
    exec(compile(src, "whale_oracle_mutant", "exec"), mod.__dict__)
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
