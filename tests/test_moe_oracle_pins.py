"""Pins of the Wukong mixture-of-experts oracle against facts that do not come from it.

  * one expert whose rows cover the layer is exactly the single-layer oracle
    (itself pinned by test_oracle_pins);
  * each expert's FMB rows, with that expert placed first, equal the
    brute-force single layer (explicit loops) built from the expert's weights;
  * the LCB rows equal those of a single layer whose W_L stacks the experts';
  * swapping two experts swaps their row blocks of the pre-LayerNorm sum less X;
  * changing one expert's MLP changes only that expert's FMB rows.
Each planted mistake in MUTANTS must fail at least one pin.
"""
import math
import types

import numpy as np
import pytest

import oracle.wukong_moe_oracle as MO
from oracle.wukong_oracle import brute_force_layer, wukong_layer


def _expert(n, d, k, n_f, n_l, hidden, seed):
    g = np.random.default_rng(seed)
    dims = [n * k] + list(hidden) + [n_f * d]
    return types.SimpleNamespace(
        phi=g.normal(size=(k, n)) / math.sqrt(n), w_l=g.normal(size=(n_l, n)) / math.sqrt(n),
        fm_gamma=1 + 0.2 * g.normal(size=n * k), fm_beta=0.2 * g.normal(size=n * k),
        mlp_w=[g.normal(size=(dims[t + 1], dims[t])) / math.sqrt(dims[t]) for t in range(len(dims) - 1)],
        mlp_b=[0.3 * g.normal(size=dims[t + 1]) for t in range(len(dims) - 1)])


def _case(seed=0, S=3, n=10, d=4):
    # three experts: (k, n_F, n_L) = (2, 2, 1), (3, 3, 2), (1, 1, 1): rows 6 + 4 = 10 = n
    shapes = [(2, 2, 1, (5,)), (3, 3, 2, (6, 4)), (1, 1, 1, (3,))]
    experts = [_expert(n, d, k, nf, nl, hid, seed + 10 * i) for i, (k, nf, nl, hid) in enumerate(shapes)]
    g = np.random.default_rng(seed + 100)
    X = g.normal(size=(S, n, d))
    og, ob = 1 + 0.2 * g.normal(size=d), 0.2 * g.normal(size=d)
    return X, experts, og, ob


def pin_single_expert(mod):
    n, d = 8, 4
    e = _expert(n, d, 3, 5, 3, (7,), seed=1)
    g = np.random.default_rng(2)
    X = g.normal(size=(2, n, d))
    og, ob = 1 + 0.2 * g.normal(size=d), 0.2 * g.normal(size=d)
    layer = types.SimpleNamespace(**vars(e), out_gamma=og, out_beta=ob)
    assert np.allclose(mod.wukong_moe_layer(X, [e], og, ob), wukong_layer(X, layer), atol=1e-13)


def pin_each_expert_first_is_brute_force(mod):
    X, experts, og, ob = _case(seed=3, S=1)
    n, d = X.shape[1], X.shape[2]
    for i, e in enumerate(experts):
        order = [e] + experts[:i] + experts[i + 1:]
        Y = mod.wukong_moe_layer(X, order, og, ob)
        n_f = e.mlp_w[-1].shape[0] // d
        single = types.SimpleNamespace(**vars(e), out_gamma=og, out_beta=ob)
        single.w_l = np.zeros((n - n_f, n))  # an LCB of the remaining rows; only the FMB rows are compared
        ref = brute_force_layer(X[0], single)
        assert np.allclose(Y[0, :n_f], ref[:n_f], atol=1e-10), i


def pin_lcb_rows_stack(mod):
    X, experts, og, ob = _case(seed=4)
    n, d = X.shape[1], X.shape[2]
    n_f = sum(e.mlp_w[-1].shape[0] // d for e in experts)
    Y = mod.wukong_moe_layer(X, experts, og, ob)
    g = np.random.default_rng(5)
    k = 2
    single = types.SimpleNamespace(
        phi=g.normal(size=(k, n)), w_l=np.concatenate([e.w_l for e in experts]), fm_gamma=None, fm_beta=None,
        mlp_w=[g.normal(size=(n_f * d, n * k))], mlp_b=None, out_gamma=og, out_beta=ob)
    assert np.allclose(Y[:, n_f:], wukong_layer(X, single)[:, n_f:], atol=1e-13)


def pin_swap_experts(mod):
    X, experts, og, ob = _case(seed=6)
    d = X.shape[2]
    _, a = mod.wukong_moe_layer(X, experts, og, ob, intermediates=True)
    swapped = [experts[1], experts[0], experts[2]]
    _, b = mod.wukong_moe_layer(X, swapped, og, ob, intermediates=True)
    fa, fb = [e.mlp_w[-1].shape[0] // d for e in experts[:2]]
    la, lb = experts[0].w_l.shape[0], experts[1].w_l.shape[0]
    n_f = sum(e.mlp_w[-1].shape[0] // d for e in experts)
    ra, rb = a["R"] - X, b["R"] - X
    assert np.allclose(rb[:, :fb], ra[:, fa:fa + fb], atol=1e-13)
    assert np.allclose(rb[:, fb:fb + fa], ra[:, :fa], atol=1e-13)
    assert np.allclose(rb[:, n_f:n_f + lb], ra[:, n_f + la:n_f + la + lb], atol=1e-13)
    assert np.allclose(rb[:, n_f + lb:n_f + lb + la], ra[:, n_f:n_f + la], atol=1e-13)


def pin_expert_locality(mod):
    X, experts, og, ob = _case(seed=7)
    d = X.shape[2]
    Y1 = mod.wukong_moe_layer(X, experts, og, ob)
    changed = [experts[0], types.SimpleNamespace(**vars(experts[1])), experts[2]]
    changed[1].mlp_w = list(experts[1].mlp_w)
    changed[1].mlp_w[-1] = experts[1].mlp_w[-1] * 1.5
    Y2 = mod.wukong_moe_layer(X, changed, og, ob)
    f0, f1 = [e.mlp_w[-1].shape[0] // d for e in experts[:2]]
    diff = np.abs(Y1 - Y2).max(axis=(0, 2))
    assert diff[f0:f0 + f1].min() > 1e-6
    assert np.all(np.delete(diff, np.arange(f0, f0 + f1)) == 0)


PINS = {f.__name__: f for f in (pin_single_expert, pin_each_expert_first_is_brute_force, pin_lcb_rows_stack,
                                 pin_swap_experts, pin_expert_locality)}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    PINS[name](MO)


def test_row_count_checked():
    X, experts, og, ob = _case()
    with pytest.raises(ValueError):
        MO.wukong_moe_layer(X, experts[:2], og, ob)


MUTANTS = {
    "lcb_rows_first": ("np.concatenate(Ms + Ls, axis=1)", "np.concatenate(Ls + Ms, axis=1)"),
    "residual_dropped": ("R = np.concatenate(Ms + Ls, axis=1) + X", "R = np.concatenate(Ms + Ls, axis=1)"),
    "first_phi_for_all": ("phi = to_f64(w.phi)", "phi = to_f64(experts[0].phi)"),
    "expert_order_reversed": ("np.concatenate(Ms + Ls, axis=1)", "np.concatenate(Ms[::-1] + Ls[::-1], axis=1)"),
    "fm_layernorm_missing": ("layer_norm(F.reshape(S, n * k), w.fm_gamma, w.fm_beta, eps)", "F.reshape(S, n * k)"),
    "lcb_of_first_expert": ("Ls.append(lcb(X, to_f64(w.w_l)))", "Ls.append(lcb(X, to_f64(experts[0].w_l))[:, :to_f64(w.w_l).shape[0]])"),
}


def make_mutant(old, new):
    src = open(MO.__file__).read()
    assert src.count(old) == 1, old
    src = src.replace(old, new).replace("from .wukong_oracle import", "from oracle.wukong_oracle import")
    mod = types.ModuleType("moe_oracle_mutant")
    mod.__file__ = MO.__file__
    exec(compile(src, "moe_oracle_mutant", "exec"), mod.__dict__)
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
