"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin is a function of the oracle module, so the same pins also run
against deliberately broken copies of the oracle (source-level mutants
planted on the CPU, see test_mutant_is_caught): every plausible mistake
listed there -- a dropped term, a wrong index or order, a transposed operand,
a wrong rounding -- must make at least one pin fail.

What pins what:
  * FM interaction: explicit pairwise dot products on tiny inputs (brute
    force), Phi = identity-row selection returning columns of the symmetric
    Gram matrix, the rank-1 closed form, exact c^2 scaling;
  * LayerNorm: the closed form of a hand row, per-vector mean 0 / variance
    sigma^2/(sigma^2+eps);
  * MLP: one-hot inputs returning weight columns, ReLU with identity weights;
  * LCB: row selection returning rows of X, linearity;
  * concat / reshape / residual: index-tagged biases with zero weights, and
    the residual-only reduction to a row LayerNorm of X;
  * the whole layer: a hand-derived 3x3 worked example (tests/golden) and an
    explicit-loop brute force on tiny inputs;
  * the stack: composition of single layers and batch independence;
  * bf16 rounding: torch's float32 -> bfloat16 conversion (round to nearest
    even) as an independent library routine;
  * the prediction head: explicit loops on tiny inputs, the logistic
    function's closed forms (sigmoid(ln 3) = 3/4, sigmoid(0) = 1/2), one-hot
    weights reading single elements of Y (row-major flatten), ReLU placement
    by sign-controlled hidden layers, and the symmetry sigmoid(-z) = 1 - sigmoid(z).
"""
import json
import os
import types

import numpy as np
import pytest

import oracle.wukong_oracle as WO

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class W:
    """Duck-typed layer weights."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def rand_weights(rng, n, d, k, n_f, n_l, hidden=(), affine=True):
    mlp = [n * k, *hidden, n_f * d]
    mlp_w = [rng.uniform(-1, 1, (b, a)) / np.sqrt(a) for a, b in zip(mlp[:-1], mlp[1:])]
    mlp_b = [rng.uniform(-0.5, 0.5, b) for b in mlp[1:]]
    if affine:
        fg, fb = rng.uniform(0.5, 1.5, n * k), rng.uniform(-0.5, 0.5, n * k)
        og, ob = rng.uniform(0.5, 1.5, d), rng.uniform(-0.5, 0.5, d)
    else:
        fg = fb = og = ob = None
    return W(phi=rng.standard_normal((k, n)) / np.sqrt(n), w_l=rng.standard_normal((n_l, n)) / np.sqrt(n),
             fm_gamma=fg, fm_beta=fb, mlp_w=mlp_w, mlp_b=mlp_b, out_gamma=og, out_beta=ob)


def gram_loops(x):
    n, d = x.shape
    g = np.zeros((n, n))
    for i in range(n):
        for m in range(n):
            s = 0.0
            for e in range(d):
                s += x[i, e] * x[m, e]
            g[i, m] = s
    return g


def standardize_rows(a, eps):
    out = np.empty_like(a, dtype=np.float64)
    for idx in np.ndindex(a.shape[:-1]):
        row = a[idx]
        m = sum(row) / len(row)
        v = sum((t - m) ** 2 for t in row) / len(row)
        out[idx] = [(t - m) / (v + eps) ** 0.5 for t in row]
    return out


# ------------------------------------------------------------------------- pins
def pin_fm_brute_force(wo):
    rng = np.random.default_rng(1)
    for S, n, d, k in [(2, 5, 3, 2), (1, 4, 4, 4), (3, 7, 2, 3)]:
        X = rng.standard_normal((S, n, d))
        phi = rng.standard_normal((k, n))
        F = wo.fm_interaction(X, phi)
        assert F.shape == (S, n, k)
        for s in range(S):
            g = gram_loops(X[s])
            for i in range(n):
                for j in range(k):
                    ref = 0.0
                    for m in range(n):
                        ref += phi[j, m] * g[i, m]
                    assert abs(F[s, i, j] - ref) <= 1e-12 * max(1.0, abs(ref))
    # small integers: Z = Phi X is exact in bf16, so the Z-first rounded form agrees exactly
    Xi = rng.integers(-3, 4, (2, 6, 4)).astype(np.float64)
    phii = rng.integers(-2, 3, (3, 6)).astype(np.float64)
    F1 = wo.fm_interaction(Xi, phii)
    F2 = wo.fm_interaction(Xi, phii, storage={"Z"})
    for s in range(2):
        g = gram_loops(Xi[s])
        assert np.array_equal(F1[s], g @ phii.T)
    assert np.array_equal(F1, F2)


def pin_gram_columns(wo):
    rng = np.random.default_rng(2)
    X = rng.standard_normal((2, 6, 4))
    sel = [4, 0, 2, 2]
    phi = np.zeros((len(sel), 6))
    for j, s in enumerate(sel):
        phi[j, s] = 1.0
    F = wo.fm_interaction(X, phi)
    for b in range(2):
        g = gram_loops(X[b])
        for j, s in enumerate(sel):
            assert np.allclose(F[b, :, j], g[:, s], rtol=0, atol=1e-12)
    # k = n and Phi = I: F is the Gram matrix itself
    F = wo.fm_interaction(X, np.eye(6))
    for b in range(2):
        assert np.allclose(F[b], F[b].T, atol=1e-12)
        assert np.linalg.eigvalsh(F[b]).min() > -1e-10
        assert np.allclose(np.diag(F[b]), (X[b] ** 2).sum(axis=1), atol=1e-12)


def pin_rank1(wo):
    rng = np.random.default_rng(3)
    a, v = rng.standard_normal(5), rng.standard_normal(3)
    phi = rng.standard_normal((2, 5))
    X = np.outer(a, v)[None]
    F = wo.fm_interaction(X, phi)[0]
    ref = (v @ v) * np.outer(a, phi @ a)
    assert np.allclose(F, ref, rtol=1e-12, atol=1e-12)


def pin_scaling(wo):
    rng = np.random.default_rng(4)
    X = rng.standard_normal((3, 6, 5))
    phi = rng.standard_normal((3, 6))
    assert np.array_equal(wo.fm_interaction(2.0 * X, phi), 4.0 * wo.fm_interaction(X, phi))
    # LN(F) is scale invariant up to eps: the FMB half of the layer ignores X -> cX
    w = rand_weights(rng, 6, 5, 3, 3, 3, hidden=(7,))
    _, a = wo.wukong_layer(X, w, intermediates=True)
    _, b = wo.wukong_layer(3.0 * X, w, intermediates=True)
    assert np.allclose(a["Fn"], b["Fn"], atol=1e-5)
    assert np.allclose(a["M"], b["M"], atol=1e-4)


def pin_ln_golden(wo):
    with open(os.path.join(GOLDEN, "ln_row_1234.json")) as f:
        g = json.load(f)
    y = wo.layer_norm(np.array(g["x"]), None, None, eps=g["eps"])
    assert np.allclose(y, g["y"], rtol=0, atol=1e-14)


def pin_ln_stats(wo):
    rng = np.random.default_rng(5)
    eps = 1e-5
    v = rng.standard_normal((4, 37)) * rng.uniform(0.01, 3, (4, 1)) + rng.uniform(-5, 5, (4, 1))
    y = wo.layer_norm(v, None, None, eps)
    var = v.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-12)
    assert np.allclose(y.var(axis=1), var / (var + eps), rtol=1e-12)
    g, b = rng.uniform(0.5, 2, 37), rng.uniform(-1, 1, 37)
    assert np.allclose(wo.layer_norm(v, g, b, eps), y * g + b, atol=1e-12)
    # inside a layer: Fn over n*k values per example and Y over d per row
    X = rng.standard_normal((2, 6, 5))
    w = rand_weights(rng, 6, 5, 3, 2, 4, hidden=(9,), affine=False)
    Y, it = wo.wukong_layer(X, w, eps=eps, intermediates=True)
    f = it["F"].reshape(2, -1)
    assert np.allclose(it["Fn"].mean(axis=1), 0, atol=1e-12)
    assert np.allclose(it["Fn"].var(axis=1), f.var(axis=1) / (f.var(axis=1) + eps), rtol=1e-10)
    rv = it["R"].var(axis=2)
    assert np.allclose(Y.mean(axis=2), 0, atol=1e-12)
    assert np.allclose(Y.var(axis=2), rv / (rv + eps), rtol=1e-10)


def pin_worked_layer(wo):
    with open(os.path.join(GOLDEN, "worked_layer_n3_d3.json")) as f:
        g = json.load(f)
    arr = lambda key: np.array(g[key], dtype=np.float64)  # noqa: E731
    w = W(phi=arr("phi"), w_l=arr("w_l"), fm_gamma=arr("fm_gamma"), fm_beta=arr("fm_beta"),
          mlp_w=[np.array(m, dtype=np.float64) for m in g["mlp_w"]],
          mlp_b=[np.array(b, dtype=np.float64) for b in g["mlp_b"]],
          out_gamma=arr("out_gamma"), out_beta=arr("out_beta"))
    Y, it = wo.wukong_layer(arr("X")[None], w, eps=g["eps"], intermediates=True)
    e = g["expected"]
    assert np.allclose(it["F"][0], e["F"], atol=1e-12)
    assert np.allclose(it["Fn"][0], e["Fn"], atol=1e-12)
    assert np.allclose(it["h"][0][0], e["h1"], atol=1e-12)
    assert np.allclose(it["M"][0], e["M"], atol=1e-12)
    assert np.allclose(it["L"][0], e["L"], atol=1e-12)
    assert np.allclose(Y[0], e["Y"], atol=1e-12)
    assert np.allclose(wo.brute_force_layer(arr("X"), w, eps=g["eps"]), e["Y"], atol=1e-12)


def pin_layer_brute_force(wo):
    rng = np.random.default_rng(6)
    for (n, d, k, n_f, hidden, affine) in [(4, 3, 2, 2, (), True), (5, 2, 3, 3, (6,), True),
                                           (6, 4, 2, 1, (5, 3), False), (3, 5, 1, 2, (4,), True)]:
        w = rand_weights(rng, n, d, k, n_f, n - n_f, hidden, affine)
        X = rng.standard_normal((2, n, d))
        Y = wo.wukong_layer(X, w)
        for s in range(2):
            assert np.allclose(Y[s], wo.brute_force_layer(X[s], w), rtol=1e-10, atol=1e-10)


def pin_mlp_onehot(wo):
    rng = np.random.default_rng(7)
    W1, b1 = rng.standard_normal((5, 4)), rng.standard_normal(5)
    out = wo.fmb_mlp(np.eye(4), [W1], [b1])
    for j in range(4):
        assert np.allclose(out[j], W1[:, j] + b1, atol=1e-14)
    x = rng.standard_normal((3, 4))
    out = wo.fmb_mlp(x, [np.eye(4), np.eye(4)], [np.zeros(4), np.zeros(4)])
    assert np.array_equal(out, np.maximum(x, 0))
    # a two-layer MLP with a negative pre-activation: explicit loops
    W2, b2 = rng.standard_normal((3, 5)), rng.standard_normal(3)
    h = wo.fmb_mlp(x, [W1, W2], [b1, b2])
    for s in range(3):
        hid = [max(sum(W1[o, i] * x[s, i] for i in range(4)) + b1[o], 0.0) for o in range(5)]
        ref = [sum(W2[o, i] * hid[i] for i in range(5)) + b2[o] for o in range(3)]
        assert np.allclose(h[s], ref, atol=1e-12)


def pin_lcb(wo):
    rng = np.random.default_rng(8)
    X1, X2 = rng.standard_normal((2, 6, 3)), rng.standard_normal((2, 6, 3))
    sel = [5, 1, 1, 0]
    wl = np.zeros((4, 6))
    for r, s in enumerate(sel):
        wl[r, s] = 1.0
    assert np.array_equal(wo.lcb(X1, wl), X1[:, sel, :])
    wl = rng.standard_normal((4, 6))
    assert np.allclose(wo.lcb(X1 + X2, wl), wo.lcb(X1, wl) + wo.lcb(X2, wl), atol=1e-12)
    assert np.allclose(wo.lcb(X1, wl)[1, 2, 1], sum(wl[2, m] * X1[1, m, 1] for m in range(6)), atol=1e-12)


def pin_concat_order(wo):
    """Zero X and zero weights leave M = b_T: tags show the reshape and concat order."""
    n, d, k, n_f = 5, 4, 2, 2
    eps = 1e-5
    rng = np.random.default_rng(9)
    tags = np.arange(n_f * d, dtype=np.float64) ** 1.5 - 3.0
    w = W(phi=rng.standard_normal((k, n)), w_l=np.zeros((n - n_f, n)), fm_gamma=None, fm_beta=None,
          mlp_w=[rng.standard_normal((7, n * k)), np.zeros((n_f * d, 7))],
          mlp_b=[rng.standard_normal(7), tags], out_gamma=None, out_beta=None)
    Y = wo.wukong_layer(np.zeros((1, n, d)), w, eps=eps)[0]
    ref_rows = standardize_rows(tags.reshape(n_f, d), eps)  # row r = tags[r*d:(r+1)*d]
    assert np.allclose(Y[:n_f], ref_rows, atol=1e-12)
    assert np.array_equal(Y[n_f:], np.zeros((n - n_f, d)))


def pin_residual_only(wo):
    """W_L = 0, W_T = 0, b_T = 0: Y is the row LayerNorm of X itself."""
    rng = np.random.default_rng(10)
    n, d, k, n_f = 6, 5, 2, 4
    eps = 1e-5
    w = W(phi=rng.standard_normal((k, n)), w_l=np.zeros((n - n_f, n)), fm_gamma=None, fm_beta=None,
          mlp_w=[rng.standard_normal((3, n * k)), np.zeros((n_f * d, 3))],
          mlp_b=[rng.standard_normal(3), np.zeros(n_f * d)], out_gamma=None, out_beta=None)
    X = rng.standard_normal((2, n, d)) * 3 + 1
    assert np.allclose(wo.wukong_layer(X, w, eps=eps), standardize_rows(X, eps), atol=1e-12)


def pin_stack(wo):
    rng = np.random.default_rng(11)
    w1 = rand_weights(rng, 6, 4, 2, 3, 3, (5,))
    w2 = rand_weights(rng, 6, 4, 3, 2, 4, (4, 3))
    X = rng.standard_normal((5, 6, 4))
    Y = wo.wukong_stack(X, [w1, w2])
    assert np.allclose(Y, wo.wukong_layer(wo.wukong_layer(X, w1), w2), atol=1e-13)
    perm = np.array([3, 0, 4, 1, 2])
    assert np.allclose(wo.wukong_stack(X[perm], [w1, w2]), Y[perm], atol=1e-13)
    assert np.allclose(wo.wukong_stack(X[1:3], [w1, w2]), Y[1:3], atol=1e-13)


def pin_bf16_rounding(wo):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-6, 6, 20000).astype(np.float32),
        # exact ties between two bf16 neighbours, odd and even lower neighbour
        (np.float32(1.0) + np.float32(2.0 ** -8) * np.arange(1, 64, 2, dtype=np.float32)),
        -(np.float32(3.0) + np.float32(2.0 ** -7) * np.arange(1, 64, 2, dtype=np.float32)),
        np.array([0.0, -0.0, 1.0, 65504.0, 3.0e38, 1e-30], dtype=np.float32),
    ])
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    got = wo.round_bf16(vals.astype(np.float64))
    assert np.array_equal(got, ref)
    bits = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wo.decode_bf16(bits), ref)


def pin_storage_points(wo):
    rng = np.random.default_rng(13)
    w = rand_weights(rng, 8, 6, 3, 4, 4, (10,))
    X = wo.round_bf16(rng.standard_normal((3, 8, 6)))
    full = frozenset({"Z", "Fn", "h", "M", "L", "Y"})
    Y, it = wo.wukong_layer(X, w, storage=full, intermediates=True)
    for name in ("Z", "Fn", "M", "L", "Y"):
        a = it[name]
        assert np.array_equal(wo.round_bf16(a), a), name
    assert np.array_equal(wo.round_bf16(it["h"][0]), it["h"][0])
    Y64 = wo.wukong_layer(X, w)
    assert np.max(np.abs(Y - Y64)) < 0.1
    assert not np.array_equal(Y, Y64)


def _head_weights(rng, dims):
    ws = [rng.standard_normal((dims[t + 1], dims[t])) / np.sqrt(dims[t]) for t in range(len(dims) - 1)]
    bs = [rng.standard_normal(dims[t + 1]) * 0.3 for t in range(len(dims) - 1)]
    return ws, bs


def pin_head_brute_force(wo):
    rng = np.random.default_rng(41)
    Y = rng.standard_normal((3, 3, 4))
    ws, bs = _head_weights(rng, [12, 7, 5, 2])
    p = wo.prediction_head(Y, ws, bs)
    for s_ in range(3):
        np.testing.assert_allclose(p[s_], wo.brute_force_head(Y[s_], ws, bs), rtol=1e-12, atol=1e-14)


def pin_head_sigmoid_closed_form(wo):
    # zero weights: the prediction is the logistic function of the bias alone
    Y = np.random.default_rng(42).standard_normal((2, 2, 3))
    ws = [np.zeros((3, 6)), np.zeros((3, 3))]
    bs = [np.zeros(3), np.array([np.log(3.0), 0.0, -np.log(3.0)])]
    p = wo.prediction_head(Y, ws, bs)
    np.testing.assert_allclose(p, [[0.75, 0.5, 0.25]] * 2, rtol=0, atol=1e-15)


def pin_head_flatten_order(wo):
    # one Linear whose rows are one-hot at r*d + e: the logits are Y[r, e]
    Y = np.arange(24, dtype=np.float64).reshape(2, 3, 4) / 24.0 - 0.4
    picks = [(0, 1), (2, 0), (1, 3)]
    W = np.zeros((3, 12))
    for o, (r, e) in enumerate(picks):
        W[o, r * 4 + e] = 1.0
    _, z = wo.prediction_head(Y, [W], [None], logits=True)
    np.testing.assert_array_equal(z, np.stack([[Y[s_, r, e] for r, e in picks] for s_ in range(2)]))


def pin_head_relu_placement(wo):
    # a hidden layer of -I on positive inputs is all zero after ReLU: only the last bias is left;
    # +I passes the inputs through; the last Linear gets no ReLU (a negative logit survives)
    Y = np.abs(np.random.default_rng(43).standard_normal((2, 2, 2))) + 0.1
    v = Y.reshape(2, 4)
    w2 = np.array([[1.0, -2.0, 0.5, 1.5]])
    _, z = wo.prediction_head(Y, [-np.eye(4), w2], [None, np.array([-0.7])], logits=True)
    np.testing.assert_allclose(z, np.full((2, 1), -0.7), rtol=0, atol=1e-15)
    _, z = wo.prediction_head(Y, [np.eye(4), -np.abs(w2)], [None, None], logits=True)
    np.testing.assert_allclose(z[:, 0], -(v @ np.abs(w2[0])), rtol=1e-14)


def pin_head_symmetry(wo):
    rng = np.random.default_rng(44)
    Y = rng.standard_normal((3, 2, 5))
    ws, bs = _head_weights(rng, [10, 6, 3])
    p = wo.prediction_head(Y, ws, bs)
    q = wo.prediction_head(Y, ws[:-1] + [-ws[-1]], bs[:-1] + [-bs[-1]])
    np.testing.assert_allclose(p + q, np.ones_like(p), rtol=0, atol=1e-14)


PINS = {name[4:]: fn for name, fn in list(globals().items()) if name.startswith("pin_")}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    PINS[name](WO)


# --------------------------------------------------------------- planted mistakes
# (old text, new text) edits of the oracle's source, each a plausible slip.
MUTANTS = {
    "gram_other_example": ("G = np.matmul(X, np.swapaxes(X, 1, 2))", "G = np.matmul(X, np.swapaxes(X[::-1], 1, 2))"),
    "phi_not_transposed": ("return np.matmul(G, phi.T)", "return np.matmul(G, phi.T[::-1])"),
    "fm_z_wrong_operand": ("return np.matmul(X, np.swapaxes(Z, 1, 2))", "return np.matmul(X[:, ::-1], np.swapaxes(Z, 1, 2))"),
    "flatten_col_major": ("f = F.reshape(S, n * k)", "f = np.swapaxes(F, 1, 2).reshape(S, n * k)"),
    "reshape_col_major": ("M = h.reshape(S, n_f, d)", "M = np.swapaxes(h.reshape(S, d, n_f), 1, 2)"),
    "concat_swapped": ("np.concatenate([M, Lc], axis=1) + X", "np.concatenate([Lc, M], axis=1) + X"),
    "residual_dropped": ("R = np.concatenate([M, Lc], axis=1) + X", "R = np.concatenate([M, Lc], axis=1)"),
    "relu_on_last": ("if t < T - 1:", "if True:"),
    "relu_missing": ("h = np.maximum(h, 0.0)", "h = h"),
    "bias_dropped": ("h = h + to_dtype(mlp_b[t], h.dtype)", "h = h"),
    "ln_unbiased": ("var = ((v - mu) ** 2).mean(axis=-1, keepdims=True)",
                    "var = ((v - mu) ** 2).sum(axis=-1, keepdims=True) / (v.shape[-1] - 1)"),
    "ln_eps_outside": ("out = (v - mu) / np.sqrt(var + eps)", "out = (v - mu) / (np.sqrt(var) + eps)"),
    "ln_beta_dropped": ("out = out + to_dtype(beta, out.dtype)", "out = out"),
    "lcb_row_shift": ("return np.matmul(w_l, X)", "return np.matmul(w_l, np.roll(X, 1, axis=1))"),
    "fm_ln_skipped": ("f_hat = layer_norm(f, w.fm_gamma, w.fm_beta, eps)", "f_hat = f"),
    "out_ln_over_rows": ("Y = layer_norm(R, w.out_gamma, w.out_beta, eps)",
                         "Y = np.swapaxes(layer_norm(np.swapaxes(R, 1, 2), None, None, eps), 1, 2)"),
    "bf16_7_bits": ("return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)", "return np.ldexp(np.round(np.ldexp(m, 7)), e - 7)"),
    "bf16_truncate": ("return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)", "return np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)"),
    "bf16_decode_shift": ("(b.astype(np.uint32) << np.uint32(16))", "(b.astype(np.uint32) << np.uint32(15))"),
    "head_flatten_col_major": ("v = Y.reshape(S, -1)", "v = np.swapaxes(Y, 1, 2).reshape(S, -1)"),
    "head_relu_on_last": ("if t + 1 < T:", "if True:"),
    "head_relu_missing": ("v = np.maximum(v, 0.0)", "v = v"),
    "head_bias_dropped": ("v = v + to_f64(head_b[t])", "v = v"),
    "head_sigmoid_sign": ("out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))", "out[pos] = 1.0 / (1.0 + np.exp(z[pos]))"),
}


def make_mutant(old, new):
    with open(WO.__file__) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = WO.__file__
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(mutant):
    mod = make_mutant(*MUTANTS[mutant])
    caught = []
    for name, pin in PINS.items():
        try:
            pin(mod)
        except Exception:  # an assertion or a shape error both expose the mistake
            caught.append(name)
    assert caught, f"no pin catches the planted mistake {mutant!r}"


def test_float32_timing_variant_follows_the_float64_oracle():
    """The float32 variant (used only to time the oracle in fp32) runs the same
    steps: on a d = 160 layer it agrees with the float64 oracle to float32
    rounding, and it refuses bf16 storage rounding, which is defined in float64."""
    import wukong_synth as ws

    cfg = ws.LAYER_D160.with_batch(3)
    w = ws.make_stack_weights(cfg, 2, "random")
    x = ws.make_input(cfg, 2)
    y64 = WO.wukong_stack(x, w)
    y32 = WO.wukong_stack(x, w, dtype=np.float32)
    assert y32.dtype == np.float32
    assert np.max(np.abs(y32 - y64)) / np.max(np.abs(y64)) < 1e-5
    with pytest.raises(ValueError):
        WO.wukong_stack(x, w, storage=("Y",), dtype=np.float32)
