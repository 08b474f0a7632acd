"""Plain CPU oracle of the Wukong layer's backward pass (gradients of one layer).

TEST INFRASTRUCTURE ONLY, like the rest of `oracle/`: imported by the tests,
the package's smoke check and the benchmark's CPU-baseline leg, never by the
library; it imports nothing from the library.  fp64 numpy, one step per line.

What it differentiates: the layer of `wukong_oracle.wukong_layer` (Wukong
paper, section 2.2, as summarised on the xdnf.cn repost of the Zhihu
article), which the pages train end to end (same repost, experiment
dataset and training setup, section 3.2.1: the dense layers are trained with
Adam; WHALE technical summaries, section 2.2: bf16 dense backbone).
Given the upstream gradient dY = dLoss/dY of the layer output, it returns
dLoss/dX and the gradient of every weight, by the chain rule through the
forward's steps taken in reverse:

  9'. output LayerNorm, per row over d, with R_hat = (R - mu) * rstd:
        d_gamma_out = sum_{b,r} dY * R_hat,  d_beta_out = sum_{b,r} dY,
        dR = rstd * (g - mean_d(g) - R_hat * mean_d(g * R_hat)),  g = dY * gamma_out
  8'. R = [M; Lc] + X:  dM = dR[:n_F],  dLc = dR[n_F:],  dX gets dR (residual)
  7'. Lc = W_L X:  d_W_L = sum_b dLc X^T,  dX gets W_L^T dLc
  6'. M = reshape(h_T):  g_T = vec(dM)
  5'. Linear t (t = T-1 .. 0) with input a_t (a_0 = f_hat, a_t = h_t):
        d_W_t = sum_b g_{t+1} a_t^T,  d_b_t = sum_b g_{t+1},
        g_t = (W_t^T g_{t+1}) * [a_t > 0] for t > 0 (ReLU),  d_f_hat = W_0^T g_1
  4'. FM LayerNorm over the n*k values, f_tilde = (f - mu) * rstd:
        d_gamma_fm = sum_b d_f_hat * f_tilde,  d_beta_fm = sum_b d_f_hat,
        df = rstd * (q - mean(q) - f_tilde * mean(q * f_tilde)),  q = d_f_hat * gamma_fm
  3'. dF = reshape(df, n x k)
  2'. F = X Z^T with Z = Phi X:  dZ = dF^T X,  dX gets dF Z + Phi^T dZ,
        d_Phi = sum_b dZ X^T

Storage rounding: besides the forward's names (see `wukong_oracle`), the
backward may round to bf16 where it produces them: "dR" (the output
LayerNorm's input gradient, which then serves as dM, as dLc and as the
residual term of dX), "dh" (each g_t, t > 0), "dFn" (d_f_hat), "dF", "dZ"
and "dX" (the final input gradient).  A rounded Z is treated as Z itself by
the chain rule (the rounding has no derivative of its own).
"""
from __future__ import annotations

from typing import Dict, Iterable

import numpy as np

from .wukong_oracle import LN_EPS, STORAGE_NAMES, round_bf16, to_f64, wukong_layer

BACKWARD_STORAGE = frozenset({"dR", "dh", "dFn", "dF", "dZ", "dX"})


def _r(x: np.ndarray, name: str, storage) -> np.ndarray:
    return round_bf16(x) if name in storage else x


def _stats(v: np.ndarray, eps: float):
    """Mean and 1 / sqrt(biased variance + eps) over the last axis."""
    mu = v.mean(axis=-1, keepdims=True)
    var = ((v - mu) ** 2).mean(axis=-1, keepdims=True)
    return mu, 1.0 / np.sqrt(var + eps)


def layer_norm_backward(g_hat: np.ndarray, v_hat: np.ndarray, rstd: np.ndarray) -> np.ndarray:
    """Input gradient of LayerNorm over the last axis from the gradient of the
    normalised value g_hat = dLoss/dv_hat (affine scale already applied)."""
    m1 = g_hat.mean(axis=-1, keepdims=True)
    m2 = (g_hat * v_hat).mean(axis=-1, keepdims=True)
    return rstd * (g_hat - m1 - v_hat * m2)


def layer_backward(X, w, dY, eps: float = LN_EPS, storage: Iterable[str] = (),
                   intermediates: bool = False) -> Dict[str, object]:
    """Gradients of one Wukong layer for a batch X [S, n, d] and upstream dY [S, n, d].

    `w` is the forward's weight object (phi, w_l, fm_gamma, fm_beta, mlp_w,
    mlp_b, out_gamma, out_beta).  Returns a dict with "dX" [S, n, d], "phi"
    [k, n], "w_l" [n_L, n], "fm_gamma" / "fm_beta" [n k], "mlp_w" (list of
    [m_{t+1}, m_t]), "mlp_b" (list of [m_{t+1}]), "out_gamma" / "out_beta" [d],
    all float64 (a missing gamma / beta / bias still gets its gradient).
    With intermediates=True, "inter" holds dR, dM, the g_t, d_f_hat, dF, dZ.
    """
    storage = frozenset(storage)
    unknown = storage - STORAGE_NAMES - BACKWARD_STORAGE
    if unknown:
        raise ValueError(f"unknown storage names {sorted(unknown)}")
    fwd_storage = storage & STORAGE_NAMES
    X = to_f64(X)
    dY = to_f64(dY)
    S, n, d = X.shape
    phi = to_f64(w.phi)
    w_l = to_f64(w.w_l)
    k, n_l = phi.shape[0], w_l.shape[0]
    n_f = n - n_l
    _, it = wukong_layer(X, w, eps, fwd_storage, intermediates=True)

    # 9'. output LayerNorm
    R = it["R"]
    mu, rstd = _stats(R, eps)
    R_hat = (R - mu) * rstd
    g_out = 1.0 if w.out_gamma is None else to_f64(w.out_gamma)
    d_out_gamma = (dY * R_hat).sum(axis=(0, 1))
    d_out_beta = dY.sum(axis=(0, 1))
    dR = _r(layer_norm_backward(dY * g_out, R_hat, rstd), "dR", storage)

    # 8'. concatenation and residual
    dM = dR[:, :n_f, :]
    dLc = dR[:, n_f:, :]
    dX = dR.copy()

    # 7'. LCB
    d_w_l = np.einsum("bre,bme->rm", dLc, X)
    dX = dX + np.matmul(w_l.T, dLc)

    # 6'-5'. MLP, last Linear first
    T = len(w.mlp_w)
    acts = [it["Fn"]] + list(it["h"][:T - 1])      # a_0 .. a_{T-1}
    g = dM.reshape(S, n_f * d)
    d_mlp_w = [None] * T
    d_mlp_b = [None] * T
    gs = []
    for t in range(T - 1, -1, -1):
        W = to_f64(w.mlp_w[t])
        d_mlp_w[t] = g.T @ acts[t]
        d_mlp_b[t] = g.sum(axis=0)
        g = g @ W
        if t > 0:
            g = _r(g * (acts[t] > 0), "dh", storage)
            gs.append(g)
    d_fn = _r(g, "dFn", storage)

    # 4'. FM LayerNorm over the n*k values of each example
    f = it["F"].reshape(S, n * k)
    mu_f, rstd_f = _stats(f, eps)
    f_tilde = (f - mu_f) * rstd_f
    g_fm = 1.0 if w.fm_gamma is None else to_f64(w.fm_gamma)
    d_fm_gamma = (d_fn * f_tilde).sum(axis=0)
    d_fm_beta = d_fn.sum(axis=0)
    df = layer_norm_backward(d_fn * g_fm, f_tilde, rstd_f)

    # 3'-2'. interaction and compression
    dF = _r(df.reshape(S, n, k), "dF", storage)
    Z = it["Z"]                                      # bf16 when the forward rounded it
    dZ = _r(np.matmul(np.swapaxes(dF, 1, 2), X), "dZ", storage)   # [S, k, d]
    dX = dX + np.matmul(dF, Z) + np.matmul(phi.T, dZ)
    d_phi = np.einsum("bje,bme->jm", dZ, X)
    dX = _r(dX, "dX", storage)

    out = {"dX": dX, "phi": d_phi, "w_l": d_w_l, "fm_gamma": d_fm_gamma, "fm_beta": d_fm_beta,
           "mlp_w": d_mlp_w, "mlp_b": d_mlp_b, "out_gamma": d_out_gamma, "out_beta": d_out_beta}
    if intermediates:
        out["inter"] = {"dR": dR, "dM": dM, "g": gs[::-1], "dFn": d_fn, "dF": dF, "dZ": dZ}
    return out


def layer_loss(X, w, dY, eps: float = LN_EPS) -> float:
    """The scalar sum(dY * layer(X)) whose gradient `layer_backward` returns (fp64, no rounding)."""
    return float((to_f64(dY) * wukong_layer(X, w, eps)).sum())


def stack_backward(X, weights, dY, eps: float = LN_EPS, storage: Iterable[str] = ()):
    """Gradients of l stacked layers (the forward of `wukong_oracle.wukong_stack`):
    the forward keeps every layer's input X_i (rounded to bf16 when "Y" is in
    storage, as the layer output it is), then `layer_backward` runs from the
    last layer to the first, each layer's dX being the upstream gradient of the
    layer before it.  Returns (dX, [per-layer gradient dicts, layer order])."""
    storage = frozenset(storage)
    xs = [to_f64(X)]
    for w in weights[:-1]:
        xs.append(wukong_layer(xs[-1], w, eps, storage & STORAGE_NAMES))
    g = to_f64(dY)
    grads = [None] * len(weights)
    for i in range(len(weights) - 1, -1, -1):
        out = layer_backward(xs[i], weights[i], g, eps, storage)
        grads[i] = out
        g = out["dX"]
    return g, grads


def stack_loss(X, weights, dY, eps: float = LN_EPS) -> float:
    """sum(dY * stack(X)) in fp64 without rounding: the scalar `stack_backward` differentiates."""
    Y = to_f64(X)
    for w in weights:
        Y = wukong_layer(Y, w, eps)
    return float((to_f64(dY) * Y).sum())
