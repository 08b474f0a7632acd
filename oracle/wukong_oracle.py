"""Plain CPU oracle of the stacked Wukong interaction layer (forward pass).

TEST INFRASTRUCTURE ONLY.  This module is the independent reference that the
HIP path is checked against.  Only the test suite, the package's smoke check
and the benchmark's CPU-baseline leg may import it; the library itself never
does, and this module imports nothing from the library.  It is deliberately
slow and literal: fp64 numpy, one step per line, no blocking or fusion.

What it computes (Wukong paper, section 2.2 "Wukong", as summarised on the
xdnf.cn repost of the Zhihu article; the page's equations were lost in
extraction, so the steps below follow its prose):

  A Wukong layer runs a Factorization Machine Block (FMB) and a Linear
  Compress Block (LCB) side by side on one example's feature matrix
  X in R^{n x d}, concatenates their outputs, adds the residual X and applies
  a LayerNorm.  The FMB "first compresses the number of features to k, then
  computes the interaction" and ends in an MLP whose output is an n_F x d
  matrix; the LCB multiplies X by a weight matrix W_L that maps the n input
  embeddings to n_L outputs.  Layers are stacked, each with its own weights
  (section 2.3 lists the knobs l, n_F, n_L, k and the MLP).

Per example and per layer, with every input exactly representable in fp64:
  1. G = X X^T                         all pairwise embedding dot products
  2. F = G Phi^T  (n x k)              the FM interaction compressed to k
                                       columns; equal to X (Phi X)^T
  3. f = vec(F) row-major              f[i*k + j] = F[i, j]
  4. f_hat = LN(f; gamma_fm, beta_fm)  over all n*k values, biased variance
  5. h_t = ReLU(W_t h_{t-1} + b_t) for t < T, h_T = W_T h_{T-1} + b_T
  6. M = reshape(h_T, n_F x d)         row-major
  7. Lc = W_L X  (n_L x d)
  8. R = [M; Lc] + X                   FMB rows first, then LCB rows
  9. Y[r] = LN(R[r]; gamma_out, beta_out) over d for each row r
 10. the next layer's X is Y.

Readings taken where the pages are silent (each is listed in the design
notes): Phi is a learned [k, n] weight shared by all examples; LayerNorm uses
eps = 1e-5 and the biased variance; ReLU follows every Linear but the last;
flatten and reshape are row-major; the FMB rows come before the LCB rows.

Storage rounding.  An implementation that keeps some intermediate tensors in
bf16 is compared against this oracle run with `storage` naming those tensors:
"Z" (Phi X, used as a product operand), "Fn" (the normalised interaction),
"h" (the hidden MLP activations), "M" (the last MLP output), "L" (the LCB
output) and "Y" (the layer output).  Each named tensor is rounded to the
nearest bf16 value (ties to even) right where it is produced; everything else
stays fp64.  When "Z" is named, step 2 is taken in its Z-first form
F = X bf16(Phi X)^T, because the rounded Z only exists in that order.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Sequence

import numpy as np

LN_EPS = 1e-5
STORAGE_NAMES = frozenset({"Z", "Fn", "h", "M", "L", "Y"})


# ---------------------------------------------------------------- number formats
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly.

    A bf16 value is the upper 16 bits of an IEEE-754 binary32 value.
    """
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("bf16 data must be passed as uint16 bit patterns")
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray) -> np.ndarray:
    """Host array (float32/float64, or uint16 bf16 bits) -> float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return decode_bf16(a)
    return a.astype(np.float64)


def to_dtype(a: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Host array (float32/float64, or uint16 bf16 bits) -> `dtype` (float64 by default)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return decode_bf16(a).astype(dtype, copy=False)
    return a.astype(dtype, copy=False)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits.  Writing x = m * 2**e with 0.5 <= |m| < 1,
    the rounded value is round_half_even(m * 2**8) * 2**(e - 8).  (Values in
    the bf16 subnormal range are not produced by this layer.)
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)  # np.round: half to even


def _maybe_round(x: np.ndarray, name: str, storage: Iterable[str]) -> np.ndarray:
    return round_bf16(x) if name in storage else x


# ---------------------------------------------------------------- building blocks
def layer_norm(v: np.ndarray, gamma, beta, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last axis: (v - mean) / sqrt(var + eps) * gamma + beta.

    var is the biased (population) variance.  gamma/beta of None mean 1/0.
    """
    mu = v.mean(axis=-1, keepdims=True)
    var = ((v - mu) ** 2).mean(axis=-1, keepdims=True)
    out = (v - mu) / np.sqrt(var + eps)
    if gamma is not None:
        out = out * to_dtype(gamma, out.dtype)
    if beta is not None:
        out = out + to_dtype(beta, out.dtype)
    return out


def fm_interaction(X: np.ndarray, phi: np.ndarray, storage: Iterable[str] = ()) -> np.ndarray:
    """FMB interaction F = (X X^T) Phi^T for a batch X [S, n, d]; returns [S, n, k].

    With "Z" in storage the compressed matrix Z = Phi X is formed and rounded
    to bf16 first, and F = X Z^T.
    """
    if "Z" in storage:
        Z = round_bf16(np.matmul(phi, X))                 # [S, k, d]
        return np.matmul(X, np.swapaxes(Z, 1, 2))          # [S, n, k]
    G = np.matmul(X, np.swapaxes(X, 1, 2))                 # [S, n, n]
    return np.matmul(G, phi.T)                              # [S, n, k]


def fmb_mlp(f_hat: np.ndarray, mlp_w: Sequence[np.ndarray], mlp_b: Sequence,
            storage: Iterable[str] = (), keep: List[np.ndarray] = None) -> np.ndarray:
    """h_t = ReLU(h_{t-1} W_t^T + b_t) for all but the last Linear; [S, m_0] -> [S, m_T]."""
    h = f_hat
    T = len(mlp_w)
    for t in range(T):
        W = to_dtype(mlp_w[t], h.dtype)
        h = h @ W.T
        if mlp_b is not None and mlp_b[t] is not None:
            h = h + to_dtype(mlp_b[t], h.dtype)
        if t < T - 1:
            h = np.maximum(h, 0.0)
            h = _maybe_round(h, "h", storage)
        else:
            h = _maybe_round(h, "M", storage)
        if keep is not None:
            keep.append(h)
        del W
    return h


def lcb(X: np.ndarray, w_l: np.ndarray) -> np.ndarray:
    """Linear Compress Block Lc = W_L X for a batch X [S, n, d]; returns [S, n_L, d]."""
    return np.matmul(w_l, X)


# ---------------------------------------------------------------- layer and stack
def wukong_layer(X, w, eps: float = LN_EPS, storage: Iterable[str] = (),
                 intermediates: bool = False, dtype=np.float64):
    """One Wukong layer on a batch X [S, n, d] (float32 / bf16 bits / float64).

    `w` carries phi [k,n], w_l [n_L,n], fm_gamma/fm_beta [n*k], mlp_w (list of
    [m_t, m_{t-1}]), mlp_b (list of [m_t]), out_gamma/out_beta [d]; any of the
    gamma/beta/bias entries may be None.  Returns Y [S, n, d] in float64, or
    (Y, dict of intermediates) when intermediates=True.

    dtype=np.float32 runs the same steps in float32 (a timing variant only: the
    parity reference is float64); storage rounding needs float64.
    """
    storage = frozenset(storage)
    unknown = storage - STORAGE_NAMES
    if unknown:
        raise ValueError(f"unknown storage names {sorted(unknown)}")
    if storage and dtype != np.float64:
        raise ValueError("storage rounding is defined on the float64 oracle")
    X = to_dtype(X, dtype)
    if X.ndim != 3:
        raise ValueError("X must be [batch, n, d]")
    S, n, d = X.shape
    phi = to_dtype(w.phi, dtype)
    w_l = to_dtype(w.w_l, dtype)
    k, n_l = phi.shape[0], w_l.shape[0]
    if phi.shape[1] != n or w_l.shape[1] != n:
        raise ValueError("Phi and W_L must have n columns")

    F = fm_interaction(X, phi, storage)                     # steps 1-2
    f = F.reshape(S, n * k)                                 # step 3
    f_hat = layer_norm(f, w.fm_gamma, w.fm_beta, eps)       # step 4
    f_hat = _maybe_round(f_hat, "Fn", storage)
    hs: List[np.ndarray] = []
    h = fmb_mlp(f_hat, w.mlp_w, w.mlp_b, storage, keep=hs)  # step 5
    if h.shape[1] % d != 0:
        raise ValueError("last MLP width must be a multiple of d")
    n_f = h.shape[1] // d
    if n_f + n_l != n:
        raise ValueError("the residual needs n_F + n_L == n")
    M = h.reshape(S, n_f, d)                                # step 6
    Lc = _maybe_round(lcb(X, w_l), "L", storage)            # step 7
    R = np.concatenate([M, Lc], axis=1) + X                 # step 8
    Y = layer_norm(R, w.out_gamma, w.out_beta, eps)         # step 9
    Y = _maybe_round(Y, "Y", storage)
    if not intermediates:
        return Y
    Z = np.matmul(phi, X)
    if "Z" in storage:
        Z = round_bf16(Z)
    return Y, {"Z": Z, "F": F, "Fn": f_hat, "h": hs, "M": M, "L": Lc, "R": R, "Y": Y}


def wukong_stack(X, weights: Sequence, eps: float = LN_EPS, storage: Iterable[str] = (), dtype=np.float64):
    """l stacked layers: X^(i+1) = wukong_layer(X^(i), weights[i]) (step 10)."""
    Y = to_dtype(X, dtype)
    for w in weights:
        Y = wukong_layer(Y, w, eps, storage, dtype=dtype)
    return Y


# ---------------------------------------------------------------- brute force
def brute_force_layer(X1, w, eps: float = LN_EPS) -> np.ndarray:
    """One layer for ONE example [n, d] with explicit Python loops (tiny inputs only).

    Every sum is written out: pairwise dot products <x_i, x_m>, their
    Phi-weighted combination, both LayerNorms, each MLP neuron, each LCB row.
    """
    X = to_f64(X1)
    n, d = X.shape
    phi, w_l = to_f64(w.phi), to_f64(w.w_l)
    k, n_l = phi.shape[0], w_l.shape[0]

    def dot(u, v):
        s = 0.0
        for a, b in zip(u, v):
            s += a * b
        return s

    def ln(vec, gamma, beta):
        m = sum(vec) / len(vec)
        var = sum((x - m) ** 2 for x in vec) / len(vec)
        g = [1.0] * len(vec) if gamma is None else list(to_f64(gamma))
        bb = [0.0] * len(vec) if beta is None else list(to_f64(beta))
        return [(x - m) / (var + eps) ** 0.5 * g[i] + bb[i] for i, x in enumerate(vec)]

    # pairwise interactions, compressed to k columns
    f = []
    for i in range(n):
        for j in range(k):
            s = 0.0
            for m in range(n):
                s += phi[j, m] * dot(X[i], X[m])
            f.append(s)
    h = ln(f, w.fm_gamma, w.fm_beta)
    T = len(w.mlp_w)
    for t in range(T):
        W = to_f64(w.mlp_w[t])
        b = None if (w.mlp_b is None or w.mlp_b[t] is None) else to_f64(w.mlp_b[t])
        out = []
        for o in range(W.shape[0]):
            s = dot(W[o], h) + (0.0 if b is None else b[o])
            out.append(max(s, 0.0) if t < T - 1 else s)
        h = out
    n_f = len(h) // d
    rows = [h[r * d:(r + 1) * d] for r in range(n_f)]
    for r in range(n_l):
        rows.append([dot(w_l[r], X[:, e]) for e in range(d)])
    Y = np.empty((n, d))
    for r in range(n):
        Y[r] = ln([rows[r][e] + X[r, e] for e in range(d)], w.out_gamma, w.out_beta)
    return Y


# ---------------------------------------------------------------- prediction head
def sigmoid(z) -> np.ndarray:
    """Logistic function 1 / (1 + e^-z), evaluated without overflow for large |z|."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def prediction_head(Y, head_w: Sequence[np.ndarray], head_b: Sequence = None,
                    storage: Iterable[str] = (), logits: bool = False):
    """Top MLP and prediction after the layer stack (Wukong paper, section 2.2:
    the Wukong layers do the feature interaction and an MLP then produces the
    prediction; the page gives no sizes for it).

    Readings: the MLP input is the last layer's output flattened row-major,
    v = vec(Y) with v[r*d + e] = Y[r, e]; every Linear but the last is followed
    by ReLU; the prediction is the logistic function of the last Linear's
    output.  `head_w` lists [m_t, m_{t-1}] weights (m_0 = n*d), `head_b` the
    [m_t] biases (None entries: no bias).  `storage` may name "h": the hidden
    activations are then rounded to bf16 where produced.  Returns the
    probabilities [S, m_T] in float64, or (probabilities, logits).
    """
    storage = frozenset(storage)
    if storage - {"h"}:
        raise ValueError(f"unknown storage names {sorted(storage - {'h'})}")
    Y = to_f64(Y)
    S = Y.shape[0]
    v = Y.reshape(S, -1)
    T = len(head_w)
    for t in range(T):
        W = to_f64(head_w[t])
        v = v @ W.T
        if head_b is not None and head_b[t] is not None:
            v = v + to_f64(head_b[t])
        if t + 1 < T:
            v = np.maximum(v, 0.0)
            v = _maybe_round(v, "h", storage)
    p = sigmoid(v)
    return (p, v) if logits else p


def brute_force_head(Y1, head_w: Sequence[np.ndarray], head_b: Sequence = None) -> List[float]:
    """The prediction head for ONE example [n, d] with explicit loops (tiny inputs only)."""
    Y = to_f64(Y1)
    n, d = Y.shape
    vec = []
    for r in range(n):
        for e in range(d):
            vec.append(Y[r, e])
    T = len(head_w)
    for t in range(T):
        W = to_f64(head_w[t])
        b = None if (head_b is None or head_b[t] is None) else to_f64(head_b[t])
        nxt = []
        for o in range(W.shape[0]):
            acc = 0.0
            for i in range(W.shape[1]):
                acc += W[o, i] * vec[i]
            if b is not None:
                acc += b[o]
            nxt.append(acc if t == T - 1 else max(acc, 0.0))
        vec = nxt
    return [1.0 / (1.0 + math.exp(-z)) for z in vec]
