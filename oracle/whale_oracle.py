"""Plain CPU oracle of WHALE's attention-based fusion step (forward pass).

TEST INFRASTRUCTURE ONLY, like the rest of `oracle/`: imported by the tests,
the package's smoke check and the benchmark's CPU-baseline leg, never by the
library; it imports nothing from the library.  fp64 numpy, one step per line.

What it computes (WHALE technical summaries, section 2.1 "attention-based
fusion module" and section 2.2 "efficiency optimizations"): in every WHALE
layer the Wukong module's interaction representation H_w is the query and
the HSTU module's behaviour representation H_s (the full sequence of L
positions) supplies the keys and the values, the keys and values being one
shared tensor (K = V).  The attention output is concatenated with H_w,
projected by a Fusion MLP, and passed through a pre-norm SwiGLU feed-forward
network whose gate and up projections are one matrix (W_gate = W_up); the
result H_f is the next layer's non-sequential input.

Per example, with H_w in R^{n x d} (the n rows of the Wukong layer output as
query tokens) and H_s in R^{L x d}:
  1. S = H_w H_s^T / sqrt(d)              (n x L) scaled dot products
  2. P = softmax(S) over the L positions  (max-subtracted)
  3. A = P H_s                            (n x d)  K = V = H_s
  4. C = [H_w, A]                         (n x 2d) concatenated per row
  5. Q = C W_f^T + b_f                    (n x d)  the Fusion MLP
  6. U = LN_d(Q; gamma, beta) W_up^T + b_up  (n x d_ff)  pre-norm
  7. G = silu(U) * U                      gate and up projection shared
  8. H_f = Q + G W_down^T + b_down        (n x d)  the pre-norm block's residual

Readings taken where the pages are silent (listed in the design notes): no
separate query / key / value projections and a single head, the scale
1/sqrt(d); the Fusion MLP is one Linear layer 2d -> d with bias; d_ff = 4d in
the measured workload; LayerNorm eps = 1e-5 with biased variance.

Storage rounding, as in the Wukong oracle: `storage` may name "P" (the
softmax weights, rounded where they multiply H_s; the normalising sum stays
unrounded), "A", "Q", "Qn" (the normalised Q), "G" and "Hf"; each named
tensor is rounded to bf16 (ties to even) where it is produced.
"""
from __future__ import annotations

import math
from typing import Iterable, List

import numpy as np

from .wukong_oracle import LN_EPS, layer_norm, round_bf16, to_f64

FUSION_STORAGE = frozenset({"P", "A", "Q", "Qn", "G", "Hf"})


def _r(x: np.ndarray, name: str, storage) -> np.ndarray:
    return round_bf16(x) if name in storage else x


def silu(u: np.ndarray) -> np.ndarray:
    """u * logistic(u), written without overflow for large |u|."""
    u = np.asarray(u, dtype=np.float64)
    e = np.exp(-np.abs(u))
    sig = np.where(u >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return u * sig


def cross_attention(Hw, Hs, storage: Iterable[str] = ()) -> np.ndarray:
    """Steps 1-3 for a batch: Hw [S, n, d] queries, Hs [S, L, d] shared keys/values -> A [S, n, d]."""
    storage = frozenset(storage)
    Hw = to_f64(Hw)
    Hs = to_f64(Hs)
    d = Hw.shape[-1]
    S = np.einsum("bqd,bkd->bqk", Hw, Hs) / math.sqrt(d)
    m = S.max(axis=-1, keepdims=True)
    E = np.exp(S - m)
    den = E.sum(axis=-1, keepdims=True)
    num = np.einsum("bqk,bkd->bqd", _r(E, "P", storage), Hs)
    return _r(num / den, "A", storage)


def whale_fusion(Hw, Hs, w, eps: float = LN_EPS, storage: Iterable[str] = (),
                 intermediates: bool = False):
    """Steps 1-8.  `w` carries w_f [d, 2d], b_f [d], gamma / beta [d] (or None),
    w_up [d_ff, d], b_up [d_ff], w_down [d, d_ff], b_down [d] (biases may be None)."""
    storage = frozenset(storage)
    if storage - FUSION_STORAGE:
        raise ValueError(f"unknown storage names {sorted(storage - FUSION_STORAGE)}")
    Hw = to_f64(Hw)
    A = cross_attention(Hw, Hs, storage)
    C = np.concatenate([Hw, A], axis=-1)
    Q = C @ to_f64(w.w_f).T
    if w.b_f is not None:
        Q = Q + to_f64(w.b_f)
    Q = _r(Q, "Q", storage)
    Qn = _r(layer_norm(Q, w.gamma, w.beta, eps), "Qn", storage)
    U = Qn @ to_f64(w.w_up).T
    if w.b_up is not None:
        U = U + to_f64(w.b_up)
    G = _r(silu(U) * U, "G", storage)
    D = G @ to_f64(w.w_down).T
    if w.b_down is not None:
        D = D + to_f64(w.b_down)
    Hf = _r(Q + D, "Hf", storage)
    if intermediates:
        return Hf, {"A": A, "Q": Q, "Qn": Qn, "G": G}
    return Hf


def brute_force_attention(Hw1, Hs1) -> List[List[float]]:
    """Steps 1-3 for ONE example with explicit loops (tiny inputs only)."""
    Q = to_f64(Hw1)
    K = to_f64(Hs1)
    n, d = Q.shape
    L = K.shape[0]
    out = []
    for i in range(n):
        logits = []
        for j in range(L):
            acc = 0.0
            for e in range(d):
                acc += Q[i, e] * K[j, e]
            logits.append(acc / math.sqrt(d))
        mx = max(logits)
        ws = [math.exp(v - mx) for v in logits]
        tot = sum(ws)
        row = []
        for e in range(d):
            acc = 0.0
            for j in range(L):
                acc += ws[j] * K[j, e]
            row.append(acc / tot)
        out.append(row)
    return out
