"""Plain CPU oracle of a Wukong mixture-of-experts layer (forward pass).

TEST INFRASTRUCTURE ONLY, like the rest of `oracle/`: imported by the tests,
the package's smoke check and the benchmark's CPU-baseline leg, never by the
library; it imports nothing from the library.  fp64 numpy, one step per line.

What it computes (Kunlun technical summary, section 2.3, "Wukong mixture of
experts"): the global interaction module runs several Wukong modules side by
side within one layer, spreading the layer's computation over them.  The
page gives no formula.  Reading taken here (listed in the design notes): each
expert e is a whole Wukong module on the layer input X, with its own
compression Phi_e [k_e, n], FM LayerNorm over its n * k_e interaction values,
MLP producing n_F,e rows of width d, and LCB W_L,e [n_L,e, n]; the experts'
outputs are concatenated along the rows, FMB rows of every expert first (in
expert order), then LCB rows (in expert order), so that
sum_e (n_F,e + n_L,e) = n; the residual X and the output LayerNorm over d
are those of a single layer:

  M_e  = reshape(MLP_e(LN(vec(X (Phi_e X)^T))), n_F,e x d)
  Lc_e = W_L,e X
  R    = [M_1; ...; M_E; Lc_1; ...; Lc_E] + X
  Y[r] = LN_d(R[r]; gamma_out, beta_out)

With one expert this is exactly `wukong_oracle.wukong_layer`.  Storage
rounding follows `wukong_oracle` (names "Z", "Fn", "h", "M", "Y").
"""
from __future__ import annotations

from typing import Iterable, Sequence

import numpy as np

from .wukong_oracle import (LN_EPS, STORAGE_NAMES, _maybe_round, fm_interaction, fmb_mlp, layer_norm, lcb,
                            to_f64)


def wukong_moe_layer(X, experts: Sequence, out_gamma=None, out_beta=None, eps: float = LN_EPS,
                     storage: Iterable[str] = (), intermediates: bool = False):
    """One mixture-of-experts layer on X [S, n, d].  `experts` holds one weight
    object per expert (phi, w_l, fm_gamma, fm_beta, mlp_w, mlp_b; any gamma,
    beta or bias may be None).  Returns Y [S, n, d] float64, or (Y, dict with
    the per-expert lists "M" and "L" and the pre-LayerNorm "R")."""
    storage = frozenset(storage)
    if storage - STORAGE_NAMES:
        raise ValueError(f"unknown storage names {sorted(storage - STORAGE_NAMES)}")
    X = to_f64(X)
    S, n, d = X.shape
    Ms, Ls = [], []
    for w in experts:
        phi = to_f64(w.phi)
        k = phi.shape[0]
        F = fm_interaction(X, phi, storage)                       # [S, n, k_e]
        f_hat = _maybe_round(layer_norm(F.reshape(S, n * k), w.fm_gamma, w.fm_beta, eps), "Fn", storage)
        h = fmb_mlp(f_hat, w.mlp_w, w.mlp_b, storage)              # [S, n_F,e * d]
        if h.shape[1] % d:
            raise ValueError("an expert's last MLP width must be a multiple of d")
        Ms.append(h.reshape(S, h.shape[1] // d, d))
        Ls.append(lcb(X, to_f64(w.w_l)))
    rows = sum(m.shape[1] for m in Ms) + sum(l.shape[1] for l in Ls)
    if rows != n:
        raise ValueError("the experts' FMB and LCB rows must add up to n")
    R = np.concatenate(Ms + Ls, axis=1) + X
    Y = _maybe_round(layer_norm(R, out_gamma, out_beta, eps), "Y", storage)
    if intermediates:
        return Y, {"M": Ms, "L": Ls, "R": R}
    return Y
