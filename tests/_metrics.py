"""Error metrics and tolerances of the parity gate.

Three views of the difference between a result g and the oracle o:
  elementwise  max_i |g_i - o_i| / max(|o_i|, rms(o))   (rms floor keeps
               LayerNorm outputs near zero and ReLU zeros from dominating)
  normwise     max_i |g_i - o_i| / max_i |o_i|          (max-norm relative error)
  rms          ||g - o||_2 / ||o||_2

The stated tolerance is a max relative error of 1e-4 for fp32 and 2e-2 for
bf16 storage with fp32 accumulation.  fp32 is gated elementwise.  For bf16 the
elementwise view has an intrinsic floor that grows with depth: two bf16
computations whose pre-rounding values differ only by fp32 accumulation
noise already differ by ~2e-2 elementwise after 2 layers of the n=512
workload and ~3e-2 after 8 layers of the n=256 one, because a rounding flip
in Fn, h, M or an inter-layer activation moves whole rows after the next
LayerNorm (test_tolerance_floor.py measures this on the CPU).  So bf16 is
gated normwise (floor ~0.7e-2 at 8 layers) plus rms <= 1e-2 at every depth,
and additionally elementwise for single layers and their intermediates,
where the elementwise floor is well inside 2e-2.
"""
import numpy as np


def _pair(got, ref):
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    if g.shape != o.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {o.shape}")
    return g, o


def rel_err(got, ref) -> float:
    """Elementwise max relative error with an rms floor."""
    g, o = _pair(got, ref)
    if o.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(o * o)))
    den = np.maximum(np.abs(o), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(g - o) / den))


def normwise_err(got, ref) -> float:
    g, o = _pair(got, ref)
    if o.size == 0:
        return 0.0
    m = float(np.max(np.abs(o)))
    return float(np.max(np.abs(g - o))) / (m if m > 0 else 1.0)


def rms_err(got, ref) -> float:
    g, o = _pair(got, ref)
    if o.size == 0:
        return 0.0
    n = float(np.sqrt(np.sum(o * o)))
    return float(np.sqrt(np.sum((g - o) ** 2))) / (n if n > 0 else 1.0)


TOL_F32 = 1e-4    # fp32 path against the pure fp64 oracle, elementwise
TOL_BF16 = 2e-2   # bf16 storage / fp32 accumulation against the bf16-storage oracle
TOL_BF16_RMS = 1e-2
