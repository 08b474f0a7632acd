"""Error metric shared by the parity tests.

err(g, o) = max_i |g_i - o_i| / max(|o_i|, rms(o)).  The rms floor keeps
LayerNorm outputs near zero and ReLU zeros from inflating a relative error.
"""
import numpy as np


def rel_err(got, ref) -> float:
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    if g.shape != o.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {o.shape}")
    if o.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(o * o)))
    den = np.maximum(np.abs(o), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(g - o) / den))


# tolerances of the parity gate
TOL_F32 = 1e-4   # fp32 path against the pure fp64 oracle
TOL_BF16 = 2e-2  # bf16 storage / fp32 accumulation against the bf16-storage oracle
