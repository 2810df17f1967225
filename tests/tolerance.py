"""Accuracy gates for attention outputs compared with the fp64 oracle.

Both bounds must hold for every output tensor:
  * max |g - r|                         <= eps_abs
  * max |g - r| / max(|r|, tau)         <= eps_rel,  tau = 1e-3 * max |r|
The floor tau keeps the relative bound meaningful where outputs are tiny
(0.088-scaled values averaged over thousands of tokens) without failing on
elements that happen to be near zero.

Integer and byte results (slot maps, cache writes, block copies) are compared
for exact equality instead.
"""

import numpy as np

TOL = {
    "bf16": (2e-3, 1e-2),       # bf16 Q/K/V, fp32 accumulation
    "fp8_e4m3": (2e-3, 3e-2),   # bf16 Q, fp8 K/V
    "f32": (1e-5, 1e-4),        # fp32 toy
}
FLOOR = 1e-3


def attention_errors(got, ref):
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0, 0.0
    err = np.abs(g - r)
    if not np.all(np.isfinite(g)):
        return float("inf"), float("inf")
    tau = FLOOR * float(np.abs(r).max())
    denom = np.maximum(np.abs(r), tau) if tau > 0 else np.ones_like(r)
    return float(err.max()), float((err / denom).max())


def assert_attention_close(got, ref, kind, what=""):
    eps_abs, eps_rel = TOL[kind]
    max_abs, max_rel = attention_errors(got, ref)
    assert max_abs <= eps_abs and max_rel <= eps_rel, (
        f"{what}: max abs err {max_abs:.3e} (limit {eps_abs:.0e}), "
        f"max rel err {max_rel:.3e} (limit {eps_rel:.0e})")
    return max_abs, max_rel
