"""Accuracy gates for attention outputs compared with the fp64 oracle.

The attention tolerance is "max abs error eps_abs / max rel error eps_rel"
(bf16: 2e-3 / 1e-2; fp8 KV: 2e-3 / 3e-2; fp32 toy: 1e-5 / 1e-4).  Read as two
element-wise conditions that must both hold for every output element i:

  (A) absolute, in the usual mixed form:  |g_i - r_i| <= eps_abs + eps_rel*|r_i|
  (B) relative, with a floor:             |g_i - r_i| <= eps_rel * max(|r_i|, tau)
      where tau = 1e-3 * max_j |r_j| over the output tensor.

(B) is the strict one: with values scaled by 1/sqrt(128) the decode outputs
are about 2e-3 in size, so (A) alone would accept an all-zero output, while
(B) rejects it.  (A) carries eps_rel*|r| because a correctly rounded bf16
output already differs from the exact value by up to 2^-8 * |r|, i.e. more
than 2e-3 once |r| > 0.5; a purely absolute 2e-3 would reject exact results.

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


def attention_errors(got, ref, kind):
    """(worst ratio to bound A, worst ratio to bound B, max abs err, max
    floored rel err); the gate passes iff both ratios are <= 1."""
    eps_abs, eps_rel = TOL[kind]
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0, 0.0, 0.0, 0.0
    if not np.all(np.isfinite(g)):
        return float("inf"), float("inf"), float("inf"), float("inf")
    err = np.abs(g - r)
    tau = FLOOR * float(np.abs(r).max())
    floor = np.maximum(np.abs(r), tau) if tau > 0 else np.ones_like(r)
    ratio_a = float((err / (eps_abs + eps_rel * np.abs(r))).max())
    rel = float((err / floor).max())
    return ratio_a, rel / eps_rel, float(err.max()), rel


def assert_attention_close(got, ref, kind, what=""):
    ratio_a, ratio_b, max_abs, max_rel = attention_errors(got, ref, kind)
    eps_abs, eps_rel = TOL[kind]
    assert ratio_a <= 1.0 and ratio_b <= 1.0, (
        f"{what}: max abs err {max_abs:.3e}, worst |err|/(eps_abs+eps_rel|r|) "
        f"{ratio_a:.3f}; max floored rel err {max_rel:.3e} (limit {eps_rel:.0e})")
    return max_abs, max_rel
