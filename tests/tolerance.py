"""Accuracy gates for attention outputs compared with the fp64 oracle.

The attention tolerance is "max abs error eps_abs / max rel error eps_rel"
(bf16: 2e-3 / 1e-2; fp8 KV: 2e-3 / 3e-2; fp32 toy: 1e-5 / 1e-4).  Read as two
element-wise conditions that must both hold for every output element i:

  (A) absolute:             |g_i - r_i| <= eps_abs + ulp_out(r_i) / 2
  (B) relative, floored:    |g_i - r_i| <= eps_rel * max(|r_i|, tau)
      where tau = 1e-3 * max_j |r_j| over the output tensor.

ulp_out(r) is the spacing of the output format (bf16 for bf16 queries, fp32
for the fp32 toy) in the binade of |r|: the output is the fp32 result
rounded to nearest in that format, and that rounding alone moves an exact
result by up to half a spacing (2^-9 |r| .. 2^-8 |r| for bf16), more than
2e-3 once |r| >= 1.  (A) grants exactly that rounding on top of eps_abs and
nothing more: for |r| < 0.5 the half spacing is below 2^-10 and (A) is
within 25% of the literal 2e-3.

(B) is the strict one: with values scaled by 1/sqrt(128) the decode outputs
are about 2e-3 in size, so (A) alone would accept an all-zero output, while
(B) rejects it.

Integer and byte results (slot maps, cache writes, block copies) are compared
for exact equality instead.
"""

import numpy as np

TOL = {
    "bf16": (2e-3, 1e-2),       # bf16 Q/K/V, fp32 accumulation
    "fp8_e4m3": (2e-3, 3e-2),   # bf16 Q, fp8 K/V
    "f32": (1e-5, 1e-4),        # fp32 toy
}
# Significand bits (with the implicit one) of the output format of each kind.
OUT_BITS = {"bf16": 8, "fp8_e4m3": 8, "f32": 24}
FLOOR = 1e-3


def half_ulp(r, kind):
    """Half the spacing of the output format at |r| (0 at r = 0)."""
    r = np.abs(np.asarray(r, dtype=np.float64))
    _, e = np.frexp(r)                    # |r| = m 2^e, m in [0.5, 1)
    out = np.ldexp(1.0, e - OUT_BITS[kind] - 1)
    return np.where(r > 0, out, 0.0)


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
    ratio_a = float((err / (eps_abs + half_ulp(r, kind))).max())
    rel = float((err / floor).max())
    return ratio_a, rel / eps_rel, float(err.max()), rel


def assert_attention_close(got, ref, kind, what=""):
    ratio_a, ratio_b, max_abs, max_rel = attention_errors(got, ref, kind)
    eps_abs, eps_rel = TOL[kind]
    assert ratio_a <= 1.0 and ratio_b <= 1.0, (
        f"{what}: max abs err {max_abs:.3e} (worst |err|/(eps_abs + ulp/2) {ratio_a:.3f}); "
        f"max floored rel err {max_rel:.3e} (limit {eps_rel:.0e}, worst ratio {ratio_b:.3f})")
    return max_abs, max_rel


U32 = 2.0 ** -24     # unit roundoff of binary32


def assert_fp32_accumulation_close(got, ref, mag, n_terms, what=""):
    """fp32 paths over long contexts, where the output is a normalised sum
    of n_terms products accumulated in binary32.  Recursive summation of n
    terms in binary32 errs by at most (n - 1) u times the sum of the terms'
    magnitudes (u = 2^-24); with the rounding of the weights, their sum
    and the final division (a few u more) the element-wise bound is

        |g_i - r_i| <= 1e-5 + (n_terms + 8) * u * mag_i,

    where mag_i is attention with |V| in place of V (the normalised sum of
    magnitudes the output is accumulated from), from the same oracle.  The
    fixed 1e-5 / 1e-4 gate of the fp32 toy assumes short contexts; this one
    grows with the number of terms, as the rounding does, and stays far
    below the change one wrong or missing key makes (about mag_i / n_eff)."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    m = np.asarray(mag, dtype=np.float64)
    assert g.shape == r.shape == m.shape, (g.shape, r.shape, m.shape)
    if r.size == 0:
        return 0.0
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    bound = 1e-5 + (n_terms + 8) * U32 * m
    ratio = float((np.abs(g - r) / bound).max())
    assert ratio <= 1.0, f"{what}: worst |err| / bound {ratio:.3f} (n_terms {n_terms})"
    return ratio
