"""The attention accuracy gate itself (CPU only)."""

import numpy as np
import pytest
import torch

from tolerance import attention_errors, half_ulp


def test_half_ulp_of_bf16_and_fp32():
    assert half_ulp(1.0, "bf16") == 2.0 ** -8          # bf16 spacing on [1, 2) is 2^-7
    assert half_ulp(0.75, "bf16") == 2.0 ** -9
    assert half_ulp(-3.0, "bf16") == 2.0 ** -7
    assert half_ulp(0.0, "bf16") == 0.0
    assert half_ulp(1.0, "f32") == 2.0 ** -24


def test_correct_bf16_rounding_passes():
    """Exact values rounded to nearest bf16 pass the gate at every magnitude."""
    rng = np.random.default_rng(0)
    r = rng.standard_normal(100000) * np.exp(rng.uniform(-6, 3, 100000))
    g = torch.from_numpy(r).to(torch.bfloat16).double().numpy()
    ratio_a, ratio_b, _, _ = attention_errors(g, r, "bf16")
    assert ratio_a <= 1.0 and ratio_b <= 1.0


def test_absolute_bound_binds_below_one():
    """An error of 7.5e-3 at |r| = 0.8 is about twice the absolute bound
    2e-3 + 2^-9 (the relative bound alone, 1e-2 * 0.8, would let it pass)."""
    r = np.array([0.8, 0.1, 0.01])
    g = r + np.array([7.5e-3, 0, 0])
    ratio_a, ratio_b, _, _ = attention_errors(g, r, "bf16")
    assert ratio_a > 1.0 and ratio_b <= 1.0


def test_floored_relative_bound_rejects_zero_output():
    r = np.full(64, 2e-3) * np.where(np.arange(64) % 2, 1, -1)
    ratio_a, ratio_b, _, _ = attention_errors(np.zeros_like(r), r, "bf16")
    assert ratio_a <= 1.0 and ratio_b > 1.0


def test_fp32_accumulation_gate():
    """The fp32 long-context gate: passes the rounding of a binary32 sum of n
    terms, fails a result that lost one of n comparable terms."""
    import numpy as np
    from tolerance import assert_fp32_accumulation_close
    rng = np.random.default_rng(5)
    n = 1500
    w = rng.random(n)
    v = rng.normal(size=(n, 64)) * 3.0
    exact = (w[:, None] * v).sum(0) / w.sum()
    mag = (w[:, None] * np.abs(v)).sum(0) / w.sum()
    acc = np.zeros(64, np.float32)
    for i in range(n):                       # plain binary32 recursive summation
        acc += np.float32(w[i]) * v[i].astype(np.float32)
    got = acc / np.float32(w.astype(np.float32).sum())
    assert_fp32_accumulation_close(got, exact, mag, n)
    dropped = ((w[1:, None] * v[1:]).sum(0)) / w.sum()
    with pytest.raises(AssertionError):
        assert_fp32_accumulation_close(dropped, exact, mag, n)
