"""Pins of the sliding-window decode in the oracle, and planted mistakes
that the pins must catch.  CPU only.  Reading: the query at position L-1
sees positions max(0, L-W) .. L-1, its own included."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import paged as P


def _placed(rng, length, d=8, hkv=1, nb=None):
    nb = nb or P.blocks_needed(length) + 3
    table = rng.permutation(nb)[:P.blocks_needed(length)].astype(np.int32)[None, :]
    kc = rng.standard_normal((nb, hkv, 16, d)).astype(np.float32)
    vc = rng.standard_normal((nb, hkv, 16, d)).astype(np.float32)
    return kc, vc, table


def pin_uniform_weights_give_the_window_mean():
    """q = 0 weighs every visible key equally, so the output is the mean of
    the visible values: with value row p = (p, 1, 0, ...) its first element
    is the mean position (L-W + L-1) / 2."""
    rng = np.random.default_rng(0)
    for length, window in [(40, 5), (40, 16), (40, 17), (33, 1), (20, 100), (64, 32)]:
        kc, vc, table = _placed(rng, length)
        for p in range(length):
            b, o = table[0, p // 16], p % 16
            vc[b, 0, o] = 0
            vc[b, 0, o, 0], vc[b, 0, o, 1] = p, 1
        q = np.zeros((1, 1, 8), np.float32)
        out = P.decode_attention_window(q, F.F32, kc, vc, F.F32, table, [length], 0.5, window)
        first = max(0, length - window)
        assert out[0, 0, 0] == pytest.approx((first + length - 1) / 2, abs=1e-12)
        assert out[0, 0, 1] == pytest.approx(1.0, abs=1e-12)


def pin_window_of_one_is_the_last_value():
    rng = np.random.default_rng(1)
    kc, vc, table = _placed(rng, 37)
    q = rng.standard_normal((1, 1, 8)).astype(np.float32)
    out = P.decode_attention_window(q, F.F32, kc, vc, F.F32, table, [37], 0.3, 1)
    b, o = table[0, 36 // 16], 36 % 16
    assert np.array_equal(out[0, 0], vc[b, 0, o].astype(np.float64))


def pin_wide_window_is_plain_decode():
    rng = np.random.default_rng(2)
    kc, vc, table = _placed(rng, 50, hkv=2)
    q = rng.standard_normal((1, 4, 8)).astype(np.float32)
    full = P.decode_attention(q, F.F32, kc, vc, F.F32, table, [50], 0.3)
    for window in (50, 51, 10 ** 6):
        assert np.array_equal(
            P.decode_attention_window(q, F.F32, kc, vc, F.F32, table, [50], 0.3, window), full)


def pin_brute_force_on_the_last_rows():
    """Against contiguous attention on explicitly listed rows."""
    rng = np.random.default_rng(3)
    for length, window in [(70, 20), (70, 64), (16, 3), (100, 48)]:
        kc, vc, table = _placed(rng, length)
        q = rng.standard_normal((1, 1, 8)).astype(np.float32)
        rows = range(max(0, length - window), length)
        keys = np.array([kc[table[0, p // 16], 0, p % 16] for p in rows], np.float64)
        vals = np.array([vc[table[0, p // 16], 0, p % 16] for p in rows], np.float64)
        want = P.contiguous_attention(q[0].astype(np.float64), keys, vals, 0.25)[0]
        got = P.decode_attention_window(q, F.F32, kc, vc, F.F32, table, [length], 0.25, window)
        assert np.allclose(got[0, 0], want, rtol=1e-12, atol=1e-12)


PINS = [pin_uniform_weights_give_the_window_mean, pin_window_of_one_is_the_last_value,
        pin_wide_window_is_plain_decode, pin_brute_force_on_the_last_rows]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_window_pin(pin):
    pin()


MUTANTS = {
    "one_more_key": lambda length, window: max(0, int(length) - int(window) - 1),
    "own_token_excluded_shift": lambda length, window: max(0, int(length) - int(window) + 1),
    "block_aligned_start": lambda length, window: max(0, int(length) - int(window)) // 16 * 16,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_window_mutant_is_caught(monkeypatch, name):
    monkeypatch.setattr(P, "window_start", MUTANTS[name])
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches {name}"
