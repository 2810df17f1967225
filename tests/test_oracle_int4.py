"""Pins of the int4 per token-head cache format in the oracle, and planted
mistakes that the pins must catch.  CPU only.

The pages only name the format ("01. vLLM", section "KV 缓存管理与前缀缓存",
the --kv-cache-dtype row); the encoding is the reading stated in
oracle/formats.py: s = max|x| / 7 per (token, kv head) row, q = round half
to even of x / s, stored as u = q + 8 nibbles, element 2i low."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import paged as P


def pin_hand_row(Fm=F):
    """max|x| = 7 gives s = 1; ties 2.5 -> 2 and 3.5 -> 4 (half to even),
    -0.5 -> 0; nibbles packed low element first (bytes derived by hand)."""
    x = np.array([7, -7, 3.5, 2.5, 0.5, -0.5, 1.5, 0], np.float32)
    packed, s = Fm.int4_quantize_row(x)
    assert s == np.float32(1.0)
    assert packed.tolist() == [0x1F, 0xAC, 0x88, 0x8A]
    assert Fm.int4_unpack_codes(packed).tolist() == [7, -7, 4, 2, 0, 0, 2, 0]


def pin_zero_row(Fm=F):
    packed, s = Fm.int4_quantize_row(np.zeros(16, np.float32))
    assert s == 0 and packed.tolist() == [0x88] * 8
    assert np.all(Fm.int4_rows_to_f64(packed[None], np.array([s]))[0] == 0)


def pin_error_bound_and_extremes(Fm=F):
    """Every element is within s/2 of its value; the largest magnitude maps
    to code +-7; codes stay in [-7, 7]."""
    rng = np.random.default_rng(0)
    for _ in range(200):
        x = (rng.standard_normal(128) * rng.uniform(0.01, 100)).astype(np.float32)
        packed, s = Fm.int4_quantize_row(x)
        assert s == np.float32(np.float32(np.max(np.abs(x))) / np.float32(7))
        back = Fm.int4_rows_to_f64(packed[None], np.array([s], np.float32))[0]
        assert np.all(np.abs(back - x) <= float(s) * (0.5 + 1e-6))
        q = Fm.int4_unpack_codes(packed)
        i = int(np.argmax(np.abs(x)))
        assert abs(int(q[i])) == 7 and np.sign(q[i]) == np.sign(x[i])
        assert q.min() >= -7 and q.max() <= 7


def pin_exact_multiples(Fm=F):
    """Rows that are integer multiples of their scale come back exactly."""
    rng = np.random.default_rng(1)
    for _ in range(50):
        s = np.float32(2.0 ** rng.integers(-8, 8))
        q = rng.integers(-7, 8, 64)
        q[0] = 7
        x = (q * s).astype(np.float32)
        packed, s2 = Fm.int4_quantize_row(x)
        assert s2 == s
        assert np.array_equal(Fm.int4_rows_to_f64(packed[None], np.array([s2]))[0], x)


def pin_attention_on_dequantised_rows():
    """Paged int4 decode equals plain attention over the dequantised rows
    gathered in order (shuffled blocks, ragged length, per-row scales)."""
    rng = np.random.default_rng(2)
    nb, hkv, hq, d, length = 9, 2, 4, 16, 37
    kc = rng.integers(0, 256, (nb, hkv, 16, d // 2)).astype(np.uint8)
    vc = rng.integers(0, 256, (nb, hkv, 16, d // 2)).astype(np.uint8)
    ks = rng.uniform(0.01, 2, (nb, hkv, 16)).astype(np.float32)
    vs = rng.uniform(0.01, 2, (nb, hkv, 16)).astype(np.float32)
    table = np.array([[7, 2, 5, 0]], np.int32)
    q = rng.standard_normal((1, hq, d)).astype(np.float32)
    got = P.decode_attention_int4(q, F.F32, kc, vc, ks, vs, table, [length], 0.25)
    for h in range(hq):
        kvh = h // 2
        keys, vals = [], []
        for p in range(length):
            b, o = table[0, p // 16], p % 16
            codes_k = [((int(kc[b, kvh, o, i // 2]) >> (4 * (i % 2))) & 15) - 8 for i in range(d)]
            codes_v = [((int(vc[b, kvh, o, i // 2]) >> (4 * (i % 2))) & 15) - 8 for i in range(d)]
            keys.append(np.array(codes_k, np.float64) * float(ks[b, kvh, o]))
            vals.append(np.array(codes_v, np.float64) * float(vs[b, kvh, o]))
        want = P.contiguous_attention(q[0, h:h + 1].astype(np.float64), np.array(keys),
                                      np.array(vals), float(np.float32(0.25)))[0]
        assert np.allclose(got[0, h], want, rtol=1e-12, atol=1e-12)


def pin_write_then_read():
    """reshape_and_cache_int4 followed by the gather returns each written row
    within half a scale, at its slot, and leaves other slots alone."""
    rng = np.random.default_rng(3)
    nb, hkv, d = 4, 2, 32
    kc = np.zeros((nb, hkv, 16, d // 2), np.uint8)
    ks = np.zeros((nb, hkv, 16), np.float32)
    key = rng.standard_normal((3, hkv, d)).astype(np.float32)
    slots = np.array([5, -1, 37])
    kc2, vc2, ks2, vs2 = P.reshape_and_cache_int4(key, key, kc, kc, ks, ks, slots, F.F32)
    for t, slot in ((0, 5), (2, 37)):
        b, o = divmod(slot, 16)
        for h in range(hkv):
            back = F.int4_rows_to_f64(kc2[b, h, o][None], ks2[b, h, o][None])[0]
            assert np.all(np.abs(back - key[t, h]) <= ks2[b, h, o] * 0.5 + 1e-7)
    touched = np.zeros((nb, 16), bool)
    touched[0, 5] = touched[2, 5] = True
    for h in range(hkv):
        assert np.all(ks2[:, h][~touched] == 0) and np.all(kc2[:, h][~touched] == 0)


def pin_one_matches_batch():
    """The per-element int4 decode helper returns exactly the batch decode's
    element for every (sequence, head), including a zero-length sequence, with
    distinct key and value scales."""
    rng = np.random.default_rng(4)
    nb, hkv, hq, d = 10, 2, 8, 16
    kc = rng.integers(0, 256, (nb, hkv, 16, d // 2)).astype(np.uint8)
    vc = rng.integers(0, 256, (nb, hkv, 16, d // 2)).astype(np.uint8)
    ks = rng.uniform(0.01, 2, (nb, hkv, 16)).astype(np.float32)
    vs = rng.uniform(3, 5, (nb, hkv, 16)).astype(np.float32)
    tables = np.array([[7, 2, 5, 0], [1, 3, 9, 4], [6, 8, 0, 0]], np.int32)
    lens = np.array([37, 0, 17], np.int32)
    q = rng.standard_normal((3, hq, d)).astype(np.float32)
    full = P.decode_attention_int4(q, F.F32, kc, vc, ks, vs, tables, lens, 0.3)
    for s in range(3):
        for h in range(hq):
            one = P.decode_attention_int4_one(q, F.F32, kc, vc, ks, vs, tables, lens, 0.3, s, h)
            assert np.array_equal(one, full[s, h]), (s, h)
    assert np.all(full[1] == 0)


PINS = [pin_hand_row, pin_zero_row, pin_error_bound_and_extremes, pin_exact_multiples,
        pin_attention_on_dequantised_rows, pin_write_then_read, pin_one_matches_batch]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_int4_pin(pin):
    pin()


# --------------------------------------------------------------------------
# planted mistakes (each replaces one oracle function for the duration)


def _swapped_nibbles(x_f32):
    packed, s = F.__dict__["_orig_quantize"](x_f32)
    return ((packed >> 4) | (packed << 4)).astype(np.uint8), s


def _scale_over_8(x_f32):
    x = np.asarray(x_f32, np.float32)
    s = np.float32(np.float32(np.max(np.abs(x))) / np.float32(8))
    q = np.zeros(x.size, np.int64) if s == 0 else np.clip(np.rint(x / s), -8, 7).astype(np.int64)
    u = (q + 8).astype(np.uint8)
    return (u[0::2] | (u[1::2] << 4)).astype(np.uint8), s


def _floor_rounding(x_f32):
    x = np.asarray(x_f32, np.float32)
    s = np.float32(np.float32(np.max(np.abs(x))) / np.float32(7))
    q = np.zeros(x.size, np.int64) if s == 0 else np.clip(np.floor(x / s), -8, 7).astype(np.int64)
    u = (q + 8).astype(np.uint8)
    return (u[0::2] | (u[1::2] << 4)).astype(np.uint8), s


def _unpack_no_offset(packed):
    packed = np.asarray(packed, np.uint8)
    u = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), np.int64)
    u[..., 0::2] = packed & 15
    u[..., 1::2] = packed >> 4
    return u


def _scales_of_next_row(packed_rows, scales):
    sc = np.roll(np.asarray(scales, np.float32), 1, axis=-1)
    q = F.int4_unpack_codes(packed_rows).astype(np.float64)
    return q * sc.astype(np.float64)[..., None]


def _one_with_swapped_scales(q, q_dtype, k_cache, v_cache, k_scales, v_scales,
                             block_tables, context_lens, softmax_scale, seq, head):
    return P.__dict__["_orig_one"](q, q_dtype, k_cache, v_cache, v_scales, k_scales,
                                   block_tables, context_lens, softmax_scale, seq, head)


MUTANTS = [("int4_quantize_row", _swapped_nibbles), ("int4_quantize_row", _scale_over_8),
           ("int4_quantize_row", _floor_rounding), ("int4_unpack_codes", _unpack_no_offset),
           ("int4_rows_to_f64", _scales_of_next_row),
           ("decode_attention_int4_one", _one_with_swapped_scales)]


@pytest.mark.parametrize("name,fn", MUTANTS, ids=[f.__name__ for _, f in MUTANTS])
def test_int4_mutant_is_caught(monkeypatch, name, fn):
    monkeypatch.setitem(F.__dict__, "_orig_quantize", F.int4_quantize_row)
    monkeypatch.setitem(P.__dict__, "_orig_one", P.decode_attention_int4_one)
    if hasattr(F, name):
        monkeypatch.setattr(F, name, fn)
    if hasattr(P, name):
        monkeypatch.setattr(P, name, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches {fn.__name__}"
