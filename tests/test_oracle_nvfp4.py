"""Pins of the nvfp4-style cache format in the oracle, and planted mistakes
that the pins must catch.  CPU only.

The pages only name the format ("01. vLLM", section "KV 缓存管理与前缀缓存",
the --kv-cache-dtype row); the encoding is the reading stated in
oracle/formats.py (FP4 E2M1 elements, an E4M3 scale per 16 elements, a
per-tensor binary32 scale)."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import paged as P

# The E2M1 magnitudes of the OCP microscaling formats, codes 0..7.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def pin_e2m1_fields():
    for c in range(16):
        want = (-1.0 if c >= 8 else 1.0) * E2M1_TABLE[c & 7]
        assert F.e2m1_code_value(c) == want


def pin_e2m1_rounding():
    """Ties go to the even mantissa (codes 0, 2, 4, 6), above 6 saturates,
    the sign of zero is kept."""
    cases = [(0.25, 0), (0.26, 1), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6),
             (5.0, 6), (5.1, 7), (6.0, 7), (1e9, 7), (0.0, 0), (-0.0, 8), (-0.1, 8), (-2.9, 13)]
    for y, code in cases:
        assert F.e2m1_encode_scalar(np.float32(y)) == code, y


def pin_hand_row():
    """A block with max 6 under g = 1: scale code E4M3(1.0) = 0x38; bytes by
    hand (element 2i low)."""
    x = np.array([6, -6, 3, 1.5, 0.75, 5, 3.5, 0.25] + [0] * 7 + [0.1], np.float32)
    packed, scales = F.nvfp4_quantize_row(x, 1.0)
    assert scales.tolist() == [0x38]
    assert packed.tolist() == [0xF7, 0x35, 0x62, 0x06, 0, 0, 0, 0]


def pin_nearest_and_block_scale():
    """Each block's scale is the E4M3 rounding of max|x| / 6 / g, and each
    element is a nearest representable multiple of S * g (brute force over
    the 15 values), for many random rows and per-tensor scales."""
    rng = np.random.default_rng(0)
    values = np.array(sorted({s * v for s in (-1, 1) for v in E2M1_TABLE}))
    for _ in range(60):
        g = np.float32(rng.uniform(0.01, 4.0))
        x = (rng.standard_normal(64) * rng.uniform(0.1, 50)).astype(np.float32)
        packed, scales = F.nvfp4_quantize_row(x, g)
        back = F.nvfp4_rows_to_f64(packed[None], scales[None], g)[0]
        for b in range(4):
            blk = x[16 * b:16 * b + 16]
            t = np.float32(np.float32(np.float32(np.max(np.abs(blk))) / np.float32(6)) / g)
            assert scales[b] == F.e4m3_encode_scalar(t)
            sg = F.E4M3_TABLE[scales[b]] * float(g)
            for i in range(16):
                best = np.min(np.abs(values * sg - float(blk[i])))
                err = abs(back[16 * b + i] - float(blk[i]))
                assert err <= best + 1e-6 * abs(float(blk[i])) + 1e-30


def pin_zero_block():
    x = np.zeros(32, np.float32)
    x[20] = 2.0
    packed, scales = F.nvfp4_quantize_row(x, 0.5)
    assert scales[0] == 0 and np.all(packed[:8] == 0)
    back = F.nvfp4_rows_to_f64(packed[None], scales[None], 0.5)[0]
    # block 1: S = E4M3(2 / 6 / 0.5 = 0.667) = 0.6875; 2 / (0.6875 * 0.5) =
    # 5.82 rounds to the E2M1 value 6; 6 * 0.6875 * 0.5 = 2.0625
    assert scales[1] == F.e4m3_encode_scalar(np.float32(0.6875))
    assert np.all(back[:16] == 0) and back[20] == 2.0625


def pin_attention_on_dequantised_rows():
    rng = np.random.default_rng(2)
    nb, hkv, hq, d, length = 7, 2, 4, 32, 29
    kc = rng.integers(0, 256, (nb, hkv, 16, d // 2)).astype(np.uint8)
    vc = rng.integers(0, 256, (nb, hkv, 16, d // 2)).astype(np.uint8)
    ks = rng.integers(0x20, 0x48, (nb, hkv, 16, d // 16)).astype(np.uint8)
    vs = rng.integers(0x20, 0x48, (nb, hkv, 16, d // 16)).astype(np.uint8)
    table = np.array([[4, 1]], np.int32)
    q = rng.standard_normal((1, hq, d)).astype(np.float32)
    got = P.decode_attention_nvfp4(q, F.F32, kc, vc, ks, vs, table, [length], 0.2, 0.5, 1.5)
    for h in range(hq):
        kvh = h // 2
        keys, vals = [], []
        for p in range(length):
            b, o = table[0, p // 16], p % 16
            kr = [E2M1_TABLE[(int(kc[b, kvh, o, i // 2]) >> (4 * (i % 2))) & 7]
                  * (-1 if (int(kc[b, kvh, o, i // 2]) >> (4 * (i % 2))) & 8 else 1)
                  * F.E4M3_TABLE[ks[b, kvh, o, i // 16]] * 0.5 for i in range(d)]
            vr = [E2M1_TABLE[(int(vc[b, kvh, o, i // 2]) >> (4 * (i % 2))) & 7]
                  * (-1 if (int(vc[b, kvh, o, i // 2]) >> (4 * (i % 2))) & 8 else 1)
                  * F.E4M3_TABLE[vs[b, kvh, o, i // 16]] * 1.5 for i in range(d)]
            keys.append(kr)
            vals.append(vr)
        want = P.contiguous_attention(q[0, h:h + 1].astype(np.float64), np.array(keys),
                                      np.array(vals), float(np.float32(0.2)))[0]
        assert np.allclose(got[0, h], want, rtol=1e-12, atol=1e-12)


def pin_write_then_read():
    """reshape_and_cache_nvfp4 with distinct key and value tensor scales: a
    row whose largest magnitude is 6 gets block scale E4M3(6 / 6 / g), i.e.
    0x38 (1.0) under g_k = 1 and 0x40 (2.0) under g_v = 0.5; in both cases
    S * g = 1, so the element codes are the hand-derived bytes of
    pin_hand_row.  Slot -1 is skipped, the written slots land at
    (slot / 16, slot % 16), every other byte keeps its poison value."""
    row = np.array([6, -6, 3, 1.5, 0.75, 5, 3.5, 0.25] + [0] * 7 + [0.1], np.float32)
    want = [0xF7, 0x35, 0x62, 0x06, 0, 0, 0, 0]
    nb, hkv, d = 3, 2, 16
    key = np.stack([np.stack([row, -row]), np.stack([row * 0.5, row])])  # [T=2][Hkv][D]
    key = np.concatenate([key, key[:1]])                                  # token 2: slot -1
    value = key.copy()
    poison = 0xA5
    kc = np.full((nb, hkv, 16, d // 2), poison, np.uint8)
    ksc = np.full((nb, hkv, 16, d // 16), poison, np.uint8)
    slots = np.array([19, 40, -1])
    kc2, vc2, ksc2, vsc2 = P.reshape_and_cache_nvfp4(key, value, kc, kc, ksc, ksc, slots,
                                                     F.F32, 1.0, 0.5)
    # token 0, head 0 -> block 1, offset 3
    assert kc2[1, 0, 3].tolist() == want and vc2[1, 0, 3].tolist() == want
    assert ksc2[1, 0, 3].tolist() == [0x38] and vsc2[1, 0, 3].tolist() == [0x40]
    # token 0, head 1 is the negated row: same bytes with every sign bit set
    # on the nonzero codes, and -0 codes (0x8) for the zeros
    neg = [b ^ 0x88 for b in want]
    assert kc2[1, 1, 3].tolist() == neg
    # token 1 -> block 2, offset 8; head 0 is row / 2, so its block scale
    # halves (E4M3(0.5) = 0x30 under g_k = 1) and the codes stay the same
    assert kc2[2, 0, 8].tolist() == want and ksc2[2, 0, 8].tolist() == [0x30]
    assert vsc2[2, 0, 8].tolist() == [0x38]
    touched = np.zeros((nb, 16), bool)
    touched[1, 3] = touched[2, 8] = True
    for a in (kc2, vc2, ksc2, vsc2):
        for h in range(hkv):
            assert np.all(a[:, h][~touched] == poison)


PINS = [pin_e2m1_fields, pin_e2m1_rounding, pin_hand_row, pin_nearest_and_block_scale,
        pin_zero_block, pin_attention_on_dequantised_rows, pin_write_then_read]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_nvfp4_pin(pin):
    pin()


# --------------------------------------------------------------------------
# planted mistakes


def _ties_away(y):
    y = np.float32(y)
    sign = int(np.array([y], dtype=np.float32).view(np.uint32)[0] >> 31)
    dist = np.abs(F.E2M1_MAGNITUDES - abs(float(y)))
    best = np.flatnonzero(dist == dist.min())
    return int(best[-1]) | (sign << 3)


def _code7_is_5(code):
    code = int(code) & 0xF
    v = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.0][code & 7]
    return -v if code & 8 else v


def _swapped_nibbles(x, g):
    packed, scales = F.__dict__["_orig_quantize"](x, g)
    return ((packed >> 4) | (packed << 4)).astype(np.uint8), scales


def _scale_without_g(packed_rows, scale_rows, g):
    return F.__dict__["_orig_rows"](packed_rows, scale_rows, 1.0)


def _writer_swapped_g(key, value, k_cache, v_cache, k_bscales, v_bscales, slots,
                      src_dtype, k_scale, v_scale):
    return P.__dict__["_orig_writer"](key, value, k_cache, v_cache, k_bscales, v_bscales,
                                      slots, src_dtype, v_scale, k_scale)


def _writer_ignoring_skip(key, value, k_cache, v_cache, k_bscales, v_bscales, slots,
                          src_dtype, k_scale, v_scale):
    slots = np.array([s if s >= 0 else 16 * k_cache.shape[0] - 1 for s in slots])
    return P.__dict__["_orig_writer"](key, value, k_cache, v_cache, k_bscales, v_bscales,
                                      slots, src_dtype, k_scale, v_scale)


MUTANTS = [("e2m1_encode_scalar", _ties_away), ("e2m1_code_value", _code7_is_5),
           ("nvfp4_quantize_row", _swapped_nibbles), ("nvfp4_rows_to_f64", _scale_without_g),
           ("reshape_and_cache_nvfp4", _writer_swapped_g),
           ("reshape_and_cache_nvfp4", _writer_ignoring_skip)]


@pytest.mark.parametrize("name,fn", MUTANTS, ids=[f.__name__ for _, f in MUTANTS])
def test_nvfp4_mutant_is_caught(monkeypatch, name, fn):
    monkeypatch.setitem(F.__dict__, "_orig_quantize", F.nvfp4_quantize_row)
    monkeypatch.setitem(F.__dict__, "_orig_rows", F.nvfp4_rows_to_f64)
    monkeypatch.setitem(P.__dict__, "_orig_writer", P.reshape_and_cache_nvfp4)
    if hasattr(F, name):
        monkeypatch.setattr(F, name, fn)
    if hasattr(P, name):
        monkeypatch.setattr(P, name, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches {fn.__name__}"
