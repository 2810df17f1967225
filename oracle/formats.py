"""Element formats of the KV cache, written out from their definitions (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the cache dtypes but not their encodings: FP16/BF16 at two
bytes and FP8 at one byte per element ("vLLM 引擎解剖", section "KV 缓存需要多少
内存？", the bytes-per-element factor), and fp8 as a --kv-cache-dtype choice
("01. vLLM：从分页 KV 起家的通用推理引擎", section "KV 缓存管理与前缀缓存").
The encodings below are the standard ones:

* bf16: the upper 16 bits of an IEEE-754 binary32.
* fp8 E4M3 (OCP "fn" variant): 1 sign bit, 4 exponent bits (bias 7), 3
  mantissa bits; exponent field 0 is subnormal; S.1111.111 is NaN; there is no
  infinity; the largest finite magnitude is 448 (code 0x7E).

* int4 per token-head (the pages only name "int4_per_token_head" among the
  lower-bit --kv-cache-dtype choices, "01. vLLM", section "KV 缓存管理与前缀
  缓存"; everything else is a reading): every (token, kv head) row of D
  values has one binary32 scale s = max|x| / 7 and D signed 4-bit codes
  q = round-half-even(x / s) in [-8, 7] (both divisions in binary32; s = 0
  and q = 0 for a zero row); a code is stored offset by 8 (u = q + 8, a
  nibble), element 2i in the low nibble and element 2i+1 in the high nibble
  of byte i.  The value is (u - 8) * s.

* nvfp4-style blocks (the pages name "nvfp4" among the lower-bit
  --kv-cache-dtype choices, same row; everything else is a reading): FP4
  E2M1 elements (1 sign, 2 exponent bits with bias 1, 1 mantissa bit;
  magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), one E4M3 scale per 16 consecutive
  elements of a (token, kv head) row, and a per-tensor binary32 scale g.
  Block scale code = E4M3(fp32(fp32(max|x| / 6) / g)); element code =
  E2M1(fp32(x / fp32(S * g))) with S the block scale's value (0 for a zero
  block: all codes 0); E2M1 rounds to nearest with ties to the even
  mantissa and saturates to +-6, keeping the sign (of zero too).  Codes are
  packed two per byte, element 2i in the low nibble.  Value = e2m1 * S * g.

Storage is always handled as raw integers (uint16 for bf16, uint8 for fp8) or
float32, exactly as the cache holds it; values are produced in float64.
"""

import numpy as np

F32, BF16, FP8_E4M3 = "f32", "bf16", "fp8_e4m3"
INT4_PTH = "int4_per_token_head"
NVFP4 = "nvfp4"

BYTES_PER_ELEM = {F32: 4, BF16: 2, FP8_E4M3: 1}

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64, exactly: the pattern is the top
    half of a binary32."""
    bits = np.asarray(bits, dtype=np.uint16)
    as_u32 = bits.astype(np.uint32) << np.uint32(16)
    return as_u32.view(np.float32).astype(np.float64)


def f32_to_f64(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def e4m3_code_value(code):
    """Real value of one E4M3 code (Python float, exact), NaN for the two NaN
    codes.  Written from the field definition, one code at a time."""
    code = int(code) & 0xFF
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * (mant / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


# Table of all 256 codes -> float64 (NaN for 0x7F and 0xFF).
E4M3_TABLE = np.array([e4m3_code_value(c) for c in range(256)], dtype=np.float64)


def fp8_bits_to_f64(codes, scale=1.0):
    """E4M3 codes (uint8) -> float64 value times the per-tensor scale."""
    codes = np.asarray(codes, dtype=np.uint8)
    return E4M3_TABLE[codes.astype(np.int64)] * float(np.float32(scale))


def storage_to_f64(raw, dtype, scale=1.0):
    """Stored cache or tensor elements of ``dtype`` -> float64 values."""
    if dtype == F32:
        return f32_to_f64(raw)
    if dtype == BF16:
        return bf16_bits_to_f64(raw)
    if dtype == FP8_E4M3:
        return fp8_bits_to_f64(raw, scale)
    raise ValueError(f"unknown dtype {dtype}")


# The 127 non-negative finite magnitudes, codes 0x00 .. 0x7E, in code order
# (which is also increasing value order).
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = E4M3_TABLE[:0x7F]


def e4m3_encode_scalar(y):
    """Quantise one binary32 value to E4M3 by brute-force nearest search.

    * NaN -> 0x7F with the input's sign bit.
    * |y| > 448 (including infinity) saturates to 448 with the sign kept.
    * Otherwise the nearest finite magnitude wins; an exact tie between two
      neighbours goes to the code whose mantissa LSB is 0 (round half to
      even).  Zero keeps its sign.
    """
    y = np.float32(y)
    sign_bit = int(np.array([y], dtype=np.float32).view(np.uint32)[0] >> 31)
    if np.isnan(y):
        return 0x7F | (sign_bit << 7)
    mag = abs(float(y))
    if mag > E4M3_MAX:
        return 0x7E | (sign_bit << 7)
    dist = np.abs(_POS_VALUES - mag)
    best = dist.min()
    cands = _POS_CODES[dist == best]
    if len(cands) == 1:
        code = int(cands[0])
    else:
        even = [int(c) for c in cands if (int(c) & 1) == 0]
        assert len(even) == 1, (y, cands)
        code = even[0]
    return code | (sign_bit << 7)


def e4m3_encode(y):
    """Vectorised form of ``e4m3_encode_scalar`` over a float32 array: the same
    nearest search, done against all 127 magnitudes at once."""
    y = np.asarray(y, dtype=np.float32)
    flat = y.reshape(-1)
    sign = (flat.view(np.uint32) >> np.uint32(31)).astype(np.int64)
    mag = np.abs(flat.astype(np.float64))
    out = np.empty(flat.shape, dtype=np.int64)
    nan = np.isnan(flat)
    sat = (~nan) & (mag > E4M3_MAX)
    rest = ~(nan | sat)
    if rest.any():
        m = mag[rest][:, None]
        dist = np.abs(_POS_VALUES[None, :] - m)
        best = dist.min(axis=1, keepdims=True)
        is_best = dist == best
        # among the nearest codes keep the even one when there are two
        n_best = is_best.sum(axis=1)
        pick_even = is_best & ((_POS_CODES[None, :] & 1) == 0)
        chosen = np.where((n_best > 1)[:, None], pick_even, is_best)
        assert (chosen.sum(axis=1) == 1).all()
        out[rest] = np.argmax(chosen, axis=1)
    out[nan] = 0x7F
    out[sat] = 0x7E
    out |= sign << 7
    return out.astype(np.uint8).reshape(y.shape)


def quantise_to_e4m3(x_f32, scale):
    """The cache-write quantiser: code = E4M3(fp32(x) / fp32(scale)), the
    division done once in binary32 (numpy's float32 divide is correctly
    rounded)."""
    x = np.asarray(x_f32, dtype=np.float32)
    y = x / np.float32(scale)
    return e4m3_encode(y.astype(np.float32))


def int4_quantize_row(x_f32):
    """One (token, kv head) row of binary32 values -> (packed codes uint8
    [D/2], binary32 scale), as described in the module docstring."""
    x = np.asarray(x_f32, dtype=np.float32)
    assert x.ndim == 1 and x.size % 2 == 0 and np.all(np.isfinite(x))
    amax = np.float32(np.max(np.abs(x)))
    s = np.float32(amax / np.float32(7.0))
    if s == 0:
        q = np.zeros(x.size, dtype=np.int64)
    else:
        q = np.clip(np.rint(x / s), -8, 7).astype(np.int64)
    u = (q + 8).astype(np.uint8)
    return (u[0::2] | (u[1::2] << np.uint8(4))).astype(np.uint8), s


def int4_unpack_codes(packed):
    """Packed bytes -> signed codes q in [-8, 7] (int64), element order."""
    packed = np.asarray(packed, dtype=np.uint8)
    u = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.int64)
    u[..., 0::2] = packed & 0x0F
    u[..., 1::2] = packed >> 4
    return u - 8


def int4_rows_to_f64(packed_rows, scales):
    """Rows of packed codes [n][D/2] with their scales [n] -> float64 [n][D]."""
    q = int4_unpack_codes(packed_rows).astype(np.float64)
    return q * np.asarray(scales, dtype=np.float32).astype(np.float64)[..., None]


E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
NVFP4_BLOCK = 16


def e2m1_code_value(code):
    """Real value of one E2M1 code (low 4 bits), written from its fields."""
    code = int(code) & 0xF
    sign = -1.0 if code & 8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    if e == 0:
        return sign * m * 0.5                    # subnormal: 0 or 0.5
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


def e2m1_encode_scalar(y):
    """Nearest E2M1 code of one binary32 value: ties to the even mantissa,
    |y| > 6 saturates, the sign bit of y is kept."""
    y = np.float32(y)
    assert np.isfinite(y)
    sign = int(np.array([y], dtype=np.float32).view(np.uint32)[0] >> 31)
    mag = abs(float(y))
    dist = np.abs(E2M1_MAGNITUDES - mag)
    best = np.flatnonzero(dist == dist.min())
    idx = int(best[0]) if len(best) == 1 else int([i for i in best if i % 2 == 0][0])
    return idx | (sign << 3)


def nvfp4_quantize_row(x_f32, g):
    """One row (D a multiple of 16) -> (packed codes uint8 [D/2], block scale
    codes uint8 [D/16]) under the per-tensor scale g."""
    x = np.asarray(x_f32, dtype=np.float32)
    g = np.float32(g)
    assert x.ndim == 1 and x.size % NVFP4_BLOCK == 0 and np.all(np.isfinite(x)) and g > 0
    codes = np.zeros(x.size, dtype=np.uint8)
    scales = np.zeros(x.size // NVFP4_BLOCK, dtype=np.uint8)
    for b in range(x.size // NVFP4_BLOCK):
        blk = x[NVFP4_BLOCK * b:NVFP4_BLOCK * (b + 1)]
        amax = np.float32(np.max(np.abs(blk)))
        t = np.float32(np.float32(amax / np.float32(6.0)) / g)
        sc = int(e4m3_encode_scalar(t))
        scales[b] = sc
        sval = np.float32(e4m3_code_value(sc))
        if sval == 0:
            continue
        denom = np.float32(sval * g)
        for i, v in enumerate(blk):
            codes[NVFP4_BLOCK * b + i] = e2m1_encode_scalar(np.float32(v / denom))
    return (codes[0::2] | (codes[1::2] << np.uint8(4))).astype(np.uint8), scales


def nvfp4_rows_to_f64(packed_rows, scale_rows, g):
    """Rows of packed codes [n][D/2] with block scale codes [n][D/16] ->
    float64 [n][D] (times the per-tensor scale g)."""
    packed = np.asarray(packed_rows, dtype=np.uint8)
    c = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.int64)
    c[..., 0::2] = packed & 0x0F
    c[..., 1::2] = packed >> 4
    vals = np.vectorize(e2m1_code_value, otypes=[np.float64])(c) if c.size else c.astype(float)
    s = E4M3_TABLE[np.asarray(scale_rows, dtype=np.uint8)]
    s = np.repeat(s, NVFP4_BLOCK, axis=-1)
    return vals * s * float(np.float32(g))
