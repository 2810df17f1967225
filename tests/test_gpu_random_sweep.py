"""Seeded random configurations against the fp64 oracle: each case draws its
own head counts, head size, cache dtype, lengths (including 0, 1 and block
edges), partition size, value scale and block placement, so that the
combinations the hand-picked cases do not name are covered too.

Decode (plain, with the new token's write inside the launch, and with a
sliding window), the chunked prefill (matrix-core tile and vector rows) and
the unified launch, also with requests that share leading blocks; every
output compared, cache bytes compared bitwise where a call writes them.
"""

import math

import numpy as np
import pytest
import torch

import paged_kv_cache_84_amd as pk
from gpu_util import announce, as_f64, host
from oracle import formats as F
from oracle import paged as P
from synth import rng as R
from synth.allocator import BlockPool, Sequence, tables_array
from tolerance import assert_attention_close, assert_fp32_accumulation_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
EDGES = [0, 1, 15, 16, 17, 31, 32, 33]


def _lengths(rng, n, hi):
    """n lengths: block edges mixed with uniform draws up to hi."""
    out = []
    for _ in range(n):
        if rng.random() < 0.4:
            out.append(int(rng.choice(EDGES)))
        else:
            out.append(int(rng.integers(1, hi + 1)))
    return out


def _pool(rng, lengths, spare=3):
    nb = sum(P.blocks_needed(max(L, 1)) for L in lengths) + spare
    pool = BlockPool(nb, rng.permutation(nb))
    seqs = [Sequence.fresh(pool, max(L, 1)) for L in lengths]
    return nb, tables_array(seqs)


def _caches(shape, kvd, seed, std):
    if kvd == F.FP8_E4M3:
        kc, ks = R.fp8_normal(shape, seed, 1, DEV)
        vc, vs = R.fp8_normal(shape, seed, 2, DEV)
        return kc.view(torch.uint8), vc.view(torch.uint8), ks, vs
    return (R.normal(shape, kvd, seed, 1, DEV, std), R.normal(shape, kvd, seed, 2, DEV, std),
            1.0, 1.0)


def _decode_case(i):
    rng = np.random.default_rng([84, 1, i])
    hkv = int(rng.choice([1, 2, 3, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 6, 8]))
    d = int(rng.choice([64, 128]))
    kvd = F.FP8_E4M3 if rng.random() < 0.4 else F.BF16
    n = int(rng.integers(1, 40))
    lengths = _lengths(rng, n, int(rng.choice([300, 3000])))
    partition = int(rng.choice([0, 0, 16, 48, 512]))
    std = float(rng.choice([0.5, 1.0, 3.0]))
    return rng, hkv, group, d, kvd, lengths, partition, std


def _kind(kvd):
    return "fp8_e4m3" if kvd == F.FP8_E4M3 else "bf16"


def _cache_as_oracle(t, kvd):
    """A device cache as the oracle's host array (fp8: the code bytes)."""
    return host(t)


@pytest.mark.parametrize("i", range(24))
def test_decode_random(i):
    rng, hkv, group, d, kvd, lengths, partition, std = _decode_case(i)
    hq = hkv * group
    announce("random decode", i, hq, hkv, d, kvd, len(lengths), partition, std)
    nb, tables = _pool(rng, lengths)
    kc, vc, ks, vs = _caches((nb, hkv, 16, d), kvd, 7000 + i, std)
    q = R.normal((len(lengths), hq, d), F.BF16, 7000 + i, 3, DEV, std)
    lens = np.array(lengths, np.int32)
    scale = float(np.float32(1 / math.sqrt(d)))
    bt, ln = torch.as_tensor(tables, device=DEV), torch.as_tensor(lens, device=DEV)
    out = pk.paged_attention_decode(q, kc, vc, bt, ln, int(lens.max()), scale, ks, vs, partition)
    torch.cuda.synchronize()
    ref = P.decode_attention(host(q), F.BF16, _cache_as_oracle(kc, kvd),
                             _cache_as_oracle(vc, kvd), kvd, tables, lens, scale, ks, vs)
    assert_attention_close(as_f64(out), ref, _kind(kvd), f"random decode {i}")


@pytest.mark.parametrize("i", range(12))
def test_decode_append_random(i):
    """The new token's K/V written inside the decode launch: cache bytes as
    the oracle's writer leaves them, outputs as the oracle's decode over
    them."""
    rng, hkv, group, d, kvd, lengths, partition, std = _decode_case(100 + i)
    lengths = [max(L, 1) for L in lengths]          # every sequence brings a token
    hq = hkv * group
    announce("random decode append", i, hq, hkv, d, kvd, len(lengths), partition)
    nb, tables = _pool(rng, lengths)
    kc, vc, ks, vs = _caches((nb, hkv, 16, d), kvd, 7100 + i, std)
    q = R.normal((len(lengths), hq, d), F.BF16, 7100 + i, 3, DEV, std)
    nk = R.normal((len(lengths), hkv, d), F.BF16, 7100 + i, 4, DEV, std)
    nv = R.normal((len(lengths), hkv, d), F.BF16, 7100 + i, 5, DEV, std)
    lens = np.array(lengths, np.int32)
    scale = float(np.float32(1 / math.sqrt(d)))
    rk, rv = _cache_as_oracle(kc, kvd), _cache_as_oracle(vc, kvd)
    bt, ln = torch.as_tensor(tables, device=DEV), torch.as_tensor(lens, device=DEV)
    out = pk.paged_attention_decode_append(q, nk, nv, kc, vc, bt, ln, int(lens.max()), scale,
                                           ks, vs, partition)
    torch.cuda.synchronize()
    slots = np.array([P.slot_of(tables[s], int(lens[s]) - 1) for s in range(len(lens))],
                     np.int64)
    rk, rv = P.reshape_and_cache(host(nk), host(nv), rk, rv, slots, F.BF16, kvd, ks, vs)
    assert np.array_equal(_cache_as_oracle(kc, kvd).view(np.uint8), rk.view(np.uint8))
    assert np.array_equal(_cache_as_oracle(vc, kvd).view(np.uint8), rv.view(np.uint8))
    ref = P.decode_attention(host(q), F.BF16, rk, rv, kvd, tables, lens, scale, ks, vs)
    assert_attention_close(as_f64(out), ref, _kind(kvd), f"random decode append {i}")


@pytest.mark.parametrize("i", range(8))
def test_sliding_window_random(i):
    rng, hkv, group, d, kvd, lengths, partition, std = _decode_case(200 + i)
    hq = hkv * group
    window = int(rng.choice([1, 16, 17, 100, 1000]))
    announce("random sliding window", i, hq, hkv, d, kvd, window, partition)
    nb, tables = _pool(rng, lengths)
    kc, vc, ks, vs = _caches((nb, hkv, 16, d), kvd, 7200 + i, std)
    q = R.normal((len(lengths), hq, d), F.BF16, 7200 + i, 3, DEV, std)
    lens = np.array(lengths, np.int32)
    scale = float(np.float32(1 / math.sqrt(d)))
    bt, ln = torch.as_tensor(tables, device=DEV), torch.as_tensor(lens, device=DEV)
    out = pk.paged_attention_decode_sliding(q, kc, vc, bt, ln, int(lens.max()), scale, window,
                                            ks, vs, partition)
    torch.cuda.synchronize()
    ref = P.decode_attention_window(host(q), F.BF16, _cache_as_oracle(kc, kvd),
                                    _cache_as_oracle(vc, kvd), kvd, tables, lens, scale, window,
                                    ks, vs)
    assert_attention_close(as_f64(out), ref, _kind(kvd), f"random window {i}")


def _prefill_case(i, d_choices=(64, 128)):
    rng = np.random.default_rng([84, 2, i])
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice(d_choices))
    n = int(rng.integers(1, 12))
    new, computed = [], []
    for _ in range(n):
        new.append(int(rng.choice([0, 1, 5, 16, 17, 100, 300])) if rng.random() < 0.5
                   else int(rng.integers(1, 200)))
        computed.append(int(rng.choice([0, 1, 15, 16, 17])) if rng.random() < 0.4
                        else int(rng.integers(0, 1500)))
    std = float(rng.choice([0.5, 1.0, 3.0]))
    return rng, hkv, group, d, new, computed, std


def _prefill_inputs(i, rng, hkv, group, d, new, computed, std, qd=F.BF16):
    lens_total = [c + n for c, n in zip(computed, new)]
    nb, tables = _pool(rng, lens_total)
    shape = (nb, hkv, 16, d)
    kc, vc = R.normal(shape, qd, 7300 + i, 1, DEV, std), R.normal(shape, qd, 7300 + i, 2, DEV, std)
    qsl = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    comp = np.array(computed, np.int32)
    q = R.normal((max(int(qsl[-1]), 1), hkv * group, d), qd, 7300 + i, 3, DEV, std)
    return lens_total, tables, kc, vc, qsl, comp, q


@pytest.mark.parametrize("i", range(16))
def test_prefill_random(i):
    rng, hkv, group, d, new, computed, std = _prefill_case(i)
    if sum(new) == 0:
        new[0] = 3
    announce("random prefill", i, hkv * group, hkv, d, new, computed)
    lens_total, tables, kc, vc, qsl, comp, q = _prefill_inputs(i, rng, hkv, group, d, new,
                                                               computed, std)
    scale = float(np.float32(1 / math.sqrt(d)))
    bt, qs, cp = (torch.as_tensor(a, device=DEV) for a in (tables, qsl, comp))
    out = pk.paged_attention_prefill_chunk(q, kc, vc, bt, qs, cp, int(max(new)), scale)
    torch.cuda.synchronize()
    ref = P.prefill_attention(host(q), F.BF16, host(kc), host(vc), F.BF16, tables, qsl, comp,
                              scale)
    assert_attention_close(as_f64(out)[:int(qsl[-1])], ref, "bf16", f"random prefill {i}")


@pytest.mark.parametrize("i", range(12))
def test_varlen_random(i):
    """The unified launch (bf16, head_dim 128) on a random mix of decodes,
    short verifications and chunks."""
    rng, hkv, group, d, new, computed, std = _prefill_case(100 + i, d_choices=(128,))
    for r in range(len(new)):              # make some requests decodes or verifications
        if rng.random() < 0.4:
            new[r] = int(rng.choice([1, 1, 2, 4]))
            computed[r] = int(rng.integers(0, 3000))
    if sum(new) == 0:
        new[0] = 1
    announce("random varlen", i, hkv * group, hkv, new, computed)
    lens_total, tables, kc, vc, qsl, comp, q = _prefill_inputs(100 + i, rng, hkv, group, d,
                                                               new, computed, std)
    scale = float(np.float32(1 / math.sqrt(d)))
    bt, qs, cp = (torch.as_tensor(a, device=DEV) for a in (tables, qsl, comp))
    out = pk.paged_attention_varlen(q, kc, vc, bt, qs, cp, int(max(lens_total)), scale)
    torch.cuda.synchronize()
    ref = P.prefill_attention(host(q), F.BF16, host(kc), host(vc), F.BF16, tables, qsl, comp,
                              scale)
    assert_attention_close(as_f64(out)[:int(qsl[-1])], ref, "bf16", f"random varlen {i}")


def _shared_tables(rng, lens_total):
    """Block tables where a request may name the same physical blocks as an
    earlier request for a random number of its leading blocks (a shared
    prefix), the rest of its blocks its own."""
    need = [P.blocks_needed(max(L, 1)) for L in lens_total]
    nb = sum(need) + 3
    free = [int(b) for b in rng.permutation(nb)]
    rows = []
    for r in range(len(lens_total)):
        row = []
        if r > 0 and rng.random() < 0.6:
            src = int(rng.integers(max(0, r - 3), r))
            row = list(rows[src][:int(rng.integers(1, min(need[r], need[src]) + 1))])
        while len(row) < need[r]:
            row.append(free.pop())
        rows.append(row)
    tables = np.full((len(rows), max(need)), -1, np.int32)
    for r, row in enumerate(rows):
        tables[r, :len(row)] = row
    return nb, tables


@pytest.mark.parametrize("path", ["chunk", "varlen"])
@pytest.mark.parametrize("i", range(8))
def test_shared_prefix_random(path, i):
    """Requests whose tables share leading blocks, so that the matrix-core
    tile stages a key tile once for several requests of a workgroup: every
    row against the oracle, and bitwise against its request computed
    alone."""
    rng = np.random.default_rng([84, 6, i])
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8]))
    n = int(rng.integers(2, 14))
    new = [int(rng.choice([1, 2, 3, 4, 5, 8, 13, 16, 17, 33, 64, 100])) for _ in range(n)]
    computed = [int(rng.choice([0, 16, 64, 100, 700])) if rng.random() < 0.5
                else int(rng.integers(0, 800)) for _ in range(n)]
    std = float(rng.choice([0.5, 1.0, 3.0]))
    announce("random shared prefix", path, i, hkv * group, hkv, new, computed)
    lens_total = [c + m for c, m in zip(computed, new)]
    nb, tables = _shared_tables(rng, lens_total)
    shape = (nb, hkv, 16, 128)
    kc = R.normal(shape, F.BF16, 7600 + i, 1, DEV, std)
    vc = R.normal(shape, F.BF16, 7600 + i, 2, DEV, std)
    qsl = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    comp = np.array(computed, np.int32)
    q = R.normal((int(qsl[-1]), hkv * group, 128), F.BF16, 7600 + i, 3, DEV, std)
    scale = float(np.float32(1 / math.sqrt(128)))
    max_len = int(max(lens_total))

    def call(q_, tables_, qsl_, comp_):
        bt, qs, cp = (torch.as_tensor(np.ascontiguousarray(a), device=DEV)
                      for a in (tables_, qsl_, comp_))
        if path == "chunk":
            return pk.paged_attention_prefill_chunk(q_, kc, vc, bt, qs, cp,
                                                    int(np.diff(qsl_).max()), scale)
        return pk.paged_attention_varlen(q_, kc, vc, bt, qs, cp, max_len, scale)

    whole = call(q, tables, qsl, comp)
    alone = [call(q[int(qsl[r]):int(qsl[r + 1])].contiguous(), tables[r:r + 1],
                  np.array([0, new[r]], np.int32), comp[r:r + 1]) for r in range(n)]
    torch.cuda.synchronize()
    for r in range(n):
        a, b = int(qsl[r]), int(qsl[r + 1])
        assert torch.equal(whole[a:b].view(torch.int16), alone[r].view(torch.int16)), (
            f"request {r}: computed {computed[r]}, {new[r]} tokens")
    ref = P.prefill_attention(host(q), F.BF16, host(kc), host(vc), F.BF16, tables, qsl, comp,
                              scale)
    assert_attention_close(as_f64(whole), ref, "bf16", f"random shared prefix {path} {i}")


def _four_bit_case(i):
    rng = np.random.default_rng([84, 3, i])
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 8]))
    n = int(rng.integers(1, 40))
    lengths = _lengths(rng, n, int(rng.choice([300, 3000])))
    partition = int(rng.choice([0, 0, 16, 48, 512]))
    return rng, hkv, group, lengths, partition


# 1003: a long-context int4 case on which the V products once lost too many
# bits to the removal of the code offset (V entered them as 136 + q)
@pytest.mark.parametrize("fmt", ["int4", "nvfp4"])
@pytest.mark.parametrize("i", list(range(8)) + [1003])
def test_four_bit_decode_random(fmt, i):
    """int4 per token-head and nvfp4-style caches with random codes and
    scales (head_dim 128, bf16 queries)."""
    rng, hkv, group, lengths, partition = _four_bit_case(i if fmt == "int4" else 50 + i)
    hq = hkv * group
    announce("random", fmt, i, hq, hkv, len(lengths), partition)
    nb, tables = _pool(rng, lengths)
    seed = 7400 + i + (50 if fmt == "nvfp4" else 0)
    kc = R.int4_codes((nb, hkv, 16, 64), seed, 1, DEV)
    vc = R.int4_codes((nb, hkv, 16, 64), seed, 2, DEV)
    q = R.normal((len(lengths), hq, 128), F.BF16, seed, 5, DEV)
    lens = np.array(lengths, np.int32)
    scale = float(np.float32(1 / math.sqrt(128)))
    bt, ln = torch.as_tensor(tables, device=DEV), torch.as_tensor(lens, device=DEV)
    if fmt == "int4":
        ks = R.int4_scales((nb, hkv, 16), seed, 3, DEV)
        vs = R.int4_scales((nb, hkv, 16), seed, 4, DEV)
        out = pk.paged_attention_decode_int4(q, kc, vc, ks, vs, bt, ln, int(lens.max()), scale,
                                             partition_tokens=partition)
        torch.cuda.synchronize()
        ref = P.decode_attention_int4(host(q), F.BF16, host(kc), host(vc), host(ks), host(vs),
                                      tables, lens, scale)
    else:
        ks = R.nvfp4_bscales((nb, hkv, 16, 8), seed, 3, DEV)
        vs = R.nvfp4_bscales((nb, hkv, 16, 8), seed, 4, DEV)
        g_k, g_v = float(rng.choice([0.25, 1.0, 3.0])), float(rng.choice([0.5, 1.0, 2.0]))
        out = pk.paged_attention_decode_nvfp4(q, kc, vc, ks, vs, bt, ln, int(lens.max()), scale,
                                              g_k, g_v, partition_tokens=partition)
        torch.cuda.synchronize()
        ref = P.decode_attention_nvfp4(host(q), F.BF16, host(kc), host(vc), host(ks), host(vs),
                                       tables, lens, scale, g_k, g_v)
    assert_attention_close(as_f64(out), ref, "bf16", f"random {fmt} {i}")


@pytest.mark.parametrize("i", range(8))
def test_prefill_other_dtypes_random(i):
    """The chunked prefill's vector rows: fp32 caches, fp8 caches with bf16
    queries, and head_dim 64."""
    rng, hkv, group, d, new, computed, std = _prefill_case(300 + i)
    if sum(new) == 0:
        new[0] = 3
    kind = ["f32", "fp8", "d64"][i % 3]
    qd, kvd = (F.F32, F.F32) if kind == "f32" else (F.BF16, F.FP8_E4M3 if kind == "fp8" else F.BF16)
    d = 64 if kind == "d64" else d
    announce("random prefill", kind, i, hkv * group, hkv, d, new, computed)
    lens_total = [c + n for c, n in zip(computed, new)]
    nb, tables = _pool(rng, lens_total)
    kc, vc, ks, vs = _caches((nb, hkv, 16, d), kvd, 7500 + i, std)
    qsl = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    comp = np.array(computed, np.int32)
    q = R.normal((int(qsl[-1]), hkv * group, d), qd, 7500 + i, 3, DEV, std)
    scale = float(np.float32(1 / math.sqrt(d)))
    bt, qs, cp = (torch.as_tensor(a, device=DEV) for a in (tables, qsl, comp))
    out = pk.paged_attention_prefill_chunk(q, kc, vc, bt, qs, cp, int(max(new)), scale, ks, vs)
    torch.cuda.synchronize()
    ref = P.prefill_attention(host(q), qd, host(kc), host(vc), kvd, tables, qsl, comp, scale,
                              ks, vs)
    if qd == F.F32:
        # contexts of up to ~1,700 keys: the gate follows the fp32 rounding
        mag = P.prefill_attention(host(q), qd, host(kc), np.abs(host(vc)), kvd, tables, qsl,
                                  comp, scale, ks, vs)
        assert_fp32_accumulation_close(as_f64(out), ref, mag, max(lens_total),
                                       f"random prefill {kind} {i}")
        return
    tol = "fp8_e4m3" if kvd == F.FP8_E4M3 else "bf16"
    assert_attention_close(as_f64(out), ref, tol, f"random prefill {kind} {i}")


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint8)


@pytest.mark.parametrize("i", range(16))
def test_cache_write_random(i):
    """reshape_and_cache (copy or fp8), and the int4 and nvfp4 writers, with
    random shapes, value scales and distinct slots, some of them -1: cache
    bytes equal the oracle's."""
    rng = np.random.default_rng([84, 4, i])
    fmt = ["copy", "fp8", "int4", "nvfp4"][i % 4]
    src = F.BF16 if rng.random() < 0.6 else F.F32
    hkv = int(rng.choice([1, 2, 3, 8]))
    d = 128 if fmt in ("int4", "nvfp4") else int(rng.choice([64, 128]))
    nb = int(rng.integers(2, 40))
    t = int(rng.integers(1, nb * 16))
    std = float(rng.choice([0.01, 1.0, 50.0]))
    slots = rng.permutation(nb * 16)[:t].astype(np.int64)
    slots[rng.random(t) < 0.1] = -1
    announce("random cache write", i, fmt, src, hkv, d, nb, t, std)
    key = R.normal((t, hkv, d), src, 7600 + i, 1, DEV, std)
    val = R.normal((t, hkv, d), src, 7600 + i, 2, DEV, std)
    sl = torch.as_tensor(slots, device=DEV)
    if fmt in ("copy", "fp8"):
        dst = src if fmt == "copy" else F.FP8_E4M3
        if dst == F.FP8_E4M3:
            kc = R.int4_codes((nb, hkv, 16, d), 7600 + i, 3, DEV)      # arbitrary bytes
            vc = R.int4_codes((nb, hkv, 16, d), 7600 + i, 4, DEV)
            ks, vs = float(rng.choice([0.05, 1.0, 3.0])), float(rng.choice([0.01, 0.5]))
        else:
            kc = R.normal((nb, hkv, 16, d), dst, 7600 + i, 3, DEV)
            vc = R.normal((nb, hkv, 16, d), dst, 7600 + i, 4, DEV)
            ks = vs = 1.0
        rk, rv = host(kc), host(vc)
        pk.reshape_and_cache(key, val, kc, vc, sl, ks, vs)
        torch.cuda.synchronize()
        rk, rv = P.reshape_and_cache(host(key), host(val), rk, rv, slots, src, dst, ks, vs)
        got = (host(kc), host(vc))
        want = (rk, rv)
    elif fmt == "int4":
        kc = R.int4_codes((nb, hkv, 16, d // 2), 7600 + i, 3, DEV)
        vc = R.int4_codes((nb, hkv, 16, d // 2), 7600 + i, 4, DEV)
        ksc = R.int4_scales((nb, hkv, 16), 7600 + i, 5, DEV)
        vsc = R.int4_scales((nb, hkv, 16), 7600 + i, 6, DEV)
        before = [host(a) for a in (kc, vc, ksc, vsc)]
        pk.reshape_and_cache_int4(key, val, kc, vc, ksc, vsc, sl)
        torch.cuda.synchronize()
        want = P.reshape_and_cache_int4(host(key), host(val), *before, slots, src)
        got = tuple(host(a) for a in (kc, vc, ksc, vsc))
    else:
        kc = R.int4_codes((nb, hkv, 16, d // 2), 7600 + i, 3, DEV)
        vc = R.int4_codes((nb, hkv, 16, d // 2), 7600 + i, 4, DEV)
        kbs = R.nvfp4_bscales((nb, hkv, 16, d // 16), 7600 + i, 5, DEV)
        vbs = R.nvfp4_bscales((nb, hkv, 16, d // 16), 7600 + i, 6, DEV)
        g_k, g_v = float(rng.choice([0.25, 1.0, 7.0])), float(rng.choice([0.5, 1.0, 2.0]))
        before = [host(a) for a in (kc, vc, kbs, vbs)]
        pk.reshape_and_cache_nvfp4(key, val, kc, vc, kbs, vbs, sl, g_k, g_v)
        torch.cuda.synchronize()
        want = P.reshape_and_cache_nvfp4(host(key), host(val), *before, slots, src, g_k, g_v)
        got = tuple(host(a) for a in (kc, vc, kbs, vbs))
    for g, w in zip(got, want):
        assert np.array_equal(_bits(g), _bits(w))


@pytest.mark.parametrize("i", range(8))
def test_copy_blocks_random(i):
    """copy_blocks over several layers with random (src, dst) pairs (distinct
    destinations, none of them a source): every block as the oracle's."""
    rng = np.random.default_rng([84, 5, i])
    layers = int(rng.integers(1, 5))
    hkv = int(rng.choice([1, 2, 8]))
    d = int(rng.choice([64, 128]))
    dt = F.BF16 if rng.random() < 0.7 else F.F32
    nb = int(rng.integers(4, 64))
    n = int(rng.integers(1, nb // 2 + 1))
    perm = rng.permutation(nb)
    src, dst = perm[:n], perm[n:2 * n]
    pairs = np.stack([rng.choice(src, n), dst], axis=1).astype(np.int64)
    announce("random copy_blocks", i, layers, hkv, d, dt, nb, n)
    kcs = [R.normal((nb, hkv, 16, d), dt, 7700 + i, 2 * l, DEV) for l in range(layers)]
    vcs = [R.normal((nb, hkv, 16, d), dt, 7700 + i, 2 * l + 1, DEV) for l in range(layers)]
    rk, rv = P.copy_blocks([host(a) for a in kcs], [host(a) for a in vcs], pairs)
    pk.copy_blocks(kcs, vcs, torch.as_tensor(pairs, device=DEV))
    torch.cuda.synchronize()
    for l in range(layers):
        assert np.array_equal(_bits(host(kcs[l])), _bits(rk[l]))
        assert np.array_equal(_bits(host(vcs[l])), _bits(rv[l]))
