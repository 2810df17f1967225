"""Checks that tie the fp64 oracle to facts fixed outside itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a
worked example printed on the pages, a closed form, a library routine on a
special case, or brute force on tiny inputs.  ``test_oracle_pins.py`` runs
them on the oracle as written, and ``test_oracle_mutants.py`` plants
plausible mistakes in the oracle (on the CPU) and checks that some pin fails.
"""

import json
import math
import os

import numpy as np
import torch

from oracle import formats as F
from oracle import paged as P
from synth.allocator import BlockPool, Sequence, tables_array

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
B = P.BLOCK_SIZE


def golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


# ---------------------------------------------------------------- helpers

def place_contiguous(keys, values, table, num_blocks, dtype=np.float64):
    """Build paged f32 caches [NB][1][16][D] holding contiguous K/V rows at
    the slots of one table (the construction used by the brute-force pins)."""
    length, d = keys.shape
    kc = np.full((num_blocks, 1, B, d), np.nan, dtype=np.float32)
    vc = np.full((num_blocks, 1, B, d), np.nan, dtype=np.float32)
    for p in range(length):
        blk, off = table[p // B], p % B
        kc[blk, 0, off] = keys[p]
        vc[blk, 0, off] = values[p]
    return kc, vc


def f32(x):
    return np.asarray(x, dtype=np.float32)


def decode1(q, kc, vc, table, length, scale, dtype=F.F32):
    """Oracle decode of a single sequence, single head."""
    out = P.decode_attention(q[None, None, :], dtype, kc, vc, dtype,
                             np.asarray([table], dtype=np.int32),
                             np.asarray([length], dtype=np.int32), scale)
    return out[0, 0]


# ------------------------------------------------------ sizes and layout

def pin_table1():
    g = golden("table1_kv_sizes.json")
    bpe = g["bytes_per_element_fp16"]
    for row in g["rows"]:
        per_tok = P.kv_bytes_per_token(row["layers"], row["kv_heads"],
                                       row["head_dim"], bpe)
        assert per_tok == row["kib_per_token"] * 1024, row
        assert per_tok * 8192 == row["gib_at_8k"] * 2 ** 30, row
    r8b = g["rows"][1]
    assert (P.kv_bytes_per_token(r8b["layers"], r8b["kv_heads"], r8b["head_dim"], bpe)
            * 128 * 1024 == g["llama31_8b_128k_context_gib"] * 2 ** 30)


def pin_fig2_slots():
    g = golden("fig2_layout.json")
    tables = np.zeros((2, 4), dtype=np.int32)
    tables[0, :3] = g["sequences"]["A"]["block_table"]
    tables[1, :2] = g["sequences"]["B"]["block_table"]
    na = g["sequences"]["A"]["prompt_tokens"]
    nb = g["sequences"]["B"]["prompt_tokens"]
    # the prompts as one prefill step: every token's slot
    slots = P.slot_mapping(tables, [0, na, na + nb], [0, 0])
    for name, row, base in (("A", 0, 0), ("B", 1, na)):
        for blk, lo, hi in g["sequences"][name]["block_contents"]:
            for p in range(lo, hi + 1):
                assert slots[base + p] // B == blk, (name, p)
    used = {int(s) // B for s in slots}
    assert used.isdisjoint(g["free_blocks"])
    # the decode step {A: 1, B: 1}
    d = g["derived_by_the_figure_layout"]
    dec = P.slot_mapping(tables, [0, 1, 2], [na, nb])
    assert list(dec) == [d["A_next_token_slot"], d["B_next_token_slot"]]
    assert P.blocks_needed(na) * B - na == d["idle_slots_before_decode"]["A"]
    assert P.blocks_needed(nb) * B - nb == d["idle_slots_before_decode"]["B"]


def pin_fig2_write_canary():
    """The decode write touches exactly the two slots of Fig. 2 and nothing
    in the free blocks."""
    g = golden("fig2_layout.json")
    rng = np.random.default_rng(0)
    kc = rng.standard_normal((12, 4, B, 64)).astype(np.float32)
    vc = rng.standard_normal((12, 4, B, 64)).astype(np.float32)
    newk = rng.standard_normal((2, 4, 64)).astype(np.float32)
    newv = rng.standard_normal((2, 4, 64)).astype(np.float32)
    d = g["derived_by_the_figure_layout"]
    slots = [d["A_next_token_slot"], d["B_next_token_slot"]]
    k2, v2 = P.reshape_and_cache(newk, newv, kc, vc, slots, F.F32, F.F32)
    changed = np.argwhere(np.any(k2 != kc, axis=-1))
    assert sorted((int(b), int(o)) for b, _, o in changed[::4]) == [(2, 8), (4, 4)]
    for blk in g["free_blocks"]:
        assert np.array_equal(k2[blk], kc[blk]) and np.array_equal(v2[blk], vc[blk])
    assert np.array_equal(k2[2, :, 8], newk[0]) and np.array_equal(v2[4, :, 4], newv[1])
    # slot -1 means "skip"
    k3, _ = P.reshape_and_cache(newk, newv, kc, vc, [-1, -1], F.F32, F.F32)
    assert np.array_equal(k3, kc)


def pin_copy_blocks():
    rng = np.random.default_rng(1)
    ks = [rng.integers(0, 65535, (10, 2, B, 8), dtype=np.uint16) for _ in range(3)]
    vs = [rng.integers(0, 65535, (10, 2, B, 8), dtype=np.uint16) for _ in range(3)]
    pairs = np.array([[1, 7], [4, 2], [1, 9]])
    k2, v2 = P.copy_blocks(ks, vs, pairs)
    for layer in range(3):
        for src, dst in pairs:
            assert np.array_equal(k2[layer][dst], ks[layer][src])
            assert np.array_equal(v2[layer][dst], vs[layer][src])
        for blk in set(range(10)) - {7, 2, 9}:
            assert np.array_equal(k2[layer][blk], ks[layer][blk])
    for bad in ([[1, 2], [3, 2]], [[1, 2], [2, 5]]):
        try:
            P.copy_blocks(ks, vs, np.array(bad))
        except AssertionError:
            continue
        raise AssertionError(f"precondition not enforced for {bad}")


def pin_swap_round_trip():
    """Swap a sequence's blocks out to a second pool and back into other
    blocks of the first: through its repointed table the sequence's logical
    K/V bytes and its decode output are unchanged, the second pool's other
    blocks are untouched, and a swap inside one pool is copy_blocks
    ([Anatomy] "抢占：RECOMPUTE", v0 SWAP; [V0/V1] §2.1)."""
    rng = np.random.default_rng(21)
    nb, hkv, d, length = 12, 2, 8, 50
    kc = f32(rng.standard_normal((nb, hkv, B, d)))
    vc = f32(rng.standard_normal((nb, hkv, B, d)))
    table = np.array([[3, 9, 0, 6]], dtype=np.int32)
    q = f32(rng.standard_normal((1, 4, d)))
    before = P.decode_attention(q, F.F32, kc, vc, F.F32, table,
                                np.array([length], np.int32), 0.37)
    host_k = [np.full((5, hkv, B, d), 7.0, dtype=np.float32)]
    host_v = [np.full((5, hkv, B, d), -7.0, dtype=np.float32)]
    out_pairs = np.array([[3, 4], [9, 0], [0, 2], [6, 1]])       # device -> host
    hk, hv = P.swap_blocks([kc], [vc], host_k, host_v, out_pairs)
    assert np.all(hk[0][3] == 7.0) and np.all(hv[0][3] == -7.0)   # untouched
    # the device blocks are reused by someone else, then the sequence comes
    # back into different blocks
    kc_clobbered = np.array(kc, copy=True); kc_clobbered[[3, 9, 0, 6]] = np.nan
    vc_clobbered = np.array(vc, copy=True); vc_clobbered[[3, 9, 0, 6]] = np.nan
    in_pairs = np.array([[4, 11], [0, 1], [2, 5], [1, 8]])        # host -> device
    (k2,), (v2,) = P.swap_blocks(hk, hv, [kc_clobbered], [vc_clobbered], in_pairs)
    table2 = np.array([[11, 1, 5, 8]], dtype=np.int32)
    after = P.decode_attention(q, F.F32, k2, v2, F.F32, table2,
                               np.array([length], np.int32), 0.37)
    assert np.array_equal(before, after)
    for j in range(4):
        assert np.array_equal(k2[table2[0, j]], kc[table[0, j]])
        assert np.array_equal(v2[table2[0, j]], vc[table[0, j]])
    # inside one pool, with disjoint pairs, a swap is a block copy
    pairs = np.array([[1, 7], [4, 2]])
    ks, vs = P.swap_blocks([kc], [vc], [kc], [vc], pairs)
    kcp, vcp = P.copy_blocks([kc], [vc], pairs)
    assert np.array_equal(ks[0], kcp[0]) and np.array_equal(vs[0], vcp[0])


# ------------------------------------------------------- softmax closed forms

def pin_hand_example():
    """Two keys whose scaled scores are 0 and ln 3 give weights 1/4 and 3/4;
    the second key sits across a block boundary from the first, behind 15
    keys with negligible weight."""
    d, scale = 4, 0.5
    q = f32([2 * math.log(3.0), 0, 0, 0])
    keys = np.zeros((17, d)); values = np.zeros((17, d))
    keys[:15, 0] = -100.0
    values[:15] = 1000.0
    keys[16, 0] = 1.0
    values[15] = [4, 0, 0, 0]
    values[16] = [0, 4, 0, 0]
    table = [3, 0]
    kc, vc = place_contiguous(keys, values, table, 5)
    out = decode1(q, kc, vc, table, 17, scale)
    s = float(np.float32(q[0])) * scale
    expect = np.array([4 / (1 + math.exp(s)), 4 * math.exp(s) / (1 + math.exp(s)), 0, 0])
    assert np.allclose(out, expect, rtol=0, atol=1e-12), out
    assert np.allclose(out, [1, 3, 0, 0], atol=1e-6), out


def pin_single_token():
    rng = np.random.default_rng(2)
    for d in (4, 64):
        keys = rng.standard_normal((1, d)); values = rng.standard_normal((1, d))
        kc, vc = place_contiguous(keys, values, [2], 3)
        q = f32(rng.standard_normal(d))
        out = decode1(q, kc, vc, [2], 1, 0.3)
        assert np.array_equal(out, vc[2, 0, 0].astype(np.float64))


def pin_zero_query_mean():
    rng = np.random.default_rng(3)
    keys = rng.standard_normal((37, 8)); values = rng.standard_normal((37, 8))
    table = [4, 1, 0]
    kc, vc = place_contiguous(keys, values, table, 5)
    out = decode1(np.zeros(8, np.float32), kc, vc, table, 37, 0.7)
    assert np.allclose(out, f32(values).astype(np.float64).mean(axis=0), atol=1e-14)
    # all keys equal: same result for any query
    kc2, _ = place_contiguous(np.tile(keys[:1], (37, 1)), values, table, 5)
    out2 = decode1(f32(rng.standard_normal(8)), kc2, vc, table, 37, 0.7)
    assert np.allclose(out2, out, atol=1e-14)


def pin_constant_values():
    rng = np.random.default_rng(4)
    keys = rng.standard_normal((50, 8))
    values = np.tile(f32(rng.standard_normal(8)), (50, 1))
    table = [3, 2, 1, 0]
    kc, vc = place_contiguous(keys, values, table, 4)
    out = decode1(f32(rng.standard_normal(8) * 3), kc, vc, table, 50, 1.0)
    assert np.allclose(out, values[0], atol=1e-12)


def pin_gqa_mapping():
    """4 q heads over 2 kv heads: heads 0,1 read kv head 0, heads 2,3 kv
    head 1 (kv values are the constant kv index + 1)."""
    rng = np.random.default_rng(5)
    kc = rng.standard_normal((3, 2, B, 8)).astype(np.float32)
    vc = np.zeros((3, 2, B, 8), np.float32)
    vc[:, 0] = 1.0
    vc[:, 1] = 2.0
    q = rng.standard_normal((1, 4, 8)).astype(np.float32)
    out = P.decode_attention(q, F.F32, kc, vc, F.F32, np.array([[2, 0]], np.int32),
                             np.array([20], np.int32), 0.5)
    assert np.allclose(out[0, :, 0], [1, 1, 2, 2], atol=1e-14)


# ----------------------------------------------- brute force and a library

def _random_case(rng, d, hq, hkv, lengths, num_blocks):
    order = rng.permutation(num_blocks)
    pool = BlockPool(num_blocks, order)
    seqs = [Sequence.fresh(pool, L) for L in lengths]
    tables = tables_array(seqs)
    kc = rng.standard_normal((num_blocks, hkv, B, d)).astype(np.float32)
    vc = rng.standard_normal((num_blocks, hkv, B, d)).astype(np.float32)
    q = rng.standard_normal((len(lengths), hq, d)).astype(np.float32)
    return q, kc, vc, tables


def _contiguous_kv(cache, table, length, kvh):
    """Independent gather for the brute force: flat slot indexing."""
    flat = cache[:, kvh].reshape(-1, cache.shape[-1])
    slots = [table[p // B] * B + p % B for p in range(length)]
    return flat[slots].astype(np.float64)


def pin_bruteforce_gather():
    rng = np.random.default_rng(6)
    for d, hq, hkv in ((4, 2, 2), (64, 4, 2), (4, 4, 1)):
        lengths = [int(x) for x in rng.integers(1, 71, size=4)]
        q, kc, vc, tables = _random_case(rng, d, hq, hkv, lengths, 24)
        scale = 1 / math.sqrt(d)
        out = P.decode_attention(q, F.F32, kc, vc, F.F32, tables,
                                 np.array(lengths, np.int32), scale)
        for s, L in enumerate(lengths):
            for h in range(hq):
                kvh = h // (hq // hkv)
                ref = P.contiguous_attention(
                    q[s, h][None].astype(np.float64), _contiguous_kv(kc, tables[s], L, kvh),
                    _contiguous_kv(vc, tables[s], L, kvh), float(np.float32(scale)))
                assert np.allclose(out[s, h], ref[0], rtol=1e-12, atol=1e-13)


def pin_torch_sdpa():
    """Decode and causal prefill agree with torch's scaled_dot_product_attention
    run in float64 on the CPU over contiguous copies of the same K/V."""
    rng = np.random.default_rng(7)
    d, hq, hkv = 16, 4, 2
    lengths = [5, 33, 48]
    q, kc, vc, tables = _random_case(rng, d, hq, hkv, lengths, 12)
    scale = float(np.float32(0.25))
    out = P.decode_attention(q, F.F32, kc, vc, F.F32, tables,
                             np.array(lengths, np.int32), scale)
    for s, L in enumerate(lengths):
        kt = torch.stack([torch.from_numpy(_contiguous_kv(kc, tables[s], L, h // 2))
                          for h in range(hq)])[None]
        vt = torch.stack([torch.from_numpy(_contiguous_kv(vc, tables[s], L, h // 2))
                          for h in range(hq)])[None]
        qt = torch.from_numpy(q[s].astype(np.float64))[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        assert np.allclose(out[s], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-13)
    # prefill: request 1 (33 tokens) as a chunk of its last 13 queries
    qs = rng.standard_normal((13, hq, d)).astype(np.float32)
    pre = P.prefill_attention(qs, F.F32, kc, vc, F.F32, tables[1:2],
                              np.array([0, 13], np.int32), np.array([20], np.int32),
                              scale)
    kt = torch.stack([torch.from_numpy(_contiguous_kv(kc, tables[1], 33, h // 2))
                      for h in range(hq)])[None]
    vt = torch.stack([torch.from_numpy(_contiguous_kv(vc, tables[1], 33, h // 2))
                      for h in range(hq)])[None]
    qt = torch.from_numpy(qs.astype(np.float64)).permute(1, 0, 2)[None]
    mask = torch.arange(33)[None, :] <= (20 + torch.arange(13))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                           scale=scale)
    assert np.allclose(pre, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def pin_decode_one_matches_batch():
    """The per-element decode helper (used to check large launches on samples
    and in worker processes) returns exactly the batch decode's element, for
    every (sequence, head), GQA groups, fp32 / bf16 / fp8 caches with their
    scales, and a zero-length sequence (zeros)."""
    rng = np.random.default_rng(31)
    lengths = [0, 1, 16, 17, 45]
    q, kc, vc, tables = _random_case(rng, 8, 8, 2, lengths, 16)
    ctx = np.array(lengths, np.int32)
    kb = (kc.view(np.uint32) >> 16).astype(np.uint16)     # any bit pattern is a bf16
    vb = (vc.view(np.uint32) >> 16).astype(np.uint16)
    k8 = F.quantise_to_e4m3(kc, np.float32(0.02))
    v8 = F.quantise_to_e4m3(vc, np.float32(0.03))
    for kv_dtype, kcache, vcache, ks, vs in ((F.F32, kc, vc, 1.0, 1.0),
                                             (F.BF16, kb, vb, 1.0, 1.0),
                                             (F.FP8_E4M3, k8, v8, 0.02, 0.03)):
        full = P.decode_attention(q, F.F32, kcache, vcache, kv_dtype, tables, ctx, 0.3,
                                  ks, vs)
        for s in range(len(lengths)):
            for h in range(q.shape[1]):
                one = P.decode_attention_one(q, F.F32, kcache, vcache, kv_dtype, tables, ctx,
                                             0.3, s, h, ks, vs)
                assert np.array_equal(one, full[s, h]), (kv_dtype, s, h)
    assert np.all(full[0] == 0)


def pin_prefill_one_matches_batch():
    """The per-row prefill helper returns exactly the chunked prefill's row
    for every (query row, head), over several requests with cached contexts
    of different lengths, chunks crossing block boundaries, and requests that
    bring no tokens this step ([Anatomy] "V1：统一调度预填充与解码", Fig. 3:
    a chunk's rows are causal rows that see keys 0..p)."""
    rng = np.random.default_rng(32)
    hq, hkv, d = 4, 2, 8
    computed = [0, 13, 5, 30, 16]
    new = [7, 0, 20, 3, 0]
    lengths = [c + n for c, n in zip(computed, new)]
    _, kc, vc, tables = _random_case(rng, d, hq, hkv, [max(L, 1) for L in lengths], 16)
    qsl = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    q = rng.standard_normal((int(qsl[-1]), hq, d)).astype(np.float32)
    nc = np.array(computed, np.int32)
    full = P.prefill_attention(q, F.F32, kc, vc, F.F32, tables, qsl, nc, 0.4)
    for row in range(q.shape[0]):
        for h in range(hq):
            one = P.prefill_attention_one(q, F.F32, kc, vc, F.F32, tables, qsl, nc, 0.4,
                                          row, h)
            assert np.array_equal(one, full[row, h]), (row, h)
    # and, independently of the batch function, the first row of request 3
    # (position 30) is dense attention over the 31 keys 0..30
    row = int(qsl[3])
    ref = P.contiguous_attention(q[row, 1][None].astype(np.float64),
                                 _contiguous_kv(kc, tables[3], 31, 0),
                                 _contiguous_kv(vc, tables[3], 31, 0), float(np.float32(0.4)))
    one = P.prefill_attention_one(q, F.F32, kc, vc, F.F32, tables, qsl, nc, 0.4, row, 1)
    assert np.allclose(one, ref[0], rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------- invariants

def pin_permutation():
    rng = np.random.default_rng(8)
    lengths = [45, 17, 64, 3]
    q, kc, vc, tables = _random_case(rng, 8, 4, 2, lengths, 14)
    ctx = np.array(lengths, np.int32)
    base = P.decode_attention(q, F.F32, kc, vc, F.F32, tables, ctx, 0.35)
    pi = rng.permutation(14)
    kc2 = np.empty_like(kc); vc2 = np.empty_like(vc)
    kc2[pi] = kc; vc2[pi] = vc
    out = P.decode_attention(q, F.F32, kc2, vc2, F.F32, pi[tables].astype(np.int32),
                             ctx, 0.35)
    assert np.array_equal(out, base)


def pin_prefix_sharing():
    """Two sequences on the same 125 shared blocks with identical tails give
    bitwise-identical outputs; a private copy of the prefix changes nothing."""
    rng = np.random.default_rng(9)
    nb, d = 260, 8
    kc = rng.standard_normal((nb, 1, B, d)).astype(np.float32)
    vc = rng.standard_normal((nb, 1, B, d)).astype(np.float32)
    shared = list(rng.permutation(nb)[:125])
    rest = [b for b in range(nb) if b not in shared]
    tail_x, tail_y, private = rest[0], rest[1], rest[2:127]
    kc[tail_y] = kc[tail_x]; vc[tail_y] = vc[tail_x]
    kc[private] = kc[shared]; vc[private] = vc[shared]
    tables = np.array([shared + [tail_x], shared + [tail_y], private + [tail_x]], np.int32)
    qv = rng.standard_normal((1, 1, d)).astype(np.float32)
    q = np.repeat(qv, 3, axis=0)
    out = P.decode_attention(q, F.F32, kc, vc, F.F32, tables,
                             np.array([2010] * 3, np.int32), 0.3)
    assert np.array_equal(out[0], out[1]) and np.array_equal(out[0], out[2])


def pin_split_lse():
    rng = np.random.default_rng(10)
    keys = rng.standard_normal((1000, 16)); values = rng.standard_normal((1000, 16))
    q = rng.standard_normal(16) * 2
    full = P.attention_row(q, keys, values, 0.25)
    for part in (16, 100, 512, 999, 1000, 4096):
        split = P.split_attention_row(q, keys, values, 0.25, part)
        assert np.allclose(split, full, rtol=1e-12, atol=1e-14), part


def pin_prefill_vs_decode():
    rng = np.random.default_rng(11)
    q, kc, vc, tables = _random_case(rng, 8, 4, 2, [30, 50], 10)
    dec = P.decode_attention(q, F.F32, kc, vc, F.F32, tables,
                             np.array([30, 50], np.int32), 0.4)
    pre = P.prefill_attention(q, F.F32, kc, vc, F.F32, tables,
                              np.array([0, 1, 2], np.int32),
                              np.array([29, 49], np.int32), 0.4)
    assert np.array_equal(dec, pre)


def _replay(schedule_steps, prompts_plus_generated, pool_order, d=8, hq=2, hkv=1,
            seed=12):
    """Run the oracle through a multi-step unified schedule: per step write
    the scheduled tokens' K/V at their slots, then attend for each of them.
    Returns (outputs by (request, position), caches, sequences)."""
    names = sorted(prompts_plus_generated)
    total = {n: prompts_plus_generated[n] for n in names}
    K, V, Q = {}, {}, {}
    for n in names:   # each request's values depend only on (seed, name)
        rng = np.random.default_rng([seed] + [ord(c) for c in n])
        K[n] = rng.standard_normal((total[n], hkv, d)).astype(np.float32)
        V[n] = rng.standard_normal((total[n], hkv, d)).astype(np.float32)
        Q[n] = rng.standard_normal((total[n], hq, d)).astype(np.float32)
    nb = len(pool_order)
    pool = BlockPool(nb, pool_order)
    seqs = {n: Sequence(pool) for n in names}
    kc = np.zeros((nb, hkv, B, d), np.float32)
    vc = np.zeros((nb, hkv, B, d), np.float32)
    done = {n: 0 for n in names}
    outs = {}
    for step in schedule_steps:
        reqs = [n for n in names if n in step]
        for n in reqs:
            seqs[n].prepare_write(done[n], step[n])
        tables = tables_array([seqs[n] for n in reqs], width=16)
        counts = [step[n] for n in reqs]
        qsl = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        comp = np.array([done[n] for n in reqs], np.int32)
        slots = P.slot_mapping(tables, qsl, comp)
        newk = np.concatenate([K[n][done[n]:done[n] + step[n]] for n in reqs])
        newv = np.concatenate([V[n][done[n]:done[n] + step[n]] for n in reqs])
        kc, vc = P.reshape_and_cache(newk, newv, kc, vc, slots, F.F32, F.F32)
        qs = np.concatenate([Q[n][done[n]:done[n] + step[n]] for n in reqs])
        o = P.prefill_attention(qs, F.F32, kc, vc, F.F32, tables, qsl, comp, 0.3)
        for i, n in enumerate(reqs):
            for j in range(step[n]):
                outs[(n, done[n] + j)] = o[qsl[i] + j]
            done[n] += step[n]
    return outs, (K, V, Q), kc, vc, seqs


def _fig3_steps():
    g = golden("fig3_schedule.json")
    steps = [dict() for _ in range(7)]
    for name, chunks in g["chunks"].items():
        for step, lo, hi in chunks:
            steps[step - 1][name] = hi - lo + 1
    for name, dsteps in g["decode_steps_used"].items():
        for step in dsteps:
            steps[step - 1][name] = 1
    totals = {n: g["prompts"][n] + len(g["decode_steps_used"][n]) for n in g["prompts"]}
    return steps, totals, g


def pin_fig3_replay():
    """Fig. 3's schedule (chunks of <=16 prompt tokens, then decodes, mixed in
    step 4) gives every token the same output as dense causal attention over
    its sequence, and the cache holds every token's K/V at its slot."""
    steps, totals, g = _fig3_steps()
    s4 = steps[3]
    assert sorted(n for n, c in s4.items() if c == 1) == sorted(g["step4"]["decodes"])
    assert [n for n, c in s4.items() if c > 1 or n in g["step4"]["chunks"]] == g["step4"]["chunks"]
    order = list(np.random.default_rng(13).permutation(40))
    outs, (K, V, Q), kc, vc, seqs = _replay(steps, totals, order)
    for n, L in totals.items():
        for kvh in range(1):
            keys = _contiguous_kv(kc, seqs[n].table, L, kvh)
            assert np.array_equal(keys, K[n][:, kvh].astype(np.float64))
        for p in range(L):
            for h in range(2):
                ref = P.contiguous_attention(
                    Q[n][p, h][None].astype(np.float64), K[n][:, 0].astype(np.float64),
                    V[n][:, 0].astype(np.float64), float(np.float32(0.3)), first_position=p)
                assert np.allclose(outs[(n, p)][h], ref[0], rtol=1e-12, atol=1e-13)


def pin_recompute():
    """Preempt by recompute: free the blocks, re-prefill from position 0 into
    whatever blocks the pool hands out next; the outputs and the logical cache
    contents are unchanged ("vLLM 引擎解剖", section "抢占：RECOMPUTE")."""
    steps = [{"X": 16, "Y": 10}, {"X": 16, "Y": 1}, {"X": 8}]
    outs1, (K, V, Q), kc, vc, seqs = _replay(steps, {"X": 40, "Y": 11},
                                             list(range(30)), seed=14)
    # replay X alone with a different free-block order (what a recompute
    # after preemption sees)
    outs2, _, kc2, vc2, seqs2 = _replay([{"X": 40}], {"X": 40},
                                        list(range(29, -1, -1)), seed=14)
    assert seqs["X"].table != seqs2["X"].table
    for p in range(40):
        assert np.allclose(outs1[("X", p)], outs2[("X", p)], rtol=1e-13, atol=1e-14)
    assert np.array_equal(_contiguous_kv(kc, seqs["X"].table, 40, 0),
                          _contiguous_kv(kc2, seqs2["X"].table, 40, 0))


def pin_spec_verify():
    """Verifying k draft tokens in one pass: a chunk of 1 + k query rows at
    positions c .. c + k, each attending causally, gives exactly the outputs
    of k + 1 separate decodes with context lengths c + 1 .. c + k + 1 over the
    same cache ("01. vLLM：从分页 KV 起家的通用推理引擎", section "调度器：统一的
    token 预算" and section "投机解码": drafts are verified by the target model
    in one step; V1 EngineCore architecture page, section "统一 token 调度":
    speculative candidates advance a request's progress by several tokens)."""
    rng = np.random.default_rng(31)
    c, k, d, hq, hkv = 37, 4, 8, 4, 2
    q, kc, vc, tables = _random_case(rng, d, hq, hkv, [c + k + 1], 12)
    rows = f32(rng.standard_normal((k + 1, hq, d)))
    chunk = P.prefill_attention(rows, F.F32, kc, vc, F.F32, tables,
                                np.array([0, k + 1], np.int32), np.array([c], np.int32), 0.3)
    singles = P.decode_attention(rows, F.F32, kc, vc, F.F32,
                                 np.repeat(tables, k + 1, axis=0),
                                 np.arange(c + 1, c + k + 2, dtype=np.int32), 0.3)
    assert np.array_equal(chunk, singles)
    # and row i does not see the drafts after it
    assert not np.allclose(singles[0], P.decode_attention(
        rows[:1], F.F32, kc, vc, F.F32, tables, np.array([c + k + 1], np.int32), 0.3)[0])


def pin_poison():
    """NaN in unused slots of the last block and in free blocks never reaches
    an output."""
    rng = np.random.default_rng(15)
    lengths = [21, 35]
    q, kc, vc, tables = _random_case(rng, 8, 2, 1, lengths, 8)
    ctx = np.array(lengths, np.int32)
    base = P.decode_attention(q, F.F32, kc, vc, F.F32, tables, ctx, 0.3)
    kp, vp = kc.copy(), vc.copy()
    used = set()
    for s, L in enumerate(lengths):
        for p in range(P.blocks_needed(L) * B):
            blk, off = tables[s][p // B], p % B
            used.add(int(blk))
            if p >= L:
                kp[blk, :, off] = np.nan; vp[blk, :, off] = np.nan
    for blk in set(range(8)) - used:
        kp[blk] = np.nan; vp[blk] = np.nan
    out = P.decode_attention(q, F.F32, kp, vp, F.F32, tables, ctx, 0.3)
    assert np.array_equal(out, base)


# ------------------------------------------------------------- formats

def pin_fp8_codec():
    t = F.E4M3_TABLE
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    finite = np.isfinite(t)
    assert finite.sum() == 254
    assert t[finite].max() == 448.0 and t[finite].min() == -448.0
    known = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x30: 0.5, 0x01: 2.0 ** -9,
             0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x7E: 448.0, 0xB8: -1.0,
             0x3C: 1.5, 0x77: 240.0}
    for c, v in known.items():
        assert t[c] == v, (hex(c), t[c], v)
    assert np.signbit(t[0x80]) and t[0x80] == 0.0
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)
    codes = [c for c in range(256) if np.isfinite(t[c])]
    enc = F.e4m3_encode(np.array([t[c] for c in codes], np.float32))
    assert list(enc) == codes
    # round half to even between neighbours, saturation, NaN, signed zero
    assert F.e4m3_encode_scalar(1.0625) == 0x38     # 1.0 | 1.125 -> even 1.0
    assert F.e4m3_encode_scalar(1.1875) == 0x3A     # 1.125 | 1.25 -> even 1.25
    assert F.e4m3_encode_scalar(1.06251) == 0x39
    assert F.e4m3_encode_scalar(2.0 ** -10) == 0x00  # half the smallest subnormal
    assert F.e4m3_encode_scalar(3 * 2.0 ** -10) == 0x02
    assert F.e4m3_encode_scalar(464.0) == 0x7E and F.e4m3_encode_scalar(1e6) == 0x7E
    assert F.e4m3_encode_scalar(-1e6) == 0xFE
    assert F.e4m3_encode_scalar(float("inf")) == 0x7E
    assert F.e4m3_encode_scalar(float("nan")) == 0x7F
    assert F.e4m3_encode_scalar(-0.0) == 0x80
    sat = F.e4m3_encode(np.array([1e6, -1e6, 464.0, 500.0, np.inf, -np.inf, np.nan],
                                 np.float32))
    assert list(sat) == [0x7E, 0xFE, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F]
    x = np.random.default_rng(16).standard_normal(4000).astype(np.float32) * 150
    assert np.array_equal(F.e4m3_encode(x),
                          np.array([F.e4m3_encode_scalar(v) for v in x], np.uint8))


def pin_fp8_vs_torch():
    """In range, the quantiser equals torch's float8_e4m3fn cast (a library
    implementation of the same standard rounding)."""
    rng = np.random.default_rng(17)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (0.01, 1, 30, 120)])
    x = np.concatenate([x, F.E4M3_TABLE[np.isfinite(F.E4M3_TABLE)]]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ours = F.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # midpoints between neighbours exercise the tie rule
    vals = F.E4M3_TABLE[:0x7F]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    ref_mid = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(mids), ref_mid)
    # the quantiser divides in binary32 before rounding
    scale = np.float32(0.0137)
    xq = x[:5000]
    assert np.array_equal(F.quantise_to_e4m3(xq, scale),
                          torch.from_numpy(xq / scale).to(torch.float8_e4m3fn)
                          .view(torch.uint8).numpy())


def pin_bf16_decode():
    rng = np.random.default_rng(18)
    bits = rng.integers(0, 65536, 50000).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    with np.errstate(invalid="ignore"):   # the random patterns include NaNs
        ours = F.bf16_bits_to_f64(bits)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    assert F.bf16_bits_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert F.bf16_bits_to_f64(np.array([0xC040], np.uint16))[0] == -3.0


# ---------------------------------------------------------- schedules

def pin_budget_example():
    g = golden("budget_example.json")
    assert sum(g["schedule"].values()) == g["budget"]
    assert g["P_prompt_tokens"] - g["schedule"]["P"] == g["P_left_after_step"]
    assert P.blocks_needed(g["prefix_tokens"]) == g["prefix_blocks"]
    assert g["prefix_tokens"] % B == 0


ALL_PINS = [
    pin_table1, pin_fig2_slots, pin_fig2_write_canary, pin_copy_blocks, pin_swap_round_trip,
    pin_hand_example, pin_single_token, pin_zero_query_mean, pin_constant_values,
    pin_gqa_mapping, pin_bruteforce_gather, pin_torch_sdpa, pin_permutation,
    pin_prefix_sharing, pin_split_lse, pin_prefill_vs_decode, pin_fig3_replay,
    pin_recompute, pin_spec_verify, pin_poison, pin_fp8_codec, pin_fp8_vs_torch, pin_bf16_decode,
    pin_budget_example, pin_decode_one_matches_batch, pin_prefill_one_matches_batch,
]


def failing_pins():
    """Names of the pins that fail on the oracle as it currently is."""
    bad = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            bad.append(pin.__name__)
    return bad
