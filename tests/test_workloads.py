"""Workload construction and the copy-on-write step, on the CPU with the oracle."""

import json
import os

import numpy as np

from oracle import formats as F
from oracle import paged as P
from synth import configs as C
from synth import rng as R
from synth.allocator import BlockPool, Sequence

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_config4_schedule_counts_match_the_pages():
    """64 x 100 new tokens on a 125-block shared prefix, one 1,022-token
    chunk and 192 decodes: 7,614 tokens, within the 8,192 default budget."""
    with open(os.path.join(GOLDEN, "budget_example.json"), encoding="utf-8") as f:
        g = json.load(f)
    s = C.config4(device="cpu", num_kv_heads=1, num_q_heads=4)
    assert s.num_tokens == 64 * g["question_tokens"] + g["schedule"]["P"] + 192 == 7614
    assert s.num_tokens <= g["default_budget_h100"]
    assert s.num_prefill_tokens == 7422 and s.num_reqs == 257
    assert len(s.copy_pairs) == 64
    ref = s.extra["refcounts"]
    assert all(ref[b] == 64 for b in s.extra["shared_prefix"])
    assert len(s.extra["shared_prefix"]) == g["prefix_blocks"]
    # every copy source is still shared with its parked fork (ref 1 left after
    # the writer moved off it) and every destination is private
    for src, dst in s.copy_pairs:
        assert ref[src] == 1 and ref[dst] == 1
    # prefix requests: positions 2000..2099 -> 7 private blocks each
    for r in range(64):
        assert s.num_computed[r] == 2000
        assert len(set(s.block_tables[r, 125:132])) == 7
        assert list(s.block_tables[r, :125]) == s.extra["shared_prefix"]
    assert s.num_computed[64] == 0 and s.query_start_loc[65] - s.query_start_loc[64] == 1022


def test_config2_pool_is_exactly_the_batch():
    s = C.config2(num_seqs=64)
    lens = s.decode_context_lens
    assert lens.min() >= 512 and lens.max() <= 4096
    assert s.num_blocks == sum(P.blocks_needed(L) for L in lens)
    used = np.concatenate([s.block_tables[i, :P.blocks_needed(L)]
                           for i, L in enumerate(lens)])
    assert sorted(used) == list(range(s.num_blocks))


def test_config1_tables():
    s = C.config1("figure")
    assert list(s.block_tables[0, :3]) == [0, 1, 2] and list(s.block_tables[1, :2]) == [3, 4]
    assert list(s.decode_context_lens) == [41, 21]
    p = C.config1("permuted")
    assert sorted(list(p.block_tables[0, :3]) + list(p.block_tables[1, :2])) != [0, 1, 2, 3, 4]


def test_allocator_refcounts_and_cow():
    pool = BlockPool(10)
    a = Sequence.fresh(pool, 20)          # blocks 0, 1
    b = a.fork()
    assert list(pool.ref[:2]) == [2, 2]
    copies = a.prepare_write(20, 1)       # lands in the shared block 1
    assert copies == [(1, 2)] and a.table == [0, 2] and b.table == [0, 1]
    assert list(pool.ref[:3]) == [2, 1, 1]
    assert a.prepare_write(32, 1) == [] and len(a.table) == 3
    b.free()
    assert pool.ref[1] == 0 and 1 in pool.free


def test_cow_step_with_the_oracle():
    """copy_blocks -> slot mapping -> reshape_and_cache on a small mixed step:
    the copied block equals its source except the written slot, the shared
    source (still read by the parked fork) is unchanged, and no write lands in
    a block that more than one sequence references."""
    s = C.config4(num_prefix_reqs=3, prefix_blocks=4, new_tokens=20, chunk_tokens=37,
                  num_decodes=8, num_writers=3, lo=40, hi=90, num_kv_heads=2,
                  num_q_heads=4)
    kc = R.to_numpy_storage(s.k_caches[0]); vc = R.to_numpy_storage(s.v_caches[0])
    (kc1,), (vc1,) = P.copy_blocks([kc], [vc], s.copy_pairs)
    slots = P.slot_mapping(s.block_tables, s.query_start_loc, s.num_computed)
    ref = s.extra["refcounts"]
    assert all(ref[int(x) // 16] == 1 for x in slots)
    nk = R.to_numpy_storage(s.new_k[0]); nv = R.to_numpy_storage(s.new_v[0])
    kc2, vc2 = P.reshape_and_cache(nk, nv, kc1, vc1, slots, F.BF16, F.BF16)
    written = {int(x) for x in slots}
    for src, dst in s.copy_pairs:
        assert np.array_equal(kc2[src], kc[src]) and np.array_equal(vc2[src], vc[src])
        for off in range(16):
            if dst * 16 + off not in written:
                assert np.array_equal(kc2[dst, :, off], kc[src, :, off])
    # the parked forks read the untouched shared blocks: same output before and after
    forks, flens = s.extra["fork_tables"], s.extra["fork_lengths"]
    q = R.to_numpy_storage(s.q[0])[-len(forks):]
    before = P.decode_attention(q, F.BF16, kc, vc, F.BF16, forks, flens, s.softmax_scale)
    after = P.decode_attention(q, F.BF16, kc2, vc2, F.BF16, forks, flens, s.softmax_scale)
    assert np.array_equal(before, after)


def test_fp8_workload_values_decode_finite():
    s = C.config5(num_seqs=2, length=64)
    codes = R.to_numpy_storage(s.k_caches[0])
    vals = F.fp8_bits_to_f64(codes, s.k_scale)
    assert np.isfinite(vals).all()
    assert abs(vals.std() - 1.0) < 0.05
