"""The unified varlen launch (decodes, speculative verification and prompt
chunks of one step in one kernel) against the fp64 oracle."""

import numpy as np
import pytest
import torch

import paged_kv_cache_84_amd as pk
from gpu_util import announce, as_f64, host, oracle_caches_after_step, snapshot
from oracle import formats as F
from oracle import paged as P
from synth import configs as C
from synth import rng as R
from synth.allocator import BlockPool, Sequence, tables_array
from tolerance import assert_attention_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def schedule_case(computed, qlens, hq, hkv, seed, poison=False):
    """Requests with `computed[r]` cached tokens bringing `qlens[r]` rows; the
    cache holds every position the rows see (random values), the block pool
    is a seeded shuffle, unused slots optionally NaN."""
    rng = np.random.default_rng(seed)
    totals = [c + n for c, n in zip(computed, qlens)]
    nb = sum(P.blocks_needed(t) for t in totals) + 5
    pool = BlockPool(nb, rng.permutation(nb))
    seqs = [Sequence.fresh(pool, t) for t in totals]
    tables = tables_array(seqs)
    kc = R.normal((nb, hkv, 16, 128), F.BF16, 400 + seed, 1, DEV)
    vc = R.normal((nb, hkv, 16, 128), F.BF16, 400 + seed, 2, DEV)
    if poison:
        for sq, t in zip(seqs, totals):
            last = sq.table[(t - 1) // 16]
            if t % 16:
                kc[last, :, t % 16:] = float("nan")
                vc[last, :, t % 16:] = float("nan")
        used = {b for sq in seqs for b in sq.table}
        free = [b for b in range(nb) if b not in used]
        kc[free] = float("nan")
        vc[free] = float("nan")
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = R.normal((int(qsl[-1]), hq, 128), F.BF16, 400 + seed, 3, DEV)
    return q, kc, vc, tables, qsl, np.array(computed, np.int32), max(totals)


def run_varlen(q, kc, vc, tables, qsl, comp, max_seq, ws=None):
    return pk.paged_attention_varlen(q, kc, vc, torch.as_tensor(tables, device=DEV),
                                     torch.as_tensor(qsl, device=DEV),
                                     torch.as_tensor(comp, device=DEV), max_seq,
                                     1.0 / 128 ** 0.5, workspace=ws)


def oracle(q, kc, vc, tables, qsl, comp):
    return P.prefill_attention(host(q), F.BF16, host(kc), host(vc), F.BF16, tables, qsl,
                               comp, float(np.float32(1.0 / 128 ** 0.5)))


@pytest.mark.parametrize("hq,hkv", [(32, 8), (64, 8), (16, 16), (16, 8)])
def test_varlen_mixed_schedule_full_compare(hq, hkv):
    """Decodes (short, across several 64-block runs, exactly on run
    boundaries), speculative verification of 1..3 drafts (one verify whose
    rows straddle a run boundary), a chunk with a cached prefix, a first
    chunk, and an empty request: every output against the oracle."""
    announce("varlen mixed", hq, hkv)
    group = hq // hkv
    k_max = max(0, 16 // group - 1)
    computed = [5, 1023, 1024, 2047, 3000, 1021, 700, 250, 0, 40]
    qlens = [1, 1, 1, 1, 1 + min(1, k_max), 1 + min(3, k_max), 90, 1, 133, 0]
    q, kc, vc, tables, qsl, comp, mx = schedule_case(computed, qlens, hq, hkv, seed=hq + hkv)
    out = run_varlen(q, kc, vc, tables, qsl, comp, mx)
    torch.cuda.synchronize()
    ref = oracle(q, kc, vc, tables, qsl, comp)
    assert_attention_close(as_f64(out), ref, "bf16", f"varlen {hq}/{hkv}")


def test_varlen_repeated_calls_with_a_reused_workspace_are_bitwise_identical():
    """A reused workspace (holding the previous call's partials, or garbage
    before the first) gives the same bits call after call."""
    announce("varlen repeat")
    q, kc, vc, tables, qsl, comp, mx = schedule_case([3000, 5000, 70, 8000], [1, 4, 1, 2],
                                                     32, 8, seed=3)
    need = pk.varlen_workspace_size(4, int(qsl[-1]), 8, 128, mx)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)
    first = run_varlen(q, kc, vc, tables, qsl, comp, mx, ws).clone()
    for _ in range(3):
        again = run_varlen(q, kc, vc, tables, qsl, comp, mx, ws)
        torch.cuda.synchronize()
        assert torch.equal(first, again)
    assert_attention_close(as_f64(first), oracle(q, kc, vc, tables, qsl, comp), "bf16",
                           "varlen repeat")


def test_varlen_poisoned_unused_slots_do_not_leak():
    announce("varlen poison")
    q, kc, vc, tables, qsl, comp, mx = schedule_case([100, 1500, 31, 0], [1, 3, 40, 20],
                                                     32, 8, seed=5, poison=True)
    out = run_varlen(q, kc, vc, tables, qsl, comp, mx)
    torch.cuda.synchronize()
    got = as_f64(out)
    assert np.all(np.isfinite(got))
    assert_attention_close(got, oracle(q, kc, vc, tables, qsl, comp), "bf16", "varlen poison")


def test_varlen_small_mixed_step_full_compare():
    """A small mixed step run with the unified launch (decodes up to 1,500
    tokens, so some span two runs): caches bit-exact, every output against
    the oracle."""
    announce("varlen small mixed step")
    s = snapshot(C.config4(num_prefix_reqs=5, prefix_blocks=6, new_tokens=37,
                           chunk_tokens=150, num_decodes=9, num_writers=3, lo=20, hi=1500,
                           device=DEV))
    ds = pk.step.DeviceStep(s)
    ds.run_varlen()
    torch.cuda.synchronize()
    rk, rv, _ = oracle_caches_after_step(s)
    assert np.array_equal(host(ds.k_caches[0]), rk)
    ref = P.prefill_attention(host(s.q[0]), F.BF16, rk, rv, F.BF16, s.block_tables,
                              s.query_start_loc, s.num_computed, s.softmax_scale)
    got = as_f64(ds.out[0])
    assert_attention_close(got, ref, "bf16", "varlen step")
