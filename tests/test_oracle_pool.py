"""The host worker pool that evaluates the oracle unit by unit returns
exactly what the oracle's batch functions return (CPU only)."""

import numpy as np

import oracle_pool as OP
from oracle import formats as F
from oracle import paged as P
from synth.allocator import BlockPool, Sequence, tables_array


def _case(seed, lengths, hq=8, hkv=2, d=16, extra_blocks=5):
    rng = np.random.default_rng(seed)
    nb = sum(P.blocks_needed(max(n, 1)) for n in lengths) + extra_blocks
    pool = BlockPool(nb, rng.permutation(nb))
    tables = tables_array([Sequence.fresh(pool, max(n, 1)) for n in lengths])
    kc = (rng.standard_normal((nb, hkv, 16, d)).astype(np.float32).view(np.uint32)
          >> 16).astype(np.uint16)
    vc = (rng.standard_normal((nb, hkv, 16, d)).astype(np.float32).view(np.uint32)
          >> 16).astype(np.uint16)
    return rng, kc, vc, tables


def test_decode_reference_equals_batch_oracle():
    lengths = [0, 1, 16, 17, 100, 37]
    rng, kc, vc, tables = _case(1, lengths)
    q = (rng.standard_normal((len(lengths), 8, 16)).astype(np.float32).view(np.uint32)
         >> 16).astype(np.uint16)
    lens = np.array(lengths, np.int32)
    want = P.decode_attention(q, F.BF16, kc, vc, F.BF16, tables, lens, 0.25)
    got = OP.decode_reference(q, kc, vc, tables, lens, F.BF16, F.BF16, 0.25)
    assert np.array_equal(got, want)


def test_prefill_reference_equals_batch_oracle():
    computed = [0, 20, 5, 0]
    new = [9, 0, 30, 1]
    lengths = [c + n for c, n in zip(computed, new)]
    rng, kc, vc, tables = _case(2, lengths)
    qsl = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    q = rng.standard_normal((int(qsl[-1]), 8, 16)).astype(np.float32)
    nc = np.array(computed, np.int32)
    want = P.prefill_attention(q, F.F32, kc, vc, F.BF16, tables, qsl, nc, 0.3)
    got = OP.prefill_reference(q, kc, vc, tables, qsl, nc, F.F32, F.BF16, 0.3)
    assert np.array_equal(got, want)
