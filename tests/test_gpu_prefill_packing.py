"""Chunk rows packed into workgroups across requests, on the GPU.

The matrix-core prefill cuts the requests' rows into 16-row units and gives
each workgroup eight consecutive units, so a workgroup may hold the end of
one request, several small requests and the start of another.  Requests
whose block tables name the same physical blocks for a key tile (a shared
prefix, "PagedAttention：为 KV 缓存分页", the sharing of blocks) are served by
one staged copy of it.  A row's arithmetic must not depend on that: every
row of a batch equals, bitwise, the same row computed with its request
alone, and all rows match the oracle."""

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
from tolerance import assert_attention_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
PREFIX_BLOCKS = 5


def _batch(seed):
    """Requests of mixed sizes: some on a shared 5-block prefix (cached up
    to a block edge of it), some on their own blocks."""
    rng = np.random.default_rng(seed)
    kinds = rng.choice(["shared", "shared", "own"], size=14)
    reqs = []
    for k in kinds:
        n = int(rng.choice([1, 2, 3, 5, 7, 16, 21, 37, 50, 130]))
        if k == "shared":
            c = 16 * int(rng.integers(1, PREFIX_BLOCKS + 1))
        else:
            c = int(rng.integers(0, 60))
        reqs.append((k, c, n))
    need = sum(P.blocks_needed(c + n) for _, c, n in reqs) + PREFIX_BLOCKS + 4
    pool = BlockPool(need, rng.permutation(need))
    first = Sequence.fresh(pool, PREFIX_BLOCKS * 16)
    seqs = []
    for k, c, n in reqs:
        if k == "shared":
            s = first.share_prefix(c // 16)
            assert not s.prepare_write(c, n)     # block-aligned: no copy needed
        else:
            s = Sequence.fresh(pool, c + n)
        seqs.append(s)
    tables = tables_array(seqs)
    comp = np.array([c for _, c, _ in reqs], np.int32)
    new = np.array([n for _, _, n in reqs], np.int32)
    qsl = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    return tables, qsl, comp, need


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("path", ["chunk", "varlen"])
@pytest.mark.parametrize("seed", [3, 4])
def test_packed_rows_equal_each_request_alone(seed, path, group):
    announce("prefill packing", seed, path, group)
    hkv, d = 2, 128
    hq = hkv * group
    tables, qsl, comp, nb = _batch(seed)
    kc = R.normal((nb, hkv, 16, d), F.BF16, 61, seed, DEV)
    vc = R.normal((nb, hkv, 16, d), F.BF16, 62, seed, DEV)
    q = R.normal((int(qsl[-1]), hq, d), F.BF16, 63, seed, DEV)
    scale = float(np.float32(1 / math.sqrt(d)))
    lens = comp + np.diff(qsl)
    max_len = int(lens.max())

    def call(q_, tables_, qsl_, comp_):
        bt, qs, cp = (torch.as_tensor(np.ascontiguousarray(a), device=DEV)
                      for a in (tables_, qsl_, comp_))
        if path == "chunk":
            return pk.paged_attention_prefill_chunk(q_, kc, vc, bt, qs, cp,
                                                    int(np.diff(qsl_).max()), scale)
        return pk.paged_attention_varlen(q_, kc, vc, bt, qs, cp, max_len, scale)

    whole = call(q, tables, qsl, comp)
    alone = []
    for r in range(len(comp)):
        a, b = int(qsl[r]), int(qsl[r + 1])
        alone.append(call(q[a:b].contiguous(), tables[r:r + 1],
                          np.array([0, b - a], np.int32), comp[r:r + 1]))
    torch.cuda.synchronize()
    for r in range(len(comp)):
        a, b = int(qsl[r]), int(qsl[r + 1])
        assert torch.equal(whole[a:b].view(torch.int16), alone[r].view(torch.int16)), (
            f"request {r}: computed {comp[r]}, {b - a} tokens")
    ref = P.prefill_attention(host(q), F.BF16, host(kc), host(vc), F.BF16, tables, qsl, comp,
                              scale)
    assert_attention_close(as_f64(whole), ref, "bf16", f"packed batch, group {group}")
