"""The five workloads of the paged-attention hot path, as seeded builders.

Every builder returns a ``Step``: the KV caches of each layer (storage
tensors ``[num_blocks][num_kv_heads][16][head_dim]``), the unified schedule of
one engine step (requests with chunks first, then decode requests), the block
tables after the allocator's copy-on-write decisions, the (src, dst) block
copies, and the new tokens' Q/K/V.  Sizes default to the full workloads and
can be shrunk for checks the oracle must finish in seconds.

The schedule format is the unified one: per request the number of tokens it
brings this step and the number already computed ("vLLM 引擎解剖", section
"V1：统一调度预填充与解码"; "v1/v0 区别", §3.1 "Token 预算").
"""

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from . import rng as R
from .allocator import BlockPool, Sequence, tables_array

BLOCK = 16

# purposes for the value generators
P_KCACHE, P_VCACHE, P_Q, P_NEWK, P_NEWV = 1, 2, 3, 4, 5
# purposes for structure generators
S_LENGTHS, S_PLACEMENT, S_WRITERS = 1, 2, 3


@dataclass
class Step:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str
    kv_dtype: str
    num_blocks: int
    k_caches: list
    v_caches: list
    block_tables: np.ndarray          # int32 [R][W], all requests of the step
    query_start_loc: np.ndarray       # int32 [R+1]
    num_computed: np.ndarray          # int32 [R]
    num_prefill_reqs: int             # requests [0, P) bring chunks, [P, R) decode
    q: list                           # per layer: [T][Hq][D] (q dtype)
    new_k: list                       # per layer: [T][Hkv][D] (q dtype)
    new_v: list
    copy_pairs: np.ndarray            # int64 [N][2]
    k_scale: float = 1.0
    v_scale: float = 1.0
    softmax_scale: float = 0.0
    extra: dict = field(default_factory=dict)

    @property
    def num_layers(self):
        return len(self.k_caches)

    @property
    def num_reqs(self):
        return len(self.num_computed)

    @property
    def num_tokens(self):
        return int(self.query_start_loc[-1])

    @property
    def num_prefill_tokens(self):
        return int(self.query_start_loc[self.num_prefill_reqs])

    # --- the decode part of the step -------------------------------------
    @property
    def decode_block_tables(self):
        return np.ascontiguousarray(self.block_tables[self.num_prefill_reqs:])

    @property
    def decode_context_lens(self):
        """Tokens each decode query sees, its own new token included."""
        return (self.num_computed[self.num_prefill_reqs:] + 1).astype(np.int32)

    # --- the chunked-prefill part ----------------------------------------
    @property
    def prefill_block_tables(self):
        return np.ascontiguousarray(self.block_tables[:self.num_prefill_reqs])

    @property
    def prefill_query_start_loc(self):
        return np.ascontiguousarray(
            self.query_start_loc[:self.num_prefill_reqs + 1]).astype(np.int32)

    @property
    def prefill_num_computed(self):
        return np.ascontiguousarray(self.num_computed[:self.num_prefill_reqs])

    def check(self):
        qsl = self.query_start_loc
        assert qsl[0] == 0 and np.all(np.diff(qsl) >= 0)
        assert len(qsl) == self.num_reqs + 1
        for r in range(self.num_prefill_reqs, self.num_reqs):
            assert qsl[r + 1] - qsl[r] == 1, "decode requests bring one token"
        return self


def _pool_tensors(config_id, num_layers, num_blocks, hkv, d, kv_dtype, device,
                  std, layer_stride=100):
    ks, vs, kscale, vscale = [], [], 1.0, 1.0
    shape = (num_blocks, hkv, BLOCK, d)
    for layer in range(num_layers):
        pk = P_KCACHE + layer * layer_stride
        pv = P_VCACHE + layer * layer_stride
        if kv_dtype == R.FP8_E4M3:
            k, kscale = R.fp8_normal(shape, config_id, pk, device)
            v, vscale = R.fp8_normal(shape, config_id, pv, device)
        else:
            k = R.normal(shape, kv_dtype, config_id, pk, device, std)
            v = R.normal(shape, kv_dtype, config_id, pv, device, std)
        ks.append(k)
        vs.append(v)
    return ks, vs, kscale, vscale


def _new_tokens(config_id, num_layers, t, hq, hkv, d, q_dtype, device, std,
                layer_stride=100):
    qs, nk, nv = [], [], []
    for layer in range(num_layers):
        o = layer * layer_stride
        qs.append(R.normal((t, hq, d), q_dtype, config_id, P_Q + o, device, std))
        nk.append(R.normal((t, hkv, d), q_dtype, config_id, P_NEWK + o, device, std))
        nv.append(R.normal((t, hkv, d), q_dtype, config_id, P_NEWV + o, device, std))
    return qs, nk, nv


def _decode_only_step(name, config_id, lengths, num_blocks, tables, hq, hkv, d,
                      q_dtype, kv_dtype, device, std, num_layers=1):
    """A step where every request is a decode of one new token at position
    length-1 (its K/V still to be written), attending to ``length`` tokens."""
    lengths = np.asarray(lengths, dtype=np.int64)
    s = len(lengths)
    ks, vs, kscale, vscale = _pool_tensors(config_id, num_layers, num_blocks,
                                           hkv, d, kv_dtype, device, std)
    qs, nk, nv = _new_tokens(config_id, num_layers, s, hq, hkv, d, q_dtype,
                             device, std)
    return Step(
        name=name, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        q_dtype=q_dtype, kv_dtype=kv_dtype, num_blocks=num_blocks,
        k_caches=ks, v_caches=vs, block_tables=tables,
        query_start_loc=np.arange(s + 1, dtype=np.int32),
        num_computed=(lengths - 1).astype(np.int32), num_prefill_reqs=0,
        q=qs, new_k=nk, new_v=nv, copy_pairs=np.zeros((0, 2), dtype=np.int64),
        k_scale=kscale, v_scale=vscale,
        softmax_scale=float(np.float32(1.0 / math.sqrt(d)))).check()


def config1(placement="figure", device="cpu"):
    """Figure-2 toy: pool of 12 blocks x 16 tokens, 4 q / 4 kv heads,
    head_dim 64, fp32.  Sequence A holds 40 tokens, B 20 ("vLLM 引擎解剖",
    Fig. 2); each gets one decode token (A at position 40, B at 20).

    ``placement="figure"`` uses the figure's tables A=[0,1,2], B=[3,4];
    ``"permuted"`` takes them from a seeded permutation of the free pool."""
    if placement == "figure":
        order = list(range(12))
    else:
        order = [int(b) for b in R.structure_rng(1, S_PLACEMENT).permutation(12)]
    pool = BlockPool(12, order)
    a = Sequence.fresh(pool, 41)   # 40 prompt tokens + the decode token
    b = Sequence.fresh(pool, 21)
    tables = tables_array([a, b], width=4)
    step = _decode_only_step("fig2-toy", 1, [41, 21], 12, tables, 4, 4, 64,
                             R.F32, R.F32, device, 1.0)
    step.extra["placement"] = placement
    return step


def config2(num_seqs=64, lo=512, hi=4096, device="cpu"):
    """Llama-3.1-8B-shaped decode layer: 32 q / 8 kv heads, head_dim 128,
    bf16; context lengths uniform on [lo, hi]; the pool holds exactly the
    blocks the batch needs, shuffled, and each sequence takes consecutive ids
    from the shuffled list; values N(0,1)/sqrt(128)."""
    rs = R.structure_rng(2, S_LENGTHS)
    lengths = rs.integers(lo, hi + 1, size=num_seqs)
    need = [(int(L) + BLOCK - 1) // BLOCK for L in lengths]
    nb = int(sum(need))
    order = R.structure_rng(2, S_PLACEMENT).permutation(nb)
    pool = BlockPool(nb, order)
    seqs = [Sequence.fresh(pool, int(L)) for L in lengths]
    tables = tables_array(seqs)
    return _decode_only_step("llama3.1-8b-decode", 2, lengths, nb, tables,
                             32, 8, 128, R.BF16, R.BF16, device,
                             1.0 / math.sqrt(128))


def config3(num_layers=32, num_seqs=32, length=8192, device="cpu"):
    """Llama-2-7B-shaped MHA decode: 32 q = 32 kv heads, head_dim 128, bf16,
    every sequence at ``length`` tokens; one shuffled placement shared by all
    layers (one block table per sequence); values N(0,1)."""
    need = (length + BLOCK - 1) // BLOCK
    nb = need * num_seqs
    order = R.structure_rng(3, S_PLACEMENT).permutation(nb)
    pool = BlockPool(nb, order)
    seqs = [Sequence.fresh(pool, length) for _ in range(num_seqs)]
    tables = tables_array(seqs)
    return _decode_only_step("llama2-7b-mha-decode", 3, [length] * num_seqs, nb,
                             tables, 32, 32, 128, R.BF16, R.BF16, device, 1.0,
                             num_layers=num_layers)


def config5(num_seqs=6, length=131072, device="cpu"):
    """Llama-3.1-70B-shaped long-context decode, one layer: 64 q / 8 kv
    heads, head_dim 128, bf16 Q, fp8 E4M3 K/V with per-tensor scales;
    values N(0,1); seeded shuffled placement."""
    need = (length + BLOCK - 1) // BLOCK
    nb = need * num_seqs
    order = R.structure_rng(5, S_PLACEMENT).permutation(nb)
    pool = BlockPool(nb, order)
    seqs = [Sequence.fresh(pool, length) for _ in range(num_seqs)]
    tables = tables_array(seqs)
    return _decode_only_step("llama3.1-70b-fp8-longctx", 5, [length] * num_seqs,
                             nb, tables, 64, 8, 128, R.BF16, R.FP8_E4M3, device,
                             1.0)


def config4(num_prefix_reqs=64, prefix_blocks=125, new_tokens=100,
            chunk_tokens=1022, num_decodes=192, num_writers=64,
            lo=1024, hi=8192, num_kv_heads=8, num_q_heads=32, device="cpu"):
    """Mixed unified step with prefix sharing (one layer, 32 q / 8 kv heads,
    head_dim 128, bf16, values N(0,1)):

    * ``num_prefix_reqs`` requests share a ``prefix_blocks``-block cached
      prefix (2,000 tokens = 125 blocks, "01. vLLM：从分页 KV 起家的通用推理引擎",
      section "一个请求怎样流过 V1") and each computes ``new_tokens`` more as a
      chunk at positions 2000..2099;
    * one first chunk of ``chunk_tokens`` from position 0 (the 1,022-token
      chunk of the 1024-token budget example, V1 EngineCore architecture page,
      section "一个 1024-token budget 的例子");
    * ``num_decodes`` decodes with context lengths uniform on [lo, hi]; the
      first ``num_writers`` of them share all their blocks with a parked fork
      (parallel sampling) and their new token lands in the partly filled last
      block, so the allocator copies that block before the write.
    """
    rs = R.structure_rng(4, S_LENGTHS)
    lengths = [int(x) for x in rs.integers(lo, hi + 1, size=num_decodes)]
    for i in range(num_writers):
        while (lengths[i] - 1) % BLOCK == 0:
            lengths[i] = int(rs.integers(lo, hi + 1))
    # pool size: everything this step touches plus the copies' destinations
    prefix_tokens = prefix_blocks * BLOCK
    per_prefix_req = (prefix_tokens + new_tokens + BLOCK - 1) // BLOCK - prefix_blocks
    nb = (prefix_blocks + num_prefix_reqs * per_prefix_req
          + (chunk_tokens + BLOCK - 1) // BLOCK
          + sum((L + BLOCK - 1) // BLOCK for L in lengths) + num_writers + 16)
    order = R.structure_rng(4, S_PLACEMENT).permutation(nb)
    pool = BlockPool(nb, order)

    copies = []
    prefix_reqs = []
    first = Sequence.fresh(pool, prefix_tokens)
    for i in range(num_prefix_reqs):
        seq = first if i == 0 else first.share_prefix(prefix_blocks)
        prefix_reqs.append(seq)
    shared_prefix = list(first.table[:prefix_blocks])
    for seq in prefix_reqs:
        copies += seq.prepare_write(prefix_tokens, new_tokens)
    chunk_req = Sequence(pool)
    copies += chunk_req.prepare_write(0, chunk_tokens)
    decodes, forks = [], []
    for i, L in enumerate(lengths):
        seq = Sequence.fresh(pool, L - 1)      # the history already cached
        if i < num_writers:
            forks.append(seq.fork())           # parked, not scheduled
        copies += seq.prepare_write(L - 1, 1)  # the new token's slot
        decodes.append(seq)
    assert len(copies) == num_writers

    reqs = prefix_reqs + [chunk_req] + decodes
    tables = tables_array(reqs)
    counts = [new_tokens] * num_prefix_reqs + [chunk_tokens] + [1] * num_decodes
    qsl = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    computed = np.array([prefix_tokens] * num_prefix_reqs + [0]
                        + [L - 1 for L in lengths], dtype=np.int32)
    t = int(qsl[-1])
    d, std = 128, 1.0
    ks, vs, kscale, vscale = _pool_tensors(4, 1, nb, num_kv_heads, d, R.BF16,
                                           device, std)
    qs, nk, nv = _new_tokens(4, 1, t, num_q_heads, num_kv_heads, d, R.BF16,
                             device, std)
    step = Step(
        name="mixed-prefix-step", num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=d, q_dtype=R.BF16, kv_dtype=R.BF16,
        num_blocks=nb, k_caches=ks, v_caches=vs, block_tables=tables,
        query_start_loc=qsl, num_computed=computed,
        num_prefill_reqs=num_prefix_reqs + 1, q=qs, new_k=nk, new_v=nv,
        copy_pairs=np.array(copies, dtype=np.int64).reshape(-1, 2),
        k_scale=kscale, v_scale=vscale,
        softmax_scale=float(np.float32(1.0 / math.sqrt(d))))
    step.extra.update(
        shared_prefix=shared_prefix,
        fork_tables=tables_array(forks) if forks else None,
        fork_lengths=np.array([lengths[i] - 1 for i in range(num_writers)],
                              dtype=np.int32),
        refcounts=pool.ref.copy(),
        decode_lengths=np.array(lengths, dtype=np.int32))
    return step.check()


BUILDERS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}
