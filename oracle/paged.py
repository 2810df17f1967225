"""Paged KV cache operations and paged attention, fp64, one element at a time.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources ("the pages"):
  [Anatomy]   "vLLM 引擎解剖" (oripoin.cn)
  [Overview]  "01. vLLM：从分页 KV 起家的通用推理引擎" (niuwancheng.cn)
  [V0/V1]     "v1/v0 区别" (llm.rainlin.net)

Conventions (the pages leave the in-block layout open; this is the reading
used throughout):
  * block size 16 tokens ([Anatomy] "PagedAttention：为 KV 缓存分页";
    [Overview] "KV 缓存管理与前缀缓存", the --block-size row);
  * per layer, K and V caches are each ``[num_blocks][num_kv_heads][16][D]``:
    one (block, kv head) tile is contiguous; ``cache_tile`` below is the only
    place that indexes a cache, so a different layout changes one function;
  * a query head ``h`` reads kv head ``h // (Hq // Hkv)`` (grouped-query
    attention, [Anatomy] "KV 缓存需要多少内存？");
  * token position ``p`` of a sequence lives in slot
    ``block_table[p // 16] * 16 + p % 16`` ([Anatomy] Fig. 2: A's tokens
    32-39 sit in its third block, physical block 2);
  * a query at position ``p`` attends to keys ``0..p`` inclusive: every token
    is compared with all tokens before it, and its own K/V are written to the
    cache before attention reads it ([Anatomy] "预填充、解码与三个时延指标").
"""

import math

import numpy as np

from .formats import (
    BF16,
    F32,
    FP8_E4M3,
    int4_quantize_row,
    int4_rows_to_f64,
    nvfp4_quantize_row,
    nvfp4_rows_to_f64,
    quantise_to_e4m3,
    storage_to_f64,
)

BLOCK_SIZE = 16


# --------------------------------------------------------------------------
# Sizes
# --------------------------------------------------------------------------

def kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_elem):
    """Bytes of KV cache one token occupies: key and value (factor 2) x bytes
    per element x layers x KV heads x head dim ([Anatomy] "KV 缓存需要多少内存？",
    the formula above Table 1)."""
    return 2 * bytes_per_elem * layers * kv_heads * head_dim


def blocks_needed(num_tokens):
    """Blocks a sequence of ``num_tokens`` tokens occupies: blocks are handed
    out as tokens arrive, so only the last one can be partly empty
    ([Anatomy] "PagedAttention：为 KV 缓存分页")."""
    return (int(num_tokens) + BLOCK_SIZE - 1) // BLOCK_SIZE


# --------------------------------------------------------------------------
# Slot mapping (token position -> physical slot)
# --------------------------------------------------------------------------

def slot_of(block_table_row, position):
    """Physical slot of logical token ``position`` through one sequence's
    block table ([Anatomy] Fig. 2)."""
    position = int(position)
    block = int(block_table_row[position // BLOCK_SIZE])
    return block * BLOCK_SIZE + position % BLOCK_SIZE


def slot_mapping(block_tables, query_start_loc, num_computed_tokens):
    """Slot of every token scheduled this step.

    The step is the unified schedule {request: num_tokens}
    ([Anatomy] "V1：统一调度预填充与解码"; [V0/V1] §3.1 "Token 预算"): request
    ``r`` contributes tokens ``query_start_loc[r] .. query_start_loc[r+1]-1``
    of the flattened batch, and its ``i``-th new token sits at position
    ``num_computed_tokens[r] + i``.
    """
    qsl = [int(x) for x in query_start_loc]
    out = []
    for r in range(len(qsl) - 1):
        for i in range(qsl[r + 1] - qsl[r]):
            p = int(num_computed_tokens[r]) + i
            out.append(slot_of(block_tables[r], p))
    return np.array(out, dtype=np.int64)


# --------------------------------------------------------------------------
# Cache writes and block copies
# --------------------------------------------------------------------------

def cache_tile(cache, block, kv_head):
    """The ``[16][D]`` tile of one (physical block, kv head)."""
    return cache[block, kv_head]


def _encode_row(src_row, src_dtype, cache_dtype, scale):
    """One token's K or V for one kv head, as the cache stores it."""
    if src_dtype == cache_dtype:
        return np.array(src_row, copy=True)
    if cache_dtype == FP8_E4M3:
        if src_dtype == F32:
            x = np.asarray(src_row, dtype=np.float32)
        elif src_dtype == BF16:
            x = storage_to_f64(src_row, BF16).astype(np.float32)  # exact
        else:
            raise ValueError(src_dtype)
        return quantise_to_e4m3(x, scale)
    raise ValueError(f"unsupported write {src_dtype} -> {cache_dtype}")


def reshape_and_cache(key, value, k_cache, v_cache, slots, src_dtype,
                      cache_dtype, k_scale=1.0, v_scale=1.0):
    """Write each scheduled token's K and V into its slot; returns new caches.

    The prefill pass computes every prompt token's K and V and stores them in
    the cache; decode reads them back ([Anatomy] "预填充、解码与三个时延指标").
    ``key``/``value`` are ``[T][Hkv][D]``; a negative slot means "skip this
    token".  Equal dtypes copy the bits; a bf16/fp32 source into an fp8 cache
    is quantised with the per-tensor scale.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    num_kv_heads = k_out.shape[1]
    for t in range(len(slots)):
        slot = int(slots[t])
        if slot < 0:
            continue
        block, offset = divmod(slot, BLOCK_SIZE)
        for h in range(num_kv_heads):
            cache_tile(k_out, block, h)[offset] = _encode_row(
                key[t, h], src_dtype, cache_dtype, k_scale)
            cache_tile(v_out, block, h)[offset] = _encode_row(
                value[t, h], src_dtype, cache_dtype, v_scale)
    return k_out, v_out


def copy_blocks(k_caches, v_caches, block_mapping):
    """Copy whole physical blocks (all kv heads, all 16 slots) for every layer.

    A block shared by several sequences is read-only; a sequence about to
    write into one gets a private copy and only its own block table is
    repointed ([Anatomy] "PagedAttention：为 KV 缓存分页", copy-on-write).  V0
    carried these copies as ``blocks_to_copy`` in each step's execute request
    ([V0/V1] §2.1 "V0 引擎循环").

    Precondition (checked): destinations are distinct and none of them is
    also a source, so the result does not depend on the order of the pairs.
    Returns new lists of caches.
    """
    pairs = [(int(s), int(d)) for s, d in np.asarray(block_mapping).reshape(-1, 2)]
    dsts = [d for _, d in pairs]
    srcs = {s for s, _ in pairs}
    assert len(set(dsts)) == len(dsts), "copy destinations must be distinct"
    assert not (set(dsts) & srcs), "a copy destination may not also be a source"
    k_new = [np.array(c, copy=True) for c in k_caches]
    v_new = [np.array(c, copy=True) for c in v_caches]
    for src, dst in pairs:
        for layer in range(len(k_new)):
            k_new[layer][dst] = k_caches[layer][src]
            v_new[layer][dst] = v_caches[layer][src]
    return k_new, v_new


def swap_blocks(src_k_caches, src_v_caches, dst_k_caches, dst_v_caches, block_mapping):
    """Copy whole blocks from one cache pool into another, every layer, K and
    V: pair (s, d) sets dst[d] = src[s].  This is the V0 engine's swap of a
    request's KV blocks between GPU memory and CPU memory ([Anatomy] "抢占：
    RECOMPUTE", the v0 SWAP mode and its --swap-space; [V0/V1] §2.1 "V0 引擎
    循环", blocks_to_swap_in / blocks_to_swap_out next to blocks_to_copy), and
    of today's KV offloading to CPU memory ([Overview] "KV 缓存管理与前缀缓存",
    --kv-offloading-size).  Which pool lives where does not change the bytes.

    Precondition (checked): destinations are distinct.  Returns new lists of
    destination caches.
    """
    pairs = [(int(s), int(d)) for s, d in np.asarray(block_mapping).reshape(-1, 2)]
    dsts = [d for _, d in pairs]
    assert len(set(dsts)) == len(dsts), "swap destinations must be distinct"
    k_new = [np.array(c, copy=True) for c in dst_k_caches]
    v_new = [np.array(c, copy=True) for c in dst_v_caches]
    for src, dst in pairs:
        for layer in range(len(k_new)):
            k_new[layer][dst] = src_k_caches[layer][src]
            v_new[layer][dst] = src_v_caches[layer][src]
    return k_new, v_new


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def gather_kv(cache, dtype, scale, block_table_row, length, kv_head):
    """K (or V) rows ``0..length-1`` of one sequence and kv head, in float64,
    gathered logical block by logical block through the block table
    ([Anatomy] Fig. 2: the table maps logical to physical blocks)."""
    rows = []
    for j in range(blocks_needed(length)):
        block = int(block_table_row[j])
        n = min(BLOCK_SIZE, length - j * BLOCK_SIZE)
        tile = cache_tile(cache, block, kv_head)
        rows.append(storage_to_f64(tile[:n], dtype, scale))
    if not rows:
        return np.zeros((0, cache.shape[-1]), dtype=np.float64)
    return np.concatenate(rows, axis=0)


def attention_row(q, keys, values, softmax_scale):
    """softmax(q . K^T * scale) V for one query vector, float64.

    The max is subtracted before exponentiating so that nothing overflows; the
    result is the same real number."""
    x = (keys @ q) * softmax_scale
    m = np.max(x)
    w = np.exp(x - m)
    return (w @ values) / np.sum(w)


def _as_f32_param(x):
    # Scalars cross the library boundary as binary32; the oracle uses the
    # same binary32 values.
    return float(np.float32(x))


def decode_attention(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                     context_lens, softmax_scale, k_scale=1.0, v_scale=1.0):
    """Decode: one query token per sequence attends to its whole paged KV
    history ([Anatomy] "预填充、解码与三个时延指标": decode streams the whole KV
    cache each step; "PagedAttention：为 KV 缓存分页").

    ``q`` is ``[S][Hq][D]`` storage; ``context_lens[s]`` counts the tokens the
    query sees, its own included.  A sequence with length 0 yields zeros.
    Returns float64 ``[S][Hq][D]``.
    """
    num_seqs, num_q_heads, head_dim = q.shape
    num_kv_heads = k_cache.shape[1]
    group = num_q_heads // num_kv_heads
    scale = _as_f32_param(softmax_scale)
    ks, vs = _as_f32_param(k_scale), _as_f32_param(v_scale)
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        length = int(context_lens[s])
        if length == 0:
            continue
        for kvh in range(num_kv_heads):
            keys = gather_kv(k_cache, kv_dtype, ks, block_tables[s], length, kvh)
            values = gather_kv(v_cache, kv_dtype, vs, block_tables[s], length, kvh)
            for h in range(kvh * group, (kvh + 1) * group):
                qv = storage_to_f64(q[s, h], q_dtype)
                out[s, h] = attention_row(qv, keys, values, scale)
    return out


def decode_attention_one(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                         context_lens, softmax_scale, seq, head,
                         k_scale=1.0, v_scale=1.0):
    """One (sequence, q head) element of ``decode_attention`` (float64 [D]);
    used to check large launches on a sample of outputs."""
    num_q_heads = q.shape[1]
    num_kv_heads = k_cache.shape[1]
    kvh = head // (num_q_heads // num_kv_heads)
    length = int(context_lens[seq])
    if length == 0:
        return np.zeros(q.shape[-1], dtype=np.float64)
    keys = gather_kv(k_cache, kv_dtype, _as_f32_param(k_scale),
                     block_tables[seq], length, kvh)
    values = gather_kv(v_cache, kv_dtype, _as_f32_param(v_scale),
                       block_tables[seq], length, kvh)
    qv = storage_to_f64(q[seq, head], q_dtype)
    return attention_row(qv, keys, values, _as_f32_param(softmax_scale))


def prefill_attention_one(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                          query_start_loc, num_computed_tokens, softmax_scale,
                          row, head, k_scale=1.0, v_scale=1.0):
    """One (query row, q head) element of ``prefill_attention`` (float64 [D]);
    used to check large launches on a sample of outputs."""
    qsl = [int(x) for x in query_start_loc]
    r = max(i for i in range(len(qsl) - 1) if qsl[i] <= row < qsl[i + 1])
    p = int(num_computed_tokens[r]) + (row - qsl[r])
    num_q_heads = q.shape[1]
    kvh = head // (num_q_heads // k_cache.shape[1])
    keys = gather_kv(k_cache, kv_dtype, _as_f32_param(k_scale),
                     block_tables[r], p + 1, kvh)
    values = gather_kv(v_cache, kv_dtype, _as_f32_param(v_scale),
                       block_tables[r], p + 1, kvh)
    qv = storage_to_f64(q[row, head], q_dtype)
    return attention_row(qv, keys, values, _as_f32_param(softmax_scale))


def prefill_attention(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                      query_start_loc, num_computed_tokens, softmax_scale,
                      k_scale=1.0, v_scale=1.0):
    """Chunked prefill: request ``r`` brings ``n_r`` new query tokens at
    positions ``c_r .. c_r + n_r - 1`` (``c_r`` = tokens already computed,
    e.g. a prefix-cache hit); the query at position ``p`` attends to keys
    ``0..p`` through the request's block table ([Anatomy] "V1：统一调度预填充与
    解码" (chunked prefill, Fig. 3); [V0/V1] §3.1 "Token 预算": attention
    metadata is query length, context length and block table per request).

    Each query row is computed on its own, as a decode row with context length
    ``p + 1``.  ``q`` is ``[Tq][Hq][D]``; returns float64 ``[Tq][Hq][D]``.
    """
    total, num_q_heads, head_dim = q.shape
    num_kv_heads = k_cache.shape[1]
    group = num_q_heads // num_kv_heads
    scale = _as_f32_param(softmax_scale)
    ks, vs = _as_f32_param(k_scale), _as_f32_param(v_scale)
    out = np.zeros((total, num_q_heads, head_dim), dtype=np.float64)
    qsl = [int(x) for x in query_start_loc]
    for r in range(len(qsl) - 1):
        n = qsl[r + 1] - qsl[r]
        if n == 0:
            continue
        c = int(num_computed_tokens[r])
        full = c + n
        for kvh in range(num_kv_heads):
            keys = gather_kv(k_cache, kv_dtype, ks, block_tables[r], full, kvh)
            values = gather_kv(v_cache, kv_dtype, vs, block_tables[r], full, kvh)
            for i in range(n):
                p = c + i
                for h in range(kvh * group, (kvh + 1) * group):
                    qv = storage_to_f64(q[qsl[r] + i, h], q_dtype)
                    out[qsl[r] + i, h] = attention_row(
                        qv, keys[: p + 1], values[: p + 1], scale)
    return out


def contiguous_attention(queries, keys, values, softmax_scale, first_position=None):
    """Dense attention on contiguous float64 arrays, no block table at all:
    ``queries [n][D]``, ``keys/values [L][D]``.  With ``first_position`` set,
    query ``i`` sits at position ``first_position + i`` and only sees keys up
    to it (causal); otherwise every query sees every key.  Only used to pin the
    paged gather."""
    scores = (queries @ keys.T) * softmax_scale
    if first_position is not None:
        pos_q = first_position + np.arange(queries.shape[0])[:, None]
        pos_k = np.arange(keys.shape[0])[None, :]
        scores = np.where(pos_k <= pos_q, scores, -np.inf)
    scores = scores - scores.max(axis=1, keepdims=True)
    w = np.exp(scores)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ values


# --------------------------------------------------------------------------
# Split-context partitions and their log-sum-exp combine
# --------------------------------------------------------------------------

def partition_state(q, keys, values, softmax_scale):
    """(m, l, o) of one partition: running max of the scaled scores, the sum
    of exp(score - m), and the unnormalised weighted sum of values."""
    x = (keys @ q) * softmax_scale
    m = np.max(x)
    w = np.exp(x - m)
    return m, np.sum(w), w @ values


def combine_partitions(states):
    """Merge partition states (m_k, l_k, o_k): with M the largest m_k,
    out = sum_k e^{m_k - M} o_k  /  sum_k e^{m_k - M} l_k."""
    big_m = max(m for m, _, _ in states)
    num = sum(math.exp(m - big_m) * o for m, _, o in states)
    den = sum(math.exp(m - big_m) * l for m, l, _ in states)
    return num / den


def split_attention_row(q, keys, values, softmax_scale, partition_len):
    """attention_row computed partition by partition and merged."""
    states = []
    for start in range(0, keys.shape[0], partition_len):
        states.append(partition_state(q, keys[start:start + partition_len],
                                      values[start:start + partition_len],
                                      softmax_scale))
    return combine_partitions(states)


# --- int4 per token-head caches (encoding: oracle/formats.py) -------------
# A cache holds packed codes [num_blocks][num_kv_heads][16][D/2] (uint8) and
# a parallel scale array [num_blocks][num_kv_heads][16] (binary32).


def reshape_and_cache_int4(key, value, k_cache, v_cache, k_scales, v_scales, slots,
                           src_dtype):
    """reshape_and_cache into int4 caches: each token's K and V row of each
    kv head is quantised with its own scale.  Returns the four new arrays."""
    outs = [np.array(a, copy=True) for a in (k_cache, v_cache, k_scales, v_scales)]
    kc, vc, ksc, vsc = outs
    for t in range(len(slots)):
        slot = int(slots[t])
        if slot < 0:
            continue
        block, offset = divmod(slot, BLOCK_SIZE)
        for h in range(kc.shape[1]):
            for src, cache, scales in ((key, kc, ksc), (value, vc, vsc)):
                x = storage_to_f64(src[t, h], src_dtype).astype(np.float32)   # exact
                cache[block, h, offset], scales[block, h, offset] = int4_quantize_row(x)
    return kc, vc, ksc, vsc


def gather_kv_int4(cache, scales, block_table_row, length, kv_head):
    """Rows 0..length-1 of one sequence and kv head from an int4 cache, float64."""
    rows = []
    for j in range(blocks_needed(length)):
        block = int(block_table_row[j])
        n = min(BLOCK_SIZE, length - j * BLOCK_SIZE)
        rows.append(int4_rows_to_f64(cache[block, kv_head][:n], scales[block, kv_head][:n]))
    if not rows:
        return np.zeros((0, 2 * cache.shape[-1]), dtype=np.float64)
    return np.concatenate(rows, axis=0)


def decode_attention_int4(q, q_dtype, k_cache, v_cache, k_scales, v_scales, block_tables,
                          context_lens, softmax_scale):
    """decode_attention over int4 caches (float64 [S][Hq][D])."""
    num_seqs, num_q_heads, head_dim = q.shape
    num_kv_heads = k_cache.shape[1]
    group = num_q_heads // num_kv_heads
    scale = _as_f32_param(softmax_scale)
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        length = int(context_lens[s])
        if length == 0:
            continue
        for kvh in range(num_kv_heads):
            keys = gather_kv_int4(k_cache, k_scales, block_tables[s], length, kvh)
            values = gather_kv_int4(v_cache, v_scales, block_tables[s], length, kvh)
            for h in range(kvh * group, (kvh + 1) * group):
                out[s, h] = attention_row(storage_to_f64(q[s, h], q_dtype), keys, values, scale)
    return out


def decode_attention_int4_one(q, q_dtype, k_cache, v_cache, k_scales, v_scales,
                              block_tables, context_lens, softmax_scale, seq, head):
    """One (sequence, q head) element of decode_attention_int4."""
    kvh = head // (q.shape[1] // k_cache.shape[1])
    length = int(context_lens[seq])
    if length == 0:
        return np.zeros(q.shape[-1])
    keys = gather_kv_int4(k_cache, k_scales, block_tables[seq], length, kvh)
    values = gather_kv_int4(v_cache, v_scales, block_tables[seq], length, kvh)
    return attention_row(storage_to_f64(q[seq, head], q_dtype), keys, values,
                         _as_f32_param(softmax_scale))


# --- sliding-window decode --------------------------------------------------
# For sliding-window layers only the most recent tokens are attended to, and
# the blocks that fall out of the window can be released early ("01. vLLM",
# section "KV 缓存管理与前缀缓存", the hybrid KV cache manager paragraph).
# Reading: a query at position L-1 sees the `window` positions
# max(0, L - window) .. L-1, its own included.


def window_start(length, window):
    """First position a decode query of a length-`length` sequence sees."""
    return max(0, int(length) - int(window))


def decode_attention_window(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                            context_lens, softmax_scale, window, k_scale=1.0, v_scale=1.0):
    """decode_attention restricted to each sequence's last `window` tokens."""
    num_seqs, num_q_heads, head_dim = q.shape
    num_kv_heads = k_cache.shape[1]
    group = num_q_heads // num_kv_heads
    scale = _as_f32_param(softmax_scale)
    ks, vs = _as_f32_param(k_scale), _as_f32_param(v_scale)
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        length = int(context_lens[s])
        if length == 0:
            continue
        first = window_start(length, window)
        for kvh in range(num_kv_heads):
            keys = gather_kv(k_cache, kv_dtype, ks, block_tables[s], length, kvh)[first:]
            values = gather_kv(v_cache, kv_dtype, vs, block_tables[s], length, kvh)[first:]
            for h in range(kvh * group, (kvh + 1) * group):
                out[s, h] = attention_row(storage_to_f64(q[s, h], q_dtype), keys, values, scale)
    return out


# --- nvfp4-style caches (encoding: oracle/formats.py) -----------------------
# Codes [num_blocks][num_kv_heads][16][D/2] (uint8), block scale codes
# [num_blocks][num_kv_heads][16][D/16] (E4M3 bytes), per-tensor k/v scales.


def reshape_and_cache_nvfp4(key, value, k_cache, v_cache, k_bscales, v_bscales, slots,
                            src_dtype, k_scale, v_scale):
    """reshape_and_cache into nvfp4 caches; returns the four new arrays."""
    kc, vc, ksc, vsc = [np.array(a, copy=True) for a in (k_cache, v_cache, k_bscales, v_bscales)]
    for t in range(len(slots)):
        slot = int(slots[t])
        if slot < 0:
            continue
        block, offset = divmod(slot, BLOCK_SIZE)
        for h in range(kc.shape[1]):
            for src, cache, sc, g in ((key, kc, ksc, k_scale), (value, vc, vsc, v_scale)):
                x = storage_to_f64(src[t, h], src_dtype).astype(np.float32)   # exact
                cache[block, h, offset], sc[block, h, offset] = nvfp4_quantize_row(x, g)
    return kc, vc, ksc, vsc


def gather_kv_nvfp4(cache, bscales, g, block_table_row, length, kv_head):
    rows = []
    for j in range(blocks_needed(length)):
        block = int(block_table_row[j])
        n = min(BLOCK_SIZE, length - j * BLOCK_SIZE)
        rows.append(nvfp4_rows_to_f64(cache[block, kv_head][:n], bscales[block, kv_head][:n], g))
    if not rows:
        return np.zeros((0, 2 * cache.shape[-1]), dtype=np.float64)
    return np.concatenate(rows, axis=0)


def decode_attention_nvfp4(q, q_dtype, k_cache, v_cache, k_bscales, v_bscales, block_tables,
                           context_lens, softmax_scale, k_scale, v_scale):
    """decode_attention over nvfp4 caches (float64 [S][Hq][D])."""
    num_seqs, num_q_heads, head_dim = q.shape
    num_kv_heads = k_cache.shape[1]
    group = num_q_heads // num_kv_heads
    scale = _as_f32_param(softmax_scale)
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        length = int(context_lens[s])
        if length == 0:
            continue
        for kvh in range(num_kv_heads):
            keys = gather_kv_nvfp4(k_cache, k_bscales, k_scale, block_tables[s], length, kvh)
            values = gather_kv_nvfp4(v_cache, v_bscales, v_scale, block_tables[s], length, kvh)
            for h in range(kvh * group, (kvh + 1) * group):
                out[s, h] = attention_row(storage_to_f64(q[s, h], q_dtype), keys, values, scale)
    return out
