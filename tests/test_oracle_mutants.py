"""Plant plausible mistakes in the oracle (on the CPU only) and check that at
least one pin catches each: the pins are strong enough to trust the oracle."""

import numpy as np
import pytest

import oracle_pins as pins
from oracle import formats as F
from oracle import paged as P


def _drop_last(q, keys, values, scale):
    if len(keys) > 1:
        keys, values = keys[:-1], values[:-1]
    x = (keys @ q) * scale
    w = np.exp(x - x.max())
    return (w @ values) / w.sum()


def _wrong_sign(q, keys, values, scale):
    x = (keys @ q) * scale
    w = np.exp(x.min() - x)
    return (w @ values) / w.sum()


def _no_scale(q, keys, values, scale):
    x = keys @ q
    w = np.exp(x - x.max())
    return (w @ values) / w.sum()


def _scores_from_values(q, keys, values, scale):
    x = (values @ q) * scale
    w = np.exp(x - x.max())
    return (w @ values) / w.sum()


def _slot_next_block(row, position):
    position = int(position)
    return int(row[(position // P.BLOCK_SIZE + 1) % len(row)]) * P.BLOCK_SIZE + position % P.BLOCK_SIZE


def _slot_wrong_offset(row, position):
    position = int(position)
    return int(row[position // P.BLOCK_SIZE]) * P.BLOCK_SIZE + (position + 1) % P.BLOCK_SIZE


def _kv_bytes_no_two(layers, kv_heads, head_dim, bpe):
    return bpe * layers * kv_heads * head_dim


def _gather_reversed_blocks(cache, dtype, scale, row, length, kv_head):
    rows = []
    nblk = P.blocks_needed(length)
    for j in range(nblk):
        block = int(row[nblk - 1 - j])
        n = min(P.BLOCK_SIZE, length - j * P.BLOCK_SIZE)
        rows.append(F.storage_to_f64(cache[block, kv_head][:n], dtype, scale))
    return np.concatenate(rows) if rows else np.zeros((0, cache.shape[-1]))


def _combine_no_rescale(states):
    num = sum(o for _, _, o in states)
    den = sum(l for _, l, _ in states)
    return num / den


def _encode_ties_away(y):
    y = np.asarray(y, dtype=np.float32)
    flat = y.reshape(-1)
    out = []
    for v in flat:
        code = F.e4m3_encode_scalar(v)
        mag = abs(float(v))
        if np.isfinite(v) and mag <= F.E4M3_MAX and (code & 0x7F) < 0x7E:
            lo, hi = F.E4M3_TABLE[code & 0x7F], F.E4M3_TABLE[(code & 0x7F) + 1]
            if mag - lo == hi - mag:
                code += 1
        out.append(code)
    return np.array(out, dtype=np.uint8).reshape(y.shape)


_ORIGINAL_ENCODE = F.e4m3_encode


def _encode_no_saturation(y):
    y = np.asarray(y, dtype=np.float32)
    out = _ORIGINAL_ENCODE(np.clip(y, -448, 448))
    big = np.abs(y) > F.E4M3_MAX
    out = out.copy()
    out[big] = 0x7F | (out[big] & 0x80)
    return out


def _copy_only_keys(k_caches, v_caches, block_mapping):
    k_new = [np.array(c, copy=True) for c in k_caches]
    v_new = [np.array(c, copy=True) for c in v_caches]
    for src, dst in np.asarray(block_mapping).reshape(-1, 2):
        for layer in range(len(k_new)):
            k_new[layer][dst] = k_caches[layer][src]
    return k_new, v_new


def _swap_source_index_from_destination(src_k, src_v, dst_k, dst_v, block_mapping):
    k_new = [np.array(c, copy=True) for c in dst_k]
    v_new = [np.array(c, copy=True) for c in dst_v]
    for src, dst in np.asarray(block_mapping).reshape(-1, 2):
        for layer in range(len(k_new)):
            k_new[layer][dst] = src_k[layer][dst % len(src_k[layer])]
            v_new[layer][dst] = src_v[layer][dst % len(src_v[layer])]
    return k_new, v_new


def _write_ignoring_skip(key, value, k_cache, v_cache, slots, src, dst, ks=1.0, vs=1.0):
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    for t in range(len(slots)):
        block, offset = divmod(int(slots[t]), P.BLOCK_SIZE)
        k_out[block, :, offset] = key[t]
        v_out[block, :, offset] = value[t]
    return k_out, v_out


def _prefill_one_without_own_key(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                                 query_start_loc, num_computed_tokens, softmax_scale,
                                 row, head, k_scale=1.0, v_scale=1.0):
    """Off by one: the query at position p sees keys 0..p-1 (its own missing)."""
    qsl = [int(x) for x in query_start_loc]
    r = max(i for i in range(len(qsl) - 1) if qsl[i] <= row < qsl[i + 1])
    p = int(num_computed_tokens[r]) + (row - qsl[r])
    kvh = head // (q.shape[1] // k_cache.shape[1])
    keys = P.gather_kv(k_cache, kv_dtype, k_scale, block_tables[r], max(p, 1), kvh)
    values = P.gather_kv(v_cache, kv_dtype, v_scale, block_tables[r], max(p, 1), kvh)
    return P.attention_row(F.storage_to_f64(q[row, head], q_dtype), keys, values,
                           float(np.float32(softmax_scale)))


def _decode_one_wrong_group(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                            context_lens, softmax_scale, seq, head, k_scale=1.0, v_scale=1.0):
    """Strided instead of consecutive GQA grouping: kv head = h mod Hkv."""
    kvh = head % k_cache.shape[1]
    length = int(context_lens[seq])
    if length == 0:
        return np.zeros(q.shape[-1])
    keys = P.gather_kv(k_cache, kv_dtype, float(np.float32(k_scale)), block_tables[seq],
                       length, kvh)
    values = P.gather_kv(v_cache, kv_dtype, float(np.float32(v_scale)), block_tables[seq],
                         length, kvh)
    return P.attention_row(F.storage_to_f64(q[seq, head], q_dtype), keys, values,
                           float(np.float32(softmax_scale)))


MUTANTS = [
    ("attention_row", P, _drop_last),
    ("attention_row", P, _wrong_sign),
    ("attention_row", P, _no_scale),
    ("attention_row", P, _scores_from_values),
    ("slot_of", P, _slot_next_block),
    ("slot_of", P, _slot_wrong_offset),
    ("kv_bytes_per_token", P, _kv_bytes_no_two),
    ("gather_kv", P, _gather_reversed_blocks),
    ("combine_partitions", P, _combine_no_rescale),
    ("e4m3_encode", F, _encode_ties_away),
    ("e4m3_encode", F, _encode_no_saturation),
    ("copy_blocks", P, _copy_only_keys),
    ("swap_blocks", P, _swap_source_index_from_destination),
    ("reshape_and_cache", P, _write_ignoring_skip),
    ("prefill_attention_one", P, _prefill_one_without_own_key),
    ("decode_attention_one", P, _decode_one_wrong_group),
]


@pytest.mark.parametrize("name,module,mutant", MUTANTS,
                         ids=[f"{n}:{m.__name__}" for n, _, m in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, module, mutant):
    monkeypatch.setattr(module, name, mutant)
    if module is F and name == "e4m3_encode":
        # the paged module imported the quantiser's helpers by name
        monkeypatch.setattr(F, "quantise_to_e4m3",
                            lambda x, s: mutant(np.asarray(x, np.float32) / np.float32(s)))
    caught = pins.failing_pins()
    assert caught, f"no pin catches the planted mistake {mutant.__name__}"


def test_oracle_as_written_passes_every_pin():
    assert pins.failing_pins() == []
