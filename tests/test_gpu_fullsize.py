"""Full-size decode workloads in the launch configuration bench.py times,
checked on sampled outputs against the fp64 oracle.

The 32-layer Llama-2-7B-shaped MHA step holds 128 GiB of KV cache and the
Llama-3.1-70B-shaped long-context batch 1.6 GB, so the oracle does not read
the whole cache: for each sampled (layer, sequence, q head) it gathers that
sequence's blocks of the matching kv head (the generator's bytes, copied as
they are) into a compact cache with an identity block table and evaluates
the one output element there.  Decode-only, like the bench legs: the caches
hold the generator's values and no token is written first.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_84_amd as pk
from gpu_util import announce, as_f64, host
from oracle import paged as P
from synth import configs as C
from tolerance import assert_attention_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def compact_reference(step, layer, seq, head):
    """Oracle output of (seq, head) from the sequence's own blocks only."""
    hq, hkv = step.num_q_heads, step.num_kv_heads
    kvh = head // (hq // hkv)
    length = int(step.decode_context_lens[seq])
    nb = P.blocks_needed(length)
    ids = torch.as_tensor(step.decode_block_tables[seq, :nb].astype(np.int64), device=DEV)
    kc = host(step.k_caches[layer][ids, kvh].unsqueeze(1).contiguous())   # [nb][1][16][D]
    vc = host(step.v_caches[layer][ids, kvh].unsqueeze(1).contiguous())
    q = host(step.q[layer][seq:seq + 1, head:head + 1].contiguous())      # [1][1][D]
    table = np.arange(nb, dtype=np.int32)[None, :]
    return P.decode_attention_one(q, step.q_dtype, kc, vc, step.kv_dtype, table,
                                  np.array([length], np.int32), step.softmax_scale, 0, 0,
                                  step.k_scale, step.v_scale)


def test_llama70b_fp8_long_context_full_size_sampled():
    """6 x 131,072 tokens, 64 q / 8 kv heads, fp8 cache, 512-token partitions
    and the log-sum-exp merge; 16 sampled (sequence, head) outputs, and the
    same outputs bitwise on a second call."""
    announce("decode config5 full size, 512-token partitions")
    s = C.config5(device=DEV)
    ds = pk.step.DeviceStep(s, partition_tokens=512)
    ds.decode(0)
    torch.cuda.synchronize()
    first = ds.out[0].clone()
    ds.decode(0)
    torch.cuda.synchronize()
    assert torch.equal(first, ds.out[0])
    rng = np.random.default_rng(55)
    got, ref = [], []
    for seq, head in zip(rng.integers(0, 6, 16), rng.integers(0, 64, 16)):
        announce("  sample seq", int(seq), "head", int(head))
        ref.append(compact_reference(s, 0, int(seq), int(head)))
        got.append(as_f64(first[seq, head]))
    assert_attention_close(np.array(got), np.array(ref), "fp8_e4m3", "config5 sampled")


def test_llama2_mha_32_layers_full_size_sampled():
    """32 layers x 32 sequences x 8,192 tokens, 32 q = 32 kv heads, bf16, the
    library's own split; 16 sampled (layer, sequence, head) outputs."""
    announce("decode config3 full size, 32 layers")
    s = C.config3(device=DEV)
    ds = pk.step.DeviceStep(s)
    for layer in range(s.num_layers):
        ds.decode(layer)
    torch.cuda.synchronize()
    rng = np.random.default_rng(33)
    got, ref = [], []
    for layer, seq, head in zip(rng.integers(0, 32, 16), rng.integers(0, 32, 16),
                                rng.integers(0, 32, 16)):
        announce("  sample layer", int(layer), "seq", int(seq), "head", int(head))
        ref.append(compact_reference(s, int(layer), int(seq), int(head)))
        got.append(as_f64(ds.out[layer][seq, head]))
    assert_attention_close(np.array(got), np.array(ref), "bf16", "config3 sampled")
