"""The workloads at full size, in the launch configuration bench.py times,
against the fp64 oracle on every output (the 32-layer MHA step, whose cache
is 128 GiB, on a seeded sample of its (layer, sequence) pairs).

Inputs are generated on the GPU (the bench's generators); the caches are
copied to the host before any GPU call writes them (``snapshot``), the
oracle applies the step's copies and writes itself, and its attention runs
in a pool of host worker processes (``oracle_pool``), one unit per
(sequence or request, kv head).
"""

import numpy as np
import pytest
import torch

import oracle_pool as OP
import paged_kv_cache_84_amd as pk
from gpu_util import announce, as_f64, host, oracle_caches_after_step, snapshot
from oracle import formats as F
from oracle import paged as P
from synth import configs as C
from tolerance import assert_attention_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def restore(step):
    """Put the snapshot's cache bytes back on the device."""
    for dev, saved in ((step.k_caches, step.extra["host_k"]),
                       (step.v_caches, step.extra["host_v"])):
        for t, h in zip(dev, saved):
            t.view(torch.uint8).copy_(torch.from_numpy(np.ascontiguousarray(h).view(np.uint8))
                                      .view(t.view(torch.uint8).shape))


def test_llama3_8b_decode_step_every_output():
    """The Llama-3.1-8B decode batch (64 sequences, 512..4096 tokens, 32 q /
    8 kv heads, bf16) through paged_attention_decode_append, the call the
    benchmark times: cache bytes after the new tokens' writes equal the
    oracle's, all 2,048 (sequence, head) outputs within tolerance, and a
    second call is bitwise identical."""
    announce("fullsize 8B decode step, every output")
    s = snapshot(C.config2(device=DEV))
    ds = pk.step.DeviceStep(s)
    ds.run_decode_append()
    torch.cuda.synchronize()
    first = ds.out[0].clone()
    ds.run_decode_append()
    torch.cuda.synchronize()
    assert torch.equal(first, ds.out[0])
    rk, rv, _ = oracle_caches_after_step(s)
    assert np.array_equal(host(ds.k_caches[0]), rk)
    assert np.array_equal(host(ds.v_caches[0]), rv)
    announce("  oracle, every output")
    ref = OP.decode_reference(host(s.q[0]), rk, rv, s.decode_block_tables,
                              s.decode_context_lens, F.BF16, F.BF16, s.softmax_scale)
    assert_attention_close(as_f64(first), ref, "bf16", "8B decode step, every output")


@pytest.fixture(scope="module")
def mixed_step():
    """The full mixed step and the oracle's caches and outputs for it."""
    announce("fullsize mixed step: inputs and oracle")
    s = snapshot(C.config4(device=DEV))
    rk, rv, slots = oracle_caches_after_step(s)
    q = host(s.q[0])
    t = s.num_prefill_tokens
    pre = OP.prefill_reference(q[:t], rk, rv, s.prefill_block_tables,
                               s.prefill_query_start_loc, s.prefill_num_computed,
                               F.BF16, F.BF16, s.softmax_scale)
    dec = OP.decode_reference(q[t:], rk, rv, s.decode_block_tables, s.decode_context_lens,
                              F.BF16, F.BF16, s.softmax_scale)
    return s, rk, rv, slots, pre, dec


def test_mixed_step_every_output(mixed_step):
    """The mixed step (64 x 100-token chunks on the 125-block shared prefix,
    a 1,022-token first chunk, 192 decodes up to 8,192 tokens, 64
    copy-on-write copies) as two calls: slots and cache bytes exact, all
    7,422 x 32 chunk rows and 192 x 32 decode outputs within tolerance."""
    s, rk, rv, slots, pre, dec = mixed_step
    announce("fullsize mixed step, two calls")
    restore(s)
    ds = pk.step.DeviceStep(s)
    ds.run()
    torch.cuda.synchronize()
    assert np.array_equal(ds.slots.cpu().numpy(), slots)
    assert np.array_equal(host(ds.k_caches[0]), rk)
    assert np.array_equal(host(ds.v_caches[0]), rv)
    t = s.num_prefill_tokens
    got = as_f64(ds.out[0])
    assert_attention_close(got[:t], pre, "bf16", "mixed step, every chunk row")
    assert_attention_close(got[t:], dec, "bf16", "mixed step, every decode")


def test_mixed_step_unified_every_output(mixed_step):
    """The same step with the unified varlen launch, as the bench times it."""
    s, rk, rv, slots, pre, dec = mixed_step
    announce("fullsize mixed step, unified launch")
    restore(s)
    ds = pk.step.DeviceStep(s)
    ds.run_varlen()
    torch.cuda.synchronize()
    assert np.array_equal(host(ds.k_caches[0]), rk)
    t = s.num_prefill_tokens
    got = as_f64(ds.out[0])
    assert_attention_close(got[:t], pre, "bf16", "unified, every chunk row")
    assert_attention_close(got[t:], dec, "bf16", "unified, every decode")


def test_llama70b_fp8_long_context_every_output():
    """6 x 131,072 tokens, 64 q / 8 kv heads, fp8 cache, 512-token
    partitions with the log-sum-exp merge, through the fused write-and-decode
    call the benchmark times: cache bytes (the six new tokens quantised)
    equal the oracle's, all 384 outputs within tolerance, a second call
    bitwise identical."""
    announce("fullsize 70B fp8 long context, every output")
    s = snapshot(C.config5(device=DEV))
    ds = pk.step.DeviceStep(s, partition_tokens=512)
    ds.run_decode_append()
    torch.cuda.synchronize()
    first = ds.out[0].clone()
    ds.run_decode_append()
    torch.cuda.synchronize()
    assert torch.equal(first, ds.out[0])
    rk, rv, _ = oracle_caches_after_step(s)
    assert np.array_equal(host(ds.k_caches[0]), rk)
    assert np.array_equal(host(ds.v_caches[0]), rv)
    announce("  oracle, every output")
    ref = OP.decode_reference(host(s.q[0]), rk, rv, s.decode_block_tables,
                              s.decode_context_lens, F.BF16, F.FP8_E4M3, s.softmax_scale,
                              s.k_scale, s.v_scale)
    assert_attention_close(as_f64(first), ref, "fp8_e4m3", "70B fp8, every output")


def test_llama2_mha_32_layers_sampled():
    """32 layers x 32 sequences x 8,192 tokens, 32 q = 32 kv heads, bf16,
    one fused write-and-decode call per layer as the benchmark runs it.  The
    cache is 128 GiB, so the oracle covers layer 0 for all 32 sequences and
    8 seeded (layer, sequence) pairs, every head of each: their blocks are
    copied out before the step, the oracle writes the new token into that
    copy (its own slot formula on the copy's identity table) and evaluates
    every head."""
    announce("fullsize 32-layer MHA step, sampled (layer, sequence) pairs")
    s = C.config3(device=DEV)
    rng = np.random.default_rng(33)
    pairs = [(0, q) for q in range(32)] + [(int(a), int(b)) for a, b in
                                          zip(rng.integers(1, 32, 8), rng.integers(0, 32, 8))]
    nb = P.blocks_needed(int(s.decode_context_lens[0]))
    saved = {}
    for layer, seq in pairs:
        ids = torch.as_tensor(s.decode_block_tables[seq, :nb].astype(np.int64), device=DEV)
        saved[(layer, seq)] = (host(s.k_caches[layer][ids]), host(s.v_caches[layer][ids]))
    ds = pk.step.DeviceStep(s)
    ds.run_decode_append()
    torch.cuda.synchronize()
    announce("  oracle on", len(pairs), "pairs")
    ident = np.arange(nb, dtype=np.int32)[None, :]
    units, where = [], []
    for layer, seq in pairs:
        kc, vc = saved[(layer, seq)]
        length = int(s.decode_context_lens[seq])
        slot = np.array([P.slot_of(ident[0], length - 1)], np.int64)
        kc, vc = P.reshape_and_cache(host(s.new_k[layer][seq:seq + 1]),
                                     host(s.new_v[layer][seq:seq + 1]), kc, vc, slot,
                                     F.BF16, F.BF16)
        q = host(s.q[layer][seq:seq + 1])
        u, _ = OP.decode_units(q, kc, vc, ident, np.array([length]), 1, F.BF16, F.BF16,
                               s.softmax_scale)
        units += u
        where += [(layer, seq)] * len(u)
    res = OP.run(OP.decode_unit, units)
    ref = np.stack([np.concatenate(res[i:i + 32]) for i in range(0, len(res), 32)])
    got = np.stack([as_f64(ds.out[layer][seq]) for layer, seq in pairs])
    assert_attention_close(got, ref, "bf16", "32-layer MHA, sampled pairs")
