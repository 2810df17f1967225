"""Helpers for the GPU parity tests: move storage tensors to numpy, run the
oracle's pipeline on the same inputs, and print which case is running."""

import sys

import numpy as np
import torch

from oracle import formats as F
from oracle import paged as P
from synth import rng as R

DTYPE_NAME = {torch.float32: F.F32, torch.bfloat16: F.BF16, torch.uint8: F.FP8_E4M3,
              torch.float8_e4m3fn: F.FP8_E4M3}


def announce(*what):
    print("CASE", *what, flush=True)
    sys.stdout.flush()


def host(t):
    return R.to_numpy_storage(t)


def kind_of(step):
    return "fp8_e4m3" if step.kv_dtype == F.FP8_E4M3 else step.q_dtype


def snapshot(step):
    """Keep host copies of the step's caches, taken before any GPU call can
    write them: a step built on the GPU shares its cache tensors with
    DeviceStep, so reading them after the step would feed the GPU's own
    writes into the oracle."""
    step.extra["host_k"] = [host(t) for t in step.k_caches]
    step.extra["host_v"] = [host(t) for t in step.v_caches]
    return step


def oracle_caches_after_step(step, layer=0):
    """Oracle copy -> slot map -> write for one layer, from the step's
    inputs as they were before the GPU step.  Returns (k_cache, v_cache,
    slots)."""
    if "host_k" in step.extra:
        kc, vc = step.extra["host_k"][layer], step.extra["host_v"][layer]
    elif step.k_caches[layer].is_cuda:
        raise AssertionError("a step built on the GPU needs snapshot(step) before it runs")
    else:
        kc = host(step.k_caches[layer])
        vc = host(step.v_caches[layer])
    if len(step.copy_pairs):
        (kc,), (vc,) = P.copy_blocks([kc], [vc], step.copy_pairs)
    slots = P.slot_mapping(step.block_tables, step.query_start_loc, step.num_computed)
    kc, vc = P.reshape_and_cache(host(step.new_k[layer]), host(step.new_v[layer]), kc, vc,
                                 slots, step.q_dtype, step.kv_dtype, step.k_scale,
                                 step.v_scale)
    return kc, vc, slots


def oracle_decode(step, kc, vc, layer=0):
    t = step.num_prefill_tokens
    q = host(step.q[layer])[t:]
    return P.decode_attention(q, step.q_dtype, kc, vc, step.kv_dtype,
                              step.decode_block_tables, step.decode_context_lens,
                              step.softmax_scale, step.k_scale, step.v_scale)


def oracle_prefill(step, kc, vc, layer=0):
    t = step.num_prefill_tokens
    q = host(step.q[layer])[:t]
    return P.prefill_attention(q, step.q_dtype, kc, vc, step.kv_dtype,
                               step.prefill_block_tables, step.prefill_query_start_loc,
                               step.prefill_num_computed, step.softmax_scale,
                               step.k_scale, step.v_scale)


def as_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)
