"""Seeded serving trace for the host block manager: requests arrive with a
prompt made of one of a few shared system prompts plus unique text, are
prefilled in one step, then decode one token per step until they finish.

The shape follows the pages' prefix-caching workloads (chat sessions and
agents resend the same system instructions, RAG resends the same documents:
"vLLM 引擎解剖", section "自动前缀缓存"; the 2,100-token new request of "01.
vLLM", section "调度器：统一的 token 预算").  Token ids are random: only their
equality matters to the block manager.
"""

import numpy as np


def serving_trace(steps=2000, max_live=256, admit_per_step=16, num_system=8,
                  system_tokens=2000, unique_tokens=(64, 512), generated=(32, 256),
                  vocab=32000, seed=11):
    """A list of engine steps; each is a dict with
    adds           [(request id, prompt int32 array)]  prefilled this step
    decode_ids     int64 array: requests that decode one token this step
    decode_tokens  int32 array: the token each of them appends
    frees          request ids that finish after this step
    """
    rng = np.random.default_rng(seed)
    systems = [rng.integers(0, vocab, system_tokens).astype(np.int32)
               for _ in range(num_system)]
    live = {}               # request id -> tokens still to generate
    out, nxt = [], 0
    for _ in range(steps):
        adds = []
        while len(live) + len(adds) < max_live and len(adds) < admit_per_step:
            sysp = systems[int(rng.integers(0, num_system))]
            tail = rng.integers(0, vocab, int(rng.integers(*unique_tokens))).astype(np.int32)
            adds.append((nxt, np.concatenate([sysp, tail])))
            nxt += 1
        decode_ids = np.array(sorted(live), dtype=np.int64)
        decode_tokens = rng.integers(0, vocab, decode_ids.size).astype(np.int32)
        frees = []
        for rid in decode_ids:
            live[int(rid)] -= 1
            if live[int(rid)] == 0:
                frees.append(int(rid))
                del live[int(rid)]
        for rid, _ in adds:
            live[rid] = int(rng.integers(*generated))
        out.append({"adds": adds, "decode_ids": decode_ids, "decode_tokens": decode_tokens,
                    "frees": frees})
    return out


def trace_ops(trace):
    """Operations of a trace: one per add, per prefill allocation, per
    decode allocation and per release."""
    return sum(2 * len(s["adds"]) + s["decode_ids"].size + len(s["frees"]) for s in trace)
