"""The fp64 oracle over many independent units, in host worker processes.

Used by the full-size parity tests to compare every output of the large
workloads.  A unit is one (sequence or request, kv head): that sequence's
cache tiles of that kv head in table order (a compact cache whose block
table is the identity), the query rows of the kv head's group, and the
context.  The worker evaluates the oracle's own decode or chunked-prefill
function on it.

Workers are started with the "spawn" method: each is a fresh interpreter
that imports numpy and the oracle only, never torch or the GPU library, so
the pool is safe to start from a process that has already used the GPU.
"""

import multiprocessing as mp
import os

import numpy as np

_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def num_workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _identity(nb):
    return np.arange(max(nb, 1), dtype=np.int32)[None, :]


def decode_unit(u):
    """u = (q [G][D], k [nb][16][D], v [nb][16][D], length, q_dtype, kv_dtype,
    softmax_scale, k_scale, v_scale) -> float64 [G][D]."""
    from oracle import paged as P
    q, k, v, length, qd, kd, scale, ks, vs = u
    out = P.decode_attention(q[None], qd, k[:, None], v[:, None], kd, _identity(k.shape[0]),
                             np.array([length], np.int32), scale, ks, vs)
    return out[0]


def prefill_unit(u):
    """u = (q [n][G][D], k, v, num_computed, q_dtype, kv_dtype, softmax_scale,
    k_scale, v_scale) -> float64 [n][G][D]: the chunk's causal rows."""
    from oracle import paged as P
    q, k, v, computed, qd, kd, scale, ks, vs = u
    n = q.shape[0]
    return P.prefill_attention(q, qd, k[:, None], v[:, None], kd, _identity(k.shape[0]),
                               np.array([0, n], np.int32), np.array([computed], np.int32),
                               scale, ks, vs)


def run(fn, units):
    """fn over units in a spawned pool (one BLAS thread per worker)."""
    saved = {k: os.environ.get(k) for k in _THREAD_VARS}
    for k in _THREAD_VARS:
        os.environ[k] = "1"
    try:
        with mp.get_context("spawn").Pool(num_workers()) as pool:
            return pool.map(fn, units, chunksize=1)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def tiles(cache, table_row, length, kv_head):
    """The compact copy of one sequence's tiles of one kv head (host array
    [NB][Hkv][16][D] -> [ceil(length/16)][16][D])."""
    nb = (int(length) + 15) // 16
    return np.ascontiguousarray(cache[np.asarray(table_row[:nb], np.int64), kv_head])


def decode_units(q, kc, vc, tables, lens, group, q_dtype, kv_dtype, scale, ks=1.0, vs=1.0):
    """One unit per (sequence, kv head) of a decode batch."""
    units, where = [], []
    for s in range(len(lens)):
        for kvh in range(kc.shape[1]):
            units.append((np.ascontiguousarray(q[s, kvh * group:(kvh + 1) * group]),
                          tiles(kc, tables[s], lens[s], kvh), tiles(vc, tables[s], lens[s], kvh),
                          int(lens[s]), q_dtype, kv_dtype, scale, ks, vs))
            where.append((s, kvh))
    return units, where


def decode_reference(q, kc, vc, tables, lens, q_dtype, kv_dtype, scale, ks=1.0, vs=1.0):
    """Every output of a decode batch (float64 [S][Hq][D]), in the pool."""
    hq, hkv = q.shape[1], kc.shape[1]
    g = hq // hkv
    units, where = decode_units(q, kc, vc, tables, lens, g, q_dtype, kv_dtype, scale, ks, vs)
    res = run(decode_unit, units)
    out = np.zeros(q.shape, np.float64)
    for (s, kvh), r in zip(where, res):
        out[s, kvh * g:(kvh + 1) * g] = r
    return out


def prefill_reference(q, kc, vc, tables, qsl, computed, q_dtype, kv_dtype, scale,
                      ks=1.0, vs=1.0):
    """Every row of a chunked-prefill call (float64 [Tq][Hq][D]), in the pool."""
    hq, hkv = q.shape[1], kc.shape[1]
    g = hq // hkv
    units, where = [], []
    for r in range(len(qsl) - 1):
        a, b = int(qsl[r]), int(qsl[r + 1])
        if b == a:
            continue
        full = int(computed[r]) + (b - a)
        for kvh in range(hkv):
            units.append((np.ascontiguousarray(q[a:b, kvh * g:(kvh + 1) * g]),
                          tiles(kc, tables[r], full, kvh), tiles(vc, tables[r], full, kvh),
                          int(computed[r]), q_dtype, kv_dtype, scale, ks, vs))
            where.append((a, b, kvh))
    res = run(prefill_unit, units)
    out = np.zeros(q.shape, np.float64)
    for (a, b, kvh), r in zip(where, res):
        out[a:b, kvh * g:(kvh + 1) * g] = r
    return out
