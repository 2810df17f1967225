"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--settle-ms MS] [--gpus 1]
                    [--no-cpu-baseline] [--no-mixed] [--no-longctx] [--no-mha]
                    [--no-swap] [--no-window] [--no-int4] [--no-nvfp4]
                    [--no-blocks] [--no-ceilings] [--no-clock] [--plain-decode]
    python bench.py --copy-calibration     (a plain 1 GiB device copy, for
                                            the HBM byte counters' scale)

A step is one pass of the hot path over one batch: the Llama-3.1-8B-shaped
decode layer (64 sequences, context 512..4096, 32 q / 8 kv heads, head_dim
128, bf16, 16-token blocks): the slots of the 64 new tokens, their cache
writes and paged decode attention, all in the one decode launch
(paged_attention_decode_append: balanced chunks + merge).  Inputs are resident
in HBM before timing starts; two copies of the KV pool alternate between
steps so that the 256 MB last-level cache cannot serve a re-read.  Each leg
first runs untimed for --settle-ms (the clock ramps up from idle), then its
warm-up steps, then the timed ones.

Prints one JSON line (rank 0): whole-step throughput in algorithmic KV GB/s,
KV tokens/s, the decode call's roofline fraction, the oracle's CPU rate on a
bounded sample, the mixed unified step with chunked prefill (MFMA
utilisation of the prefill call), the fp8 long-context decode, the
32-layer MHA decode step, the 8B batch with a sliding window and over an
int4 per token-head cache and over an nvfp4-style cache, a device <-> host
block swap of one long sequence, measured ceilings (a streaming HBM read
with the decode's loads, a register-only bf16 MFMA loop, and that loop with
softmax-like vector work from the same waves) that the decode and prefill
rates are also read against, and the host block manager's operations per
second on a serving trace (with the oracle's rate on a bounded sample
beside it).  The roofline's "traffic" is the HBM bytes per step call that
rocprofv3's FETCH_SIZE and WRITE_SIZE counters measured
(profiles/decode_llama3_8b_64seq_traffic.md), used only while the decode
sources are the ones those counters were taken on.
"""

import argparse
import hashlib
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure


def decode_bytes(step):
    """Algorithmic bytes of one decode call: every context token's K and V
    once, the queries and outputs, and the block-table entries used."""
    lens = step.decode_context_lens.astype(np.int64)
    kvb = 1 if step.kv_dtype == "fp8_e4m3" else (4 if step.kv_dtype == "f32" else 2)
    qb = 4 if step.q_dtype == "f32" else 2
    kv = int(lens.sum()) * 2 * step.num_kv_heads * step.head_dim * kvb
    qo = len(lens) * 2 * step.num_q_heads * step.head_dim * qb
    bt = int(sum((L + 15) // 16 for L in lens)) * 4
    return kv + qo + bt


def prefill_flops(step):
    """4 * D * Hq flops per attended (query, key) pair, causal pairs only."""
    qsl = step.prefill_query_start_loc
    comp = step.prefill_num_computed
    pairs = 0
    for r in range(len(comp)):
        n = int(qsl[r + 1] - qsl[r])
        c = int(comp[r])
        pairs += n * c + n * (n + 1) // 2
    return 4.0 * step.head_dim * step.num_q_heads * pairs, pairs


# Sources whose kernels the decode call runs; the traffic counters in
# profiles/ are used only while these hash to the value recorded with them.
DECODE_SOURCES = ("paged_kv_cache_84_amd/csrc/decode.hip",
                  "paged_kv_cache_84_amd/csrc/decode_mfma.hip",
                  "paged_kv_cache_84_amd/csrc/decode_mfma.h",
                  "paged_kv_cache_84_amd/csrc/decode_sched.h",
                  "paged_kv_cache_84_amd/csrc/common.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_llama3_8b_64seq_traffic.md")


def strip_comments(text):
    """C++ source without its comments and blank lines, each line's trailing
    spaces dropped (string and character literals kept whole): what the
    compiler sees, so that editing a comment keeps the hash."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (line.rstrip() for line in "".join(out).split("\n"))
    return "\n".join(line for line in lines if line)


def decode_source_hash():
    """Hash of the decode kernels' sources, comments aside."""
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(strip_comments(f.read()).encode("utf-8"))
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode call from the committed counter summary (the
    line starting 'traffic-json:'), or None if absent or taken on other
    decode sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if line.startswith("traffic-json:"):
                    rec = json.loads(line.split(":", 1)[1])
                    if rec.get("decode_source_hash") == decode_source_hash():
                        return rec
    except (OSError, ValueError):
        pass
    return None


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size, for scaling the HBM
    byte counters (run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def settle(run, ms):
    """Untimed calls of `run` for about `ms` of wall time (at least one), so
    that every leg is timed at the clock the GPU holds under steady load
    rather than while it ramps up from idle."""
    t0 = time.perf_counter()
    i = 0
    while True:
        run(i)
        i += 1
        if i % 4 == 0 or ms <= 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= ms:
                return i


def time_region(fn, iters, stream):
    """Mean ms per call over `iters` calls bracketed by two HIP events on the
    stream (synchronised before and after)."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(iters):
        fn(i)
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters        # ms


def time_each(fn, iters, stream):
    """Per-call ms of `iters` calls, each between its own pair of HIP events
    on the stream: median, min and p90 (a pass of its own, after the
    bracketed mean, so the events do not enter the mean)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    torch.cuda.synchronize()
    for i in range(iters):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return {"median_ms": round(float(np.median(t)), 4), "min_ms": round(float(t.min()), 4),
            "p90_ms": round(float(np.percentile(t, 90)), 4), "calls": iters}


def timed(fn, iters, stream):
    """(bracketed mean ms, per-call statistics)."""
    return time_region(fn, iters, stream), time_each(fn, iters, stream)


# ----------------------------------------------------------- CPU baseline

_CPU = {}


def _one_blas_thread():
    from threadpoolctl import threadpool_limits
    _CPU["limits"] = threadpool_limits(1)


def _cpu_unit(seq):
    from oracle import paged as P
    d = _CPU
    return P.decode_attention(d["q"][seq:seq + 1], d["q_dtype"], d["kc"], d["vc"],
                              d["kv_dtype"], d["tables"][seq:seq + 1],
                              d["lens"][seq:seq + 1], d["scale"])


def cpu_baseline(step, budget_s=15.0):
    """The fp64 oracle, as written, over a sample of the decode batch's
    sequences, one process per core with one BLAS thread each."""
    from synth import rng as R
    _CPU.update(q=R.to_numpy_storage(step.q[0]), kc=R.to_numpy_storage(step.k_caches[0]),
                vc=R.to_numpy_storage(step.v_caches[0]), tables=step.block_tables,
                lens=step.decode_context_lens, q_dtype=step.q_dtype,
                kv_dtype=step.kv_dtype, scale=step.softmax_scale)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    nseq = len(step.decode_context_lens)
    # time one sequence on one core, then size the sample (whole passes over
    # the batch) to about `budget_s` seconds of wall time
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        t0 = time.perf_counter()
        _cpu_unit(0)
        one = time.perf_counter() - t0
    per_pass = one * nseq / workers
    passes = int(max(1, min(2000, round(budget_s / max(per_pass, 1e-3)))))
    units = list(range(nseq)) * passes
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers, initializer=_one_blas_thread) as pool:
        pool.map(_cpu_unit, units, chunksize=1)
    wall = time.perf_counter() - t0
    tokens = int(step.decode_context_lens.astype(np.int64).sum()) * passes
    kv_bytes = tokens * 2 * step.num_kv_heads * step.head_dim * 2
    seq0_bytes = int(step.decode_context_lens[0]) * 2 * step.num_kv_heads * step.head_dim * 2
    return {"value": round(kv_bytes / wall / 1e9, 4), "unit": "GB/s", "cores": workers,
            "kind": "oracle",
            "single_core": {"value": round(seq0_bytes / one / 1e9, 4), "unit": "GB/s",
                            "seconds": round(one, 3),
                            "sample": "sequence 0 of the batch (32 heads), one process, "
                                      "one BLAS thread"},
            "sample": f"{passes} pass(es) over all {nseq} sequences x 32 heads of the "
                      f"decode batch ({tokens} KV tokens), {wall:.1f} s wall on "
                      f"{workers} worker processes with one BLAS thread each",
            "kv_tokens_per_s": round(tokens / wall, 1)}


def _cpu_decode_unit(u):
    """The oracle's decode over one (sequence, kv head) sample unit: the
    sequence's tiles of that head as a compact cache with the identity table."""
    from oracle import paged as P
    q, k, v, length, qd, kd, scale, ks, vs = u
    table = np.arange(k.shape[0], dtype=np.int32)[None, :]
    return P.decode_attention(q[None], qd, k[:, None], v[:, None], kd, table,
                              np.array([length], np.int32), scale, ks, vs)


def _cpu_prefill_unit(u):
    """The oracle's chunked prefill over one (request, kv head) sample unit."""
    from oracle import paged as P
    q, k, v, computed, qd, kd, scale = u
    n = q.shape[0]
    table = np.arange(k.shape[0], dtype=np.int32)[None, :]
    return P.prefill_attention(q, qd, k[:, None], v[:, None], kd, table,
                               np.array([0, n], np.int32), np.array([computed], np.int32),
                               scale)


def _bf16_bits(rng, shape):
    """N(0,1) samples as bf16 bit patterns (truncated from binary32)."""
    return (rng.standard_normal(shape, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _fp8_codes(rng, shape):
    """Uniformly drawn finite E4M3 codes (any finite code serves for timing)."""
    c = rng.integers(0, 0x7F, size=shape, dtype=np.uint8)           # magnitudes, no NaN
    return c | (rng.integers(0, 2, size=shape, dtype=np.uint8) << 7)


def _timed_pool(fn, units, workers):
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_one_blas_thread) as pool:
        t0 = time.perf_counter()
        pool.map(fn, units, chunksize=1)
        return time.perf_counter() - t0


def cpu_extra_baselines(workers):
    """The oracle on bounded samples of the other workloads, in their own
    units, each extrapolated to the whole workload by its rate (labelled):
    the mixed step's chunked prefill (flop/s over two 100-row requests on the
    2,000-token shared prefix, 94% of the step's pairs are of this kind), the
    70B fp8 long-context decode (one of the six sequences) and the 32-layer
    MHA step (two (layer, sequence) pairs of the 1,024).  Values are seeded
    N(0,1) bf16 or finite fp8 codes; the oracle's time does not depend on them."""
    rng = np.random.default_rng(2026)
    d, out = 128, {}
    # mixed-step prefill: request rows at positions 2000..2099, 32 q / 8 kv heads
    n, c, hkv, group = 100, 2000, 8, 4
    nb = (c + n + 15) // 16
    units = [(_bf16_bits(rng, (n, group, d)), _bf16_bits(rng, (nb, 16, d)),
              _bf16_bits(rng, (nb, 16, d)), c, "bf16", "bf16", float(np.float32(d ** -0.5)))
             for _ in range(2 * hkv)]
    wall = _timed_pool(_cpu_prefill_unit, units, workers)
    pairs = 2 * (n * c + n * (n + 1) // 2)
    flops = 4.0 * d * hkv * group * pairs
    out["mixed_step_prefill"] = {
        "value": round(flops / wall / 1e9, 3), "unit": "GFLOP/s", "cores": workers,
        "kind": "oracle",
        "sample": f"2 requests x 100 chunk rows on a 2,000-token prefix x 32 heads "
                  f"({pairs} (query, key) pairs per head), {wall:.2f} s wall",
        "extrapolated_prefill_s": round(223.6e9 / (flops / wall), 2)}
    # 70B fp8 long context: one sequence of 131,072 tokens, 64 q / 8 kv heads
    L, hkv, group = 131072, 8, 8
    nb = L // 16
    units = [(_bf16_bits(rng, (group, d)), _fp8_codes(rng, (nb, 16, d)),
              _fp8_codes(rng, (nb, 16, d)), L, "bf16", "fp8_e4m3", 1.0, 0.01, 0.01)
             for _ in range(hkv)]
    wall = _timed_pool(_cpu_decode_unit, units, workers)
    nbytes = L * hkv * d * 2
    out["longctx_decode"] = {
        "value": round(nbytes / wall / 1e9, 3), "unit": "GB/s", "cores": workers,
        "kind": "oracle",
        "sample": f"1 of the 6 sequences (131,072 tokens) x 8 kv heads x 64 q heads, "
                  f"{wall:.2f} s wall",
        "extrapolated_step_s": round(6 * wall, 2)}
    # 32-layer MHA: two (layer, sequence) pairs of 8,192 tokens, 32 / 32 heads
    L, hkv = 8192, 32
    nb = L // 16
    units = [(_bf16_bits(rng, (1, d)), _bf16_bits(rng, (nb, 16, d)),
              _bf16_bits(rng, (nb, 16, d)), L, "bf16", "bf16", float(np.float32(d ** -0.5)),
              1.0, 1.0) for _ in range(2 * hkv)]
    wall = _timed_pool(_cpu_decode_unit, units, workers)
    nbytes = 2 * L * hkv * d * 2 * 2
    out["mha_decode"] = {
        "value": round(nbytes / wall / 1e9, 3), "unit": "GB/s", "cores": workers,
        "kind": "oracle",
        "sample": f"2 of the 1,024 (layer, sequence) pairs (8,192 tokens, 32 heads), "
                  f"{wall:.2f} s wall",
        "extrapolated_step_s": round(512 * wall, 1)}
    return out


def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cpus_usable": len(os.sched_getaffinity(0))}


def gpu_clock_under_load(busy, seconds=1.5):
    """The shader clock rocm-smi reports while `busy` keeps the GPU loaded
    (its own thread samples it mid-way); None where rocm-smi is missing or
    prints no sclk."""
    import re
    import subprocess
    import threading
    got = {}

    def sample():
        time.sleep(seconds / 3)
        try:
            r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                               text=True, timeout=30)
            got["text"] = r.stdout
        except (OSError, subprocess.SubprocessError) as e:
            got["error"] = str(e)

    th = threading.Thread(target=sample)
    th.start()
    t0 = time.perf_counter()
    while th.is_alive() or time.perf_counter() - t0 < seconds:
        busy()
        torch.cuda.synchronize()
    th.join()
    text = got.get("text") or ""
    mhz = [int(x) for x in re.findall(r"sclk[^(]*\((\d+)\s*Mhz\)", text, flags=re.I)]
    return {"sclk_mhz": max(mhz) if mhz else None, "source": "rocm-smi --showclocks, "
            "sampled while the decode step runs", "error": got.get("error")}


# ----------------------------------------------------------- GPU legs

def bench_decode(args, pk, step):
    # two device copies of the same batch, used in turn
    dss = [pk.step.DeviceStep(step) for _ in range(2)]
    stream = torch.cuda.current_stream()

    def one_step(i):
        # the 64 new tokens' slots and cache writes, then the decode: one launch
        if args.plain_decode:
            dss[i % 2].decode(0)
        else:
            dss[i % 2].decode_append(0)

    settle(one_step, args.settle_ms)
    for i in range(args.warmup):
        one_step(i)
    ms_step = time_region(one_step, args.steps, stream)
    stats_step = time_each(one_step, args.steps, stream)
    settle(lambda i: dss[i % 2].decode(0), args.settle_ms)
    ms_decode, stats_decode = timed(lambda i: dss[i % 2].decode(0), args.steps, stream)
    nbytes = decode_bytes(step)
    tokens = int(step.decode_context_lens.sum())
    return dss, {"ms_step": ms_step, "ms_decode": ms_decode, "bytes": nbytes,
                 "tokens": tokens, "stats_step": stats_step, "stats_decode": stats_decode}


def bench_mixed(args, pk, C):
    s = C.config4(device="cuda")
    ds = pk.step.DeviceStep(s)
    stream = torch.cuda.current_stream()
    settle(lambda i: ds.run(), args.settle_ms)
    for _ in range(max(2, args.warmup)):
        ds.run()
    iters = max(5, args.steps // 2)
    ms_step, st_step = timed(lambda i: ds.run(), iters, stream)
    settle(lambda i: ds.prefill(0), args.settle_ms)
    ms_prefill, st_prefill = timed(lambda i: ds.prefill(0), iters, stream)
    settle(lambda i: ds.decode(0), args.settle_ms)
    ms_decode, st_decode = timed(lambda i: ds.decode(0), iters, stream)
    # the same step with one unified attention launch for all requests
    settle(lambda i: ds.run_varlen(), args.settle_ms)
    for _ in range(2):
        ds.run_varlen()
    ms_step_varlen = time_region(lambda i: ds.run_varlen(), iters, stream)
    ms_varlen = time_region(lambda i: ds.varlen(0), iters, stream)
    flops, pairs = prefill_flops(s)
    tflops = flops / (ms_prefill * 1e-3) / 1e12
    return {"workload": "mixed unified step: 64 x 100-token chunks on a 125-block "
                        "shared prefix + 1,022-token first chunk + 192 decodes "
                        "(1024..8192) + 64 copy-on-write copies, 32q/8kv, d128, bf16",
            "ms_per_step": round(ms_step, 4), "step_stats": st_step,
            "prefill_ms": round(ms_prefill, 4), "prefill_stats": st_prefill,
            "prefill_tflops": round(tflops, 2),
            "prefill_mfma_frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "prefill_pairs": pairs,
            "decode_ms": round(ms_decode, 4), "decode_stats": st_decode,
            "decode_gbs": round(decode_bytes(s) / (ms_decode * 1e-3) / 1e9, 1),
            "unified": unified_roofline(ms_varlen, ms_prefill + ms_decode, ms_step_varlen,
                                        flops, decode_bytes(s))}


def unified_roofline(ms, ms_two, ms_step, flops, nbytes):
    """The unified call does the chunks' products (matrix-core bound) and
    streams the decodes' K/V (HBM bound) side by side: its floor is the
    larger of the two ideal times."""
    t_mfma = flops / (BF16_MFMA_PEAK_TFLOPS * 1e12) * 1e3
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9) * 1e3
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    return {"attention_ms": round(ms, 4), "two_launch_attention_ms": round(ms_two, 4),
            "ms_per_step": round(ms_step, 4),
            "roofline": {"bound": bound, "ideal_ms": round(max(t_mfma, t_hbm), 4),
                         "ideal_mfma_ms": round(t_mfma, 4), "ideal_hbm_ms": round(t_hbm, 4),
                         "frac": round(max(t_mfma, t_hbm) / ms, 4)}}


PCIE5_X16_GBS = 64.0   # host link of one MI355X, per direction


def swap_workload(num_layers=32, hkv=32, d=128, seq_blocks=512, pool_blocks=600):
    """One 8,192-token sequence of the Llama-2-7B-shaped 32-layer cache
    (512 blocks of 128 KiB per layer and K/V, seeded scattered placement in
    a 600-block device pool) with a pinned host pool for it and a second
    device pool to bring it back into (a seeded scattered set of blocks)."""
    from synth import rng as R
    rs = R.structure_rng(3, 7)
    dev_ids = rs.permutation(pool_blocks)[:seq_blocks]
    back_ids = rs.permutation(pool_blocks)[:seq_blocks]
    shape = (pool_blocks, hkv, 16, d)
    dev_k = [R.normal(shape, R.BF16, 3, 200 + l, "cuda") for l in range(num_layers)]
    dev_v = [R.normal(shape, R.BF16, 3, 300 + l, "cuda") for l in range(num_layers)]
    host_k = [torch.empty((seq_blocks, hkv, 16, d), dtype=torch.bfloat16, pin_memory=True)
              for _ in range(num_layers)]
    host_v = [torch.empty_like(t, pin_memory=True) for t in host_k]
    back_k = [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(num_layers)]
    back_v = [torch.zeros_like(t) for t in back_k]
    slots = np.arange(seq_blocks)
    out_pairs = torch.as_tensor(np.stack([dev_ids, slots], 1).astype(np.int64), device="cuda")
    in_pairs = torch.as_tensor(np.stack([slots, back_ids], 1).astype(np.int64), device="cuda")
    return {"dev_k": dev_k, "dev_v": dev_v, "host_k": host_k, "host_v": host_v,
            "back_k": back_k, "back_v": back_v, "out_pairs": out_pairs, "in_pairs": in_pairs,
            "bytes": 2 * num_layers * seq_blocks * hkv * 16 * d * 2}


def bench_swap(args, pk):
    """Swap one sequence out to pinned host memory and back in (one
    swap_blocks call each way), GB/s against the host link's peak."""
    w = swap_workload()
    stream = torch.cuda.current_stream()
    out = lambda i: pk.swap_blocks(w["dev_k"], w["dev_v"], w["host_k"], w["host_v"],
                                   w["out_pairs"])
    back = lambda i: pk.swap_blocks(w["host_k"], w["host_v"], w["back_k"], w["back_v"],
                                    w["in_pairs"])
    out(0)
    back(0)
    iters = 3
    ms_out = time_region(out, iters, stream)
    ms_in = time_region(back, iters, stream)
    gb = w["bytes"] / 1e9
    return {"workload": "swap one 8,192-token sequence of the Llama-2-7B-shaped 32-layer "
                        "cache (512 blocks x 128 KiB per layer and K/V = 4 GiB) to pinned "
                        "host memory and back into scattered device blocks",
            "bytes_each_way": w["bytes"],
            "out_ms": round(ms_out, 3), "out_gbs": round(gb / (ms_out * 1e-3), 1),
            "in_ms": round(ms_in, 3), "in_gbs": round(gb / (ms_in * 1e-3), 1),
            "link_peak_gbs": PCIE5_X16_GBS,
            "out_frac": round(gb / (ms_out * 1e-3) / PCIE5_X16_GBS, 3),
            "in_frac": round(gb / (ms_in * 1e-3) / PCIE5_X16_GBS, 3)}


def _serve(m, trace, batched):
    """One pass of a serving trace through a block manager (library: batched
    calls per engine step; oracle: one call per request)."""
    for st in trace:
        for rid, prompt in st["adds"]:
            m.allocate(rid, len(prompt) - m.add_request(rid, prompt))
        ids, toks = st["decode_ids"], st["decode_tokens"]
        if batched:
            m.append_tokens_batch(ids, toks)
            if m.allocate_batch(ids, np.ones(ids.size, np.int32)).any():
                raise RuntimeError("block pool too small for the trace")
        else:
            for rid, t in zip(ids.tolist(), toks.tolist()):
                m.append_tokens(rid, [t])
                m.allocate(rid, 1)
        for rid in st["frees"]:
            m.free_request(rid)


def bench_block_manager(args, oracle_budget_s=5.0):
    """Host block manager on a serving trace: 2,000 engine steps, up to 256
    live requests, prompts = one of 8 shared 2,000-token system prompts + 64..511
    unique tokens, 32..255 generated tokens each; pool of 32,768 blocks."""
    from paged_kv_cache_84_amd import blocks as PB
    from synth.serving import serving_trace, trace_ops
    trace = serving_trace()
    ops = trace_ops(trace)
    adds = sum(len(st["adds"]) for st in trace)
    m = PB.BlockManager(32768)
    t0 = time.perf_counter()
    cached = 0
    for st in trace:     # the same pass as _serve, counting prefix hits
        for rid, prompt in st["adds"]:
            c = m.add_request(rid, prompt)
            cached += c
            m.allocate(rid, len(prompt) - c)
        ids = st["decode_ids"]
        m.append_tokens_batch(ids, st["decode_tokens"])
        if m.allocate_batch(ids, np.ones(ids.size, np.int32)).any():
            raise RuntimeError("block pool too small for the trace")
        for rid in st["frees"]:
            m.free_request(rid)
    lib_s = time.perf_counter() - t0
    prompt_tokens = sum(len(p) for st in trace for _, p in st["adds"])
    out = {"workload": " ".join(bench_block_manager.__doc__.split(":", 1)[1].split()),
           "ops": ops, "requests": adds, "seconds": round(lib_s, 4),
           "ops_per_s": round(ops / lib_s, 1),
           "prefix_hit_tokens_frac": round(cached / prompt_tokens, 4)}
    if not args.no_cpu_baseline:
        from oracle import blocks as OB
        om = OB.BlockManager(32768)
        done_ops, t0 = 0, time.perf_counter()
        for i, st in enumerate(trace):
            _serve(om, [st], batched=False)
            done_ops += 2 * len(st["adds"]) + st["decode_ids"].size + len(st["frees"])
            if time.perf_counter() - t0 > oracle_budget_s:
                break
        osec = time.perf_counter() - t0
        out["oracle"] = {"ops_per_s": round(done_ops / osec, 1), "steps": i + 1,
                         "ops": done_ops, "cores": 1, "kind": "oracle",
                         "sample": f"the first {i + 1} engine steps of the same trace"}
    return out


def bench_extra_decode(args, pk, C, which):
    """Optional legs: the fp8 long-context decode (64/8 heads, 6 x 131,072
    tokens, 512-token partitions) or the 32-layer MHA decode step (32 x 8,192
    tokens), each timed as whole decode steps on inputs resident in HBM: per
    layer, one paged_attention_decode_append call (the new tokens' cache
    writes inside the decode launch)."""
    if which == "longctx":
        s = C.config5(device="cuda")
        # two device copies of the 1.6 GB cache, used in turn (the inputs
        # were made on the GPU, so the second step gets cloned caches)
        dss = [pk.step.DeviceStep(s, partition_tokens=512) for _ in range(2)]
        dss[1].k_caches = [t.clone() for t in dss[1].k_caches]
        dss[1].v_caches = [t.clone() for t in dss[1].v_caches]
        layers = [0]
        name = ("Llama-3.1-70B-shaped long-context decode, one layer: 6 x 131072 "
                "tokens, 64 q / 8 kv heads, d128, bf16 q, fp8 e4m3 K/V, 512-token "
                "partitions; new tokens' fp8 write + decode in one call; two copies "
                "of the cache used in turn")
    else:
        s = C.config3(device="cuda")
        # one copy: each step reads 128 GiB, far past the last-level cache
        dss = [pk.step.DeviceStep(s)]
        layers = list(range(s.num_layers))
        name = ("Llama-2-7B-shaped MHA decode, 32 layers back to back: 32 x 8192 "
                "tokens, 32/32 heads, d128, bf16; per layer, new tokens' write + "
                "decode in one call")
    stream = torch.cuda.current_stream()

    def run(i):
        ds = dss[i % len(dss)]
        for layer in layers:
            ds.decode_append(layer)

    settle(run, args.settle_ms)
    for i in range(2):
        run(i)
    iters = max(3, min(args.steps, 10 if which == "mha" else args.steps))
    ms, stats = timed(run, iters, stream)
    nbytes = decode_bytes(s) * len(layers)
    tokens = int(s.decode_context_lens.sum()) * len(layers)
    return {"workload": name, "ms_per_step": round(ms, 4), "step_stats": stats,
            "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kv_tokens_per_s": round(tokens / (ms * 1e-3), 1),
            "algorithmic_bytes": nbytes}


def bench_window(args, pk, ds, step, window=1024):
    """The 8B decode batch with a 1,024-token sliding window on the decode
    leg's device inputs: only the window's K/V are read (algorithmic bytes
    count min(L, W) tokens per sequence)."""
    lens = step.decode_context_lens
    stream = torch.cuda.current_stream()
    q = ds.q[0][ds.num_prefill_tokens:]
    out = torch.empty_like(q)
    ws = torch.empty(pk.decode_workspace_size(len(lens), step.num_q_heads, step.num_kv_heads,
                                              step.head_dim, int(lens.max())),
                     dtype=torch.uint8, device="cuda")

    def run(i):
        pk.paged_attention_decode_sliding(q, ds.k_caches[0], ds.v_caches[0], ds.dec_tables,
                                          ds.dec_lens, int(lens.max()), step.softmax_scale,
                                          window, out=out, workspace=ws)

    settle(run, args.settle_ms)
    for i in range(args.warmup):
        run(i)
    ms, stats = timed(run, args.steps, stream)
    seen = np.minimum(lens.astype(np.int64), window)
    nbytes = (int(seen.sum()) * 2 * step.num_kv_heads * step.head_dim * 2
              + 2 * len(lens) * step.num_q_heads * step.head_dim * 2)
    return {"workload": f"Llama-3.1-8B-shaped decode batch with a {window}-token sliding "
                        "window (64 sequences, context 512..4096, 32/8 heads, d128, bf16)",
            "window": window, "ms_per_call": round(ms, 4), "call_stats": stats,
            "algorithmic_bytes": nbytes,
            "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def bench_int4(args, pk, step, copies=3):
    """The 8B decode batch (64 sequences, 512..4096 tokens, 32 q / 8 kv heads)
    over an int4 per token-head cache: decode calls on resident inputs,
    several copies of the pool in turn so the last-level cache cannot serve a
    re-read.  Algorithmic bytes: per token and kv head, 64 code bytes and a
    4-byte scale for K and for V, plus Q and the output."""
    from synth import rng as R
    lens = step.decode_context_lens
    tables = torch.as_tensor(step.decode_block_tables, device="cuda")
    lens_d = torch.as_tensor(lens, device="cuda")
    nb = int(step.num_blocks)
    hq, hkv, d = step.num_q_heads, step.num_kv_heads, step.head_dim
    q = R.normal((len(lens), hq, d), "bf16", 950, 1, "cuda")
    pools = [(R.int4_codes((nb, hkv, 16, d // 2), 950, 10 + c, "cuda"),
              R.int4_codes((nb, hkv, 16, d // 2), 950, 20 + c, "cuda"),
              R.int4_scales((nb, hkv, 16), 950, 30 + c, "cuda"),
              R.int4_scales((nb, hkv, 16), 950, 40 + c, "cuda")) for c in range(copies)]
    out = torch.empty_like(q)
    ws = torch.empty(pk.decode_workspace_size(len(lens), hq, hkv, d, int(lens.max())),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def run(i):
        kc, vc, ks, vs = pools[i % copies]
        pk.paged_attention_decode_int4(q, kc, vc, ks, vs, tables, lens_d, int(lens.max()),
                                       step.softmax_scale, out=out, workspace=ws)

    settle(run, args.settle_ms)
    for i in range(args.warmup):
        run(i)
    ms, stats = timed(run, args.steps, stream)
    tokens = int(lens.sum())
    nbytes = tokens * hkv * 2 * (d // 2 + 4) + 2 * len(lens) * hq * d * 2
    return {"workload": "Llama-3.1-8B-shaped decode layer over an int4 per token-head "
                        "cache: 64 sequences, context 512..4096, 32 q / 8 kv heads, d128, "
                        "bf16 q",
            "ms_per_call": round(ms, 4), "call_stats": stats, "algorithmic_bytes": nbytes,
            "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kv_tokens_per_s": round(tokens / (ms * 1e-3), 1)}


def bench_nvfp4(args, pk, step, copies=3):
    """The 8B decode batch over an nvfp4-style cache (E2M1 codes, an E4M3
    scale per 16 elements, per-tensor scales): decode calls on resident
    inputs, several pool copies in turn.  Algorithmic bytes: per token and kv
    head, 64 code bytes and 8 block-scale bytes for K and for V, plus Q and
    the output."""
    from synth import rng as R
    lens = step.decode_context_lens
    tables = torch.as_tensor(step.decode_block_tables, device="cuda")
    lens_d = torch.as_tensor(lens, device="cuda")
    nb = int(step.num_blocks)
    hq, hkv, d = step.num_q_heads, step.num_kv_heads, step.head_dim
    q = R.normal((len(lens), hq, d), "bf16", 960, 1, "cuda")
    pools = [(R.int4_codes((nb, hkv, 16, d // 2), 960, 10 + c, "cuda"),
              R.int4_codes((nb, hkv, 16, d // 2), 960, 20 + c, "cuda"),
              R.nvfp4_bscales((nb, hkv, 16, d // 16), 960, 30 + c, "cuda"),
              R.nvfp4_bscales((nb, hkv, 16, d // 16), 960, 40 + c, "cuda"))
             for c in range(copies)]
    out = torch.empty_like(q)
    ws = torch.empty(pk.decode_workspace_size(len(lens), hq, hkv, d, int(lens.max())),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def run(i):
        kc, vc, ks, vs = pools[i % copies]
        pk.paged_attention_decode_nvfp4(q, kc, vc, ks, vs, tables, lens_d, int(lens.max()),
                                        step.softmax_scale, 1.0, 1.0, out=out, workspace=ws)

    settle(run, args.settle_ms)
    for i in range(args.warmup):
        run(i)
    ms, stats = timed(run, args.steps, stream)
    tokens = int(lens.sum())
    nbytes = tokens * hkv * 2 * (d // 2 + d // 16) + 2 * len(lens) * hq * d * 2
    return {"workload": "Llama-3.1-8B-shaped decode layer over an nvfp4-style cache (E2M1, "
                        "E4M3 scale per 16 elements): 64 sequences, context 512..4096, "
                        "32 q / 8 kv heads, d128, bf16 q",
            "ms_per_call": round(ms, 4), "call_stats": stats, "algorithmic_bytes": nbytes,
            "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kv_tokens_per_s": round(tokens / (ms * 1e-3), 1)}


def xor_of_range(n):
    """XOR of the integers 0 .. n-1 (closed form by n mod 4)."""
    x = n - 1
    return [x, 1, x + 1, 0][x % 4] if n > 0 else 0


def bench_ceilings(args, pk, read_bytes=4 << 30, mfma_waves=4096, mfma_iters=4096):
    """Measured ceilings: a streaming read of 4 GiB with the decode's
    16-byte non-temporal loads (the buffer holds the word ramp 0, 1, 2, ...,
    whose XOR checks that every word was read), a register-only loop of
    the prefill's bf16 MFMA on 4 waves per SIMD (each wave's result checks
    that every product was issued), and that loop with the softmax's kind
    of vector work from the same waves, alone and together: the share of
    the vector time the matrix cores do not hide."""
    stream = torch.cuda.current_stream()
    words = torch.arange(read_bytes // 4, dtype=torch.int32, device="cuda")
    checksum = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        pk.measure_hbm_read(words, checksum)
    ms_read = time_region(lambda i: pk.measure_hbm_read(words, checksum), 5, stream)
    got = int(checksum.cpu().numpy().view(np.uint32)[0])
    assert got == xor_of_range(read_bytes // 4), "HBM read checksum mismatch"
    del words
    result = torch.zeros(mfma_waves, dtype=torch.float32, device="cuda")
    pk.measure_mfma_bf16(mfma_iters, result)
    ms_mfma = time_region(lambda i: pk.measure_mfma_bf16(mfma_iters, result), 3, stream)
    assert bool(torch.all(result == 32.0 * mfma_iters)), "MFMA loop result mismatch"
    pair = torch.zeros(2 * mfma_waves, dtype=torch.float32, device="cuda")
    ms_mode = []
    for mode in range(3):
        pk.measure_mfma_valu(mfma_iters, mode, pair)
        ms_mode.append(time_region(lambda i: pk.measure_mfma_valu(mfma_iters, mode, pair),
                                   3, stream))
        r = pair.view(-1, 2).cpu()
        assert bool(torch.all(r[:, 0] == (0.0 if mode == 1 else 32.0 * mfma_iters))) and \
            bool(torch.all(r[:, 1] == r[0, 1])) and (float(r[0, 1]) > 0) == (mode > 0), \
            "MFMA + vector loop result mismatch"
    del pair
    read_gbs = read_bytes / (ms_read * 1e-3) / 1e9
    tflops = mfma_waves * mfma_iters * 8 * 16384 / (ms_mfma * 1e-3) / 1e12
    return {"hbm_read": {"bytes": read_bytes, "ms": round(ms_read, 4),
                         "gbs": round(read_gbs, 1),
                         "frac_of_peak": round(read_gbs / HBM_PEAK_GBS, 4)},
            "mfma_bf16": {"waves": mfma_waves, "mfma_per_wave": mfma_iters * 8,
                          "ms": round(ms_mfma, 4), "tflops": round(tflops, 1),
                          "frac_of_peak": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4)},
            "mfma_with_vector_work": {
                "waves": mfma_waves, "iterations": mfma_iters,
                "ms_mfma_only": round(ms_mode[0], 4), "ms_vector_only": round(ms_mode[1], 4),
                "ms_both": round(ms_mode[2], 4),
                "vector_share_not_hidden": round((ms_mode[2] - ms_mode[0]) / ms_mode[1], 4)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed calls of each leg for this many ms before its warm-up "
                         "steps (the GPU clock ramps up from idle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mixed", action="store_true")
    ap.add_argument("--no-longctx", action="store_true",
                    help="skip the fp8 long-context decode (1.6 GB of KV)")
    ap.add_argument("--no-mha", action="store_true",
                    help="skip the 32-layer MHA decode step (128 GiB of KV)")
    ap.add_argument("--no-swap", action="store_true",
                    help="skip the device <-> host block swap of one long sequence")
    ap.add_argument("--no-window", action="store_true",
                    help="skip the sliding-window decode of the 8B batch")
    ap.add_argument("--no-int4", action="store_true",
                    help="skip the int4 per token-head decode of the 8B batch")
    ap.add_argument("--no-nvfp4", action="store_true",
                    help="skip the nvfp4-style decode of the 8B batch")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the shader clock with rocm-smi (e.g. under a "
                         "profiler, whose preloaded library the rocm-smi child inherits)")
    ap.add_argument("--plain-decode", action="store_true",
                    help="time the plain paged_attention_decode call as the step (for "
                         "builds whose decode kernel has no fused cache write, e.g. one "
                         "built with -DPKV_DECODE_USE_MFMA=0)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured HBM-read and MFMA ceilings")
    ap.add_argument("--no-blocks", action="store_true",
                    help="skip the host block manager on a serving trace")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter scale)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the paged-attention path here is "
              "built and measured on a single MI355X (no collectives); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        torch.cuda.set_device(0)
        copy_calibration()
        return
    import paged_kv_cache_84_amd as pk
    from synth import configs as C
    # The workload is built on the host; the CPU baseline runs before the GPU
    # is touched (its worker processes are forked from this one).
    step = C.config2(device="cpu")
    cpu = None if args.no_cpu_baseline else cpu_baseline(step)
    if cpu is not None:
        cpu["other_workloads"] = cpu_extra_baselines(cpu["cores"])
        cpu["host"] = host_info()
    torch.cuda.set_device(0)
    pk.library()

    dss, r = bench_decode(args, pk, step)
    gbs_step = r["bytes"] / (r["ms_step"] * 1e-3) / 1e9
    gbs_decode = r["bytes"] / (r["ms_decode"] * 1e-3) / 1e9
    line = {
        "metric": "paged decode attention HBM GB/s (% of peak) + KV tokens/s; "
                  "prefill MFMA util",
        "value": round(gbs_step, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(r["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped decode layer: 64 sequences, "
                               "context uniform in [512, 4096], 32 q / 8 kv heads, "
                               "head_dim 128, bf16 Q/K/V, 16-token blocks, shuffled "
                               "block placement; step = slots + cache writes of the 64 "
                               "new tokens inside the paged decode launch "
                               "(paged_attention_decode_append: balanced chunks + merge)",
                   "num_seqs": 64, "kv_tokens": r["tokens"],
                   "algorithmic_bytes": r["bytes"],
                   "decode_chunks_per_kv_head": pk.decode_num_chunks(
                       64, 32, 8, int(step.decode_context_lens.max()))},
        "pct_of_hbm_peak": round(100 * gbs_step / HBM_PEAK_GBS, 2),
        "kv_tokens_per_s": round(r["tokens"] / (r["ms_step"] * 1e-3), 1),
        "step_stats": r["stats_step"],
        "roofline": {"bound": "hbm",
                     "kernel": "the step's call, paged_attention_decode_append (chunk kernel "
                               "with the new rows' writes + merge kernel)",
                     "achieved": round(gbs_step, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs_step / HBM_PEAK_GBS, 4), "traffic": None,
                     "launch_ms": round(r["ms_step"], 4),
                     "plain_decode_call": {"ms": round(r["ms_decode"], 4),
                                           "gbs": round(gbs_decode, 1),
                                           "frac": round(gbs_decode / HBM_PEAK_GBS, 4),
                                           "stats": r["stats_decode"]}},
    }
    if args.plain_decode:
        line["config"]["workload"] += "; timed as the plain paged_attention_decode call"
        line["roofline"]["kernel"] = "paged_attention_decode (chunk kernel + merge kernel)"
    if not args.no_clock:
        line["gpu_clock"] = gpu_clock_under_load(
            lambda: [(dss[i % 2].decode(0) if args.plain_decode else dss[i % 2].decode_append(0))
                     for i in range(20)])
    tr = measured_traffic()
    if tr is not None:
        key = "bytes_per_call" if args.plain_decode else "append_call_bytes"
        line["roofline"]["traffic"] = tr[key]
        line["roofline"]["traffic_over_algorithmic"] = round(tr[key] / r["bytes"], 3)
    if not args.no_mixed:
        line["mixed_step"] = bench_mixed(args, pk, C)
    if not args.no_longctx:
        line["longctx_decode"] = bench_extra_decode(args, pk, C, "longctx")
    if not args.no_mha:
        line["mha_decode"] = bench_extra_decode(args, pk, C, "mha")
    if not args.no_window:
        line["window_decode"] = bench_window(args, pk, dss[0], step)
    if not args.no_int4:
        line["int4_decode"] = bench_int4(args, pk, step)
    if not args.no_nvfp4:
        line["nvfp4_decode"] = bench_nvfp4(args, pk, step)
    if not args.no_ceilings:
        ceil = bench_ceilings(args, pk)
        ceil["decode_call_frac_of_read_ceiling"] = round(
            line["roofline"]["achieved"] / ceil["hbm_read"]["gbs"], 4)
        if "mixed_step" in line:
            ceil["prefill_frac_of_mfma_ceiling"] = round(
                line["mixed_step"]["prefill_tflops"] / ceil["mfma_bf16"]["tflops"], 4)
        line["ceilings"] = ceil
    if not args.no_swap:
        line["swap_blocks"] = bench_swap(args, pk)
    if not args.no_blocks:
        line["block_manager"] = bench_block_manager(args)
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
