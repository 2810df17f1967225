"""The C ABI library: it loads, exports every declared entry point, and rejects
bad host-side arguments with the documented status codes.  No call here
reaches a kernel launch, so this runs without a GPU."""

import ctypes
import os
import re
import subprocess

import pytest

from paged_kv_cache_84_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")
OK, NULL, ALIGN, SHAPE, UNSUP, WS, LAUNCH = range(7)
F32, BF16, FP8 = 0, 1, 2


def _sources_newer_than(lib):
    csrc = os.path.join(ROOT, "paged_kv_cache_84_amd", "csrc")
    newest = max(os.path.getmtime(os.path.join(csrc, f)) for f in os.listdir(csrc))
    return newest > os.path.getmtime(lib) or os.path.getmtime(HEADER) > os.path.getmtime(lib)


@pytest.fixture(scope="module")
def lib():
    path = B.library_path()
    if not os.path.exists(path) or _sources_newer_than(path):
        # cross-compiles for gfx950 on the CPU; no GPU needed
        from paged_kv_cache_84_amd import build
        build.build()
    return B.library()


def declared_functions():
    import glob
    text = "\n".join(open(h, encoding="utf-8").read()
                     for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?([a-z_][a-z_0-9]*)\s*\(",
                                 text, flags=re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert "paged_attention_decode" in names and len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", B.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert sorted(B.EXPORTED) == names


def test_small_host_calls(lib):
    assert lib.pkv_block_size() == 16
    assert lib.kv_bytes_per_token(32, 8, 128, 2) == 131072
    assert lib.kv_bytes_per_token(-1, 8, 128, 2) == -1
    for code in range(9):
        assert lib.pkv_status_string(code)
    assert lib.pkv_status_string(99) == b"unknown status"


def test_slot_mapping_errors(lib):
    f = lib.compute_slot_mapping
    assert f(None, 4, None, None, 0, 10, None, 0, None) == OK          # nothing to do
    assert f(None, 4, None, None, 2, 10, None, 5, None) == NULL
    assert f(0x1000, 4, 0x1000, 0x1000, -1, 10, 0x1000, 5, None) == SHAPE
    assert f(0x1000, 4, 0x1000, 0x1000, 2, 10, 0x1004, 5, None) == ALIGN


def test_reshape_and_cache_errors(lib):
    f = lib.reshape_and_cache
    p = 0x10000
    args = lambda **k: [k.get("key", p), p, p, p, p, k.get("t", 3), k.get("hkv", 2),
                        k.get("d", 64), 10, k.get("src", BF16), k.get("dst", BF16),
                        k.get("ks", 1.0), 1.0, None]
    assert f(*args(t=0)) == OK
    assert f(*args(key=None)) == NULL
    assert f(*args(key=p + 8)) == ALIGN
    assert f(*args(d=60)) == UNSUP
    assert f(*args(t=-1)) == SHAPE
    assert f(*args(src=FP8, dst=FP8)) == UNSUP
    assert f(*args(src=BF16, dst=F32)) == UNSUP
    assert f(*args(dst=FP8, ks=0.0)) == SHAPE


def test_copy_blocks_errors(lib):
    f = lib.copy_blocks
    arr = (ctypes.c_void_p * 1)(0x10000)
    assert f(arr, arr, 1, 0x10000, 0, 10, 4096, None) == OK
    assert f(arr, arr, 1, 0x10000, 2, 10, 4095, None) == SHAPE
    assert f(None, arr, 1, 0x10000, 2, 10, 4096, None) == NULL
    bad = (ctypes.c_void_p * 1)(0x10008)
    assert f(bad, arr, 1, 0x10000, 2, 10, 4096, None) == ALIGN
    nul = (ctypes.c_void_p * 1)(None)
    assert f(nul, arr, 1, 0x10000, 2, 10, 4096, None) == NULL


def test_swap_blocks_errors(lib):
    f = lib.swap_blocks
    arr = (ctypes.c_void_p * 1)(0x10000)
    assert f(arr, arr, arr, arr, 1, 0x10000, 0, 10, 10, 4096, None) == OK
    assert f(arr, arr, arr, arr, 0, 0x10000, 2, 10, 10, 4096, None) == OK
    assert f(arr, arr, arr, arr, 1, 0x10000, 2, 10, 10, 4095, None) == SHAPE
    assert f(arr, arr, arr, arr, 1, 0x10000, 2, -1, 10, 4096, None) == SHAPE
    assert f(arr, arr, None, arr, 1, 0x10000, 2, 10, 10, 4096, None) == NULL
    assert f(arr, arr, arr, arr, 1, None, 2, 10, 10, 4096, None) == NULL
    assert f(arr, arr, arr, arr, 1, 0x10004, 2, 10, 10, 4096, None) == ALIGN
    bad = (ctypes.c_void_p * 1)(0x10008)
    assert f(arr, arr, bad, arr, 1, 0x10000, 2, 10, 10, 4096, None) == ALIGN
    nul = (ctypes.c_void_p * 1)(None)
    assert f(arr, nul, arr, arr, 1, 0x10000, 2, 10, 10, 4096, None) == NULL


def _decode(lib, **k):
    p = 0x100000
    a = dict(out=p, q=p, kc=p, vc=p, nb=100, bt=p, maxb=64, lens=p, s=4, maxlen=1000,
             hq=32, hkv=8, d=128, scale=0.088, qd=BF16, kvd=BF16, ks=1.0, vs=1.0,
             part=0, ws=p, wsb=1 << 30)
    a.update(k)
    return lib.paged_attention_decode(a["out"], a["q"], a["kc"], a["vc"], a["nb"],
                                      a["bt"], a["maxb"], a["lens"], a["s"],
                                      a["maxlen"], a["hq"], a["hkv"], a["d"],
                                      a["scale"], a["qd"], a["kvd"], a["ks"], a["vs"],
                                      a["part"], a["ws"], a["wsb"], None)


def test_decode_errors(lib):
    assert _decode(lib, s=0) == OK
    assert _decode(lib, out=None) == NULL
    assert _decode(lib, q=0x100008) == ALIGN
    assert _decode(lib, hq=30) == SHAPE                    # not a multiple of hkv
    assert _decode(lib, hq=72) == UNSUP                    # group 9
    assert _decode(lib, d=96) == UNSUP
    assert _decode(lib, qd=F32) == UNSUP                   # f32 q with bf16 cache
    assert _decode(lib, qd=FP8, kvd=FP8) == UNSUP
    assert _decode(lib, maxb=10) == SHAPE                  # 160 tokens < max_context_len
    assert _decode(lib, part=100) == SHAPE                 # not a multiple of 16
    assert _decode(lib, part=-16) == SHAPE
    assert _decode(lib, kvd=FP8, ks=0.0) == SHAPE
    assert _decode(lib, nb=0) == SHAPE
    need = lib.paged_attention_decode_workspace_size(4, 32, 8, 128, 1000, 0)
    chunks = lib.paged_attention_decode_num_chunks(4, 32, 8, 1000, 0)
    # one partial per (chunk, sequence) pair that overlaps: at most chunks + seqs
    assert need >= (chunks + 4) * 32 * (128 + 2) * 4
    assert _decode(lib, wsb=need - 1) == WS
    assert _decode(lib, ws=None) == WS
    # 4 x 63 blocks at most; chunks of at least 4 blocks
    assert 1 <= chunks <= 63
    assert lib.paged_attention_decode_num_chunks(4, 32, 8, 1000, 64) == 63
    assert lib.paged_attention_decode_num_chunks(4, 32, 8, 1000, 48) == 84
    assert lib.paged_attention_decode_num_chunks(4, 32, 8, 1000, 40) == -1


def test_decode_noalloc_host_errors(lib):
    """The allocation-free decode refuses a split larger than its scratch
    array, and bad sizes, before it touches any device state."""
    f = lib.paged_attention_decode_noalloc
    p = 0x100000
    base = [p, p, p, p, 100, p, 1 << 20, p, 1, 1 << 24, 64, 8, 128, 0.088, BF16, BF16,
            1.0, 1.0, 16, None]
    assert f(*base) == WS                               # one partial per 16 tokens of 16 M
    assert lib.paged_attention_decode_workspace_size(1, 64, 8, 128, 1 << 24, 16) > 64 << 20
    bad = list(base)
    bad[18] = 24                                        # partition not a multiple of 16
    assert f(*bad) == SHAPE
    bad = list(base)
    bad[10] = 60                                        # q heads not a multiple of kv heads
    assert f(*bad) == SHAPE


def test_prefill_errors(lib):
    f = lib.paged_attention_prefill_chunk
    p = 0x100000
    base = [p, p, p, p, 100, p, 64, p, p, 3, 50, 20, 32, 8, 128, 0.088, BF16, BF16,
            1.0, 1.0, None]

    def call(**k):
        a = list(base)
        for i, v in k.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a9=0) == OK
    assert call(a0=None) == NULL
    assert call(a1=p + 4) == ALIGN
    assert call(a12=31) == SHAPE
    assert call(a14=80) == UNSUP
    assert call(a16=F32) == UNSUP
    assert call(a4=0) == SHAPE


def test_varlen_errors(lib):
    f = lib.paged_attention_varlen
    p = 0x100000
    need = lib.paged_attention_varlen_workspace_size(3, 50, 8, 128, 2000)

    def a256(n):
        return (n + 255) // 256 * 256

    # the queue counters (256 bytes apart), totals and per-CU arrivals; the tile list (50 tokens in tiles of at
    # least 16, plus one partial tile per request) and the run list (2 runs of
    # 64 blocks per request), 8 bytes an entry; then per (request, kv head,
    # run) 16 columns of 128 fp32 values and 16 (max, sum) pairs
    assert need == (12544 + a256((4 + 3) * 8) + a256(3 * 2 * 8) + 3 * 8 * 2 * 16 * 128 * 4
                    + 3 * 8 * 2 * 16 * 2 * 4)
    assert lib.paged_attention_varlen_workspace_size(3, 50, 8, 96, 2000) == 0
    assert lib.paged_attention_varlen_workspace_size(3, -1, 8, 128, 2000) == 0
    assert lib.paged_attention_varlen_workspace_size(1, 1, 8, 128, 0) == (
        12544 + 256 + 256 + 8 * 16 * 130 * 4)
    base = [p, p, p, p, 100, p, 125, p, p, 3, 50, 2000, 32, 8, 128, 0.088, BF16, BF16,
            p, need, None]

    def call(**k):
        a = list(base)
        for i, v in k.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a9=0) == OK
    assert call(a10=0) == OK
    assert call(a0=None) == NULL
    assert call(a1=p + 4) == ALIGN
    assert call(a12=30) == SHAPE                 # not a multiple of hkv
    assert call(a12=72) == UNSUP                 # group 9
    assert call(a14=96) == UNSUP
    assert call(a17=FP8) == UNSUP
    assert call(a15=0.0) == UNSUP
    assert call(a15=-0.5) == UNSUP
    assert call(a6=124) == SHAPE                 # 1,984 tokens < max_seq_len
    assert call(a4=0) == SHAPE
    assert call(a11=-1) == SHAPE
    assert call(a18=None) == WS
    assert call(a19=need - 1) == WS
    assert call(a18=p + 8) == ALIGN


def test_int4_errors(lib):
    f = lib.reshape_and_cache_int4
    p = 0x100000
    base = [p, p, p, p, p, p, p, 4, 8, 128, 100, BF16, None]

    def call(**k):
        a = list(base)
        for i, v in k.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a7=0) == OK
    assert call(a4=None) == NULL
    assert call(a0=p + 4) == ALIGN
    assert call(a9=130) == UNSUP          # more than 128 elements per row
    assert call(a9=63) == UNSUP           # odd
    assert call(a11=FP8) == UNSUP
    assert call(a8=0) == SHAPE
    d = lib.paged_attention_decode_int4
    need = lib.paged_attention_decode_workspace_size(4, 32, 8, 128, 1000, 0)
    dbase = [p, p, p, p, p, p, 100, p, 63, p, 4, 1000, 32, 8, 128, 0.088, BF16, 0, p, need,
             None]

    def dcall(**k):
        a = list(dbase)
        for i, v in k.items():
            a[int(i[1:])] = v
        return d(*a)

    assert dcall(a10=0) == OK
    assert dcall(a4=None) == NULL
    assert dcall(a5=p + 4) == ALIGN
    assert dcall(a14=64) == UNSUP
    assert dcall(a16=F32) == UNSUP
    assert dcall(a12=72) == UNSUP         # group 9
    assert dcall(a8=62) == SHAPE          # 992 tokens < max_context_len
    assert dcall(a17=100) == SHAPE        # partition not a multiple of 16
    assert dcall(a19=need - 1) == WS


def _append(lib, **k):
    p = 0x100000
    a = dict(out=p, q=p, nk=p, nv=p, kc=p, vc=p, nb=100, bt=p, maxb=64, lens=p, s=4,
             maxlen=1000, hq=32, hkv=8, d=128, scale=0.088, qd=BF16, kvd=BF16, ks=1.0,
             vs=1.0, part=0, ws=p, wsb=1 << 30)
    a.update(k)
    return lib.paged_attention_decode_append(
        a["out"], a["q"], a["nk"], a["nv"], a["kc"], a["vc"], a["nb"], a["bt"], a["maxb"],
        a["lens"], a["s"], a["maxlen"], a["hq"], a["hkv"], a["d"], a["scale"], a["qd"],
        a["kvd"], a["ks"], a["vs"], a["part"], a["ws"], a["wsb"], None)


def test_decode_append_errors(lib):
    assert _append(lib, s=0) == OK
    assert _append(lib, s=0, nk=None) == OK            # no rows to write
    assert _append(lib, nk=None) == NULL
    assert _append(lib, nv=None) == NULL
    assert _append(lib, out=None) == NULL
    assert _append(lib, nk=0x100008) == ALIGN
    assert _append(lib, nv=0x100004) == ALIGN
    assert _append(lib, qd=F32, kvd=F32) == UNSUP       # the write is in the matrix-core kernel
    assert _append(lib, kvd=F32) == UNSUP
    assert _append(lib, d=96) == UNSUP
    assert _append(lib, hq=72) == UNSUP                 # group 9
    assert _append(lib, hq=30) == SHAPE
    assert _append(lib, maxb=10) == SHAPE
    assert _append(lib, part=100) == SHAPE
    assert _append(lib, kvd=FP8, ks=0.0) == SHAPE
    need = lib.paged_attention_decode_workspace_size(4, 32, 8, 128, 1000, 0)
    assert _append(lib, wsb=need - 1) == WS


def test_sliding_errors(lib):
    f = lib.paged_attention_decode_sliding
    p = 0x100000
    need = lib.paged_attention_decode_workspace_size(4, 32, 8, 128, 1000, 0)
    base = [p, p, p, p, 100, p, 63, p, 4, 1000, 32, 8, 128, 0.088, BF16, BF16, 1.0, 1.0, 256,
            0, p, need, None]

    def call(**k):
        a = list(base)
        for i, v in k.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a8=0) == OK
    assert call(a18=0) == SHAPE           # window must be positive
    assert call(a18=-5) == SHAPE
    assert call(a14=F32, a15=F32) == UNSUP  # the window is built into the matrix-core path
    assert call(a0=None) == NULL
    assert call(a21=need - 1) == WS


def test_nvfp4_errors(lib):
    f = lib.reshape_and_cache_nvfp4
    p = 0x100000
    base = [p, p, p, p, p, p, p, 4, 8, 128, 100, BF16, 1.0, 1.0, None]

    def call(**k):
        a = list(base)
        for i, v in k.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a7=0) == OK
    assert call(a5=None) == NULL
    assert call(a4=p + 4) == ALIGN
    assert call(a9=144) == UNSUP          # more than 128 elements per row
    assert call(a9=40) == UNSUP           # not a multiple of 16
    assert call(a11=FP8) == UNSUP
    assert call(a8=0) == SHAPE
    assert call(a12=0.0) == SHAPE
    assert call(a13=-1.0) == SHAPE
    assert call(a13=float("inf")) == SHAPE
    d = lib.paged_attention_decode_nvfp4
    need = lib.paged_attention_decode_workspace_size(4, 32, 8, 128, 1000, 0)
    dbase = [p, p, p, p, p, p, 100, p, 63, p, 4, 1000, 32, 8, 128, 0.088, BF16, 1.0, 1.0, 0,
             p, need, None]

    def dcall(**k):
        a = list(dbase)
        for i, v in k.items():
            a[int(i[1:])] = v
        return d(*a)

    assert dcall(a10=0) == OK
    assert dcall(a4=None) == NULL
    assert dcall(a5=p + 4) == ALIGN
    assert dcall(a14=64) == UNSUP
    assert dcall(a16=F32) == UNSUP
    assert dcall(a12=72) == UNSUP         # group 9
    assert dcall(a8=62) == SHAPE          # 992 tokens < max_context_len
    assert dcall(a19=100) == SHAPE        # partition not a multiple of 16
    assert dcall(a17=0.0) == SHAPE
    assert dcall(a18=-2.0) == SHAPE
    assert dcall(a21=need - 1) == WS
    assert dcall(a20=None) == WS


def test_measure_errors(lib):
    p = 0x100000
    f = lib.pkv_measure_hbm_read
    assert f(p, 0, p, None) == SHAPE
    assert f(p, 24, p, None) == SHAPE            # not a multiple of 16
    assert f(p, 1 << 40, p, None) == SHAPE
    assert f(None, 64, p, None) == NULL
    assert f(p, 64, None, None) == NULL
    assert f(p + 8, 64, p, None) == ALIGN
    assert f(p, 64, p + 2, None) == ALIGN
    g = lib.pkv_measure_mfma_bf16
    assert g(0, 8, p, None) == SHAPE
    assert g(524289, 8, p, None) == SHAPE
    assert g(10, 12, p, None) == SHAPE           # not a multiple of 8
    assert g(10, 0, p, None) == SHAPE
    assert g(10, 8, None, None) == NULL
    assert g(10, 8, p + 2, None) == ALIGN
    h = lib.pkv_measure_mfma_valu
    assert h(0, 8, 0, p, None) == SHAPE
    assert h(524289, 8, 2, p, None) == SHAPE
    assert h(10, 12, 1, p, None) == SHAPE
    assert h(10, 8, 3, p, None) == SHAPE
    assert h(10, 8, -1, p, None) == SHAPE
    assert h(10, 8, 2, None, None) == NULL
    assert h(10, 8, 2, p + 2, None) == ALIGN
