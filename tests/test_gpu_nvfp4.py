"""nvfp4-style KV cache on the GPU (E2M1 codes, an E4M3 scale per 16
elements, a per-tensor scale): the cache write bit-exact with the oracle's
encoder, the decode against the fp64 oracle over the dequantised rows."""

import numpy as np
import pytest
import torch

import paged_kv_cache_84_amd as pk
from gpu_util import announce, as_f64, host
from oracle import formats as F
from oracle import paged as P
from synth import rng as R
from synth.allocator import BlockPool, Sequence, tables_array
from tolerance import assert_attention_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALE = 1.0 / 128 ** 0.5


def _write_case(src, d, g_k, g_v, t=40, nb=12, hkv=4, seed=0):
    sdt = F.BF16 if src == "bf16" else F.F32
    key = R.normal((t, hkv, d), sdt, 900 + seed, 1, DEV, std=3.0)
    value = R.normal((t, hkv, d), sdt, 900 + seed, 2, DEV)
    key[3] = 0                                    # zero rows: scale code 0, codes 0
    key[4, :, :16] = -0.0                         # a zero block with negative zeros
    value[5, 1, :] = 1e-30 if src == "f32" else 1e-36   # scale rounds to 0
    value[6, 0, :] = 5e4                          # block scale saturates at 448
    if d >= 32:   # E2M1 ties under S * g = 1
        key[8, 2, 16:32] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 2,
                                        device=DEV).to(key.dtype)
    rng = np.random.default_rng(4 + seed)
    slots = rng.permutation(nb * 16)[:t].astype(np.int64)
    slots[[7, 20]] = -1
    kc = R.int4_codes((nb, hkv, 16, d // 2), 900 + seed, 3, DEV)
    vc = R.int4_codes((nb, hkv, 16, d // 2), 900 + seed, 4, DEV)
    ks = R.int4_codes((nb, hkv, 16, d // 16), 900 + seed, 5, DEV)
    vs = R.int4_codes((nb, hkv, 16, d // 16), 900 + seed, 6, DEV)
    return sdt, key, value, kc, vc, ks, vs, slots


@pytest.mark.parametrize("src,d,g_k,g_v", [("bf16", 128, 1.0, 1.0), ("f32", 128, 0.37, 2.5),
                                            ("bf16", 64, 0.01, 0.5), ("f32", 16, 1.0, 1e-3)])
def test_nvfp4_cache_write_bit_exact(src, d, g_k, g_v):
    announce("nvfp4 write", src, d, g_k, g_v)
    sdt, key, value, kc, vc, ks, vs, slots = _write_case(src, d, g_k, g_v)
    if d >= 32 and g_k == 1.0:
        # the tie row really is one: block max 6 under g = 1 gives S = 1
        assert float(key[8, 2, 16:32].abs().max()) == 6.0
    want = P.reshape_and_cache_nvfp4(host(key), host(value), host(kc), host(vc), host(ks),
                                     host(vs), slots, sdt, g_k, g_v)
    pk.reshape_and_cache_nvfp4(key, value, kc, vc, ks, vs, torch.as_tensor(slots, device=DEV),
                               g_k, g_v)
    torch.cuda.synchronize()
    for got, ref, what in zip((kc, vc, ks, vs), want, ("k codes", "v codes", "k scales",
                                                        "v scales")):
        assert np.array_equal(host(got), ref), what


def _nvfp4_batch(lengths, hq, hkv, seed, poison=False):
    rng = np.random.default_rng(seed)
    nb = sum(P.blocks_needed(n) for n in lengths) + 7
    pool = BlockPool(nb, rng.permutation(nb))
    seqs = [Sequence.fresh(pool, n) for n in lengths]
    tables = tables_array(seqs)
    kc = R.int4_codes((nb, hkv, 16, 64), 950 + seed, 1, DEV)
    vc = R.int4_codes((nb, hkv, 16, 64), 950 + seed, 2, DEV)
    ks = R.nvfp4_bscales((nb, hkv, 16, 8), 950 + seed, 3, DEV)
    vs = R.nvfp4_bscales((nb, hkv, 16, 8), 950 + seed, 4, DEV)
    if poison:
        # NaN block scales (0x7F) in the unused slots of last blocks and in
        # every block no sequence owns
        used = {b for sq in seqs for b in sq.table}
        for sq, n in zip(seqs, lengths):
            if n % 16:
                last = sq.table[(n - 1) // 16]
                ks[last, :, n % 16:] = 0x7F
                vs[last, :, n % 16:] = 0xFF
        free = [b for b in range(nb) if b not in used]
        ks[free] = 0x7F
        vs[free] = 0x7F
    q = R.normal((len(lengths), hq, 128), F.BF16, 950 + seed, 5, DEV)
    return q, kc, vc, ks, vs, tables, np.array(lengths, np.int32)


def _run(q, kc, vc, ks, vs, tables, lens, g_k, g_v, partition=0):
    return pk.paged_attention_decode_nvfp4(q, kc, vc, ks, vs, torch.as_tensor(tables, device=DEV),
                                           torch.as_tensor(lens, device=DEV), int(lens.max()),
                                           SCALE, g_k, g_v, partition_tokens=partition)


def _oracle(q, kc, vc, ks, vs, tables, lens, g_k, g_v):
    return P.decode_attention_nvfp4(host(q), F.BF16, host(kc), host(vc), host(ks), host(vs),
                                    tables, lens, float(np.float32(SCALE)),
                                    float(np.float32(g_k)), float(np.float32(g_v)))


@pytest.mark.parametrize("hq,hkv", [(32, 8), (64, 8), (16, 16), (8, 2)])
@pytest.mark.parametrize("partition", [0, 64])
def test_nvfp4_decode_ragged_batch(hq, hkv, partition):
    """Ragged lengths (1 token, partial and exact blocks, several partitions),
    shuffled blocks, per-tensor scales other than 1, every output against
    the oracle."""
    announce("nvfp4 decode", hq, hkv, partition)
    lengths = [1, 15, 16, 17, 100, 333, 512, 700]
    args = _nvfp4_batch(lengths, hq, hkv, seed=hq + hkv + partition)
    out = _run(*args, 0.75, 1.5, partition=partition)
    torch.cuda.synchronize()
    assert_attention_close(as_f64(out), _oracle(*args, 0.75, 1.5), "bf16",
                           f"nvfp4 decode {hq}/{hkv}")


def test_nvfp4_decode_poisoned_scales_do_not_leak():
    """NaN block scales in unused slots and free blocks never reach an output."""
    announce("nvfp4 decode poison")
    args = _nvfp4_batch([3, 40, 129, 250], 32, 8, seed=9, poison=True)
    out = _run(*args, 1.0, 1.0)
    torch.cuda.synchronize()
    got = as_f64(out)
    assert np.all(np.isfinite(got))
    assert_attention_close(got, _oracle(*args, 1.0, 1.0), "bf16", "nvfp4 poison")


def test_nvfp4_write_then_decode():
    """The GPU writer fills an nvfp4 cache from bf16 rows; the decode over it
    matches the oracle's decode over the oracle's own encoding of the same
    rows (the two encodings are bit-equal, so this checks the pair end to
    end)."""
    announce("nvfp4 write + decode")
    lengths = [37, 160, 255]
    hq, hkv = 32, 8
    rng = np.random.default_rng(21)
    nb = sum(P.blocks_needed(n) for n in lengths) + 3
    pool = BlockPool(nb, rng.permutation(nb))
    seqs = [Sequence.fresh(pool, n) for n in lengths]
    tables = tables_array(seqs)
    slots = np.concatenate([[sq.table[p // 16] * 16 + p % 16 for p in range(n)]
                            for sq, n in zip(seqs, lengths)]).astype(np.int64)
    t = len(slots)
    key = R.normal((t, hkv, 128), F.BF16, 970, 1, DEV)
    value = R.normal((t, hkv, 128), F.BF16, 970, 2, DEV)
    kc = torch.zeros((nb, hkv, 16, 64), dtype=torch.uint8, device=DEV)
    vc = torch.zeros_like(kc)
    ks = torch.zeros((nb, hkv, 16, 8), dtype=torch.uint8, device=DEV)
    vs = torch.zeros_like(ks)
    g_k, g_v = 0.5, 0.25
    pk.reshape_and_cache_nvfp4(key, value, kc, vc, ks, vs, torch.as_tensor(slots, device=DEV),
                               g_k, g_v)
    q = R.normal((len(lengths), hq, 128), F.BF16, 970, 3, DEV)
    lens = np.array(lengths, np.int32)
    out = _run(q, kc, vc, ks, vs, tables, lens, g_k, g_v)
    torch.cuda.synchronize()
    okc, ovc, oks, ovs = P.reshape_and_cache_nvfp4(
        host(key), host(value), np.zeros((nb, hkv, 16, 64), np.uint8),
        np.zeros((nb, hkv, 16, 64), np.uint8), np.zeros((nb, hkv, 16, 8), np.uint8),
        np.zeros((nb, hkv, 16, 8), np.uint8), slots, F.BF16, g_k, g_v)
    ref = P.decode_attention_nvfp4(host(q), F.BF16, okc, ovc, oks, ovs, tables, lens,
                                   float(np.float32(SCALE)), g_k, g_v)
    assert_attention_close(as_f64(out), ref, "bf16", "nvfp4 write + decode")


def test_nvfp4_decode_llama8b_batch_sampled():
    """The 8B decode batch (64 sequences, 512..4096 tokens, 32 q / 8 kv
    heads) over an nvfp4 cache, as the benchmark times it: sampled outputs
    against the oracle, and bitwise equal on a second call."""
    announce("nvfp4 decode 8B sampled")
    rng = np.random.default_rng(64)
    lengths = [int(x) for x in rng.integers(512, 4097, 64)]
    q, kc, vc, ks, vs, tables, lens = _nvfp4_batch(lengths, 32, 8, seed=64)
    out = _run(q, kc, vc, ks, vs, tables, lens, 1.0, 1.0).clone()
    again = _run(q, kc, vc, ks, vs, tables, lens, 1.0, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    hq_, kc_, vc_, ks_, vs_ = host(q), host(kc), host(vc), host(ks), host(vs)
    got, ref = [], []
    for seq, head in zip(rng.integers(0, 64, 12), rng.integers(0, 32, 12)):
        seq, head = int(seq), int(head)
        kvh = head // 4
        keys = P.gather_kv_nvfp4(kc_, ks_, 1.0, tables[seq], int(lens[seq]), kvh)
        values = P.gather_kv_nvfp4(vc_, vs_, 1.0, tables[seq], int(lens[seq]), kvh)
        ref.append(P.attention_row(F.bf16_bits_to_f64(hq_[seq, head]), keys, values,
                                   float(np.float32(SCALE))))
        got.append(as_f64(out[seq, head]))
    assert_attention_close(np.array(got), np.array(ref), "bf16", "nvfp4 8B sampled")
