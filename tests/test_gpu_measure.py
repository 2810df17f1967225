"""The ceiling kernels do the work they are timed for: the HBM read folds
every word of its buffer into the checksum, the MFMA loop accumulates the
products it issues, the MFMA-with-vector-work loop runs each part its mode
asks for."""

import numpy as np
import pytest
import torch

import paged_kv_cache_84_amd as pk
from gpu_util import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (64 << 20) + 16 * 77])
def test_hbm_read_checksum_covers_every_word(nbytes):
    announce("hbm read checksum", nbytes)
    g = torch.Generator(device=DEV).manual_seed(nbytes)
    words = torch.randint(-(1 << 31), (1 << 31) - 1, (nbytes // 4,), generator=g,
                          device=DEV, dtype=torch.int64).to(torch.int32)
    checksum = torch.full((1,), 12345, dtype=torch.int32, device=DEV)   # cleared by the call
    pk.measure_hbm_read(words, checksum)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(words.cpu().numpy().view(np.uint32))
    assert int(checksum.cpu().numpy().view(np.uint32)[0]) == int(want)


@pytest.mark.parametrize("iterations,waves", [(1, 8), (37, 64), (4096, 2048)])
def test_mfma_loop_accumulates_every_product(iterations, waves):
    announce("mfma loop", iterations, waves)
    result = torch.zeros(waves, dtype=torch.float32, device=DEV)
    pk.measure_mfma_bf16(iterations, result)
    torch.cuda.synchronize()
    assert torch.all(result == 32.0 * iterations)


def _vector_sum(iterations):
    """The vector chains' sum in float64: x <- 0.5 x + 0.25 from x0 = j / 8,
    p = 2^(x - 1) on chains 0 and 3 (else p = x), y += p - (p with its low
    16 bits cleared)."""
    total = 0.0
    for j in range(5):
        x = np.float32(0.125 * j)
        y = 0.0
        for _ in range(iterations):
            x = np.float32(x * np.float32(0.5) + np.float32(0.25))
            p = np.float32(2.0 ** (float(x) - 1.0)) if j % 3 == 0 else x
            hi = np.array([p], np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
            y += float(p) - float(hi.view(np.float32)[0])
        total += y
    return total


@pytest.mark.parametrize("iterations,waves", [(1, 8), (37, 64), (512, 2048)])
def test_mfma_valu_modes(iterations, waves):
    announce("mfma + vector loop", iterations, waves)
    want_v = _vector_sum(iterations)
    assert want_v > 0
    got = []
    for mode in range(3):
        r = torch.full((2 * waves,), -7.0, dtype=torch.float32, device=DEV)
        pk.measure_mfma_valu(iterations, mode, r)
        torch.cuda.synchronize()
        r = r.view(-1, 2).cpu()
        assert torch.all(r[:, 0] == (0.0 if mode == 1 else 32.0 * iterations))
        assert torch.all(r[:, 1] == r[0, 1])
        got.append(float(r[0, 1]))
    assert got[0] == 0.0
    assert got[1] == got[2]
    assert abs(got[1] - want_v) <= 1e-2 * want_v
