"""The ceiling kernels do the work they are timed for: the HBM read folds
every word of its buffer into the checksum, the MFMA loop accumulates the
products it issues."""

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
