"""Seeded value generators.

Structure (lengths, placements) comes from ``numpy.random.default_rng`` seeded
with ``[config_id, purpose]``; tensor values from a ``torch.Generator`` seeded
with ``config_id * 1000 + purpose`` on the device the values are made on.
Values are returned as storage: float32, bf16 bit patterns (uint16 / int16
views) or fp8 E4M3 codes (uint8).
"""

import numpy as np
import torch

F32, BF16, FP8_E4M3 = "f32", "bf16", "fp8_e4m3"

TORCH_STORAGE = {F32: torch.float32, BF16: torch.bfloat16,
                 FP8_E4M3: torch.float8_e4m3fn}


def structure_rng(config_id, purpose):
    return np.random.default_rng([int(config_id), int(purpose)])


def value_generator(config_id, purpose, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(config_id) * 1000 + int(purpose))
    return g


def normal(shape, dtype, config_id, purpose, device="cpu", std=1.0):
    """i.i.d. N(0, std^2) values stored as ``dtype`` (bf16 rounds to nearest
    even through torch's cast).  Returns a torch tensor on ``device``."""
    g = value_generator(config_id, purpose, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if dtype == F32:
        return x
    if dtype == BF16:
        return x.to(torch.bfloat16)
    raise ValueError(dtype)


def fp8_normal(shape, config_id, purpose, device="cpu", chunk=1 << 26):
    """fp8 E4M3 cache contents whose values are N(0,1) samples under a
    per-tensor scale.

    The samples are drawn in bf16, the scale is amax/448 over them, and each
    code is torch's own float8_e4m3fn cast of sample/scale (a library cast,
    not this project's quantiser).  Returns (codes uint8 tensor, scale)."""
    x = normal(shape, BF16, config_id, purpose, device)
    amax = float(x.abs().max().float())
    scale = float(np.float32(amax / 448.0))
    codes = torch.empty(shape, dtype=torch.uint8, device=device)
    flat_x, flat_c = x.view(-1), codes.view(-1)
    for start in range(0, flat_x.numel(), chunk):
        part = flat_x[start:start + chunk].float() / scale
        flat_c[start:start + chunk] = part.to(torch.float8_e4m3fn).view(torch.uint8)
    del x
    return codes, scale


def to_numpy_storage(t):
    """Torch storage tensor -> numpy array of the raw storage type."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def storage_dtype_of(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise ValueError(t.dtype)


def int4_codes(shape, config_id, purpose, device="cpu"):
    """Packed int4 codes: uniform random bytes (every byte is two valid
    codes), uint8 ``shape`` (the last dim is head_dim / 2)."""
    g = value_generator(config_id, purpose, device)
    return torch.randint(0, 256, shape, generator=g, device=device, dtype=torch.int32).to(
        torch.uint8)


def int4_scales(shape, config_id, purpose, device="cpu", lo=0.05, hi=0.6):
    """Per-row int4 scales: float32 uniform in [lo, hi) (max|x| / 7 of N(0, 1)
    rows of 128 values lies near 0.4)."""
    g = value_generator(config_id, purpose, device)
    return lo + (hi - lo) * torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def nvfp4_bscales(shape, config_id, purpose, device="cpu", lo=0x28, hi=0x3A):
    """nvfp4 block-scale bytes: E4M3 codes uniform in [lo, hi) (0x28 .. 0x39
    are 0.25 .. 1.125, the range max|x| / 6 of N(0, 1) blocks of 16 lands
    in under a unit per-tensor scale); uint8 ``shape``."""
    g = value_generator(config_id, purpose, device)
    return torch.randint(lo, hi, shape, generator=g, device=device, dtype=torch.int32).to(
        torch.uint8)
