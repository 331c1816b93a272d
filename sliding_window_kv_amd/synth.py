"""Seeded synthetic inputs shared by the tests and the benchmark.

Only random numbers and integer structure (permutations, lengths, offsets)
come from here; nothing in this module computes any part of the method.
Host-side draws use numpy's PCG64; multi-GB device fills use torch's
generator on the device.
"""
from __future__ import annotations

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(shape, seed: int) -> np.ndarray:
    """N(0, 1) float32 array."""
    return rng(seed).standard_normal(shape, dtype=np.float32)


def block_table_permutation(batch: int, max_blocks: int, num_blocks: int, seed: int) -> np.ndarray:
    """[batch, max_blocks] int32: distinct physical blocks drawn from a random permutation of the pool."""
    if batch * max_blocks > num_blocks:
        raise ValueError("pool too small for the table")
    perm = rng(seed).permutation(num_blocks)[: batch * max_blocks]
    return perm.reshape(batch, max_blocks).astype(np.int32)


def uniform_lengths(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """n integers uniform in [lo, hi] (inclusive)."""
    return rng(seed).integers(lo, hi + 1, size=n).astype(np.int32)


def uniform_ints(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """n integers uniform in [lo, hi) (exclusive)."""
    return rng(seed).integers(lo, hi, size=n).astype(np.int32)


def device_normal_(tensor, seed: int):
    """Fill a device tensor in place with N(0, 1) from a seeded device generator."""
    import torch

    g = torch.Generator(device=tensor.device)
    g.manual_seed(seed)
    if tensor.dtype in (torch.float32, torch.float16, torch.bfloat16):
        tensor.normal_(0.0, 1.0, generator=g)
    else:
        raise TypeError(f"unsupported dtype {tensor.dtype}")
    return tensor


def device_int8_codes_(tensor, seed: int):
    """Fill an int8 device tensor in place with codes uniform in [-127, 127] (seeded device generator)."""
    import torch

    if tensor.dtype != torch.int8:
        raise TypeError(f"expected int8, got {tensor.dtype}")
    g = torch.Generator(device=tensor.device)
    g.manual_seed(seed)
    tensor.copy_(torch.randint(-127, 128, tensor.shape, generator=g, device=tensor.device, dtype=torch.int16))
    return tensor


def device_fp8_codes_(tensor, seed: int):
    """Fill a uint8 device tensor in place with bytes uniform over [0, 255] minus 127 and 255
    (the two bytes an E4M3 cache never holds: they are NaN), seeded device generator."""
    import torch

    if tensor.dtype != torch.uint8:
        raise TypeError(f"expected uint8, got {tensor.dtype}")
    g = torch.Generator(device=tensor.device)
    g.manual_seed(seed)
    x = torch.randint(0, 254, tensor.shape, generator=g, device=tensor.device, dtype=torch.int16)
    tensor.copy_(x + (x >= 127).to(torch.int16))
    return tensor


def device_uniform_(tensor, lo: float, hi: float, seed: int):
    """Fill a float device tensor in place with U(lo, hi) from a seeded device generator."""
    import torch

    g = torch.Generator(device=tensor.device)
    g.manual_seed(seed)
    tensor.uniform_(lo, hi, generator=g)
    return tensor
