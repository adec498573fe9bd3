"""Seeded synthetic rank buffers, shared by the tests, the smoke check and the bench.

This module only draws numbers: it holds none of the collectives' arithmetic.
Every draw uses numpy's PCG64 ``default_rng(seed)``; rank r's buffer is the
r-th draw of N values from one generator (rank-major order).  bf16 buffers are
fp32 draws converted by PyTorch's CPU ``to(torch.bfloat16)`` (round to nearest
even) and returned as uint16 bit patterns; fp16 buffers likewise through numpy's
``astype(float16)``.

Distributions (the workloads the reduce/copy data plane is measured on):
  ``uniform``  2*U - 1 with U ~ U[0,1) in float32, i.e. values in [-1, 1)
  ``normal``   standard normal, float32
  ``w002``     0.02 * standard normal (weight-like tensors for reshard)
  ``int20``    integers uniform in [-2**20, 2**20], int32
"""
from __future__ import annotations

import numpy as np

NP_TYPES = {"f32": np.float32, "bf16": np.uint16, "i32": np.int32, "f16": np.uint16}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns (PyTorch's RNE conversion)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 values (PyTorch's widening)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(h, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).float().numpy()


def _draw(rng: np.random.Generator, dist: str, n: int, dtype: str) -> np.ndarray:
    if dist == "int20":
        if dtype != "i32":
            raise ValueError("int20 draws are int32")
        return rng.integers(-(2**20), 2**20, size=n, dtype=np.int32, endpoint=True)
    if dist == "uniform":
        x = rng.random(n, dtype=np.float32)
        x *= np.float32(2.0)
        x -= np.float32(1.0)
    elif dist == "normal":
        x = rng.standard_normal(n, dtype=np.float32)
    elif dist == "w002":
        x = rng.standard_normal(n, dtype=np.float32)
        x *= np.float32(0.02)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return to_bf16_bits(x)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "i32":
        raise ValueError("float draws cannot fill int32 buffers")
    raise ValueError(f"unknown dtype {dtype!r}")


def rank_buffers(P: int, n: int, dtype: str, dist: str, seed: int = 0) -> list[np.ndarray]:
    """P buffers of n elements; buffer r is the r-th draw from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    return [_draw(rng, dist, n, dtype) for _ in range(P)]


def tensor(shape, dtype: str, dist: str, seed: int = 0) -> np.ndarray:
    """One global tensor of the given shape (row-major), drawn like one rank buffer."""
    rng = np.random.default_rng(seed)
    return _draw(rng, dist, int(np.prod(shape)), dtype).reshape(shape)


def sample_indices(n: int, k: int, seed: int = 1) -> np.ndarray:
    """k distinct-ish sorted indices in [0, n) plus both ends, for sampled checks."""
    if n <= 0:
        return np.zeros(0, np.uint64)
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, n, size=min(k, n), dtype=np.int64)
    idx = np.unique(np.concatenate([idx, [0, n - 1]]))
    return idx.astype(np.uint64)


def device_rank_buffers(P: int, n: int, dtype: str, dist: str, seed: int, device):
    """P device tensors drawn on the GPU with PyTorch's seeded generator.

    For sizes whose host-side draw would take too long (e.g. 1 GiB per rank);
    the tests copy back only sampled values for the oracle.  Returns a list of
    contiguous torch tensors (bf16 as torch.bfloat16, f32, i32).
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for _ in range(P):
        if dist == "uniform":
            x = torch.rand(n, generator=g, device=device, dtype=torch.float32)
            x.mul_(2.0).sub_(1.0)
        elif dist == "normal":
            x = torch.randn(n, generator=g, device=device, dtype=torch.float32)
        elif dist == "int20":
            x = torch.randint(-(2**20), 2**20 + 1, (n,), generator=g, device=device,
                              dtype=torch.int32)
        else:
            raise ValueError(dist)
        if dtype == "bf16":
            x = x.to(torch.bfloat16)
        elif dtype == "i32" and dist != "int20":
            raise ValueError("float draws cannot fill int32 buffers")
        out.append(x.contiguous())
    return out
