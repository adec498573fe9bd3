"""Parity bar between the HIP path and the CPU oracle, plus GPU buffer helpers.

The bar:
  * int32, min/max and every copy: bit-exact.
  * fp32 sum: bit-equal, or |got - want| <= 1e-6 * max(|want|, 2^-126).
  * bf16 and fp16 sum: the two values are at most 1 ulp apart (their
    sign-magnitude ordinals differ by <= 1).
Both sides fold in fp32 in rank order 0..P-1, so bit equality is expected;
the tolerance is the stated bar, and non-bit-equal counts are reported.
"""
from __future__ import annotations

import numpy as np

CANARY = 0xA5


def _ordinal_bf16(h: np.ndarray) -> np.ndarray:
    h = h.astype(np.int64)
    mag = h & 0x7FFF
    return np.where(h & 0x8000, -mag, mag)


def assert_parity(got: np.ndarray, want: np.ndarray, dtype: str, op: str, what: str = "") -> int:
    """Assert the bar; returns the number of elements that are not bit-equal."""
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    half = dtype in ("bf16", "f16")
    gb = got.view(np.uint16 if half else np.uint32)
    wb = want.view(np.uint16 if half else np.uint32)
    neq = gb != wb
    n_neq = int(np.count_nonzero(neq))
    if n_neq == 0:
        return 0
    if dtype == "i32" or op != "sum":
        i = int(np.argmax(neq))
        raise AssertionError(f"{what}: {n_neq} elements differ (first at {i}: {got[i]!r} vs {want[i]!r})")
    if dtype == "f32":
        g = got.astype(np.float64)
        w = want.astype(np.float64)
        tol = 1e-6 * np.maximum(np.abs(w), 2.0 ** -126)
        bad = neq & ~(np.abs(g - w) <= tol)
    else:
        bad = neq & (np.abs(_ordinal_bf16(gb) - _ordinal_bf16(wb)) > 1)
    nbad = int(np.count_nonzero(bad))
    if nbad:
        i = int(np.argmax(bad))
        raise AssertionError(f"{what}: {nbad} elements outside tolerance (first at {i}: "
                             f"{got[i]!r} vs {want[i]!r})")
    return n_neq


class DevBuf:
    """A device byte buffer with canary guard bands around the payload."""

    def __init__(self, nbytes: int, device, offset: int = 0, pad: int = 256, fill: int = CANARY):
        import torch

        self.nbytes = nbytes
        self.pad = pad + offset
        self.base = torch.full((self.pad + nbytes + pad,), fill, dtype=torch.uint8, device=device)
        self.tail = pad
        self.fill = fill

    @property
    def ptr(self) -> int:
        return self.base.data_ptr() + self.pad

    def upload(self, arr: np.ndarray) -> "DevBuf":
        import torch

        b = np.ascontiguousarray(arr).view(np.uint8).ravel()
        assert b.size == self.nbytes
        self.base[self.pad:self.pad + self.nbytes].copy_(torch.from_numpy(b.copy()))
        return self

    def download(self, dtype) -> np.ndarray:
        return self.base[self.pad:self.pad + self.nbytes].cpu().numpy().view(dtype)

    def guards_intact(self) -> bool:
        lo = self.base[: self.pad]
        hi = self.base[self.pad + self.nbytes:]
        return bool((lo == self.fill).all().item()) and bool((hi == self.fill).all().item())


def upload_all(arrays, device, offset: int = 0):
    return [DevBuf(a.nbytes, device, offset).upload(a) for a in arrays]


def assert_rmsnorm_parity(got: np.ndarray, want: np.ndarray, dtype: str, hidden: int,
                          what: str = "") -> int:
    """The fused all-reduce + RMSNorm bar.  The kernel sums squares in fp32 in
    its own order while the oracle works in fp64, so the fp32 result may
    differ by (hidden/2 + 4) * 2^-24 relative (recursive-summation bound on
    the sum of squares, halved by the square root, plus the final products);
    that is below one bf16 or fp16 ulp, so those must be within 1 ulp."""
    half = dtype in ("bf16", "f16")
    gb = got.view(np.uint16 if half else np.uint32)
    wb = want.view(np.uint16 if half else np.uint32)
    neq = gb != wb
    if not np.any(neq):
        return 0
    if half:
        bad = neq & (np.abs(_ordinal_bf16(gb) - _ordinal_bf16(wb)) > 1)
    else:
        g = got.astype(np.float64)
        w = want.astype(np.float64)
        tol = (hidden / 2 + 4) * 2.0 ** -24 * np.abs(w) + 2.0 ** -126
        bad = neq & ~(np.abs(g - w) <= tol)
    nbad = int(np.count_nonzero(bad))
    if nbad:
        i = int(np.argmax(bad))
        raise AssertionError(f"{what}: {nbad} elements outside tolerance (first at {i}: "
                             f"{got[i]!r} vs {want[i]!r})")
    return int(np.count_nonzero(neq))
