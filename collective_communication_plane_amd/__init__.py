"""MI355X-native reduce/copy data plane for collectives over P rank buffers on one GPU.

The product is ``libccl.so`` (C ABI in ``include/ccl.h``, HIP kernels for
gfx950 in ``csrc/``); ``ccl`` is its thin ctypes binding.
"""
from . import ccl  # noqa: F401

__all__ = ["ccl"]
