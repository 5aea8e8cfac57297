"""MI355X (gfx950) denoising-step library for masked-diffusion LMs.

One denoising iteration over the current block -- vicinity KV refresh,
bidirectional attention over the cached KV, LM head with fused vocab
statistics, and the parallel-decode commit -- in hand-written HIP kernels
behind the C ABI of include/dinfer.h (libdinfer.so).  This package is the thin
Python binding: argument marshalling, with PyTorch providing device memory and
streams.
"""
from .binding import load, DinferError, LIB_PATH, EXPORTS  # noqa: F401


def Engine(*args, **kwargs):  # noqa: N802 - thin factory, keeps import light
    from .engine import Engine as _E
    return _E(*args, **kwargs)
