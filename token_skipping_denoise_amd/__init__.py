"""MI355X (gfx950) library for one token-skipping denoising iteration of a
bidirectional masked-diffusion transformer.

The compute path is the HIP library ``libdllm.so`` (C ABI in include/dllm.h);
``api`` is a thin torch binding that marshals pointers and streams.
"""
from . import _ffi  # noqa: F401

__all__ = ["api", "build"]
