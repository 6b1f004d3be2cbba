"""MI355X (gfx950) decode-step hot path of ECHO's lossless KV-cache offloading.

`abi` binds the C ABI of libecho.so (include/echo.h); `runtime` allocates the
buffers it needs (device memory through torch, the host pool through HIP).
"""
from . import abi  # noqa: F401

__all__ = ["abi"]
