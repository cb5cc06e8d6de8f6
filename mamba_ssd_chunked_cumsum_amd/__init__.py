"""libssd: Mamba-2 SSD chunked selective-scan forward for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library libssd.so (hand-written HIP kernels); ``forward`` is its
Python binding. The library is loaded on first use and must have been built beforehand.
"""

from .libssd import SSDError, forward, load, status_string, version  # noqa: F401

__all__ = ["forward", "load", "status_string", "version", "SSDError"]
