"""libssd: Mamba-2 SSD chunked selective-scan forward for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library libssd.so (hand-written HIP kernels); ``forward`` (the
chunked forward), ``backward`` (its gradients) and ``step`` (one recurrent decode step) are its
Python bindings. The library is loaded on first use and must have been built beforehand.
"""

from .libssd import SSDError, backward, forward, load, status_string, step, version  # noqa: F401

__all__ = ["forward", "backward", "step", "load", "status_string", "version", "SSDError"]
