"""Paged sliding-window KV cache and paged attention for MI355X (gfx950).

The work happens in libkvc.so (C ABI, include/kvc.h): a C++ host page manager
and HIP kernels for the K/V scatter, the bf16 MFMA paged attention and the
split merge.  This package is the thin Python binding over it; PyTorch is
used for device memory and streams only.  Importing the package does not load
the library; the first call does, and raises if it has not been built.
"""
from ._lib import KvcError, NoUndo, OutOfPages, lib  # noqa: F401
from .cache import KvCache, attend_batch, attend_batch_workspace_bytes, shared_pool_caches  # noqa: F401
from .attention import paged_attention, merge_partials  # noqa: F401
from .windowed import WindowedStream  # noqa: F401
