"""Windowed inference over one cache ("LingBot-Map Paged KV Cache", section 4).

For very long streams the cache is restarted once per window: a window holds
`window_slots` kept units (KV slots, i.e. stored keyframes, not raw frames),
and adjacent windows share `overlap` units.  The restart policy (reset, then
re-append the last `overlap` kept units oldest first, with their appended
K/V) runs in libkvc.so (kvc_windowed_*); this module allocates the two device
rings that hold the shared units' K/V and marshals the calls.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional

from . import _lib as L
from .cache import KvCache, current_stream_ptr, torch_dtype


class WindowedStream:
    """Windowed appends over `cache`: append(k, v), then keep() or drop() the unit."""

    def __init__(self, cache: KvCache, window_slots: int = 128, overlap: int = 16):
        lib = L.lib()
        self.cache = cache
        self.window_slots = window_slots
        self.overlap = overlap
        self._ring = (None, None)
        nb = C.c_size_t()
        L.check(lib.kvc_windowed_ring_bytes(cache.handle, overlap, C.byref(nb)), "kvc_windowed_ring_bytes")
        if nb.value:
            import torch
            shp = (overlap + 1, cache.unit_tokens, cache.num_heads, cache.head_dim)  # shared units + a free slot
            dt = torch_dtype(cache.dtype)
            self._ring = tuple(torch.empty(shp, dtype=dt, device=cache.k_pool.device) for _ in range(2))
            assert self._ring[0].numel() * self._ring[0].element_size() == nb.value
        kr, vr = (None if r is None else r.data_ptr() for r in self._ring)
        h = C.c_void_p()
        L.check(lib.kvc_windowed_create(cache.handle, window_slots, overlap, kr, vr, C.byref(h)),
                "kvc_windowed_create")
        self._h = h
        self._pending = None  # keeps the appended tensors alive until keep()/drop()

    def close(self) -> None:
        if getattr(self, "_h", None):
            L.lib().kvc_windowed_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _state(self) -> L.KvcWindowedState:
        st = L.KvcWindowedState()
        L.check(L.lib().kvc_windowed_get_state(self._h, C.byref(st)), "kvc_windowed_get_state")
        return st

    @property
    def slots(self) -> int:
        return self._state().slots

    @property
    def windows(self) -> int:
        return self._state().windows

    def append(self, k=None, v=None, stream: Optional[int] = None) -> bool:
        """Append one unit; returns True when this append started a new window."""
        c = self.cache
        if c.device is None:
            if k is not None or v is not None:
                raise ValueError("host-only cache takes no K/V")
            kp = vp = s = None
        else:
            c._check_unit(k, "k")
            c._check_unit(v, "v")
            kp, vp = k.data_ptr(), v.data_ptr()
            s = current_stream_ptr(k.device) if stream is None else stream
        r = C.c_int32()
        L.check(L.lib().kvc_windowed_append(self._h, kp, vp, s, C.byref(r)), "kvc_windowed_append")
        self._pending = (k, v)
        return bool(r.value)

    def keep(self, stream: Optional[int] = None) -> None:
        """The last unit is a keyframe: it stays, takes one slot, and its ring slot (written by the append)
        becomes one of the shared units."""
        s = None
        if self.cache.device is not None:
            s = current_stream_ptr(self.cache.k_pool.device) if stream is None else stream
        L.check(L.lib().kvc_windowed_keep(self._h, s), "kvc_windowed_keep")
        self._pending = None

    def drop(self) -> None:
        """The last unit is not kept (keyframe skip): roll it back."""
        L.check(L.lib().kvc_windowed_drop(self._h), "kvc_windowed_drop")
        self._pending = None
