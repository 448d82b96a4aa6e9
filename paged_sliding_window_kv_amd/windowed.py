"""Windowed inference over one cache ("LingBot-Map Paged KV Cache", section 4).

For very long streams the cache is restarted once per window: a window holds
`window_slots` kept units (KV slots, i.e. stored keyframes, not raw frames),
and adjacent windows share `overlap` units so that the next window starts
aligned with the previous one.  Reading used (the page fixes neither the
restart order nor where the shared units' K/V come from): when a window is
full, the next append first resets the cache and re-appends the last
`overlap` kept units of the finished window, oldest first.  Their K/V are the
ones that were appended (in the model they would be recomputed in the new
window).  The driver keeps those units in a fixed device ring, allocated
once, so device memory stays constant however long the stream runs.

Marshalling only: reset, append and rollback run in libkvc.so.
"""
from __future__ import annotations

from typing import Optional

from .cache import KvCache


class WindowedStream:
    """Windowed appends over `cache`: append(k, v), then keep() or drop() the unit."""

    def __init__(self, cache: KvCache, window_slots: int = 128, overlap: int = 16):
        if window_slots < 1 or not (0 <= overlap < window_slots):
            raise ValueError("need window_slots >= 1 and 0 <= overlap < window_slots")
        self.cache = cache
        self.window_slots = window_slots
        self.overlap = overlap
        self.slots = 0          # kept units in the current window
        self.windows = 0        # restarts so far
        self._pending = None    # (k, v) of the unit appended last, until keep()/drop()
        self._ring = None
        self._ring_len = 0      # kept units in the ring (at most `overlap`)
        self._ring_head = 0     # next ring slot to write
        if cache.device is not None and overlap > 0:
            import torch
            shp = (overlap, cache.unit_tokens, cache.num_heads, cache.head_dim)
            dt = cache.k_pool.dtype
            self._ring = (torch.empty(shp, dtype=dt, device=cache.k_pool.device),
                          torch.empty(shp, dtype=dt, device=cache.k_pool.device))

    def _restart(self, stream: Optional[int]) -> None:
        self.cache.reset()
        n = self._ring_len
        for j in range(n):
            slot = (self._ring_head - n + j) % self.overlap
            if self._ring is None:
                self.cache.append(stream=stream)
            else:
                self.cache.append(self._ring[0][slot], self._ring[1][slot], stream=stream)
        self.slots = n
        self.windows += 1

    def append(self, k=None, v=None, stream: Optional[int] = None) -> bool:
        """Append one unit; returns True when this append started a new window."""
        if self._pending is not None:
            raise RuntimeError("keep() or drop() the previous unit first")
        restarted = False
        if self.slots >= self.window_slots:
            self._restart(stream)
            restarted = True
        if self.cache.device is None:
            self.cache.append()
        else:
            self.cache.append(k, v, stream=stream)
        self._pending = (k, v)
        return restarted

    def keep(self) -> None:
        """The last unit is a keyframe: it stays, takes one slot and enters the overlap ring."""
        if self._pending is None:
            raise RuntimeError("nothing appended")
        k, v = self._pending
        self._pending = None
        self.slots += 1
        if self.overlap > 0:
            if self._ring is not None:
                self._ring[0][self._ring_head].copy_(k)
                self._ring[1][self._ring_head].copy_(v)
            self._ring_head = (self._ring_head + 1) % self.overlap
            self._ring_len = min(self._ring_len + 1, self.overlap)

    def drop(self) -> None:
        """The last unit is not kept (keyframe skip): roll it back."""
        if self._pending is None:
            raise RuntimeError("nothing appended")
        self._pending = None
        self.cache.rollback()
