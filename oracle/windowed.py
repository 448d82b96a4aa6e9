"""Windowed inference over the oracle cache (test infrastructure).

"LingBot-Map Paged KV Cache", section 4: the KV cache is reset once per
window of `window_slots` stored units (KV slots, not raw frames), and
adjacent windows share `overlap` units.  Reading: when a window is full, the
next append first resets the cache and re-appends the last `overlap` kept
units of the finished window (oldest first, the K/V that were appended);
non-kept units (keyframe skips) take no slot and are rolled back.

Pinned by tests/test_oracle_windowed.py: a 15-frame trace derived by hand
from these readings (tests/golden/windowed_trace.json: restart frames, tables
and the frame every visible token comes from), which planted mistakes (a
restart one slot late or early, the shared units re-appended newest first,
dropped units entering the shared ring or taking slots) each fail.
"""
from __future__ import annotations

import collections

from .page_cache import OracleCache


class OracleWindowed:
    def __init__(self, cache: OracleCache, window_slots: int, overlap: int):
        self.cache = cache
        self.window_slots = window_slots
        self.overlap = overlap
        self.slots = 0
        self.windows = 0
        self.kept = collections.deque(maxlen=overlap if overlap > 0 else None)  # (k, v) of recent kept units
        self.pending = None

    def append(self, k=None, v=None) -> bool:
        restarted = False
        if self.slots >= self.window_slots:
            self.cache.reset()
            shared = list(self.kept) if self.overlap > 0 else []
            for kk, vv in shared:
                self.cache.append(kk, vv)
            self.slots = len(shared)
            self.windows += 1
            restarted = True
        self.cache.append(k, v)
        self.pending = (k, v)
        return restarted

    def keep(self) -> None:
        self.slots += 1
        if self.overlap > 0:
            self.kept.append(self.pending)
        self.pending = None

    def drop(self) -> None:
        self.pending = None
        self.cache.rollback()
