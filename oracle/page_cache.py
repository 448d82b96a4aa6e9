"""Oracle page cache: pool, free list, scale / window / special streams (test infrastructure).

Follows "LingBot-Map Paged KV Cache", section 2 (the cache manager cuts each
layer's KV into fixed-size pages held in two logical streams and three page
types: scale pages that are never evicted, sliding-window patch pages that go
back to a free list once outside the window and are reused by the next frame,
and append-only special pages that pack 42 frames of 6 special tokens per
256-slot page; the visible table is scale -> window -> special and the partly
filled last page is described by its length) and section 3 (a non-keyframe is
appended, attended and then rolled back).  The chunked form follows "vLLM-Omni
RFC #2727: Reconstruction Engine", section 1 and section 2.3 (frames grouped
into chunks; global attention over the most recent sliding_window_num chunks;
sliding_window_num = 1 gives independent chunks, infinity gives full global
attention).

Readings where the pages are silent or at odds (the same list is kept with the
design notes):
  R1  Special packing: frame-aligned by default (a page holds floor(page/X)
      frames, 42 for X = 6, so every full special page holds 252 tokens and
      page lengths are passed per page); "contiguous" packs tokens across page
      boundaries and is a create option.
  R2  The window counts units (frames or chunks) including the one just
      appended; eviction happens after all pops of the same append.
  R3  Free list: LIFO stack, initially ordered so pops return 0, 1, 2, ...;
      an evicted unit's pages are pushed in reverse so a later pop returns its
      first page first; a unit's patch pops precede the special pop.
  R4  Table order inside a stream: scale units chronologically, window units
      oldest to newest, special pages in opening order.
  R5  Every unit, scale units included, sends its special tokens to the
      special stream.
  R6  Rollback is single level and undoes the last append exactly (pages,
      lists, special fill, free-stack order).
  R7  Keyframes: t < S or (t - S) mod N == 0.
  R8  Unbounded window when window_units <= 0.

Pool arrays hold the exact input bit patterns (uint16 for bf16, float32 for
fp32) in a natural [page][head][slot][dim] layout for both K and V; this layout
is the oracle's own and is unrelated to the device pools.
"""
from __future__ import annotations

import collections
import dataclasses
from typing import List, Optional, Tuple

import numpy as np

from .attention import bf16_bits_to_f64
from .fp8 import dequantize_rows, quantize_rows

FRAME_ALIGNED = 0
CONTIGUOUS = 1


class OutOfPages(RuntimeError):
    pass


class NoUndo(RuntimeError):
    pass


@dataclasses.dataclass
class OracleConfig:
    num_heads: int
    head_dim: int
    page_size: int = 256
    patch_tokens: int = 256
    special_tokens: int = 6
    num_scale_units: int = 8
    window_units: int = 64          # <= 0: unbounded (R8)
    special_packing: int = FRAME_ALIGNED
    max_units: int = 1000
    num_pages: int = 0              # 0: derive with required_pages
    store_dtype: str = "bf16"       # "bf16" -> uint16 patterns, "f32" -> float32, "fp8" -> E4M3 codes + exponents

    @property
    def unit_pages(self) -> int:
        return -(-self.patch_tokens // self.page_size)

    @property
    def frames_per_special_page(self) -> int:
        # 256 slots / 6 tokens -> 42 frames ("LingBot-Map Paged KV Cache", section 2).
        return self.page_size // self.special_tokens if self.special_tokens else 0


def special_pages_for(cfg: OracleConfig, units: int) -> int:
    if cfg.special_tokens == 0 or units <= 0:
        return 0
    if cfg.special_packing == FRAME_ALIGNED:
        f = cfg.frames_per_special_page
        return -(-units // f)
    return -(-(units * cfg.special_tokens) // cfg.page_size)


def required_pages(cfg: OracleConfig) -> int:
    """Pages needed so that max_units appends never run out.

    A bounded window holds S + W units; one more unit is popped before the
    oldest is evicted (R2), so S + W + 1 units at most.
    """
    u = cfg.unit_pages
    if cfg.window_units > 0:
        units = min(cfg.max_units, cfg.num_scale_units + cfg.window_units + 1)
    else:
        units = cfg.max_units
    return units * u + special_pages_for(cfg, cfg.max_units)


def is_keyframe(t: int, num_scale: int, interval: int) -> bool:
    """Keyframe rule R7 ("LingBot-Map Paged KV Cache", section 3: KV kept every N frames)."""
    if interval <= 1 or t < num_scale:
        return True
    return (t - num_scale) % interval == 0


@dataclasses.dataclass
class _Undo:
    unit: List[int]
    evicted: Optional[List[int]]
    new_special: List[int]
    prev_fill: int
    to_scale: bool


class OracleCache:
    """One layer's paged KV cache with the policy of the module docstring."""

    def __init__(self, cfg: OracleConfig, with_pool: bool = True):
        if cfg.page_size <= 0 or cfg.patch_tokens <= 0 or cfg.num_heads <= 0 or cfg.head_dim <= 0:
            raise ValueError("bad config")
        if cfg.special_tokens < 0 or cfg.special_tokens > cfg.page_size:
            raise ValueError("special_tokens must be in [0, page_size]")
        self.cfg = cfg
        self.num_pages = cfg.num_pages or required_pages(cfg)
        self.with_pool = with_pool
        dt = {"bf16": np.uint16, "f32": np.float32, "fp8": np.uint8}[cfg.store_dtype]
        if with_pool:
            shape = (self.num_pages, cfg.num_heads, cfg.page_size, cfg.head_dim)
            self.k_pool = np.zeros(shape, dt)
            self.v_pool = np.zeros(shape, dt)
            if cfg.store_dtype == "fp8":
                # per-(token, head) row exponents of the FP8 pages (oracle/fp8.py)
                self.k_exp = np.zeros(shape[:3], np.int8)
                self.v_exp = np.zeros(shape[:3], np.int8)
        self.reset()

    # -- state ---------------------------------------------------------------
    def reset(self) -> None:
        """Empty cache; free stack ordered so that pops return 0, 1, 2, ... (R3)."""
        self.free: List[int] = list(range(self.num_pages - 1, -1, -1))  # top = end
        self.scale_units: List[List[int]] = []
        self.window: collections.deque = collections.deque()
        self.special_pages: List[int] = []
        self.fill = 0          # frames (frame-aligned) or tokens (contiguous) in the last special page
        self.n = 0             # units cached
        self.undo: Optional[_Undo] = None

    def state(self) -> dict:
        return {
            "free": list(self.free),
            "scale_pages": [p for u in self.scale_units for p in u],
            "window_pages": [p for u in self.window for p in u],
            "window_units": len(self.window),
            "special_pages": list(self.special_pages),
            "special_fill": self.fill,
            "num_units": self.n,
            "has_undo": self.undo is not None,
        }

    def patch_page_count(self) -> int:
        return sum(len(u) for u in self.scale_units) + sum(len(u) for u in self.window)

    # -- append ----------------------------------------------------------------
    def _special_slots(self) -> Tuple[int, List[Tuple[int, int]]]:
        """(new pages needed, [(page index in special stream, slot)] for each special token)."""
        cfg = self.cfg
        x = cfg.special_tokens
        if x == 0:
            return 0, []
        npg = len(self.special_pages)
        if cfg.special_packing == FRAME_ALIGNED:
            f = cfg.frames_per_special_page
            if npg == 0 or self.fill == f:
                return 1, [(npg, j) for j in range(x)]
            return 0, [(npg - 1, x * self.fill + j) for j in range(x)]
        # contiguous: tokens fill the last page, the rest go to one new page (x <= page)
        slots = []
        page_idx, pos = (npg - 1, self.fill) if npg else (-1, cfg.page_size)
        new = 0
        for _ in range(x):
            if pos == cfg.page_size:      # current page full (or none yet): open the next one
                page_idx = npg + new
                new += 1
                pos = 0
            slots.append((page_idx, pos))
            pos += 1
        return new, slots

    def append(self, k_unit: Optional[np.ndarray] = None, v_unit: Optional[np.ndarray] = None) -> None:
        """Append one unit ("LingBot-Map Paged KV Cache", section 2; RFC #2727, section 3.3 data flow).

        k_unit, v_unit: [patch_tokens + special_tokens, H, d] in the store dtype,
        patch tokens first.  Raises OutOfPages with the state unchanged.
        """
        cfg = self.cfg
        u = cfg.unit_pages
        new_special, sslots = self._special_slots()
        if len(self.free) < u + new_special:
            raise OutOfPages(f"need {u + new_special} pages, {len(self.free)} free")
        if self.with_pool:
            t = cfg.patch_tokens + cfg.special_tokens
            if k_unit is None or v_unit is None:
                raise ValueError("pool-backed cache needs K and V")
            assert k_unit.shape == (t, cfg.num_heads, cfg.head_dim), k_unit.shape
            assert v_unit.shape == k_unit.shape
        # patch pages first, then the special page (R3)
        unit = [self.free.pop() for _ in range(u)]
        opened = [self.free.pop() for _ in range(new_special)]
        prev_fill = self.fill
        self.special_pages.extend(opened)
        if self.with_pool:
            fp8 = cfg.store_dtype == "fp8"
            if fp8:
                # bf16 input rows quantised per (token, head) as they are appended
                kc, ke = quantize_rows(bf16_bits_to_f64(k_unit))
                vc, ve = quantize_rows(bf16_bits_to_f64(v_unit))
            else:
                kc, vc = k_unit, v_unit

            def put(pg, slot, i):
                self.k_pool[pg, :, slot, :] = kc[i]
                self.v_pool[pg, :, slot, :] = vc[i]
                if fp8:
                    self.k_exp[pg, :, slot] = ke[i]
                    self.v_exp[pg, :, slot] = ve[i]

            for i in range(cfg.patch_tokens):
                put(unit[i // cfg.page_size], i % cfg.page_size, i)
            for j, (pidx, slot) in enumerate(sslots):
                put(self.special_pages[pidx], slot, cfg.patch_tokens + j)
        if cfg.special_tokens:
            if cfg.special_packing == FRAME_ALIGNED:
                self.fill = 1 if new_special else self.fill + 1
            else:
                self.fill = sslots[-1][1] + 1
        to_scale = self.n < cfg.num_scale_units
        evicted = None
        if to_scale:
            self.scale_units.append(unit)
        else:
            self.window.append(unit)
            if cfg.window_units > 0 and len(self.window) > cfg.window_units:
                evicted = self.window.popleft()
                for p in reversed(evicted):
                    self.free.append(p)
        self.undo = _Undo(unit, evicted, opened, prev_fill, to_scale)
        self.n += 1

    # -- rollback ------------------------------------------------------------
    def rollback(self) -> None:
        """Undo the last append exactly ("LingBot-Map Paged KV Cache", section 3; reading R6)."""
        ud = self.undo
        if ud is None:
            raise NoUndo("no append to roll back")
        if ud.evicted is not None:
            got = [self.free.pop() for _ in ud.evicted]
            assert got == ud.evicted, (got, ud.evicted)
            self.window.appendleft(ud.evicted)
        for p in reversed(ud.new_special):
            assert self.special_pages[-1] == p
            self.special_pages.pop()
            self.free.append(p)
        self.fill = ud.prev_fill
        self.n -= 1
        if ud.to_scale:
            assert self.scale_units[-1] == ud.unit
            self.scale_units.pop()
        else:
            assert self.window[-1] == ud.unit
            self.window.pop()
        for p in reversed(ud.unit):
            self.free.append(p)
        self.undo = None

    # -- visible table -------------------------------------------------------
    def visible_table(self) -> Tuple[List[int], List[int]]:
        """Pages in the order scale -> window -> special with per-page valid lengths.

        "LingBot-Map Paged KV Cache", section 2: the visible table lists scale
        pages, then window pages, then special pages last; the partly filled
        last page is described by its length, so no mask is needed.
        """
        cfg = self.cfg
        ids: List[int] = []
        lens: List[int] = []
        tail = cfg.patch_tokens - cfg.page_size * (cfg.unit_pages - 1)
        for unit in list(self.scale_units) + list(self.window):
            for i, p in enumerate(unit):
                ids.append(p)
                lens.append(tail if i == len(unit) - 1 else cfg.page_size)
        ns = len(self.special_pages)
        for i, p in enumerate(self.special_pages):
            ids.append(p)
            if cfg.special_packing == FRAME_ALIGNED:
                full = cfg.special_tokens * cfg.frames_per_special_page
                lens.append(cfg.special_tokens * self.fill if i == ns - 1 else full)
            else:
                lens.append(self.fill if i == ns - 1 else cfg.page_size)
        return ids, lens

    def last_page_len(self) -> int:
        _, lens = self.visible_table()
        return lens[-1] if lens else 0

    # -- gather --------------------------------------------------------------
    def gather(self, ids: Optional[List[int]] = None, lens: Optional[List[int]] = None):
        """Visible K and V as [H, Lk, d] arrays in the store dtype, in table order.

        FP8 caches return the dequantised values (float64, code * 2^e)."""
        if ids is None:
            ids, lens = self.visible_table()
        cfg = self.cfg
        if cfg.store_dtype == "fp8":
            if not ids:
                e = np.zeros((cfg.num_heads, 0, cfg.head_dim))
                return e, e.copy()
            ks = [dequantize_rows(self.k_pool[p, :, :n, :], self.k_exp[p, :, :n]) for p, n in zip(ids, lens)]
            vs = [dequantize_rows(self.v_pool[p, :, :n, :], self.v_exp[p, :, :n]) for p, n in zip(ids, lens)]
            return np.concatenate(ks, axis=1), np.concatenate(vs, axis=1)
        dt = self.k_pool.dtype
        if not ids:
            e = np.zeros((cfg.num_heads, 0, cfg.head_dim), dt)
            return e, e.copy()
        ks = [self.k_pool[p, :, :n, :] for p, n in zip(ids, lens)]
        vs = [self.v_pool[p, :, :n, :] for p, n in zip(ids, lens)]
        return np.concatenate(ks, axis=1), np.concatenate(vs, axis=1)
